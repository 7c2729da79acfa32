"""The seeded input generators: determinism, shapes and the stated structure."""
import numpy as np

from synth import inputs as S


def test_host_generation_is_seeded_and_shaped():
    a = S.activations_host(512, 64, "t4", outliers=4, gain=30.0, wid=9)
    b = S.activations_host(512, 64, "t4", outliers=4, gain=30.0, wid=9)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (512, 64) and a.dtype == np.float32
    loud = S.outlier_channels(64, 4, 9)
    quiet = np.setdiff1d(np.arange(64), loud)
    assert np.median(np.abs(a[:, loud])) > 10 * np.median(np.abs(a[:, quiet]))


def test_relu_sparse_fraction_and_bf16_values():
    x = S.activations_host(4096, 32, "t4_relu", dtype="bfloat16", wid=4)
    frac = np.mean(x == 0)
    assert 0.57 < frac < 0.63
    # bf16-representable: the low 16 bits of every float32 are zero
    assert np.all((x.view(np.uint32) & 0xFFFF) == 0)


def test_workload_table_matches_stated_shapes():
    w = S.WORKLOADS["llama7b_attn_4096x4096"]
    assert (w.rows, w.cols, w.tokens, w.bits, w.groupsize, w.blocksize) == (4096, 4096, 128 * 2048, 4, 128, 128)
    t = S.WORKLOADS["tiny_fp32_128x256"]
    assert (t.rows, t.cols, t.tokens, t.groupsize, t.outliers) == (128, 256, 2048, -1, 4)
    assert round(0.005 * 4096) == S.WORKLOADS["llama7b_attn_4096x4096"].outliers
    assert round(0.001 * 49152) == S.WORKLOADS["opt175b_fc2_12288x49152"].outliers


def test_decoder_sweep_table():
    layers = S.llama7b_sweep()
    assert len(layers) == 32 * 7
    shapes = [(w.rows, w.cols) for w, _ in layers[:7]]
    assert shapes == [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    assert [i for _, i in layers] == list(range(224))          # each linear its own seed
    assert all(w.bits == 4 and w.groupsize == 128 and w.tokens == 262144 for w, _ in layers)
    assert sum(w.rows * w.cols for w, _ in layers) == 32 * (4 * 4096 * 4096 + 3 * 11008 * 4096)
