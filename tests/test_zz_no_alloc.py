"""The allocation-free prepare entry point (gptq_prepare_noalloc), called
through the C ABI, against gptq_prepare with a caller workspace: the same
kernels on the same inputs, so U, perm, dead and info must agree bit for bit
(stronger than the parity bar; U is also checked against the oracle's factor
of the same H within 1e-4).  Three calls in a row on one device share the one
static scratch array: the largest supported d first, then smaller ones with
act-order and a dead input, so stale scratch contents from a bigger call must
not leak into a smaller one."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import gptq_ref as ref

pytestmark = pytest.mark.gpu


def _h_from_x(d, n, seed, dead_col=None):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    X = torch.randn((n, d), generator=g, device="cuda")
    X[:, : max(1, d // 100)] *= 20.0                     # a few loud channels
    if dead_col is not None:
        X[:, dead_col] = 0.0
    return 2.0 * (X.T @ X)


def _run(name, H, act_order, ws=None):
    from post_weight_quantization_23_amd import _lib
    d = H.shape[0]
    perm = torch.full((d,), -7, dtype=torch.int32, device="cuda")
    dead = torch.full((d,), 9, dtype=torch.uint8, device="cuda")
    info = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: C.c_void_p(t.data_ptr())
    if name == "gptq_prepare":
        _lib.call(name, p(H), d, C.c_float(0.01), act_order, p(perm), p(dead), p(info), p(ws), ws.numel(), stream)
    else:
        _lib.call(name, p(H), d, C.c_float(0.01), act_order, p(perm), p(dead), p(info), stream)
    return perm, dead, info


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import post_weight_quantization_23_amd  # noqa: F401  (loads the library, raises if missing)


def test_prepare_noalloc_matches_prepare_on_consecutive_calls():
    from post_weight_quantization_23_amd import _lib
    cases = [(4096, 0, None, 4096 + 512), (1000, 1, 17, 3000), (300, 0, 5, 1200)]
    for k, (d, ao, dead_col, n) in enumerate(cases):
        print(f"\n[no-alloc] call {k}: d={d} act_order={ao} dead={dead_col}", flush=True)
        H = _h_from_x(d, n, 100 + k, dead_col)
        need = _lib.query("gptq_prepare_workspace_size", d, ao)
        ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
        U_ws, U_na = H.clone(), H.clone()
        ref_out = _run("gptq_prepare", U_ws, ao, ws)
        na_out = _run("gptq_prepare_noalloc", U_na, ao)
        torch.cuda.synchronize()
        assert int(ref_out[2].item()) == 0 and int(na_out[2].item()) == 0
        assert torch.equal(U_ws.view(torch.int32), U_na.view(torch.int32)), "U differs from gptq_prepare"
        assert torch.equal(ref_out[0], na_out[0]) and torch.equal(ref_out[1], na_out[1])
        if dead_col is not None:
            assert int(na_out[1][dead_col].item()) == 1
        # the parity bar: the oracle's factor of the same (fp32) H
        Hh = H.double().cpu().numpy()
        Hd, perm_ref, dead_ref, _ = ref.prepare(Hh, 0.01, bool(ao))
        np.testing.assert_array_equal(na_out[0].cpu().numpy().astype(np.int64) if ao else np.arange(d),
                                      perm_ref)
        np.testing.assert_array_equal(na_out[1].cpu().numpy().astype(bool), dead_ref)
        Ur = ref.upper_cholesky_of_inverse(Hd)
        rel = np.linalg.norm(U_na.double().cpu().numpy() - Ur) / np.linalg.norm(Ur)
        print(f"  bitwise equal to gptq_prepare; U vs oracle {rel:.3g}", flush=True)
        assert rel <= 1e-4
