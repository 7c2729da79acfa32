"""Throughput of the GPTQ layer quantizer on one MI355X.

One step = the whole path for one layer of the named workload, with the
weights and the calibration activations already resident in HBM:
    H = 0;  H += 2 X^T X  (gptq_hessian_accumulate)
    U = chol_upper((H + damp)^{-1})  (gptq_prepare)
    codes, rulers = GPTQ column loop  (gptq_quantize_layer)
    packed words  (gptq_pack)
Prints ONE JSON line: weights/s for the whole layer (value), seconds per layer,
Hessian TFLOP/s, per-stage milliseconds, the roofline of the dominant kernel
(the Hessian SYRK, timed with HIP events on the stream it runs on), and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]
    python bench.py --copy-probe      # plain copy of known size (PMC calibration)
    python bench.py --gemv [--gemv-model llama7b|opt175b] [--fused-inputs] [--steps K] [--warmup W]
    python bench.py --hadamard [--workload NAME] [--steps K] [--warmup W]
    python bench.py --stack [--blocks B] [--steps K] [--warmup W]
    python bench.py --sweep [--sweep-blocks 32] [--rotate]
    python bench.py --hessian [--workload NAME] [--x-fill workload|uniform|zeros]

--gemv measures the dequantizing matrix-vector product over packed layers
instead: one step = one generated token (batch 1) through every linear layer
of the named model, each a separate gptq_dequant_gemv launch over its own
packed words (distinct memory, so the words come from HBM, not cache).  It
prints its own JSON line: weights/s and effective GB/s for the token, the
roofline of the largest layer's launch (HIP events around back-to-back
launches over distinct layers of that shape), the same token through bf16 /
fp16 torch matrix-vector products for comparison, and the oracle on a bounded
sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sec per layer & weights/s for GPTQ 4-bit g128 on 4096×4096; Hessian TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_syrk16_{workload}.json")
SYRK_SOURCE = os.path.join(ROOT, "post_weight_quantization_23_amd", "csrc", "syrk.hip")
GEMV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_{workload}.json")
GEMV_SOURCE = os.path.join(ROOT, "post_weight_quantization_23_amd", "csrc", "gemv.hip")
LINEAR_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_linear_{workload}.json")
LINEAR_SOURCE = os.path.join(ROOT, "post_weight_quantization_23_amd", "csrc", "linear.hip")
HADAMARD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_hadamard_{workload}.json")
HADAMARD_SOURCE = os.path.join(ROOT, "post_weight_quantization_23_amd", "csrc", "hadamard.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(workload: str, path_fmt: str = TRAFFIC_FILE, source: str = SYRK_SOURCE):
    """HBM bytes per launch of the dominant kernel from committed PMC counters,
    or None when the kernel source changed since they were taken."""
    path = path_fmt.format(workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_hash(source):
        return None
    return t.get("bytes_per_launch")


def copy_probe(nbytes: int = 1 << 30, reps: int = 5) -> None:
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {nbytes} bytes (read {nbytes}, write {nbytes} each)")


def cpu_baseline(W_dev, X_dev, w, tokens_sample=16384, rows_sample=128, cols_sample=4096):
    """The oracle as it stands, on a bounded sample, extrapolated to one layer.

    The sample: the first `cols_sample` input channels (all of them up to
    d = 4096), `tokens_sample` tokens and `rows_sample` rows.  The oracle's H
    costs tokens x d^2, its factor d^3 and its column loop rows x d^2, so the
    three measured times are scaled by those ratios."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gptq_ref as ref

    dc = min(w.cols, cols_sample)
    tokens_sample = min(tokens_sample, w.tokens)
    rows_sample = min(rows_sample, w.rows)
    X = X_dev[:tokens_sample, :dc].float().cpu().numpy()
    W = W_dev[:rows_sample, :dc].float().cpu().numpy()
    t0 = time.perf_counter()
    H = ref.hessian(X)
    t_h = time.perf_counter() - t0
    t0 = time.perf_counter()
    Hd, perm, dead, lam = ref.prepare(H, w.percdamp, w.act_order)
    U = ref.upper_cholesky_of_inverse(Hd)
    t_p = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref.gptq_quantize(W.astype(np.float64), H, w.bits, w.groupsize, w.percdamp, w.act_order, U=U)
    t_q = time.perf_counter() - t0
    fc = w.cols / dc
    scale_h = (w.tokens / tokens_sample) * fc ** 2
    scale_p = fc ** 3
    scale_q = (w.rows / rows_sample) * fc ** 2
    sec_layer = t_h * scale_h + t_p * scale_p + t_q * scale_q
    threads = [p.get("num_threads", 0) for p in threadpool_info()]
    cores = max(threads) if threads else 1
    cols_note = "" if dc == w.cols else f", the first {dc} of {w.cols} input channels"
    return {
        "value": (w.rows * w.cols) / sec_layer,
        "unit": "weights/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{tokens_sample} of {w.tokens} tokens, {rows_sample} of {w.rows} rows{cols_note}; "
                   f"H (x{scale_h:g}), factor (x{scale_p:g}), column loop (x{scale_q:g}) extrapolated by "
                   f"tokens*d^2, d^3, rows*d^2; measured s: H {t_h:.2f}, prepare {t_p:.2f}, loop {t_q:.2f}"),
        "sec_per_layer_extrapolated": sec_layer,
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


GEMV_MODELS = {
    # name: (blocks, [(layer, rows, cols), ...] per block, bits, groupsize, x dtype)
    "llama7b": (32, [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                     ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)],
                4, 128, "bfloat16"),
    "opt175b": (96, [("q", 12288, 12288), ("k", 12288, 12288), ("v", 12288, 12288), ("out", 12288, 12288),
                     ("fc1", 49152, 12288), ("fc2", 12288, 49152)],
                3, 128, "float16"),
}


# The same models with the projections that read one input stored as one
# matrix (rows concatenated): q, k and v; gate and up (Llama); fc1 alone and
# q, k, v (OPT).  One launch then serves what were two or three.
GEMV_FUSED = {
    "llama7b": [("qkv", 3 * 4096, 4096), ("o", 4096, 4096), ("gate_up", 2 * 11008, 4096), ("down", 4096, 11008)],
    "opt175b": [("qkv", 3 * 12288, 12288), ("out", 12288, 12288), ("fc1", 49152, 12288), ("fc2", 12288, 49152)],
}


def gemv_bytes(r: int, c: int, bits: int, groupsize: int, xbytes: int = 2) -> int:
    """Algorithmic HBM bytes of one launch: packed words, fp32 scales and int32
    zeros (one per row and group), x once, y once."""
    G = (c + groupsize - 1) // groupsize if 0 < groupsize < c else 1
    return r * c * bits // 8 + r * G * 8 + c * xbytes + r * 4


def gemv_cpu_baseline(layers, bits, groupsize, xs, total_weights, codes_sample=8_000_000):
    """The oracle's dequantizing product on a few rows of each layer shape
    (about codes_sample codes in all), extrapolated to the token by weight
    count."""
    import numpy as np

    from oracle import gptq_ref as ref
    cols = sum({(L["r"], L["c"]): L["c"] for L in layers}.values())
    rows_sample = max(8, codes_sample // cols)
    seen, t_sum, w_sum = set(), 0.0, 0
    for L in layers:
        key = (L["r"], L["c"])
        if key in seen:
            continue
        seen.add(key)
        words = L["packed"][:rows_sample].cpu().numpy()
        sc = L["scales"][:rows_sample].cpu().numpy()
        zr = L["zeros"][:rows_sample].cpu().numpy()
        x = xs[L["c"]].float().cpu().numpy()
        g = np.arange(L["c"]) // groupsize
        t0 = time.perf_counter()
        ref.dequant_gemv(words, bits, L["c"], sc, zr, g, x)
        t_sum += time.perf_counter() - t0
        w_sum += rows_sample * L["c"]
    rate = w_sum / t_sum
    return {
        "value": rate,
        "unit": "weights/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{rows_sample} rows of each distinct layer shape ({w_sum} weights, {t_sum:.2f} s); "
                   f"single-threaded Python unpacking; extrapolated: "
                   f"{total_weights / rate:.1f} s per token"),
    }


def bench_gemv(args) -> int:
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    blocks, shapes, bits, gs, xdt = GEMV_MODELS[args.gemv_model]
    if args.fused_inputs:
        shapes = GEMV_FUSED[args.gemv_model]
    tag = f"{args.gemv_model}_decode_token_{bits}bit_g{gs}" + ("_fused_inputs" if args.fused_inputs else "")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xdtype = getattr(torch, xdt)
    gen = torch.Generator(device=dev)
    gen.manual_seed(S.torch_seed(900, 0, 3))
    layers = []
    log(f"building {blocks} x {len(shapes)} packed layers of {args.gemv_model} ({bits}-bit, g{gs}) ...")
    for b in range(blocks):
        for name, r, c in shapes:
            G = S.n_groups(c, gs)
            words = torch.randint(-2 ** 31, 2 ** 31, (r, c * bits // 32), generator=gen, device=dev,
                                  dtype=torch.int32).view(torch.uint32)
            scales = (0.02 * 5.0 / (2 ** bits - 1)) * torch.exp(
                0.3 * torch.randn((r, G), generator=gen, device=dev))
            zeros = torch.randint(0, 2 ** bits, (r, G), generator=gen, device=dev, dtype=torch.int32)
            layers.append({"name": f"{name}{b}", "r": r, "c": c, "packed": words, "scales": scales.float(),
                           "zeros": zeros, "y": torch.empty(r, dtype=torch.float32, device=dev)})
    xs = {}
    for _, r, c in shapes:
        if c not in xs:
            xs[c] = torch.from_numpy(S.token_host(c, 900 + c % 101, xdt, "t4", outliers=max(1, c // 200),
                                                  gain=30.0)).to(dev).to(xdtype)
    torch.cuda.synchronize()
    total_w = sum(L["r"] * L["c"] for L in layers)
    total_b = sum(gemv_bytes(L["r"], L["c"], bits, gs) for L in layers)
    log(f"{len(layers)} layers, {total_w / 1e9:.2f} G weights, {total_b / 1e9:.2f} GB per token")

    def token():
        for L in layers:
            q.dequant_gemv(L["packed"], L["scales"], L["zeros"], xs[L["c"]], bits, gs, out=L["y"])

    # Eager launches are bound by Python's per-call cost (~10 us); the token
    # is captured once in a HIP graph and replayed, as a decode loop would.
    token()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        token()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / 3
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_tok = e0.elapsed_time(e1) / args.steps
    log(f"token: {ms_tok:.4f} ms (graph replay, events), wall {wall * 1e3 / args.steps:.4f} ms, "
        f"eager launches {ms_eager:.4f} ms")

    # Dominant kernel: the launch shape with the most bytes per token; its
    # launches over distinct layers, back to back in one graph, bracketed by
    # events.
    by_shape = {}
    for L in layers:
        by_shape.setdefault((L["r"], L["c"]), []).append(L)
    dom = max(by_shape, key=lambda k: gemv_bytes(k[0], k[1], bits, gs) * len(by_shape[k]))
    dl = by_shape[dom]
    reps = max(1, 64 // len(dl))
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        for _ in range(reps):
            for L in dl:
                q.dequant_gemv(L["packed"], L["scales"], L["zeros"], xs[L["c"]], bits, gs, out=L["y"])
    g2.replay()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(4):
        g2.replay()
    f1.record()
    torch.cuda.synchronize()
    us_launch = f0.elapsed_time(f1) * 1e3 / (4 * reps * len(dl))
    b_launch = gemv_bytes(dom[0], dom[1], bits, gs)
    achieved = b_launch / (us_launch * 1e-6) / 1e9

    # The same token through 16-bit torch matrix-vector products (weights in
    # the activation dtype), for the pages' "faster than fp16" comparison.
    ref16 = None
    if args.gemv_model == "llama7b":
        w16 = [torch.empty((L["r"], L["c"]), dtype=xdtype, device=dev).normal_(0.0, 0.02, generator=gen)
               for L in layers]
        y16 = {r: torch.empty(r, dtype=xdtype, device=dev) for _, r, _ in shapes}

        def token16():
            for Wt, L in zip(w16, layers):
                torch.mv(Wt, xs[L["c"]], out=y16[L["r"]])

        for _ in range(2):
            token16()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            token16()
        g1.record()
        torch.cuda.synchronize()
        ms16 = g0.elapsed_time(g1) / args.steps
        ref16 = {"ms_per_token": ms16, "speedup": ms16 / ms_tok,
                 "what": f"torch.mv on {xdt} weights of the same shapes ({len(layers)} launches, distinct memory)"}
        del w16

    rec = {
        "metric": f"dequantizing GEMV, one generated token (batch 1) through {args.gemv_model}'s "
                  f"{len(layers)} linear " + ("launches (projections of one input stored as one matrix)"
                                              if args.fused_inputs else "layers") + f", {bits}-bit g{gs}: weights/s",
        "value": total_w / (ms_tok * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_tok,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 dot (codes x activations), f32 sums",
        "data": "synthetic (seeded random packed words, log-normal scales, uniform zero points, "
                "Student-t(4) activations with outlier channels)",
        "config": {"workload": tag, "layers": len(layers), "weights": total_w, "bytes_per_token": total_b,
                   "x_dtype": xdt, "fused_inputs": bool(args.fused_inputs)},
        "effective_GBps": total_b / (ms_tok * 1e-3) / 1e9,
        "ms_per_token_eager_launches": ms_eager,
        "roofline": {
            "kernel": f"dq_gemv_kernel<{bits},*> on the {dom[0]}x{dom[1]} layers ({len(dl)} per token; "
                      f"{4 * reps * len(dl)} launches back to back in graph replays between HIP events, "
                      f"gaps between launches included)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": load_traffic(tag, GEMV_TRAFFIC_FILE, GEMV_SOURCE),
            "algorithmic_bytes_per_launch": b_launch,
            "us_per_launch": us_launch,
        },
        "fp16_reference": ref16,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        rec["cpu_baseline"] = gemv_cpu_baseline(layers, bits, gs, xs, total_w)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_hadamard(args) -> int:
    """Hadamard pre-rotation of the workload's calibration activations (one
    step = the whole X, rotated into a second buffer of the same dtype)."""
    import numpy as np
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    w = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _, X = S.workload_device(w, device=dev)
    Xr = torch.empty_like(X)
    block = min(X.shape[1] & -X.shape[1], 8192)
    for _ in range(max(1, args.warmup)):
        q.hadamard_rotate(X, out=Xr)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        q.hadamard_rotate(X, out=Xr)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * X.numel() * X.element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": f"Hadamard pre-rotation of the calibration activations ({w.tokens}x{w.cols} {w.x_dtype}, "
                  f"block {block}): GB/s",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 butterflies, " + w.x_dtype + " in/out", "data": "synthetic (the workload's activations)",
        "config": {"workload": w.name + "_hadamard", "rows": w.tokens, "cols": w.cols, "block": block},
        "roofline": {"kernel": f"fwht_kernel<{block.bit_length() - 1},*> (HIP events around back-to-back launches)",
                     "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": load_traffic(w.name + "_hadamard", HADAMARD_TRAFFIC_FILE, HADAMARD_SOURCE),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        from oracle import gptq_ref as ref
        sample = 8192
        A = X[:sample].float().cpu().numpy()
        t0 = time.perf_counter()
        ref.hadamard_rotate(A, block)
        t = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": 2 * sample * w.cols * X.element_size() / t / 1e9, "unit": "GB/s",
                               "cores": int(torch.get_num_threads()), "kind": "oracle",
                               "sample": f"{sample} of {w.tokens} rows ({t:.2f} s), float64 matrix product per block"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def bench_stack(args) -> int:
    """Layer-by-layer GPTQ over Llama-7B-shaped gated MLP blocks (d 4096,
    h 11008), 4-bit g128, calibrated on 262144 bf16 tokens: one step = the
    whole stack (every Hessian, factor, quantization and quantized forward)."""
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from post_weight_quantization_23_amd import gptq
    from synth import inputs as S

    w = S.WORKLOADS["llama7b_attn_4096x4096"]
    d, h, nb = w.cols, 11008, args.blocks
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _, X0 = S.workload_device(w, device=dev)
    blocks = [(S.weights_device(h, d, 7, 3 * k, "bfloat16", device=dev),
               S.weights_device(h, d, 7, 3 * k + 1, "bfloat16", device=dev),
               S.weights_device(d, h, 7, 3 * k + 2, "bfloat16", device=dev)) for k in range(nb)]
    torch.cuda.synchronize()

    def step():
        return q.quantize_mlp_stack(X0, blocks, bits=4, groupsize=128, percdamp=0.01, act_order=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    weights = nb * 3 * h * d
    # the quantized forward on the block's largest product, timed alone: the
    # weights rounded once to bf16 (as the stack runs it), and for comparison
    # the same call on fp32 weights (rounded inside the kernel)
    Wh = torch.empty((h, d), dtype=torch.float32, device=dev).normal_(0.0, 0.02)
    Wh16 = gptq.round16(Wh, torch.bfloat16)
    Y = torch.empty((w.tokens, h), dtype=torch.bfloat16, device=dev)

    def time_fwd(Wt):
        gptq.linear_forward(X0, Wt, out=Y)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(3):
            gptq.linear_forward(X0, Wt, out=Y)
        f1.record()
        torch.cuda.synchronize()
        return f0.elapsed_time(f1) / 3

    fwd_ms = time_fwd(Wh16)
    fwd_f32_ms = time_fwd(Wh)
    flops = 2.0 * w.tokens * d * h
    tfl = flops / (fwd_ms * 1e-3) / 1e12
    rec = {
        "metric": f"layer-by-layer GPTQ over {nb} gated MLP blocks (d {d}, h {h}; gate, up, down), "
                  f"{w.tokens} bf16 calibration tokens, 4-bit g128: weights/s",
        "value": weights / (ms * 1e-3), "unit": "weights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 MFMA (Hessians, forwards), fp32 (factor, quantizer)",
        "data": "synthetic (seeded N(0, 0.02^2) weights, Student-t(4) activations with outlier channels)",
        "config": {"workload": "llama7b_mlp_stack", "blocks": nb, "d": d, "h": h, "tokens": w.tokens,
                   "bits": 4, "groupsize": 128},
        "roofline": {"kernel": "linear_kernel<bf16, 16-bit weights> (quantized forward 262144 x 4096 -> 11008, "
                               "HIP events)",
                     "bound": "mfma", "achieved": tfl, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tfl / PEAK_BF16_TFLOPS,
                     "traffic": load_traffic("llama7b_mlp_forward_262144x4096x11008", LINEAR_TRAFFIC_FILE, LINEAR_SOURCE),
                     "algorithmic_flops_per_launch": flops,
                     "ms_per_launch": fwd_ms, "ms_per_launch_fp32_weights": fwd_f32_ms},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


GRID_VARIANTS = [
    # name, bits, groupsize, symmetric
    ("asym_b4_g128", 4, 128, False),
    ("sym_b4_g128", 4, 128, True),
    ("asym_b2_g128", 2, 128, False),
    ("asym_b3_g128", 3, 128, False),
    ("asym_b8_g128", 8, 128, False),
    ("asym_b4_g64", 4, 64, False),
    ("asym_b4_g32", 4, 32, False),
    ("asym_b4_row", 4, -1, False),
]


def bench_grid(args) -> int:
    """The quantize stage (ruler fits, the column loop with its block repairs
    and the deferred products) on the 4096 x 4096 layer for every grid
    variant, on one factor U of that layer's Hessian."""
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    w = S.WORKLOADS["llama7b_attn_4096x4096"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W, X = S.workload_device(w, device=dev)
    r, c = w.rows, w.cols
    U = torch.zeros((c, c), dtype=torch.float32, device=dev)
    q.hessian_accumulate(U, X)
    perm, dead, _ = q.prepare(U, w.percdamp, False)
    del X
    ws = q.Workspace()
    res = {}
    steps = max(1, args.steps)
    for name, bits, gs, sym in GRID_VARIANTS:
        def one():
            return q.quantize_layer(W, U, perm, dead, bits=bits, groupsize=gs, blocksize=w.blocksize, ws=ws,
                                    sym=sym)
        for _ in range(max(1, args.warmup)):
            one()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            one()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"bits": bits, "groupsize": gs, "sym": sym, "ms": e0.elapsed_time(e1) / steps}
        log(f"{name}: {res[name]['ms']:.3f} ms")
    # the column loop's repairs: every column updates all later columns of
    # every row, r * c (c - 1) / 2 multiply-adds, however they are blocked
    flops = float(r) * c * (c - 1)
    tot_ms = sum(v["ms"] for v in res.values())
    worst = max(res.values(), key=lambda v: v["ms"])
    for v in res.values():
        v["weights_per_s"] = r * c / (v["ms"] * 1e-3)
    ach = flops / (worst["ms"] * 1e-3) / 1e12
    rec = {
        "metric": "GPTQ quantize stage per grid variant on 4096x4096 (ruler fits, column loop, deferred "
                  "products): weights/s over all variants",
        "value": len(res) * r * c / (tot_ms * 1e-3), "unit": "weights/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": tot_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0, 0.02^2) weights; U from the Hessian of Student-t(4) activations)",
        "config": {"workload": "llama7b_attn_4096x4096_grid_variants", "rows": r, "cols": c,
                   "blocksize": w.blocksize, "variants": res},
        "roofline": {"kernel": "gptq_quantize_layer, slowest variant (HIP events around the call)", "bound": "mfma",
                     "achieved": ach, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_FP32_TFLOPS, "traffic": None, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_layer(q, w, W, X, ws, rotate: bool):
    """One layer through the whole path with HIP events between the stages;
    returns per-stage milliseconds (the rotation, when asked for, included)."""
    import torch
    d, r, c = w.cols, w.rows, w.cols
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    H = torch.zeros((d, d), dtype=torch.float32, device=W.device)
    ev[0].record()
    if rotate:
        X = q.hadamard_rotate(X, out=X)
        W = q.hadamard_rotate(W, out=W)
    ev[1].record()
    q.hessian_accumulate(H, X, ws=ws[0])
    ev[2].record()
    perm, dead, info = q.prepare(H, w.percdamp, w.act_order, check=False, ws=ws[1])
    ev[3].record()
    out = q.quantize_layer(W, H, perm, dead, bits=w.bits, groupsize=w.groupsize, blocksize=w.blocksize,
                           ws=ws[2])
    ev[4].record()
    q.pack(out["codes"], w.bits)
    ev[5].record()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise RuntimeError(f"prepare reported info = {int(info.item())}")
    names = ["rotate", "hessian", "prepare", "quantize", "pack"]
    ms = {k: ev[i].elapsed_time(ev[i + 1]) for i, k in enumerate(names)}
    ms["layer"] = ev[0].elapsed_time(ev[5])
    return ms


def bench_sweep(args) -> int:
    """The 7B-shaped decoder sweep: all 224 linear layers, each with its own
    weights and calibration activations (generated on the device before its
    timed pass), optionally pre-rotated (rotation inside the timed pass)."""
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = S.llama7b_sweep(args.sweep_blocks)
    ws = [q.Workspace(), q.Workspace(), q.Workspace()]
    # one untimed pass per layer shape first (first-call set-up, workspaces)
    for w, li in {(lw.rows, lw.cols): (lw, i) for lw, i in layers}.values():
        W, X = S.workload_device(w, layer=li, device=dev)
        run_layer(q, w, W, X, ws, args.rotate)
        del W, X
    per_class, total_ms, total_w, wall_gen = {}, 0.0, 0, 0.0
    stage_tot = {}
    for n, (w, li) in enumerate(layers):
        t0 = time.perf_counter()
        W, X = S.workload_device(w, layer=li, device=dev)
        torch.cuda.synchronize()
        wall_gen += time.perf_counter() - t0
        ms = run_layer(q, w, W, X, ws, args.rotate)
        del W, X
        key = f"{w.rows}x{w.cols}"
        pc = per_class.setdefault(key, {"layers": 0, "ms": 0.0})
        pc["layers"] += 1
        pc["ms"] += ms["layer"]
        for k, v in ms.items():
            stage_tot[k] = stage_tot.get(k, 0.0) + v
        total_ms += ms["layer"]
        total_w += w.rows * w.cols
        if (n + 1) % 7 == 0:
            log(f"block {(n + 1) // 7}/{len(layers) // 7}: {total_ms:.1f} ms of quantization so far "
                f"(inputs generated in {wall_gen:.1f} s)")
    for pc in per_class.values():
        pc["ms_per_layer"] = pc["ms"] / pc["layers"]
    flops_h = sum(w.cols * (w.cols + 1) * w.tokens for w, _ in layers)
    rec = {
        "metric": METRIC,
        "value": total_w / (total_ms / 1e3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 1,
        "ms_per_step": total_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; per-linear N(0,0.02^2) weights and Student-t(4) activations, 0.5% outlier "
                "channels x30)",
        "config": {"workload": f"llama7b_decoder_sweep_{len(layers)}_linears", "blocks": len(layers) // 7,
                   "linears": len(layers), "tokens": 262144, "bits": 4, "groupsize": 128, "blocksize": 128,
                   "percdamp": 0.01, "act_order": False, "hadamard_rotation": bool(args.rotate)},
        "sec_for_sweep": total_ms / 1e3,
        "weights": total_w,
        "hessian_tflops": flops_h / (stage_tot["hessian"] / 1e3) / 1e12,
        "stage_ms_total": {k: round(v, 2) for k, v in stage_tot.items()},
        "per_class": per_class,
        "roofline": {
            "kernel": "gptq_hessian_accumulate over the sweep (HIP events around each call)",
            "bound": "mfma",
            "achieved": flops_h / (stage_tot["hessian"] / 1e3) / 1e12,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops_h / (stage_tot["hessian"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": flops_h / len(layers),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample of each layer shape ...")
        sec = 0.0
        samples = []
        for w, li in {(lw.rows, lw.cols): (lw, i) for lw, i in layers}.values():
            W, X = S.workload_device(w, layer=li, device=dev)
            cb = cpu_baseline(W, X, w)
            del W, X
            n_cls = sum(1 for lw, _ in layers if (lw.rows, lw.cols) == (w.rows, w.cols))
            sec += n_cls * cb["sec_per_layer_extrapolated"]
            samples.append(f"{w.rows}x{w.cols} (x{n_cls}): {cb['sample']}")
            cores = cb["cores"]
        rec["cpu_baseline"] = {"value": total_w / sec, "unit": "weights/s", "cores": cores, "kind": "oracle",
                               "sample": " | ".join(samples), "sec_for_sweep_extrapolated": sec}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def library_reference(X, d: int, n_tok: int, reps: int = 3):
    """The vendor library's product X^T X on the same activations: torch.mm
    (hipBLASLt) of the transposed copy and X, the full d x d product in the
    activations' 16-bit type with fp32 accumulation, timed back to back after
    the benchmark's own timed region.  Context for the Hessian's rate: the
    library computes both triangles, the SYRK only the upper one."""
    import torch
    if X.dtype not in (torch.bfloat16, torch.float16):
        return None
    Xt = X.t().contiguous()
    out = torch.empty((d, d), dtype=X.dtype, device=X.device)
    torch.mm(Xt, X, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(Xt, X, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del Xt, out
    torch.cuda.empty_cache()
    full = 2.0 * d * d * n_tok
    return {"what": "torch.mm(X^T, X) (hipBLASLt): the full d x d product, 16-bit output, fp32 accumulation",
            "ms": ms, "tflops_full_product": full / (ms / 1e3) / 1e12,
            "tflops_upper_triangle_equiv": d * (d + 1) * n_tok / (ms / 1e3) / 1e12}


def bench_hessian(args) -> int:
    """gptq_hessian_accumulate alone, back to back, on the workload's X or on
    an X of the same shape filled with uniform random values in [-1, 1) or
    zeros (the SYRK's clock depends on the operands' values)."""
    import torch

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    w = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = getattr(torch, w.x_dtype)
    if args.x_fill == "workload":
        _, X = S.workload_device(w, device=dev)
    else:
        X = torch.empty((w.tokens, w.cols), dtype=dt, device=dev)
        if args.x_fill == "zeros":
            X.zero_()
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(S.torch_seed(w.wid, 0, 5))
            X.uniform_(-1.0, 1.0, generator=g)
    H = torch.zeros((w.cols, w.cols), dtype=torch.float32, device=dev)
    ws = q.Workspace()
    for _ in range(args.warmup):
        q.hessian_accumulate(H, X, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        q.hessian_accumulate(H, X, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = w.cols * (w.cols + 1) * w.tokens
    tf = flops / (ms / 1e3) / 1e12
    peak = PEAK_FP16_TFLOPS if w.x_dtype == "float16" else PEAK_BF16_TFLOPS
    print(json.dumps({
        "metric": "Hessian TFLOP/s (gptq_hessian_accumulate alone)", "value": tf, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.x_dtype == "bfloat16" else "fp16",
        "data": f"synthetic ({args.x_fill} activations)",
        "config": {"workload": w.name, "cols": w.cols, "tokens": w.tokens, "x_fill": args.x_fill},
        "roofline": {"kernel": "syrk16_dma_kernel + reduce_partials_kernel", "bound": "mfma", "achieved": tf,
                     "peak": peak, "unit": "TFLOP/s", "frac": tf / peak, "traffic": None,
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama7b_attn_4096x4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--gemv", action="store_true")
    ap.add_argument("--gemv-model", default="llama7b", choices=sorted(GEMV_MODELS))
    ap.add_argument("--fused-inputs", action="store_true",
                    help="--gemv: projections that read one input stored as one matrix (q|k|v, gate|up)")
    ap.add_argument("--hadamard", action="store_true")
    ap.add_argument("--stack", action="store_true")
    ap.add_argument("--grid", action="store_true")
    ap.add_argument("--blocks", type=int, default=2)
    ap.add_argument("--sweep", action="store_true", help="the 7B-shaped decoder sweep (224 linear layers)")
    ap.add_argument("--sweep-blocks", type=int, default=32)
    ap.add_argument("--rotate", action="store_true", help="--sweep: Hadamard pre-rotation of X and W")
    ap.add_argument("--hessian", action="store_true", help="gptq_hessian_accumulate alone, back to back")
    ap.add_argument("--x-fill", default="workload", choices=["workload", "uniform", "zeros"],
                    help="--hessian: the workload's X, or uniform random / zero values of its shape")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the quantizer's path runs on a single MI355X here "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if args.copy_probe:
        copy_probe()
        return 0
    if args.gemv:
        return bench_gemv(args)
    if args.hadamard:
        return bench_hadamard(args)
    if args.stack:
        return bench_stack(args)
    if args.grid:
        return bench_grid(args)
    if args.sweep:
        return bench_sweep(args)
    if args.hessian:
        return bench_hessian(args)

    from post_weight_quantization_23_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build as b
        b.build()
    import post_weight_quantization_23_amd as q
    from synth import inputs as S

    w = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {w.name}: W {w.rows}x{w.cols} {w.w_dtype}, X {w.tokens}x{w.cols} {w.x_dtype}")
    W, X = S.workload_device(w, device=dev)
    torch.cuda.synchronize()

    d, r, c = w.cols, w.rows, w.cols
    H = torch.empty((d, d), dtype=torch.float32, device=dev)
    G = (c + w.groupsize - 1) // w.groupsize if w.groupsize > 0 else 1
    out = {
        "codes": torch.empty((r, c), dtype=torch.uint8, device=dev),
        "scales": torch.empty((r, G), dtype=torch.float32, device=dev),
        "zeros": torch.empty((r, G), dtype=torch.int32, device=dev),
        "g_idx": torch.empty(c, dtype=torch.int32, device=dev),
        "row_loss": torch.empty(r, dtype=torch.float32, device=dev),
    }
    packed = torch.empty((r, c * w.bits // 32), dtype=torch.uint32, device=dev)
    ws_h, ws_p, ws_q = q.Workspace(), q.Workspace(), q.Workspace()

    # Events are recorded on torch's current stream, the stream the bindings
    # hand to the library, so they bracket exactly the library's launches.
    def step(ev):
        ev[0].record()
        H.zero_()
        ev[1].record()
        q.hessian_accumulate(H, X, ws=ws_h)
        ev[2].record()
        perm, dead, info = q.prepare(H, w.percdamp, w.act_order, check=False, ws=ws_p)
        ev[3].record()
        q.quantize_layer(W, H, perm, dead, bits=w.bits, groupsize=w.groupsize, blocksize=w.blocksize,
                         ws=ws_q, out=out)
        ev[4].record()
        q.pack(out["codes"], w.bits, out=packed)
        ev[5].record()
        return info

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        info = step(mk())
    torch.cuda.synchronize()
    if args.warmup and int(info.item()) != 0:
        raise RuntimeError(f"prepare reported info = {int(info.item())}")

    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage = {"zero_h": [], "hessian": [], "prepare": [], "quantize": [], "pack": [], "step": []}
    for ev in evs:
        stage["zero_h"].append(ev[0].elapsed_time(ev[1]))
        stage["hessian"].append(ev[1].elapsed_time(ev[2]))
        stage["prepare"].append(ev[2].elapsed_time(ev[3]))
        stage["quantize"].append(ev[3].elapsed_time(ev[4]))
        stage["pack"].append(ev[4].elapsed_time(ev[5]))
        stage["step"].append(ev[0].elapsed_time(ev[5]))
    avg = {k: sum(v) / len(v) for k, v in stage.items()}
    ms_step = wall * 1e3 / args.steps
    sec_layer = ms_step / 1e3
    flops_h = d * (d + 1) * w.tokens
    hess_tflops = flops_h / (avg["hessian"] / 1e3) / 1e12
    peak = PEAK_FP16_TFLOPS if w.x_dtype == "float16" else PEAK_BF16_TFLOPS
    traffic = load_traffic(w.name)
    rec = {
        "metric": METRIC,
        "value": (r * c) / sec_layer,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.x_dtype == "bfloat16" else ("fp16" if w.x_dtype == "float16" else "f32"),
        "data": "synthetic (seeded; N(0,0.02^2) weights, Student-t(4) activations with outlier channels)",
        "config": {"workload": w.name, "rows": r, "cols": c, "tokens": w.tokens, "bits": w.bits,
                   "groupsize": w.groupsize, "blocksize": w.blocksize, "percdamp": w.percdamp,
                   "act_order": w.act_order, "w_dtype": w.w_dtype, "x_dtype": w.x_dtype},
        "sec_per_layer": sec_layer,
        "hessian_tflops": hess_tflops,
        "stage_ms": {k: round(v, 4) for k, v in avg.items()},
        "roofline": {
            "kernel": "gptq_hessian_accumulate: syrk16_dma_kernel + reduce_partials_kernel (HIP events around the call)",
            "bound": "mfma",
            "achieved": hess_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": hess_tflops / peak,
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops_h,
        },
    }
    # The other stages against their own bounds, from the same HIP events (a
    # stage's time includes all of its kernels, so these are lower bounds of
    # the rate of its dominant kernel): the factor's 2d^3/3 flops and the
    # lazy updates' r*c*(c - blocksize) flops against the fp32 matrix-core
    # peak, the pack's (1 + bits/8) bytes per weight against HBM.
    f_prep = 2.0 * d ** 3 / 3.0
    f_lazy = float(r) * c * max(c - w.blocksize, 0)
    b_pack = r * c * (1.0 + w.bits / 8.0)
    rec["stage_roofline"] = {
        "prepare": {"bound": "mfma", "achieved": f_prep / (avg["prepare"] / 1e3) / 1e12, "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": f_prep / (avg["prepare"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
                    "algorithmic_flops": f_prep},
        "quantize": {"bound": "mfma", "achieved": f_lazy / (avg["quantize"] / 1e3) / 1e12, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": f_lazy / (avg["quantize"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
                     "algorithmic_flops": f_lazy, "note": "lazy-update flops over the whole call (chain included)"},
        "pack": {"bound": "hbm", "achieved": b_pack / (avg["pack"] / 1e3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": b_pack / (avg["pack"] / 1e3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": b_pack},
    }
    # The pack is one short launch: the events around a single call hold the
    # host's launch time as well.  50 calls captured in a HIP graph and
    # replayed (after the timed steps, on the same codes) run back to back on
    # the device and give the kernel's own rate.
    n_pack = 50
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            q.pack(out["codes"], w.bits, out=packed)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n_pack):
                q.pack(out["codes"], w.bits, out=packed)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us_pack = e0.elapsed_time(e1) * 1e3 / n_pack
        del graph
        rec["stage_roofline"]["pack_graph_replay"] = {
            "bound": "hbm", "us_per_call": us_pack, "achieved": b_pack / (us_pack / 1e6) / 1e9,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": b_pack / (us_pack / 1e6) / 1e9 / PEAK_HBM_GBS,
            "calls": n_pack}
    except Exception as e:   # noqa: BLE001  (context only)
        rec["stage_roofline"]["pack_graph_replay"] = {"error": f"{type(e).__name__}: {e}"}
    try:   # context only: the benchmark line stands without it
        lib = library_reference(X, d, w.tokens)
        if lib is not None:
            lib["hessian_speedup"] = lib["ms"] / avg["hessian"]
    except Exception as e:   # noqa: BLE001
        lib = {"error": f"{type(e).__name__}: {e}"}
    rec["library_reference"] = lib
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(W, X, w)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
