"""The C-ABI library without a GPU: it loads, exports every symbol include/gptq.h
declares, and rejects bad arguments on the host before touching HIP (so none
of these calls reaches the device)."""
import ctypes as C
import os
import re

import pytest

from post_weight_quantization_23_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")
BAD = C.c_void_p(0x1000)   # never dereferenced: validation fails first
ALIGNED = C.c_void_p(0x10000)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from post_weight_quantization_23_amd import build
        build.build()
    return _lib.load()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gptq_status|const char\s*\*)\s*(gptq_\w+)\s*\(", src, re.M)))


def test_header_symbols_are_exported(lib):
    names = _declared()
    assert len(names) == 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def _st(lib, name, *args):
    return getattr(lib, name)(*args)


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.gptq_status_string(code).decode().startswith(name)


def test_workspace_queries(lib):
    out = C.c_size_t(7)
    assert _st(lib, "gptq_hessian_workspace_size", 4096, 262144, 1, C.byref(out)) == 0
    assert out.value > 0
    assert _st(lib, "gptq_hessian_workspace_size", 256, 2048, 0, C.byref(out)) == 0 and out.value == 0
    assert _st(lib, "gptq_hessian_workspace_size", 16, 16, 9, C.byref(out)) == 2
    assert _st(lib, "gptq_hessian_workspace_size", -1, 16, 1, C.byref(out)) == 1
    assert _st(lib, "gptq_hessian_workspace_size", 16, 16, 1, None) == 1
    assert _st(lib, "gptq_prepare_workspace_size", 4096, 0, C.byref(out)) == 0
    assert out.value >= 4096 * 4096 * 4
    assert _st(lib, "gptq_prepare_workspace_size", 4096, 2, C.byref(out)) == 1
    assert _st(lib, "gptq_prepare_workspace_size", 70000, 0, C.byref(out)) == 5
    assert _st(lib, "gptq_quantize_layer_workspace_size", 4096, 4096, 128, C.byref(out)) == 0
    assert out.value >= 4096 * 4096 * 4 + 128 * 4096 * 4
    assert _st(lib, "gptq_quantize_layer_workspace_size", 4096, 4096, 0, C.byref(out)) == 5
    assert _st(lib, "gptq_quantize_layer_workspace_size", 4096, 4096, 129, C.byref(out)) == 5


def test_hessian_argument_errors(lib):
    f = "gptq_hessian_accumulate"
    # no-op sizes succeed without touching the device
    assert _st(lib, f, None, 0, None, 1, 10, 0, None, 0, None) == 0
    assert _st(lib, f, None, 8, None, 1, 0, 8, None, 0, None) == 0
    assert _st(lib, f, None, 8, BAD, 1, 4, 8, None, 0, None) == 1          # H NULL
    assert _st(lib, f, ALIGNED, 8, None, 1, 4, 8, None, 0, None) == 1      # X NULL
    assert _st(lib, f, ALIGNED, 8, ALIGNED, 7, 4, 8, None, 0, None) == 2   # dtype
    assert _st(lib, f, ALIGNED, 8, ALIGNED, 1, 4, 4, None, 0, None) == 3   # ldx < d
    assert _st(lib, f, ALIGNED, 8, C.c_void_p(0x10001), 1, 4, 8, None, 0, None) == 4  # X misaligned
    assert _st(lib, f, ALIGNED, 8, C.c_void_p(0x10002), 0, 4, 8, None, 0, None) == 4  # fp32 X misaligned
    # bf16 at a size that needs split partials: workspace required
    assert _st(lib, f, ALIGNED, 4096, ALIGNED, 1, 262144, 4096, None, 0, None) == 6
    assert "workspace" in lib.gptq_last_error().decode()


def test_prepare_argument_errors(lib):
    f = "gptq_prepare"
    info = ALIGNED
    assert _st(lib, f, ALIGNED, 16, C.c_float(0.01), 0, None, ALIGNED, None, None, 0, None) == 1   # info NULL
    assert _st(lib, f, ALIGNED, 16, C.c_float(-1.0), 0, None, ALIGNED, info, None, 0, None) == 1   # damp < 0
    assert _st(lib, f, ALIGNED, 16, C.c_float(float("nan")), 0, None, ALIGNED, info, None, 0, None) == 1
    assert _st(lib, f, ALIGNED, 16, C.c_float(0.01), 1, None, ALIGNED, info, None, 0, None) == 1   # perm NULL
    assert _st(lib, f, ALIGNED, 16, C.c_float(0.01), 0, None, None, info, None, 0, None) == 1      # dead NULL
    assert _st(lib, f, ALIGNED, 16, C.c_float(0.01), 0, None, ALIGNED, info, None, 0, None) == 6   # no workspace
    assert _st(lib, f, C.c_void_p(0x10004), 16, C.c_float(0.01), 0, None, ALIGNED, info, ALIGNED, 1 << 20, None) == 4
    assert _st(lib, f, ALIGNED, 16, C.c_float(0.01), 0, None, ALIGNED, info, C.c_void_p(0x10010), 1 << 20, None) == 4


def test_quantize_argument_errors(lib):
    f = "gptq_quantize_layer"
    A = ALIGNED

    def q(W=A, wt=1, r=8, c=256, ldw=256, U=A, bits=4, g=128, B=128, codes=A, ws=A, nws=1 << 30, sym=0):
        return _st(lib, f, W, wt, r, c, ldw, U, None, None, bits, sym, g, B, codes, A, A, A, None, None, ws, nws,
                   None)

    assert q(r=0) == 0 and q(c=0) == 0
    assert q(bits=5) == 5 and q(bits=1) == 5
    assert q(sym=2) == 1 and q(sym=-1) == 1
    assert q(B=0) == 5 and q(B=256) == 5
    assert q(g=96, B=128) == 5            # neither a multiple nor a divisor
    assert q(wt=3) == 2
    assert q(ldw=100) == 3
    assert q(W=None) == 1 and q(U=None) == 1 and q(codes=None) == 1
    assert q(W=C.c_void_p(0x10001)) == 4
    assert q(ws=None) == 6 and q(nws=16) == 6


def test_pack_argument_errors(lib):
    f = "gptq_pack"
    A = ALIGNED
    assert _st(lib, f, A, 4, 12, 4, None, A, 2, None) == 3     # c % 8
    assert _st(lib, f, A, 4, 48, 3, None, A, 5, None) == 3     # c % 32
    assert _st(lib, f, A, 4, 64, 3, None, A, 5, None) == 3     # ld_words < 6
    assert _st(lib, f, A, 4, 64, 8, None, A, 16, None) == 5    # bits
    assert _st(lib, f, None, 4, 64, 4, None, A, 8, None) == 1
    assert _st(lib, f, C.c_void_p(0x10008), 4, 64, 4, None, A, 8, None) == 4
    assert _st(lib, f, A, 4, 64, 4, C.c_void_p(0x10002), A, 8, None) == 4   # col_perm alignment
    assert _st(lib, f, None, 0, 64, 4, None, None, 8, None) == 0


def test_dequant_gemv_argument_errors(lib):
    f = "gptq_dequant_gemv"
    A = ALIGNED

    def g(packed=A, r=8, c=256, bits=4, ldw=32, s=A, z=A, ldg=2, gs=128, perm=None, x=A, xt=1, y=A):
        return _st(lib, f, packed, r, c, bits, ldw, s, z, ldg, gs, perm, x, xt, y, None)

    assert g(r=0, y=None) == 0                 # nothing to do
    assert g(r=-1) == 1 and g(c=-32) == 1
    assert g(bits=2) == 5 and g(bits=8) == 5
    assert g(xt=0) == 2                        # fp32 activations are not a 16-bit input
    assert g(xt=7) == 1
    assert g(c=48, ldw=6) == 3                 # c % 32
    assert g(c=49152 + 32, ldw=6148, ldg=385) == 5
    assert g(gs=48) == 5                       # groupsize not a multiple of 32
    assert g(ldw=31) == 3                      # ld_words < c * bits / 32
    assert g(ldg=1) == 3                       # 2 groups of 128
    assert g(gs=-1, ldg=1) != 3 and g(gs=256, ldg=1) != 3 and g(gs=512, ldg=1) != 3
    assert g(packed=None) == 1 and g(s=None) == 1 and g(z=None) == 1 and g(x=None) == 1 and g(y=None) == 1
    assert g(packed=C.c_void_p(0x10004)) == 4  # 4-bit words need 16-byte alignment
    assert g(ldw=34) == 4                      # ... and ld_words % 4 == 0
    assert g(bits=3, ldw=24, packed=C.c_void_p(0x10004), y=C.c_void_p(0x10002)) == 4
    assert g(x=C.c_void_p(0x10002)) == 4       # x 16-byte aligned without perm
    assert g(perm=C.c_void_p(0x10002)) == 4


def test_hadamard_argument_errors(lib):
    f = "gptq_hadamard_rotate"
    A, O = ALIGNED, C.c_void_p(0x40000000)

    def h(a=A, at=1, rows=4, d=4096, lda=4096, block=0, out=O, ot=1, ldo=4096):
        return _st(lib, f, a, at, rows, d, lda, block, out, ot, ldo, None)

    assert h(rows=0) == 0 and h(d=0) == 0
    assert h(rows=-1) == 1
    assert h(at=5) == 2 and h(ot=-1) == 2
    assert h(block=16) == 5 and h(block=96) == 5 and h(block=16384) == 5
    assert h(d=4000, lda=4000, ldo=4000, block=64) == 3           # 64 does not divide 4000
    assert h(d=48, lda=48, ldo=48) == 5                           # default block 16 is too small
    assert h(lda=100) == 3 and h(ldo=100) == 3
    assert h(a=None) == 1 and h(out=None) == 1
    assert h(a=C.c_void_p(0x10001)) == 4
    assert h(out=C.c_void_p(0x10000 + 2 * 4096)) == 1             # overlaps A without being A
    assert h(out=A, ot=0) == 1                                     # in place needs the same dtype


def test_linear_forward_argument_errors(lib):
    f = "gptq_linear_forward"
    X, W, Y, G = ALIGNED, C.c_void_p(0x1000000), C.c_void_p(0x40000000), C.c_void_p(0x80000000)

    def l(x=X, xt=1, n=8, d=256, ldx=256, w=W, wt=0, r=64, ldw=256, act=0, g=None, ldg=0, y=Y, yt=1, ldy=64):
        return _st(lib, f, x, xt, n, d, ldx, w, wt, r, ldw, act, g, ldg, y, yt, ldy, None)

    # only calls that fail validation (or have nothing to do) are made here:
    # a call that passes would launch on made-up addresses
    assert l(n=0) == 0 and l(r=0) == 0
    assert l(n=-1) == 1 and l(act=2) == 1 and l(yt=9) == 1 and l(wt=7) == 1
    assert l(xt=0) == 2                           # fp32 activations
    assert l(wt=2) == 2                           # 16-bit weights of another type than X
    assert l(d=100, ldx=100, ldw=100) == 5 and l(d=0) == 5
    assert l(ldx=200) == 3 and l(ldw=128) == 3 and l(ldy=32) == 3
    assert l(act=1, g=G, ldg=32) == 3
    assert l(x=None) == 1 and l(w=None) == 1 and l(y=None) == 1 and l(act=1, ldg=64) == 1
    assert l(x=C.c_void_p(0x10008)) == 4 and l(ldx=260) == 4 and l(ldw=258) == 4
    assert l(wt=1, ldw=260) == 4                  # 16-bit weights: rows on 16 bytes
    assert l(wt=1, ldx=1 << 22, ldw=256) == 5     # 16-bit weights: strides below 2^22
    assert l(n=1 << 29, r=1 << 29, ldy=1 << 29) == 5   # more 256 x 256 tiles than a grid holds
    assert l(y=C.c_void_p(0x10000 + 512)) == 1    # Y inside X
    assert l(act=1, g=G, ldg=64, y=C.c_void_p(0x80000000 + 2), yt=1, ldy=64) == 1


def test_round16_argument_errors(lib):
    f = "gptq_round16"
    S, D = ALIGNED, C.c_void_p(0x40000000)

    def r(s=S, rows=4, cols=64, lds=64, dt=1, d=D, ldd=64):
        return _st(lib, f, s, rows, cols, lds, dt, d, ldd, None)

    assert r(rows=0) == 0 and r(cols=0) == 0
    assert r(rows=-1) == 1 and r(dt=5) == 1
    assert r(dt=0) == 2
    assert r(lds=32) == 3 and r(ldd=32) == 3
    assert r(s=None) == 1 and r(d=None) == 1
    assert r(s=C.c_void_p(0x10002)) == 4 and r(d=C.c_void_p(0x40000001)) == 4
    assert r(d=C.c_void_p(0x10000 + 64)) == 1     # dst inside src


def test_python_binding_rejects_cpu_tensors():
    import torch
    from post_weight_quantization_23_amd import gptq
    with pytest.raises(ValueError):
        gptq.hessian_accumulate(torch.zeros(4, 4), torch.zeros(2, 4))
    with pytest.raises(ValueError):
        gptq.pack(torch.zeros(2, 8, dtype=torch.uint8), 4)
    with pytest.raises(ValueError):
        gptq.dequant_gemv(torch.zeros(2, 4, dtype=torch.uint32), torch.zeros(2, 1), torch.zeros(2, 1, dtype=torch.int32),
                          torch.zeros(32, dtype=torch.bfloat16), 4, -1)


def test_python_quantize_layer_checks_lengths_and_outputs_before_the_device():
    # The kernels index perm / dead by column and write every output with
    # strides r and c, so the binding rejects a short or mis-shaped tensor
    # (these are CPU tensors: the shape checks come before the device check).
    import torch
    from post_weight_quantization_23_amd import gptq
    r, c = 4, 64
    W = torch.zeros(r, c)
    U = torch.zeros(c, c)
    ok_perm = torch.zeros(c, dtype=torch.int32)
    ok_dead = torch.zeros(c, dtype=torch.uint8)

    def q(**kw):
        args = dict(W=W, U=U, perm=ok_perm, dead=ok_dead)
        args.update(kw)
        return gptq.quantize_layer(args.pop("W"), args.pop("U"), args.pop("perm"), args.pop("dead"), **args)

    with pytest.raises(ValueError, match="perm"):
        q(perm=torch.zeros(c - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="dead"):
        q(dead=torch.zeros(c + 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="perm"):
        q(perm=torch.zeros(2 * c, dtype=torch.int32)[::2])
    with pytest.raises(TypeError, match="perm"):
        q(perm=torch.zeros(c, dtype=torch.int64))
    with pytest.raises(ValueError, match="U"):
        q(U=torch.zeros(c, c + 1))
    bad_outs = {
        "codes": torch.zeros(r, c - 1, dtype=torch.uint8),
        "scales": torch.zeros(r, 2),                 # groupsize 128 > c: one group
        "zeros": torch.zeros(r + 1, 1, dtype=torch.int32),
        "g_idx": torch.zeros(c + 8, dtype=torch.int32),
        "w_hat": torch.zeros(c, r),
        "row_loss": torch.zeros(2 * r)[::2],
    }
    for k, t in bad_outs.items():
        with pytest.raises(ValueError, match=k):
            q(out={k: t})
    with pytest.raises(TypeError, match="codes"):
        q(out={"codes": torch.zeros(r, c, dtype=torch.int32)})
    with pytest.raises(ValueError, match="unknown"):
        q(out={"code": torch.zeros(r, c, dtype=torch.uint8)})
    # Everything well formed: only then does the device check fire.
    with pytest.raises(ValueError, match="GPU"):
        q(out={"codes": torch.zeros(r, c, dtype=torch.uint8)})


def test_launch_grids_are_bounded_at_the_exact_limit(lib):
    # A launch's grid.x * 256 threads must fit in 32 bits: at most 2^24 - 1
    # workgroups.  Each size is tried one past the limit (rejected as
    # unsupported) and at the limit (accepted by the size check, then stopped
    # by a NULL pointer or a missing workspace, so nothing is launched).
    A = ALIGNED
    lim = (1 << 24) - 1
    q = lambda r, ws: _st(lib, "gptq_quantize_layer", A, 1, r, 256, 256, A, None, None, 4, 0, 128, 128, A, A, A, A,
                          None, None, ws, 1 << 40 if ws else 0, None)
    assert q(lim + 1, A) == 5 and q(lim, None) == 6                    # one workgroup per row
    l = lambda x, r: _st(lib, "gptq_linear_forward", x, 1, 1 << 20, 256, 256, C.c_void_p(0x1000000), 0, r, 256,
                         0, None, 0, C.c_void_p(0x40000000), 1, r, None)
    assert l(A, 1 << 20) == 5 and l(None, (1 << 20) - 256) == 1        # 2^12 x 2^12 tiles vs 2^12 x (2^12 - 1)
    rr = lambda s, rows: _st(lib, "gptq_round16", s, rows, 1024, 1024, 1, C.c_void_p(0x40000000), 1024, None)
    assert rr(A, lim + 1) == 5 and rr(None, lim) == 1                  # 256 four-element items per row
    p = lambda c, r, perm: _st(lib, "gptq_pack", c, r, 2048, 4, perm, A, 256, None)
    assert p(A, lim + 1, None) == 5 and p(None, lim, None) == 1        # 256 chunks of 8 codes per row
    assert p(A, 4 * (lim + 1), A) == 5 and p(None, 4 * lim, A) == 1    # 64 chunks of 32 codes per row
    h = lambda a, rows: _st(lib, "gptq_hadamard_rotate", a, 1, rows, 4096, 4096, 4096, C.c_void_p(0x40000000), 1,
                            4096, None)
    assert h(A, lim + 1) == 5 and h(None, lim) == 1                    # one tile of 4096 per workgroup


def test_hessian_workspace_must_be_256_byte_aligned(lib):
    f = "gptq_hessian_accumulate"
    base = lambda ws: _st(lib, f, ALIGNED, 4096, ALIGNED, 1, 262144, 4096, ws, 1 << 40, None)
    assert base(C.c_void_p(0x10010)) == 4 and base(C.c_void_p(0x10080)) == 4


def test_prepare_noalloc_argument_errors(lib):
    f = "gptq_prepare_noalloc"
    A = ALIGNED

    def p(H=A, d=256, damp=0.01, ao=0, perm=None, dead=A, info=A):
        return _st(lib, f, H, d, C.c_float(damp), ao, perm, dead, info, None)

    assert p(d=-1) == 1 and p(ao=2) == 1 and p(damp=-1.0) == 1 and p(damp=float("nan")) == 1
    assert p(d=4097) == 5                         # beyond the static scratch
    assert p(d=0) == 1 and p(info=None) == 1 and p(H=None) == 1 and p(dead=None) == 1
    assert p(ao=1, perm=None) == 1                # act-order needs perm
    assert p(H=C.c_void_p(0x10004)) == 4 and p(info=C.c_void_p(0x10002)) == 4


# ---------------------------------------------------------------------------
# The same host checks built with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; the kernels' launch functions that the driver would need are
# stubs that abort, and every call in it must fail validation before a launch).
ASAN_SOURCES = ["gptq_api.hip", "workspace.hip", "syrk.hip", "prepare.hip", "gemv.hip", "gemm_f32.hip", "pack.hip",
                "hadamard.hip"]
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_driver():
    import hashlib
    import shutil
    import subprocess
    from concurrent.futures import ThreadPoolExecutor
    from post_weight_quantization_23_amd import build as b
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    gxx = shutil.which("g++")
    if not os.path.exists(hipcc) or gxx is None:
        pytest.skip("hipcc or g++ not available")
    csrc = os.path.join(ROOT, "post_weight_quantization_23_amd", "csrc")
    driver = os.path.join(ROOT, "tests", "asan", "boundary_driver.cpp")
    h = hashlib.sha256(" ".join(SAN_HOST).encode())
    for f in sorted(os.listdir(csrc)) + [driver, HEADER]:
        path = f if os.path.isabs(f) else os.path.join(csrc, f)
        with open(path, "rb") as fh:
            h.update(fh.read())
    out = os.path.join(ROOT, "post_weight_quantization_23_amd", "_build", "asan", h.hexdigest()[:16])
    exe = os.path.join(out, "boundary_driver")
    if os.path.exists(exe):
        return exe
    os.makedirs(out, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]

    def compile_one(src):
        obj = os.path.join(out, src.replace(".hip", ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", *SAN_HOST,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               *inc, "-c", os.path.join(csrc, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, ASAN_SOURCES))
    dobj = os.path.join(out, "boundary_driver.o")
    r = subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", *inc, "-c", driver, "-o", dobj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([gxx, "-fsanitize=address,undefined", "-o", exe + ".tmp", dobj, *objs, "-L/opt/rocm/lib",
                        "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    os.replace(exe + ".tmp", exe)
    return exe


def test_host_validation_under_address_and_undefined_behavior_sanitizers():
    import subprocess
    exe = _asan_driver()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all validation checks passed" in r.stdout
