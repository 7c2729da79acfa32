// C ABI of the gfx950 GPTQ layer quantizer (declared in include/gptq.h).
//
// Every entry point validates all of its arguments on the host before it
// touches HIP, so an error return means nothing was enqueued.  The library
// allocates nothing; scratch space is the caller's workspace.
#include <climits>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/gptq.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

gptq_status fail(gptq_status st, const char* fn, const std::string& what) {
  g_last_error = std::string(fn) + ": " + what;
  return st;
}

gptq_status ok() {
  g_last_error.clear();
  return GPTQ_OK;
}

gptq_status check_launch(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPTQ_EHIP, fn, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = 65535;       // H / U edge (grid y limit, int kernels)
constexpr int64_t kMaxRows = INT_MAX / 2; // rows of W, tokens of X
// A launch's grid.x times its 256 threads per workgroup must fit in 32 bits.
constexpr int64_t kMaxGroups256 = ((int64_t(1) << 32) - 1) / 256;

// Workgroups of 256 threads needed for n items at `per` items per workgroup.
int64_t groups_for(int64_t n, int64_t per) { return (n + per - 1) / per; }

// Bytes spanned by a rows x cols matrix with row stride ld (elements of
// `elem` bytes), or -1 when that does not fit in 63 bits.
int64_t extent_bytes(int64_t rows, int64_t ld, int64_t cols, int64_t elem) {
  int64_t e = 0;
  if (rows <= 0 || cols <= 0) return 0;
  if (__builtin_mul_overflow(rows - 1, ld, &e) || __builtin_add_overflow(e, cols, &e) ||
      __builtin_mul_overflow(e, elem, &e))
    return -1;
  return e;
}

// Whether [p, p + bytes) and [q, q + bytes_q) overlap (extents already known to fit).
bool overlaps(const void* p, int64_t bytes, const void* q, int64_t bytes_q) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uint64_t)bytes_q && b < a + (uint64_t)bytes;
}

size_t elem_size(gptq_dtype t) { return t == GPTQ_F32 ? 4 : 2; }
bool valid_dtype(int t) { return t == GPTQ_F32 || t == GPTQ_BF16 || t == GPTQ_F16; }

// Scratch of gptq_prepare_noalloc: one array per GPU, as large as
// gptq_prepare's workspace at the largest supported d.  In host code the
// name `scratch` is only a stand-in; its device address on the current
// device comes from hipGetSymbolAddress (looked up once per device and kept).
static __device__ __align__(256) unsigned char scratch[GPTQ_PREPARE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* gptq_status_string(gptq_status s) {
  switch (s) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_EINVAL: return "GPTQ_EINVAL: invalid argument";
    case GPTQ_EDTYPE: return "GPTQ_EDTYPE: unsupported dtype";
    case GPTQ_ESHAPE: return "GPTQ_ESHAPE: inconsistent shape or leading dimension";
    case GPTQ_EALIGN: return "GPTQ_EALIGN: misaligned pointer or leading dimension";
    case GPTQ_EUNSUPPORTED: return "GPTQ_EUNSUPPORTED: outside what this library supports";
    case GPTQ_EWORKSPACE: return "GPTQ_EWORKSPACE: workspace missing or too small";
    case GPTQ_EHIP: return "GPTQ_EHIP: HIP launch failed";
  }
  return "unknown gptq_status";
}

const char* gptq_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ Hessian
gptq_status gptq_hessian_workspace_size(int64_t d, int64_t n_tok, gptq_dtype xt, size_t* bytes) {
  const char* fn = "gptq_hessian_workspace_size";
  if (!bytes) return fail(GPTQ_EINVAL, fn, "bytes is NULL");
  if (d < 0 || n_tok < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(xt)) return fail(GPTQ_EDTYPE, fn, "xt must be GPTQ_F32, GPTQ_BF16 or GPTQ_F16");
  if (d > kMaxDim || n_tok > kMaxRows) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  *bytes = 0;
  if (xt != GPTQ_F32 && d > 0 && n_tok > 0) *bytes = gptq::syrk_workspace_bytes(gptq::plan_syrk(d, n_tok));
  return ok();
}

gptq_status gptq_hessian_accumulate(float* H, int64_t d, const void* X, gptq_dtype xt, int64_t n_tok,
                                    int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "gptq_hessian_accumulate";
  if (d < 0 || n_tok < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(xt)) return fail(GPTQ_EDTYPE, fn, "xt must be GPTQ_F32, GPTQ_BF16 or GPTQ_F16");
  if (d > kMaxDim || n_tok > kMaxRows) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if (d == 0 || n_tok == 0) return ok();
  if (!H) return fail(GPTQ_EINVAL, fn, "H is NULL");
  if (!X) return fail(GPTQ_EINVAL, fn, "X is NULL");
  if (ldx < d) return fail(GPTQ_ESHAPE, fn, "ldx < d");
  if (!aligned(H, 4)) return fail(GPTQ_EALIGN, fn, "H not 4-byte aligned");
  if (xt == GPTQ_F32) {
    if (!aligned(X, 4)) return fail(GPTQ_EALIGN, fn, "X not 4-byte aligned");
  } else {
    if (!aligned(X, 2)) return fail(GPTQ_EALIGN, fn, "16-bit X not 2-byte aligned");
  }
  size_t need = 0;
  if (xt != GPTQ_F32) need = gptq::syrk_workspace_bytes(gptq::plan_syrk(d, n_tok));
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(GPTQ_EWORKSPACE, fn, "workspace needs " + std::to_string(need) + " bytes");
  if (need > 0 && !aligned(ws, 256)) return fail(GPTQ_EALIGN, fn, "workspace not 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (xt == GPTQ_F32) {
    gptq::GemmArgs g;
    g.M = (int)d; g.N = (int)d; g.K = (int)n_tok;
    g.A = reinterpret_cast<const float*>(X); g.lda = ldx; g.a_trans = 1; g.a_mask = gptq::MASK_NONE; g.a_off = 0;
    g.B = reinterpret_cast<const float*>(X); g.ldb = ldx; g.b_trans = 0; g.b_mask = gptq::MASK_NONE; g.b_off = 0;
    g.C = H; g.ldc = d; g.alpha = 2.f; g.beta = 1.f; g.upper_only = 1;
    gptq::launch_gemm_f32(g, s);
  } else {
    const gptq::SyrkPlan p = gptq::plan_syrk(d, n_tok);
    gptq::launch_syrk16(H, d, X, xt == GPTQ_BF16 ? 1 : 2, n_tok, ldx, p, reinterpret_cast<float*>(ws), s);
  }
  return check_launch(fn);
}

// ------------------------------------------------------------------ prepare
gptq_status gptq_prepare_workspace_size(int64_t d, int act_order, size_t* bytes) {
  const char* fn = "gptq_prepare_workspace_size";
  if (!bytes) return fail(GPTQ_EINVAL, fn, "bytes is NULL");
  if (d < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (act_order != 0 && act_order != 1) return fail(GPTQ_EINVAL, fn, "act_order must be 0 or 1");
  if (d > kMaxDim) return fail(GPTQ_EUNSUPPORTED, fn, "d too large");
  *bytes = d > 0 ? gptq::prepare_workspace_bytes(d, act_order) : 0;
  return ok();
}

gptq_status gptq_prepare(float* H, int64_t d, float percdamp, int act_order, int32_t* perm,
                         uint8_t* dead, int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "gptq_prepare";
  if (d < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (act_order != 0 && act_order != 1) return fail(GPTQ_EINVAL, fn, "act_order must be 0 or 1");
  if (!(percdamp >= 0.f) || !(percdamp < 1e30f)) return fail(GPTQ_EINVAL, fn, "percdamp must be finite and >= 0");
  if (d > kMaxDim) return fail(GPTQ_EUNSUPPORTED, fn, "d too large");
  if (!info) return fail(GPTQ_EINVAL, fn, "info is NULL");
  if (d == 0) return fail(GPTQ_EINVAL, fn, "d == 0 (nothing to factor)");
  if (!H) return fail(GPTQ_EINVAL, fn, "H is NULL");
  if (!dead) return fail(GPTQ_EINVAL, fn, "dead is NULL");
  if (act_order && !perm) return fail(GPTQ_EINVAL, fn, "perm is NULL with act_order");
  if (!aligned(H, 16) || !aligned(info, 4) || (perm && !aligned(perm, 4)))
    return fail(GPTQ_EALIGN, fn, "H must be 16-byte aligned, perm and info 4-byte aligned");
  const size_t need = gptq::prepare_workspace_bytes(d, act_order);
  if (!ws || ws_bytes < need) return fail(GPTQ_EWORKSPACE, fn, "workspace needs " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(GPTQ_EALIGN, fn, "workspace not 256-byte aligned");
  gptq::launch_prepare(H, d, percdamp, act_order, perm, dead, info, ws, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

gptq_status gptq_prepare_noalloc(float* H, int64_t d, float percdamp, int act_order, int32_t* perm,
                                 uint8_t* dead, int32_t* info, void* stream) {
  const char* fn = "gptq_prepare_noalloc";
  if (d < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (act_order != 0 && act_order != 1) return fail(GPTQ_EINVAL, fn, "act_order must be 0 or 1");
  if (!(percdamp >= 0.f) || !(percdamp < 1e30f)) return fail(GPTQ_EINVAL, fn, "percdamp must be finite and >= 0");
  if (d > GPTQ_PREPARE_NOALLOC_MAX_D)
    return fail(GPTQ_EUNSUPPORTED, fn, "d > " + std::to_string(GPTQ_PREPARE_NOALLOC_MAX_D) +
                                           ": the static scratch is too small; use gptq_prepare with a workspace");
  if (!info) return fail(GPTQ_EINVAL, fn, "info is NULL");
  if (d == 0) return fail(GPTQ_EINVAL, fn, "d == 0 (nothing to factor)");
  if (!H) return fail(GPTQ_EINVAL, fn, "H is NULL");
  if (!dead) return fail(GPTQ_EINVAL, fn, "dead is NULL");
  if (act_order && !perm) return fail(GPTQ_EINVAL, fn, "perm is NULL with act_order");
  if (!aligned(H, 16) || !aligned(info, 4) || (perm && !aligned(perm, 4)))
    return fail(GPTQ_EALIGN, fn, "H must be 16-byte aligned, perm and info 4-byte aligned");
  static_assert(GPTQ_PREPARE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
  if (gptq::prepare_workspace_bytes(d, act_order) > GPTQ_PREPARE_NOALLOC_SCRATCH_BYTES)
    return fail(GPTQ_EUNSUPPORTED, fn, "workspace exceeds the static scratch");
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return fail(GPTQ_EHIP, fn, std::string("scratch lookup: ") + hipGetErrorString(e));
  gptq::launch_prepare(H, d, percdamp, act_order, perm, dead, info, ws, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

// ------------------------------------------------------------------ quantize
gptq_status gptq_quantize_layer_workspace_size(int64_t r, int64_t c, int64_t blocksize, size_t* bytes) {
  const char* fn = "gptq_quantize_layer_workspace_size";
  if (!bytes) return fail(GPTQ_EINVAL, fn, "bytes is NULL");
  if (r < 0 || c < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (blocksize < 1 || blocksize > 128) return fail(GPTQ_EUNSUPPORTED, fn, "blocksize must be 1..128");
  if (r > kMaxRows || c > kMaxDim) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  *bytes = (r > 0 && c > 0) ? gptq::quantize_workspace_bytes(r, c, blocksize) : 0;
  return ok();
}

gptq_status gptq_quantize_layer(const void* W, gptq_dtype wt, int64_t r, int64_t c, int64_t ldw,
                                const float* U, const int32_t* perm, const uint8_t* dead, int bits,
                                int sym, int64_t groupsize, int64_t blocksize, uint8_t* codes, float* scales,
                                int32_t* zeros, int32_t* g_idx, float* W_hat, float* row_loss, void* ws,
                                size_t ws_bytes, void* stream) {
  const char* fn = "gptq_quantize_layer";
  if (r < 0 || c < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(wt)) return fail(GPTQ_EDTYPE, fn, "wt must be GPTQ_F32, GPTQ_BF16 or GPTQ_F16");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return fail(GPTQ_EUNSUPPORTED, fn, "bits must be 2, 3, 4 or 8");
  if (sym != 0 && sym != 1) return fail(GPTQ_EINVAL, fn, "sym must be 0 or 1");
  if (blocksize < 1 || blocksize > 128) return fail(GPTQ_EUNSUPPORTED, fn, "blocksize must be 1..128");
  if (groupsize > 0 && (groupsize % blocksize) != 0 && (blocksize % groupsize) != 0)
    return fail(GPTQ_EUNSUPPORTED, fn, "groupsize must be a multiple or a divisor of blocksize");
  if (r > kMaxRows || c > kMaxDim) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if (r > kMaxGroups256) return fail(GPTQ_EUNSUPPORTED, fn, "r too large: one 256-thread workgroup per row");
  if (r == 0 || c == 0) return ok();
  if (ldw < c) return fail(GPTQ_ESHAPE, fn, "ldw < c");
  if (!W || !U || !codes || !scales || !zeros || !g_idx) return fail(GPTQ_EINVAL, fn, "a required pointer is NULL");
  if (!aligned(W, elem_size(wt)) || !aligned(U, 4) || !aligned(scales, 4) || !aligned(zeros, 4) ||
      !aligned(g_idx, 4) || (perm && !aligned(perm, 4)) || (W_hat && !aligned(W_hat, 4)) ||
      (row_loss && !aligned(row_loss, 4)))
    return fail(GPTQ_EALIGN, fn, "misaligned pointer");
  const size_t need = gptq::quantize_workspace_bytes(r, c, blocksize);
  if (!ws || ws_bytes < need) return fail(GPTQ_EWORKSPACE, fn, "workspace needs " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(GPTQ_EALIGN, fn, "workspace not 256-byte aligned");
  gptq::QuantArgs a;
  a.W = W; a.wt = (int)wt; a.r = r; a.c = c; a.ldw = ldw; a.U = U; a.perm = perm; a.dead = dead;
  a.bits = bits; a.sym = sym; a.groupsize = groupsize; a.blocksize = blocksize; a.codes = codes; a.scales = scales;
  a.zeros = zeros; a.g_idx = g_idx; a.W_hat = W_hat; a.row_loss = row_loss; a.ws = ws;
  gptq::launch_quantize(a, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

// ------------------------------------------------------------------ pack
gptq_status gptq_pack(const uint8_t* codes, int64_t r, int64_t c, int bits, const int32_t* col_perm,
                      uint32_t* packed, int64_t ld_words, void* stream) {
  const char* fn = "gptq_pack";
  if (r < 0 || c < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (bits != 3 && bits != 4) return fail(GPTQ_EUNSUPPORTED, fn, "packing supports 3 and 4 bits");
  if (bits == 4 && c % 8 != 0) return fail(GPTQ_ESHAPE, fn, "4-bit packing needs c % 8 == 0");
  if (bits == 3 && c % 32 != 0) return fail(GPTQ_ESHAPE, fn, "3-bit packing needs c % 32 == 0");
  if (r > kMaxRows || c > (int64_t)INT_MAX) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if (ld_words < (bits == 4 ? c / 8 : c / 32 * 3)) return fail(GPTQ_ESHAPE, fn, "ld_words < c * bits / 32");
  // one thread per packed chunk (8 codes at 4 bits, 32 codes at 3 bits or with col_perm)
  if (groups_for(r * groups_for(c, (bits == 4 && !col_perm) ? 8 : 32), 256) > kMaxGroups256)
    return fail(GPTQ_EUNSUPPORTED, fn, "too many packed chunks for one launch");
  if (r == 0 || c == 0) return ok();
  if (!codes || !packed) return fail(GPTQ_EINVAL, fn, "codes or packed is NULL");
  if (!aligned(codes, 16) || !aligned(packed, 4)) return fail(GPTQ_EALIGN, fn, "codes must be 16-byte aligned");
  if (col_perm && !aligned(col_perm, 4)) return fail(GPTQ_EALIGN, fn, "col_perm misaligned");
  gptq::launch_pack(codes, r, c, bits, col_perm, packed, ld_words, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

// ------------------------------------------------------------------ dequantizing product
gptq_status gptq_dequant_gemv(const uint32_t* packed, int64_t r, int64_t c, int bits, int64_t ld_words,
                              const float* scales, const int32_t* zeros, int64_t ld_groups, int64_t groupsize,
                              const int32_t* col_perm, const void* x, gptq_dtype xt, float* y, void* stream) {
  const char* fn = "gptq_dequant_gemv";
  if (r < 0 || c < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (bits != 3 && bits != 4) return fail(GPTQ_EUNSUPPORTED, fn, "bits must be 3 or 4");
  if (!valid_dtype(xt)) return fail(GPTQ_EINVAL, fn, "xt must be a gptq_dtype");
  if (xt == GPTQ_F32) return fail(GPTQ_EDTYPE, fn, "x must be GPTQ_BF16 or GPTQ_F16 (16-bit activations)");
  if (c % 32 != 0) return fail(GPTQ_ESHAPE, fn, "c % 32 != 0");
  if (r > kMaxRows) return fail(GPTQ_EUNSUPPORTED, fn, "r too large");
  if (c > 0 && gptq::plan_gemv(c).S == 0) return fail(GPTQ_EUNSUPPORTED, fn, "c > 49152");
  const bool grouped = groupsize > 0 && groupsize < c;
  if (grouped && groupsize % 32 != 0) return fail(GPTQ_EUNSUPPORTED, fn, "groupsize must be a multiple of 32");
  const int64_t n_groups = grouped ? (c + groupsize - 1) / groupsize : 1;
  if (r == 0) return ok();
  if (!y) return fail(GPTQ_EINVAL, fn, "y is NULL");
  if (!aligned(y, 4)) return fail(GPTQ_EALIGN, fn, "y misaligned");
  if (c > 0) {
    if (ld_words < c / 32 * bits) return fail(GPTQ_ESHAPE, fn, "ld_words < c * bits / 32");
    if (ld_groups < n_groups) return fail(GPTQ_ESHAPE, fn, "ld_groups < number of groups");
    if (!packed || !scales || !zeros || !x) return fail(GPTQ_EINVAL, fn, "a required pointer is NULL");
    if (bits == 4 && (!aligned(packed, 16) || ld_words % 4 != 0))
      return fail(GPTQ_EALIGN, fn, "4-bit words need a 16-byte aligned base and ld_words % 4 == 0");
    if (!aligned(packed, 4) || !aligned(scales, 4) || !aligned(zeros, 4) || (col_perm && !aligned(col_perm, 4)))
      return fail(GPTQ_EALIGN, fn, "misaligned pointer");
    if (!aligned(x, col_perm ? 2 : 16)) return fail(GPTQ_EALIGN, fn, "x must be 16-byte aligned");
  }
  gptq::launch_dequant_gemv(packed, r, c, bits, ld_words, scales, zeros, ld_groups, groupsize, col_perm, x,
                            xt == GPTQ_F16 ? 1 : 0, y, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

// ------------------------------------------------------------------ Hadamard pre-rotation
gptq_status gptq_hadamard_rotate(const void* A, gptq_dtype at, int64_t rows, int64_t d, int64_t lda,
                                 int64_t block, void* out, gptq_dtype ot, int64_t ldo, void* stream) {
  const char* fn = "gptq_hadamard_rotate";
  if (rows < 0 || d < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(at) || !valid_dtype(ot)) return fail(GPTQ_EDTYPE, fn, "at and ot must be gptq_dtype values");
  if (block <= 0 && d > 0) {
    block = d & -d;
    if (block > 8192) block = 8192;
  }
  if (d > 0 && (block < 32 || block > 8192 || (block & (block - 1)) != 0))
    return fail(GPTQ_EUNSUPPORTED, fn, "block must be a power of two in 32 .. 8192");
  if (d > 0 && d % block != 0) return fail(GPTQ_ESHAPE, fn, "block must divide d");
  if (rows == 0 || d == 0) return ok();
  if (lda < d || ldo < d) return fail(GPTQ_ESHAPE, fn, "lda and ldo must be >= d");
  if (rows > kMaxRows || d > kMaxRows) return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if ((rows * (d / block)) >= (int64_t)INT_MAX) return fail(GPTQ_EUNSUPPORTED, fn, "too many blocks");
  // one workgroup per tile of 4096 elements (8192 for b = 8192)
  if (groups_for(rows * (d / block), block == 8192 ? 1 : 4096 / block) > kMaxGroups256)
    return fail(GPTQ_EUNSUPPORTED, fn, "too many tiles for one launch");
  if (!A || !out) return fail(GPTQ_EINVAL, fn, "A or out is NULL");
  if (!aligned(A, elem_size(at)) || !aligned(out, elem_size(ot))) return fail(GPTQ_EALIGN, fn, "misaligned pointer");
  const int64_t ea = extent_bytes(rows, lda, d, (int64_t)elem_size(at));
  const int64_t eo = extent_bytes(rows, ldo, d, (int64_t)elem_size(ot));
  if (ea < 0 || eo < 0) return fail(GPTQ_EUNSUPPORTED, fn, "matrix extent exceeds 2^63 bytes");
  if (overlaps(A, ea, out, eo) && !(A == out && at == ot && lda == ldo))
    return fail(GPTQ_EINVAL, fn, "out overlaps A (only exact in-place use is allowed)");
  gptq::launch_hadamard(A, (int)at, lda, rows, d, block, out, (int)ot, ldo, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

// ------------------------------------------------------------------ quantized linear forward
gptq_status gptq_linear_forward(const void* X, gptq_dtype xt, int64_t n_tok, int64_t d, int64_t ldx,
                                const void* W_hat, gptq_dtype wt, int64_t r, int64_t ldw, int act, const void* G,
                                int64_t ldg, void* Y, gptq_dtype yt, int64_t ldy, void* stream) {
  const char* fn = "gptq_linear_forward";
  if (n_tok < 0 || d < 0 || r < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(xt) || !valid_dtype(yt) || !valid_dtype(wt))
    return fail(GPTQ_EINVAL, fn, "xt, wt and yt must be gptq_dtype values");
  if (xt == GPTQ_F32) return fail(GPTQ_EDTYPE, fn, "X must be GPTQ_BF16 or GPTQ_F16");
  if (wt != GPTQ_F32 && wt != xt) return fail(GPTQ_EDTYPE, fn, "W_hat must be GPTQ_F32 or of X's type");
  if (act != 0 && act != 1) return fail(GPTQ_EINVAL, fn, "act must be 0 (none) or 1 (silu(G) * up)");
  if (d < 64 || d % 64 != 0) return fail(GPTQ_EUNSUPPORTED, fn, "d must be a positive multiple of 64");
  if (r > (int64_t)INT_MAX / 2 || d > (int64_t)INT_MAX / 2 || n_tok > kMaxRows ||
      groups_for(n_tok, 256) * groups_for(r, 256) > kMaxGroups256)   // one workgroup per 256 x 256 tile
    return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if (n_tok == 0 || r == 0) return ok();
  if (ldx < d || ldw < d || ldy < r || (act == 1 && ldg < r)) return fail(GPTQ_ESHAPE, fn, "leading dimension too small");
  if (!X || !W_hat || !Y || (act == 1 && !G)) return fail(GPTQ_EINVAL, fn, "a required pointer is NULL");
  const bool w16 = wt != GPTQ_F32;
  if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(W_hat, 16) || ldw % (w16 ? 8 : 4) != 0)
    return fail(GPTQ_EALIGN, fn, "X and W_hat rows must start on 16 bytes");
  if (w16 && (ldx >= (int64_t(1) << 22) || ldw >= (int64_t(1) << 22)))
    return fail(GPTQ_EUNSUPPORTED, fn, "16-bit W_hat needs ldx and ldw below 2^22");
  if (!aligned(Y, elem_size(yt)) || (act == 1 && !aligned(G, 2))) return fail(GPTQ_EALIGN, fn, "misaligned pointer");
  const int64_t ey = extent_bytes(n_tok, ldy, r, (int64_t)elem_size(yt));
  const int64_t ex = extent_bytes(n_tok, ldx, d, 2);
  const int64_t ew = extent_bytes(r, ldw, d, (int64_t)elem_size(wt));
  const int64_t eg = act == 1 ? extent_bytes(n_tok, ldg, r, 2) : 0;
  if (ey < 0 || ex < 0 || ew < 0 || eg < 0) return fail(GPTQ_EUNSUPPORTED, fn, "matrix extent exceeds 2^63 bytes");
  if (overlaps(Y, ey, X, ex) || overlaps(Y, ey, W_hat, ew)) return fail(GPTQ_EINVAL, fn, "Y overlaps X or W_hat");
  if (act == 1 && overlaps(Y, ey, G, eg) && !(Y == G && yt == xt && ldy == ldg))
    return fail(GPTQ_EINVAL, fn, "Y overlaps G (only Y == G with the same type and stride is allowed)");
  gptq::launch_linear(X, (int)xt, n_tok, d, ldx, W_hat, w16, r, ldw, act, G, ldg, Y, (int)yt, ldy,
                      reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

gptq_status gptq_round16(const float* src, int64_t rows, int64_t cols, int64_t lds, gptq_dtype dt, void* dst,
                         int64_t ldd, void* stream) {
  const char* fn = "gptq_round16";
  if (rows < 0 || cols < 0) return fail(GPTQ_EINVAL, fn, "negative size");
  if (!valid_dtype(dt)) return fail(GPTQ_EINVAL, fn, "dt must be a gptq_dtype value");
  if (dt == GPTQ_F32) return fail(GPTQ_EDTYPE, fn, "dt must be GPTQ_BF16 or GPTQ_F16");
  if (rows > kMaxRows || cols > kMaxRows || groups_for(rows * ((cols + 3) / 4), 256) > kMaxGroups256)
    return fail(GPTQ_EUNSUPPORTED, fn, "size too large");
  if (rows == 0 || cols == 0) return ok();
  if (lds < cols || ldd < cols) return fail(GPTQ_ESHAPE, fn, "leading dimension too small");
  if (!src || !dst) return fail(GPTQ_EINVAL, fn, "a required pointer is NULL");
  if (!aligned(src, 4) || !aligned(dst, 2)) return fail(GPTQ_EALIGN, fn, "misaligned pointer");
  const int64_t es = extent_bytes(rows, lds, cols, 4), ed = extent_bytes(rows, ldd, cols, 2);
  if (es < 0 || ed < 0) return fail(GPTQ_EUNSUPPORTED, fn, "matrix extent exceeds 2^63 bytes");
  if (overlaps(src, es, dst, ed)) return fail(GPTQ_EINVAL, fn, "dst overlaps src");
  gptq::launch_round16(src, rows, cols, lds, (int)dt, dst, ldd, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

}  // extern "C"
