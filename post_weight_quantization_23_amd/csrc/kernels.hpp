// Host-side launch interfaces of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

enum { MASK_NONE = 0, MASK_UPPER = 1, MASK_LOWER = 2 };

// See gemm_f32.hip for the exact contract.
struct GemmArgs {
  int M, N, K;
  const float* A;
  int64_t lda;
  int a_trans, a_mask, a_off;
  const float* B;
  int64_t ldb;
  int b_trans, b_mask, b_off;
  float* C;
  int64_t ldc;
  float alpha, beta;
  int upper_only;
};
void launch_gemm_f32(const GemmArgs& g, hipStream_t s);
// Two independent products in one launch (one grid, the second problem's
// tiles after the first's).
void launch_gemm_f32_pair(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s);

// --- Hessian (syrk.hip) ---
struct SyrkPlan {
  int tile;        // output tile edge
  int tiles;       // upper-triangle tiles
  int splits;      // token splits (1 = accumulate straight into H)
  int64_t chunk;   // tokens per split (multiple of the K-step)
};
SyrkPlan plan_syrk(int64_t d, int64_t n_tok);
size_t syrk_workspace_bytes(const SyrkPlan& p);
// dtype: 1 = bf16, 2 = fp16.  ws holds the split partials (may be null when
// p.splits == 1).
void launch_syrk16(float* H, int64_t d, const void* X, int dtype, int64_t n_tok, int64_t ldx,
                   const SyrkPlan& p, float* ws, hipStream_t s);

// --- Preparation (prepare.hip) ---
size_t prepare_workspace_bytes(int64_t d, int act_order);
void launch_prepare(float* H, int64_t d, float percdamp, int act_order, int32_t* perm,
                    uint8_t* dead, int32_t* info, void* ws, hipStream_t s);

// --- Quantization (quantize.hip) ---
// Blocks per super-block: repairs inside it are applied as the loop goes,
// repairs beyond it deferred to one product (quantize.hip).
constexpr int64_t kSuperBlocks = 4;
// The fp32 working copy of W (r x c) and the scaled errors of one
// super-block (r x kSuperBlocks * blocksize), each 256-byte aligned
// (workspace.hip).
size_t quantize_workspace_bytes(int64_t r, int64_t c, int64_t blocksize);
struct QuantArgs {
  const void* W;
  int wt;  // 0 f32, 1 bf16, 2 f16
  int64_t r, c, ldw;
  const float* U;
  const int32_t* perm;
  const uint8_t* dead;
  int bits;
  int sym;  // symmetric ruler
  int64_t groupsize, blocksize;
  uint8_t* codes;
  float* scales;
  int32_t* zeros;
  int32_t* g_idx;
  float* W_hat;
  float* row_loss;
  void* ws;
};
void launch_quantize(const QuantArgs& a, hipStream_t s);

// --- Pack (pack.hip) ---
// perm (nullable): packed column j takes the code of original column perm[j].
void launch_pack(const uint8_t* codes, int64_t r, int64_t c, int bits, const int32_t* perm,
                 uint32_t* packed, int64_t ld_words, hipStream_t s);

// --- Hadamard pre-rotation (hadamard.hip) ---
// at / ot: 0 f32, 1 bf16, 2 f16; block a power of two in 32 .. 8192 dividing d.
void launch_hadamard(const void* A, int at, int64_t lda, int64_t rows, int64_t d, int64_t block, void* out,
                     int ot, int64_t ldo, hipStream_t s);

// --- Quantized linear forward over the calibration tokens (linear.hip) ---
// xt: 1 bf16, 2 f16; yt: 0 f32, 1 bf16, 2 f16; act: 0 none, 1 silu(G) * up.
// W: fp32, or (w16) already rounded to xt's 16-bit type.
void launch_linear(const void* X, int xt, int64_t n_tok, int64_t d, int64_t ldx, const void* W, bool w16,
                   int64_t r, int64_t ldw, int act, const void* G, int64_t ldg, void* Y, int yt, int64_t ldy,
                   hipStream_t s);
// dst[rows x cols] (16-bit type dt: 1 bf16, 2 f16) = round16(src), element-wise.
void launch_round16(const float* src, int64_t rows, int64_t cols, int64_t lds, int dt, void* dst, int64_t ldd,
                    hipStream_t s);

// --- Dequantize-on-the-fly product (gemv.hip) ---
struct GemvPlan {
  int S;         // waves sharing one row's columns (0: c too large)
  int nch_lane;  // 32-column chunks per lane
};
GemvPlan plan_gemv(int64_t c);
void launch_dequant_gemv(const uint32_t* packed, int64_t r, int64_t c, int bits, int64_t ld_words,
                         const float* scales, const int32_t* zeros, int64_t ld_groups, int64_t groupsize,
                         const int32_t* perm, const void* x, int x_f16, float* y, hipStream_t s);

}  // namespace gptq
