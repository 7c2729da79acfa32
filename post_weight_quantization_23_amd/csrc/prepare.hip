// Preparation of H: dead inputs, act-order, damping, and the upper Cholesky
// factor of the inverse ("GPTQ, with the code open", sections "Paper vs. code"
// and "From one repair to a whole model").
//
// The page's own route is three steps (Cholesky of H, inverse, Cholesky of
// the inverse, 4d^3/3 flops).  Here U comes from one recursion over H (2d^3/3
// flops): if H = V V^T with V upper triangular (a Cholesky factorisation run
// from the last column backwards), then H^{-1} = V^{-T} V^{-1}, so U = V^{-1} is
// upper triangular with U^T U = H^{-1} -- the unique factor the method uses.
// For H = [[A, B], [B^T, C]] (C the trailing block):
//     U22 = rec(C)            (so V22 = U22^{-1})
//     T   = B U22^T           (= V12, the off-diagonal block of V)
//     A'  = A - T T^T         (what remains of A after C is eliminated)
//     U11 = rec(A')
//     U12 = -U11 T U22
// All products are fp32 matrix-core GEMMs (gemm_f32.hip).  Blocks of <= 128
// are factored by one workgroup in LDS with the same recursion down to 16,
// where one wave runs the column-by-column factorisation and inversion (the
// 32-level products of that wave on 16 x 16 matrix-core tiles).
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 128;      // leaf block handled by one workgroup
constexpr int LDM = NB + 1;  // LDS row stride of the leaf block

// ---------------------------------------------------------------------------
// Diagonal pass, one workgroup: dead inputs (H[j][j] == 0 becomes 1), the
// NaN/Inf check and the info reset, the undamped diagonal for act-order, the
// identity permutation when perm is given without act-order, and the damping
// lambda = percdamp * mean(diag) (after the dead inputs' 1s), summed in a
// fixed order, added to every diagonal entry.  The damping commutes with the
// symmetric permutation of act-order (it adds the same lambda to every
// diagonal entry), so it is applied here in both cases.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void diag_prep_kernel(float* H, int64_t d, uint8_t* dead, int32_t* info,
                                                         float* diag_out, int32_t* perm_identity,
                                                         float percdamp) {
  __shared__ int bad;
  __shared__ float part[1024];
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  float sum = 0.f;
  for (int64_t j = threadIdx.x; j < d; j += 1024) {
    float v = H[j * d + j];
    if (!__builtin_isfinite(v)) atomicOr(&bad, 1);
    const bool dj = (v == 0.0f);
    dead[j] = dj ? 1 : 0;
    if (dj) v = 1.0f;
    diag_out[j] = v;
    sum += v;
    if (perm_identity) perm_identity[j] = (int32_t)j;
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float lam = percdamp * (part[0] / (float)d);
  for (int64_t j = threadIdx.x; j < d; j += 1024) H[j * d + j] = diag_out[j] + lam;
  if (threadIdx.x == 0) *info = bad ? -1 : 0;
}

// Act-order: rank of column i = #{j : diag_j > diag_i} + #{j < i : diag_j == diag_i}
// (a stable descending sort); perm[rank] = i.  A NaN diagonal (already
// reported through info) sorts as -inf so the ranks always form a permutation.
GPTQ_DEV float sort_key(float v) { return __builtin_isnan(v) ? -__builtin_inff() : v; }

// One workgroup per 64 columns i; its four waves count over the four
// quarters of j and the partial counts are summed through LDS.  The scan
// over j reads the same diag[j] in every lane of a wave (a broadcast).
__global__ __launch_bounds__(256) void rank_kernel(const float* diag, int64_t d, int32_t* perm) {
  __shared__ int64_t part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  const float di = i < d ? sort_key(diag[i]) : 0.f;
  const int64_t q = (d + 3) / 4;
  const int64_t j0 = wave * q, j1 = min(d, j0 + q);
  int64_t rank = 0;
  int64_t j = j0;
  for (; j + 8 <= j1; j += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = sort_key(diag[j + u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += (v[u] > di) || (v[u] == di && j + u < i);
  }
  for (; j < j1; ++j) {
    const float v = sort_key(diag[j]);
    rank += (v > di) || (v == di && j < i);
  }
  part[wave][lane] = rank;
  __syncthreads();
  if (wave == 0 && i < d) perm[part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane]] = (int32_t)i;
}

// dst[a][b] = src[min(pa,pb)][max(pa,pb)] for a <= b (upper triangle of the
// symmetrically permuted matrix).  One row a per blockIdx.y.
__global__ __launch_bounds__(256) void permute_upper_kernel(const float* src, int64_t d,
                                                            const int32_t* perm, float* dst) {
  const int64_t a = blockIdx.y;
  const int64_t pa = perm[a];
  for (int64_t b = a + (int64_t)blockIdx.x * 256 + threadIdx.x; b < d; b += (int64_t)gridDim.x * 256) {
    const int64_t pb = perm[b];
    const int64_t r = min(pa, pb), c = max(pa, pb);
    dst[a * d + b] = src[r * d + c];
  }
}

__global__ __launch_bounds__(256) void copy_block_kernel(const float* src, float* dst, int64_t ld,
                                                         int rows, int cols) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * cols) return;
  const int64_t r = idx / cols, c = idx % cols;
  dst[r * ld + c] = src[r * ld + c];
}

// Zeros strictly below the diagonal, one row per blockIdx.y; rows of a d with
// d % 4 == 0 start 16-byte aligned and take four columns per thread.
__global__ __launch_bounds__(256) void zero_lower_kernel(float* H, int64_t d) {
  const int64_t r = blockIdx.y;
  float* row = H + r * d;
  if ((d & 3) == 0) {
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t c = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); c < r; c += 4 * (int64_t)gridDim.x * 256) {
      if (c + 4 <= r) {
        *reinterpret_cast<floatx4*>(row + c) = z;
      } else {
        for (int64_t e = c; e < r; ++e) row[e] = 0.f;
      }
    }
  } else {
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < r; c += (int64_t)gridDim.x * 256) row[c] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Leaf: U of one diagonal block of <= 128 in LDS.
// ---------------------------------------------------------------------------

// One wave: the S x S diagonal block of M at (o, o) (S = 16) holds the upper
// triangle of the (updated) H block; it is replaced by U = V^{-1} where
// V V^T = block, V upper.  One backward sweep j = S-1 .. 0 does both:
//   factor : V[:, j] = A[:, j] / sqrt(A[j][j]);  A[0:j, 0:j] -= V[0:j, j] V[0:j, j]^T
//   invert : X[j, :] /= V[j][j];  X[0:j, :] -= V[0:j, j] X[j, :]   (X starts as I)
// (row j of X is final at step j: every later row has already been removed).
// Registers only: lane k of a 16-lane row holds column k of the symmetric
// block A and column k of X.  With p = A[j][j] and a_i = A[i][j] (lane j's
// A[i]), both updates are  col[i] -= a_i * col[j] / p  for i < j -- on the A
// side col[j] = A[j][k] = A[k][j] by symmetry, on the X side col[j] = X[j][k]
// before its scaling -- and the X side then scales col[j] by 1/sqrt(p).  A
// non-positive or NaN pivot is recorded as the sweep goes (the first one
// found) and reported once at the end.
template <int S>
__device__ __forceinline__ void leaf_sweep(float* M, int o, int32_t* info, int64_t gbase, int pad) {
  static_assert(S == 16, "the row broadcast spans 16 lanes");
  // Every 16-lane row of the wave holds the symmetric block, lane k of a row
  // column k (col[i] = A[i][k]); row 1 also holds X (lane 16 + c: column c).
  // A[i][j] reaches every lane of a row from its lane j by a DPP row
  // broadcast, so each row updates its own copy without leaving the VALU.
  const int lane = threadIdx.x & 63;
  const int k = lane & 15;
  const bool xside = (lane >> 4) == 1;
  float col[S], xc[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    col[i] = M[(o + min(i, k)) * LDM + o + max(i, k)];
    xc[i] = i == k ? 1.f : 0.f;
  }
  // row_newbcast: lane src of each 16-lane row to the whole row (src is a
  // constant in every unrolled step, so the switch folds away)
  auto bc = [](float v, int src) {
    const int iv = __float_as_int(v);
    int r;
    switch (src) {
#define GPTQ_RB(n) \
  case n: r = __builtin_amdgcn_mov_dpp(iv, 0x150 + n, 0xF, 0xF, true); break;
      GPTQ_RB(0) GPTQ_RB(1) GPTQ_RB(2) GPTQ_RB(3) GPTQ_RB(4) GPTQ_RB(5) GPTQ_RB(6) GPTQ_RB(7)
      GPTQ_RB(8) GPTQ_RB(9) GPTQ_RB(10) GPTQ_RB(11) GPTQ_RB(12) GPTQ_RB(13) GPTQ_RB(14)
      default: r = __builtin_amdgcn_mov_dpp(iv, 0x150 + 15, 0xF, 0xF, true); break;
#undef GPTQ_RB
    }
    return __int_as_float(r);
  };
  int bad = -1;   // sweep position of the first non-positive pivot found
#pragma unroll
  for (int j = S - 1; j >= 0; --j) {
    const float piv = bc(col[j], j);
    const float rv = __builtin_amdgcn_rsqf(piv);   // 1/sqrt(pivot), ~1 ulp
    const float inv = rv * rv;
    const float fa = col[j] * inv, fx = xc[j] * inv;
    {
      const float ps = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(piv)));
      bad = (bad < 0 && !(ps > 0.f)) ? j : bad;
    }
#pragma unroll
    for (int i = 0; i < j; ++i) {
      const float ai = bc(col[i], j);
      col[i] = __builtin_fmaf(-ai, fa, col[i]);
      xc[i] = __builtin_fmaf(-ai, fx, xc[i]);
    }
    xc[j] *= rv;
  }
  if (xside) {
#pragma unroll
    for (int i = 0; i < S; ++i) M[(o + i) * LDM + o + k] = (k >= i) ? xc[i] : 0.f;
  }
  if (lane == 0 && bad >= 0 && (o + bad) >= pad) {
    if (*info == 0) *info = (int32_t)(gbase + (o + bad - pad) + 1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One wave: C (16 x 16) = alpha * A (16 x 16) * op(B) [+ C] on LDS arrays with
// v_mfma_f32_16x16x4f32 (four steps of K = 4).  op(B) = B^T (B stored 16 x 16
// as [n][k]) when bt, else B ([k][n]).  With upper_only only entries on and
// above the diagonal are written.  Operand layout of the instruction: lane l
// supplies A[l % 16][4s + l / 16] and B[4s + l / 16][l % 16]; it receives
// D[4 (l / 16) + v][l % 16] in accumulator v.
__device__ __forceinline__ void wave_gemm16(const float* A, int lda, const float* B, int ldb, bool bt, float* C,
                                            int ldc, float alpha, bool accumulate, bool upper_only) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int kk = 4 * s4 + kq;
    const float a = A[r * lda + kk];
    const float b = bt ? B[r * ldb + kk] : B[kk * ldb + r];
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, d, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = 4 * kq + v;
    if (!upper_only || r >= i) {
      float* p = C + i * ldc + r;
      *p = accumulate ? __builtin_fmaf(alpha, d[v], *p) : alpha * d[v];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Which K-blocks (of the output block's edge) can hold non-zero products for
// output block (bi, bj)
// when one operand is triangular (its zeros below the diagonal are exact
// zeros in LDS): KM_NONE all; KM_A_UPPER A upper (kb >= bi); KM_BT_UPPER
// op(B) = B^T with B upper (kb >= bj); KM_B_UPPER op(B) = B upper (kb <= bj).
enum { KM_NONE = 0, KM_A_UPPER = 1, KM_BT_UPPER = 2, KM_B_UPPER = 3 };

GPTQ_DEV bool k_block_live(int km, int kb, int bi, int bj) {
  if (km == KM_A_UPPER) return kb >= bi;
  if (km == KM_BT_UPPER) return kb >= bj;
  if (km == KM_B_UPPER) return kb <= bj;
  return true;
}

// C (H x H) = alpha * A * op(B) [+ C] on LDS arrays, K = H, on the fp32
// matrix cores.  op(B) = B^T (B stored H x K) when bt, else B (K x H).
// K-blocks that a triangular operand zeroes are skipped, and with upper_only
// blocks strictly below the diagonal are skipped.
//   H = 64: 32 x 32 output blocks (v_mfma_f32_32x32x2f32), one per wave.
//     Lane l supplies A[l % 32][k + l / 32] and B[k + l / 32][l % 32] and
//     receives D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32] in accumulator v.
//     Diagonal blocks are written whole (their entries below the diagonal
//     are never read as U).
//   H = 32: 16 x 16 output blocks (v_mfma_f32_16x16x4f32), one per wave, so
//     all four waves work.  Lane l supplies A[l % 16][k + l / 16] and
//     B[k + l / 16][l % 16] and receives D[4 (l / 16) + v][l % 16].  With
//     upper_only only entries on and above the diagonal are written.
// Even and odd K-steps go to two accumulators, so consecutive MFMAs do not
// wait on each other.
template <int H>
__device__ __forceinline__ void lds_gemm(const float* A, int lda, const float* B, int ldb, int bt, float* C, int ldc,
                                         float alpha, bool accumulate, bool upper_only, int km) {
  constexpr int BS = H / 2, NBK = 2;   // output block edge; blocks per dimension
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bi = wave / NBK, bj = wave % NBK;
  if (upper_only && bj < bi) return;
  if constexpr (H == 64) {
    floatx16 acc0, acc1;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc0[v] = acc1[v] = 0.f;
    const int r = BS * bi + (lane & 31), c = BS * bj + (lane & 31), kh = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) {
      if (!k_block_live(km, kb, bi, bj)) continue;   // wave-uniform
#pragma unroll
      for (int k = BS * kb; k < BS * kb + BS; k += 4) {
        const float a0 = A[r * lda + k + kh], a1 = A[r * lda + k + 2 + kh];
        const float b0 = bt ? B[c * ldb + k + kh] : B[(k + kh) * ldb + c];
        const float b1 = bt ? B[c * ldb + k + 2 + kh] : B[(k + 2 + kh) * ldb + c];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc1, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = BS * bi + 8 * (v >> 2) + 4 * kh + (v & 3);
      float* p = C + i * ldc + c;
      const float sum = acc0[v] + acc1[v];
      *p = accumulate ? __builtin_fmaf(alpha, sum, *p) : alpha * sum;
    }
  } else {
    static_assert(H == 32, "the leaf's products are 64 or 32 wide");
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) {
      if (!k_block_live(km, kb, bi, bj)) continue;   // wave-uniform
#pragma unroll
      for (int s4 = 0; s4 < BS / 4; ++s4) {
        const int k = BS * kb + 4 * s4 + kq;
        const float a = A[(BS * bi + r) * lda + k];
        const float b = bt ? B[(BS * bj + r) * ldb + k] : B[k * ldb + BS * bj + r];
        if (s4 & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = BS * bi + 4 * kq + v, j = BS * bj + r;
      if (upper_only && j < i) continue;
      float* p = C + i * ldc + j;
      const float sum = acc0[v] + acc1[v];
      *p = accumulate ? __builtin_fmaf(alpha, sum, *p) : alpha * sum;
    }
  }
}

// In-LDS recursion on the diagonal block (o, n), n in {32, 64, 128}; level
// temporaries T1/T2 of each size are separate (T64a/T64b for n == 128,
// T32a/T32b for n == 64, T16a/T16b for n == 32).  On return M[o:o+n, o:o+n]
// holds U with exact zeros below the diagonal.  With H = [[A, B], [B^T, C]]:
//   U22 = rec(C);  T = B U22^T;  A -= T T^T;  U11 = rec(A);  U12 = -(U11 T) U22.
// A block of 32 is done by wave 0 alone (16-wide sweeps and 16 x 16 products),
// larger ones by all four waves.
struct LeafScratch {
  float *T64a, *T64b, *T32a, *T32b, *T16a, *T16b;
};

template <int N>
__device__ __forceinline__ void leaf_rec(float* M, int o, const LeafScratch& ts, int32_t* info, int64_t gbase, int pad) {
  if constexpr (N == 32) {
    if ((threadIdx.x >> 6) == 0) {
      constexpr int h = 16, ldt = 17;
      const int o2 = o + h;
      float* Bm = M + o * LDM + o2;
      float* U22 = M + o2 * LDM + o2;
      float* U11 = M + o * LDM + o;
      leaf_sweep<16>(M, o2, info, gbase, pad);
      wave_gemm16(Bm, LDM, U22, LDM, true, ts.T16a, ldt, 1.f, false, false);      // T = B U22^T
      wave_gemm16(ts.T16a, ldt, ts.T16a, ldt, true, U11, LDM, -1.f, true, true);  // A -= T T^T
      leaf_sweep<16>(M, o, info, gbase, pad);
      wave_gemm16(U11, LDM, ts.T16a, ldt, false, ts.T16b, ldt, 1.f, false, false);  // T2 = U11 T
      wave_gemm16(ts.T16b, ldt, U22, LDM, false, Bm, LDM, -1.f, false, false);      // U12 = -T2 U22
      // The 32 x 32 block's lower-left quarter received the level above's
      // update of this diagonal block (those products work on whole 32 x 32
      // tiles); U is zero there.
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int v = 0; v < 4; ++v) M[(o2 + 4 * (lane >> 4) + v) * LDM + o + (lane & 15)] = 0.f;
    }
    __syncthreads();
  } else {
    constexpr int h = N / 2;
    const int o2 = o + h;
    float* T1 = (h == 64) ? ts.T64a : ts.T32a;
    float* T2 = (h == 64) ? ts.T64b : ts.T32b;
    constexpr int ldt = h + 1;
    float* Bm = M + o * LDM + o2;
    float* U22 = M + o2 * LDM + o2;
    float* U11 = M + o * LDM + o;
    leaf_rec<h>(M, o2, ts, info, gbase, pad);
    lds_gemm<h>(Bm, LDM, U22, LDM, 1, T1, ldt, 1.f, false, false, KM_BT_UPPER);   // T1 = B U22^T
    __syncthreads();
    lds_gemm<h>(T1, ldt, T1, ldt, 1, U11, LDM, -1.f, true, true, KM_NONE);        // A -= T1 T1^T
    __syncthreads();
    leaf_rec<h>(M, o, ts, info, gbase, pad);
    lds_gemm<h>(U11, LDM, T1, ldt, 0, T2, ldt, 1.f, false, false, KM_A_UPPER);    // T2 = U11 T1
    __syncthreads();
    lds_gemm<h>(T2, ldt, U22, LDM, 0, Bm, LDM, -1.f, false, false, KM_B_UPPER);   // U12 = -T2 U22
    __syncthreads();
  }
}

constexpr int LEAF_FLOATS = NB * LDM + 2 * 64 * 65 + 2 * 32 * 33 + 2 * 16 * 17;

__global__ __launch_bounds__(256) void leaf_kernel(float* H, int64_t d, int64_t o, int n,
                                                   int32_t* info) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* M = sm;
  LeafScratch ts;
  ts.T64a = M + NB * LDM;
  ts.T64b = ts.T64a + 64 * 65;
  ts.T32a = ts.T64b + 64 * 65;
  ts.T32b = ts.T32a + 32 * 33;
  ts.T16a = ts.T32b + 32 * 33;
  ts.T16b = ts.T16a + 16 * 17;
  const int pad = NB - n;
  const bool fast = pad == 0 && (d % 4) == 0 && (o % 4) == 0;
  if (fast) {
    // 16 float4 per thread, all issued before any is used: element group
    // e = tid + 256 u is row e / 32, columns 4 (e % 32) .. +3.
    floatx4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = threadIdx.x + 256 * u, i = e >> 5, k4 = (e & 31) * 4;
      v[u] = *reinterpret_cast<const floatx4*>(H + (o + i) * d + o + k4);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = threadIdx.x + 256 * u, i = e >> 5, k4 = (e & 31) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) M[i * LDM + k4 + c] = (k4 + c >= i) ? v[u][c] : 0.f;
    }
  } else {
    for (int e = threadIdx.x; e < NB * NB; e += 256) {
      const int i = e / NB, k = e % NB;
      float v;
      if (i < pad || k < pad) {
        v = (i == k) ? 1.f : 0.f;
      } else if (k >= i) {
        v = H[(o + i - pad) * d + (o + k - pad)];
      } else {
        v = 0.f;
      }
      M[i * LDM + k] = v;
    }
  }
  __syncthreads();
  leaf_rec<NB>(M, 0, ts, info, o, pad);
  if (fast) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = threadIdx.x + 256 * u, i = e >> 5, k4 = (e & 31) * 4;
      floatx4 w;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = (k4 + c >= i) ? M[i * LDM + k4 + c] : 0.f;
      *reinterpret_cast<floatx4*>(H + (o + i) * d + o + k4) = w;
    }
  } else {
    for (int e = threadIdx.x; e < n * n; e += 256) {
      const int i = e / n, k = e % n;
      H[(o + i) * d + (o + k)] = (k >= i) ? M[(i + pad) * LDM + (k + pad)] : 0.f;
    }
  }
}

constexpr size_t leaf_smem_bytes() { return (size_t)LEAF_FLOATS * sizeof(float); }

GemmArgs gemm_args(int M, int N, int K, const float* A, int64_t lda, int at, int am, const float* B, int64_t ldb,
                   int bt, int bm, float* C, int64_t ldc, float alpha, float beta, int upper_only) {
  GemmArgs g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.a_trans = at; g.a_mask = am; g.a_off = 0;
  g.B = B; g.ldb = ldb; g.b_trans = bt; g.b_mask = bm; g.b_off = 0;
  g.C = C; g.ldc = ldc; g.alpha = alpha; g.beta = beta; g.upper_only = upper_only;
  return g;
}

// Recursive U for the diagonal block (o, n) of H.  Wk is a d x d scratch
// matrix: each node keeps T in its upper-right block position and X^T in its
// lower-left one, so nodes never share scratch.  With U12 = -U11 (T U22), the
// product X = T U22 needs only T and U22 and shares one launch with the
// update of A; U12 is then written straight into H.
void factor_rec(float* H, float* Wk, int64_t d, int64_t o, int64_t n, int32_t* info, hipStream_t s) {
  if (n <= NB) {
    hipLaunchKernelGGL(leaf_kernel, dim3(1), dim3(256), leaf_smem_bytes(), s, H, d, o, (int)n, info);
    return;
  }
  const int64_t nblk = (n + NB - 1) / NB;
  const int64_t n2 = NB * (nblk / 2);
  const int64_t n1 = n - n2;
  float* A = H + o * d + o;
  float* B = H + o * d + (o + n1);
  float* C = H + (o + n1) * d + (o + n1);
  float* T = Wk + o * d + (o + n1);
  float* Xt = Wk + (o + n1) * d + o;   // n2 x n1
  factor_rec(H, Wk, d, o + n1, n2, info, s);
  // T = B * U22^T : op(B) = U22^T, stored as U22 [n][k] -> b_trans, keep k >= n
  launch_gemm_f32(gemm_args((int)n1, (int)n2, (int)n2, B, d, 0, MASK_NONE, C, d, 1, MASK_LOWER, T, d, 1.f, 0.f, 0), s);
  // A' = A - T T^T (upper tiles)  and  X^T = U22^T T^T (op(A) = U22^T: keep m >= k)
  launch_gemm_f32_pair(
      gemm_args((int)n1, (int)n1, (int)n2, T, d, 0, MASK_NONE, T, d, 1, MASK_NONE, A, d, -1.f, 1.f, 1),
      gemm_args((int)n2, (int)n1, (int)n2, C, d, 1, MASK_LOWER, T, d, 1, MASK_NONE, Xt, d, 1.f, 0.f, 0), s);
  factor_rec(H, Wk, d, o, n1, info, s);
  // U12 = -U11 X  (U11 upper: keep k >= m; op(B) = X, stored as X^T -> b_trans)
  launch_gemm_f32(gemm_args((int)n1, (int)n2, (int)n1, A, d, 0, MASK_UPPER, Xt, d, 1, MASK_NONE, B, d, -1.f, 0.f, 0), s);
}

}  // namespace

size_t prepare_workspace_bytes(int64_t d, int act_order) {
  (void)act_order;
  // d x d scratch (node temporaries; also the permuted copy) + diagonal.
  const size_t mat = (size_t)d * (size_t)d * sizeof(float);
  return ((mat + 255) / 256) * 256 + (size_t)d * sizeof(float) + 256;
}

void launch_prepare(float* H, int64_t d, float percdamp, int act_order, int32_t* perm, uint8_t* dead,
                    int32_t* info, void* ws, hipStream_t s) {
  static const bool attr_set = [] {   // once, thread-safe (function-local static)
    (void)hipFuncSetAttribute((const void*)leaf_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)leaf_smem_bytes());
    return true;
  }();
  (void)attr_set;
  const size_t mat = (size_t)d * (size_t)d * sizeof(float);
  float* Wk = reinterpret_cast<float*>(ws);
  float* diag = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ((mat + 255) / 256) * 256);
  hipLaunchKernelGGL(diag_prep_kernel, dim3(1), dim3(1024), 0, s, H, d, dead, info, diag,
                     act_order ? nullptr : perm, percdamp);
  if (act_order) {
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((d + 63) / 64)), dim3(256), 0, s, (const float*)diag, d, perm);
    const unsigned gx = (unsigned)std::min<int64_t>((d + 255) / 256, 64);
    hipLaunchKernelGGL(permute_upper_kernel, dim3(gx, (unsigned)d), dim3(256), 0, s, (const float*)H, d,
                       (const int32_t*)perm, Wk);
    const int64_t cnt = d * d;
    hipLaunchKernelGGL(copy_block_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                       (const float*)Wk, H, d, (int)d, (int)d);
  }
  factor_rec(H, Wk, d, 0, d, info, s);
  const unsigned gz = (unsigned)std::min<int64_t>((d + 1023) / 1024, 64);
  hipLaunchKernelGGL(zero_lower_kernel, dim3(gz, (unsigned)d), dim3(256), 0, s, H, d);
}

}  // namespace gptq
