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
// are factored by one workgroup in LDS with the same recursion down to 32,
// where one wave runs the column-by-column factorisation and inversion.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 128;      // leaf block handled by one workgroup
constexpr int LDM = NB + 1;  // LDS row stride of the leaf block

// ---------------------------------------------------------------------------
// Diagonal pass: dead inputs, NaN/Inf check, info reset.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void diag_dead_kernel(float* H, int64_t d, uint8_t* dead,
                                                         int32_t* info, float* diag_out) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int64_t j = threadIdx.x; j < d; j += blockDim.x) {
    float v = H[j * d + j];
    if (!__builtin_isfinite(v)) atomicOr(&bad, 1);
    const bool dj = (v == 0.0f);
    dead[j] = dj ? 1 : 0;
    if (dj) {
      v = 1.0f;
      H[j * d + j] = 1.0f;
    }
    diag_out[j] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) *info = bad ? -1 : 0;
}

// Act-order: rank of column i = #{j : diag_j > diag_i} + #{j < i : diag_j == diag_i}
// (a stable descending sort); perm[rank] = i.  A NaN diagonal (already
// reported through info) sorts as -inf so the ranks always form a permutation.
GPTQ_DEV float sort_key(float v) { return __builtin_isnan(v) ? -__builtin_inff() : v; }

__global__ __launch_bounds__(256) void rank_kernel(const float* diag, int64_t d, int32_t* perm) {
  __shared__ float tile[1024];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float di = i < d ? sort_key(diag[i]) : 0.f;
  int64_t rank = 0;
  for (int64_t base = 0; base < d; base += 1024) {
    __syncthreads();
    for (int k = threadIdx.x; k < 1024; k += 256) tile[k] = base + k < d ? sort_key(diag[base + k]) : 0.f;
    __syncthreads();
    const int lim = (int)min<int64_t>(1024, d - base);
    for (int k = 0; k < lim; ++k) {
      const float v = tile[k];
      rank += (v > di) || (v == di && base + k < i);
    }
  }
  if (i < d) perm[rank] = (int32_t)i;
}

__global__ void identity_perm_kernel(int32_t* perm, int64_t d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < d) perm[i] = (int32_t)i;
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

// lambda = percdamp * mean(diag), summed in a fixed order; H[j][j] += lambda.
__global__ __launch_bounds__(1024) void damp_kernel(float* H, int64_t d, float percdamp) {
  __shared__ float part[1024];
  float s = 0.f;
  for (int64_t j = threadIdx.x; j < d; j += 1024) s += H[j * d + j];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float lam = percdamp * (part[0] / (float)d);
  for (int64_t j = threadIdx.x; j < d; j += 1024) H[j * d + j] += lam;
}

__global__ __launch_bounds__(256) void copy_block_kernel(const float* src, float* dst, int64_t ld,
                                                         int rows, int cols) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * cols) return;
  const int64_t r = idx / cols, c = idx % cols;
  dst[r * ld + c] = src[r * ld + c];
}

__global__ __launch_bounds__(256) void zero_lower_kernel(float* H, int64_t d) {
  const int64_t r = blockIdx.y;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < r; c += (int64_t)gridDim.x * 256)
    H[r * d + c] = 0.f;
}

// ---------------------------------------------------------------------------
// Leaf: U of one diagonal block of <= 128 in LDS.
// ---------------------------------------------------------------------------

// One wave: the 32 x 32 diagonal block of M at (o, o) holds the upper
// triangle of the (updated) H block; it is replaced by U = V^{-1} where
// V V^T = block, V upper.  One backward sweep j = 31 .. 0 does both:
//   factor : V[:, j] = A[:, j] / sqrt(A[j][j]);  A[0:j, 0:j] -= V[0:j, j] V[0:j, j]^T
//   invert : X[j, :] /= V[j][j];  X[0:j, :] -= V[0:j, j] X[j, :]   (X starts as I)
// (row j of X is final at step j: every later row has already been removed).
// Registers only: lane k < 32 holds column k of the symmetric block A, lane
// 32 + c column c of X.  With p = A[j][j] and a_i = A[i][j] (read from lane j),
// both updates are  col[i] -= a_i * col[j] / p  for i < j  -- on the A side
// col[j] = A[j][k] = A[k][j] by symmetry, on the X side col[j] = X[j][c] before
// its scaling -- and the X side then scales col[j] by 1/sqrt(p).  A non-positive
// or NaN pivot sets *info once.
__device__ __forceinline__ void leaf32(float* M, int o, float* /*unused*/, int32_t* info, int64_t gbase,
                                       int pad) {
  const int lane = threadIdx.x & 63;
  const int k = lane & 31;
  const bool xside = lane >= 32;
  float col[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float av = M[(o + min(i, k)) * LDM + o + max(i, k)];
    col[i] = xside ? (i == k ? 1.f : 0.f) : av;
  }
#pragma unroll
  for (int j = 31; j >= 0; --j) {
    const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(col[j]), j));
    if (lane == 0 && !(piv > 0.f) && (o + j) >= pad) {
      if (*info == 0) *info = (int32_t)(gbase + (o + j - pad) + 1);
    }
    const float rv = __builtin_amdgcn_rsqf(piv);   // 1/sqrt(pivot), ~1 ulp
    const float f = col[j] * (rv * rv);
#pragma unroll
    for (int i = 0; i < j; ++i) {
      const float ai = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(col[i]), j));
      col[i] = __builtin_fmaf(-ai, f, col[i]);
    }
    if (xside) col[j] *= rv;
  }
  if (xside) {
#pragma unroll
    for (int i = 0; i < 32; ++i) M[(o + i) * LDM + o + k] = (k >= i) ? col[i] : 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// C (n x m) = alpha * A * op(B) [+ C] on LDS arrays with the fp32 matrix
// cores; n, m, K multiples of 32.  op(B) = B^T (B stored m x K) when bt, else
// B (K x m).  32 x 32 output blocks are spread over the 4 waves; with
// upper_only, blocks strictly below the diagonal are skipped.
__device__ __forceinline__ void lds_gemm(int n, int m, int K, const float* A, int lda, const float* B, int ldb, int bt,
                         float* C, int ldc, float alpha, bool accumulate, bool upper_only) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nbm = m / 32, blocks = (n / 32) * nbm;
  for (int blk = wave; blk < blocks; blk += 4) {
    const int bi = blk / nbm, bj = blk % nbm;
    if (upper_only && bj < bi) continue;
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    const int r = 32 * bi + (lane & 31), c = 32 * bj + (lane & 31), kh = lane >> 5;
#pragma unroll 8
    for (int k = 0; k < K; k += 2) {
      const float a = A[r * lda + k + kh];
      const float b = bt ? B[c * ldb + k + kh] : B[(k + kh) * ldb + c];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 32 * bi + 8 * (v >> 2) + 4 * kh + (v & 3);
      float* p = C + i * ldc + c;
      *p = accumulate ? __builtin_fmaf(alpha, acc[v], *p) : alpha * acc[v];
    }
  }
}

// In-LDS recursion on the diagonal block (o, n), n in {32, 64, 128}; level
// temporaries T1/T2 of each size are separate (T64a/T64b for n == 128,
// T32a/T32b for n == 64).  On return M[o:o+n, o:o+n] holds U with exact
// zeros below the diagonal.
struct LeafScratch {
  float *T64a, *T64b, *T32a, *T32b, *X32;
};

template <int N>
__device__ __forceinline__ void leaf_rec(float* M, int o, const LeafScratch& ts, int32_t* info, int64_t gbase, int pad) {
  if constexpr (N == 32) {
    if ((threadIdx.x >> 6) == 0) leaf32(M, o, ts.X32, info, gbase, pad);  // X32: 64-float exchange buffer
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
    lds_gemm(h, h, h, Bm, LDM, U22, LDM, 1, T1, ldt, 1.f, false, false);    // T1 = B U22^T
    __syncthreads();
    lds_gemm(h, h, h, T1, ldt, T1, ldt, 1, U11, LDM, -1.f, true, true);     // A -= T1 T1^T
    __syncthreads();
    leaf_rec<h>(M, o, ts, info, gbase, pad);
    lds_gemm(h, h, h, U11, LDM, T1, ldt, 0, T2, ldt, 1.f, false, false);    // T2 = U11 T1
    __syncthreads();
    lds_gemm(h, h, h, T2, ldt, U22, LDM, 0, Bm, LDM, -1.f, false, false);   // U12 = -T2 U22
    __syncthreads();
  }
}

constexpr int LEAF_FLOATS = NB * LDM + 2 * 64 * 65 + 2 * 32 * 33 + 32 * 33;

__global__ __launch_bounds__(256) void leaf_kernel(float* H, int64_t d, int64_t o, int n,
                                                   int32_t* info) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* M = sm;
  LeafScratch ts;
  ts.T64a = M + NB * LDM;
  ts.T64b = ts.T64a + 64 * 65;
  ts.T32a = ts.T64b + 64 * 65;
  ts.T32b = ts.T32a + 32 * 33;
  ts.X32 = ts.T32b + 32 * 33;
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
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)leaf_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)leaf_smem_bytes());
    attr_set = true;
  }
  const size_t mat = (size_t)d * (size_t)d * sizeof(float);
  float* Wk = reinterpret_cast<float*>(ws);
  float* diag = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ((mat + 255) / 256) * 256);
  hipLaunchKernelGGL(diag_dead_kernel, dim3(1), dim3(1024), 0, s, H, d, dead, info, diag);
  const unsigned gb = (unsigned)((d + 255) / 256);
  if (act_order) {
    hipLaunchKernelGGL(rank_kernel, dim3(gb), dim3(256), 0, s, (const float*)diag, d, perm);
    const unsigned gx = (unsigned)std::min<int64_t>((d + 255) / 256, 64);
    hipLaunchKernelGGL(permute_upper_kernel, dim3(gx, (unsigned)d), dim3(256), 0, s, (const float*)H, d,
                       (const int32_t*)perm, Wk);
    const int64_t cnt = d * d;
    hipLaunchKernelGGL(copy_block_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                       (const float*)Wk, H, d, (int)d, (int)d);
  } else if (perm != nullptr) {
    hipLaunchKernelGGL(identity_perm_kernel, dim3(gb), dim3(256), 0, s, perm, d);
  }
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, s, H, d, percdamp);
  factor_rec(H, Wk, d, 0, d, info, s);
  const unsigned gx = (unsigned)std::min<int64_t>((d + 255) / 256, 64);
  hipLaunchKernelGGL(zero_lower_kernel, dim3(gx, (unsigned)d), dim3(256), 0, s, H, d);
}

}  // namespace gptq
