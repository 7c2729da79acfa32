// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32), true fp32
// throughout -- no reduced-precision fp32 mode ("GPTQ, with the code open",
// "Paper vs. code": the Cholesky chain needs full 32-bit precision).
//
//   C[M x N] = alpha * op(A) * op(B) + beta * C
//
// op(A) is logical M x K: row-major A[m][k] (a_trans == 0, lda >= K) or the
// transpose of a row-major K x M array (a_trans == 1, lda >= M).  op(B) is
// logical K x N: row-major B[k][n] (b_trans == 0) or the transpose of a
// row-major N x K array (b_trans == 1).  Either operand may be declared
// triangular; elements outside its triangle are treated as exactly zero
// whatever the memory holds, and K-tiles that are entirely zero are skipped.
// With upper_only, output tiles strictly below the diagonal are skipped (a
// SYRK-shaped update; M == N).  beta == 0 never reads C.
//
// Tiling: TM x TN output tile per 256-thread workgroup, 2 x 2 waves, each
// wave (TM/2) x (TN/2) as 32x32 MFMA blocks; K-steps of KT staged through LDS
// in k-major rows (As[k][m], Bs[k][n]) with double buffering.  One launch may
// carry two independent problems: workgroups past the first problem's tiles
// work on the second.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int PAD = 4;

GPTQ_DEV bool keep_a(int mask, int off, int m, int k) {
  // A logical [m][k]
  if (mask == MASK_UPPER) return k + off >= m;
  if (mask == MASK_LOWER) return m + off >= k;
  return true;
}
GPTQ_DEV bool keep_b(int mask, int off, int k, int n) {
  // B logical [k][n]
  if (mask == MASK_UPPER) return n + off >= k;
  if (mask == MASK_LOWER) return k + off >= n;
  return true;
}

// Read 4 consecutive floats of a row (columns c .. c+3 of row `row`), zero
// outside [0, rows) x [0, cols).  Vector path when the whole float4 is in
// bounds and the address is 16-byte aligned.
GPTQ_DEV floatx4 load4(const float* base, int64_t ld, int row, int col, int rows, int cols,
                       bool aligned) {
  floatx4 v = {0.f, 0.f, 0.f, 0.f};
  if (row >= rows || row < 0) return v;
  const float* p = base + (int64_t)row * ld + col;
  if (aligned && col + 3 < cols) {
    v = *reinterpret_cast<const floatx4*>(p);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (col + c < cols && col + c >= 0) v[c] = p[c];
  }
  return v;
}

struct GemmPair {
  GemmArgs g[2];
  int tiles0;   // tiles of g[0]; workgroups from here on belong to g[1]
};

template <int TM, int TN, int KT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmPair pr) {
  constexpr int WM = TM / 2, WN = TN / 2;   // per-wave tile
  constexpr int MB = WM / 32, NB = WN / 32; // 32x32 blocks per wave
  constexpr int LDA_S = TM + PAD, LDB_S = TN + PAD;
  extern __shared__ __attribute__((aligned(16))) float gemm_smem[];
  // LDS: A buffers 0/1 (KT x LDA_S each), then B buffers 0/1 (KT x LDB_S).
  auto As = [&](int b) { return gemm_smem + b * (KT * LDA_S); };
  auto Bs = [&](int b) { return gemm_smem + 2 * (KT * LDA_S) + b * (KT * LDB_S); };

  const bool second = (int)blockIdx.x >= pr.tiles0;
  const GemmArgs& g = second ? pr.g[1] : pr.g[0];
  const int bid = second ? (int)blockIdx.x - pr.tiles0 : (int)blockIdx.x;
  const int tiles_n = (g.N + TN - 1) / TN;
  const int bm = bid / tiles_n, bn = bid % tiles_n;
  const int m0 = bm * TM, n0 = bn * TN;
  if (g.upper_only && n0 + TN <= m0) return;  // tile strictly below the diagonal

  // K range that can hold non-zero products for this tile.
  int k_lo = 0, k_hi = g.K;
  if (g.a_mask == MASK_UPPER) k_lo = max(k_lo, m0 - g.a_off);
  if (g.a_mask == MASK_LOWER) k_hi = min(k_hi, m0 + TM + g.a_off);
  if (g.b_mask == MASK_UPPER) k_hi = min(k_hi, n0 + TN + g.b_off);
  if (g.b_mask == MASK_LOWER) k_lo = max(k_lo, n0 - g.b_off);
  k_lo = (k_lo / KT) * KT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  constexpr int NVA = TM * KT / 4 / 256;
  constexpr int NVB = TN * KT / 4 / 256;
  floatx4 ra[NVA], rb[NVB];

  const bool a_al = ((g.lda & 3) == 0) && ((reinterpret_cast<uintptr_t>(g.A) & 15) == 0);
  const bool b_al = ((g.ldb & 3) == 0) && ((reinterpret_cast<uintptr_t>(g.B) & 15) == 0);

  // ---- global -> registers ----
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NVA; ++u) {
      int idx = tid + 256 * u;
      if (!g.a_trans) {          // A[m][k]: float4 along k
        int m = idx / (KT / 4), k4 = idx % (KT / 4);
        int gm = m0 + m, gk = k0 + 4 * k4;
        floatx4 v = load4(g.A, g.lda, gm, gk, g.M, g.K, a_al);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!keep_a(g.a_mask, g.a_off, gm, gk + c)) v[c] = 0.f;
        ra[u] = v;
      } else {                   // A stored [k][m]: float4 along m
        int k = idx / (TM / 4), m4 = idx % (TM / 4);
        int gk = k0 + k, gm = m0 + 4 * m4;
        floatx4 v = load4(g.A, g.lda, gk, gm, g.K, g.M, a_al);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!keep_a(g.a_mask, g.a_off, gm + c, gk)) v[c] = 0.f;
        ra[u] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < NVB; ++u) {
      int idx = tid + 256 * u;
      if (!g.b_trans) {          // B[k][n]: float4 along n
        int k = idx / (TN / 4), n4 = idx % (TN / 4);
        int gk = k0 + k, gn = n0 + 4 * n4;
        floatx4 v = load4(g.B, g.ldb, gk, gn, g.K, g.N, b_al);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!keep_b(g.b_mask, g.b_off, gk, gn + c)) v[c] = 0.f;
        rb[u] = v;
      } else {                   // B stored [n][k]: float4 along k
        int n = idx / (KT / 4), k4 = idx % (KT / 4);
        int gn = n0 + n, gk = k0 + 4 * k4;
        floatx4 v = load4(g.B, g.ldb, gn, gk, g.N, g.K, b_al);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!keep_b(g.b_mask, g.b_off, gk + c, gn)) v[c] = 0.f;
        rb[u] = v;
      }
    }
  };
  // ---- registers -> LDS (k-major rows) ----
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NVA; ++u) {
      int idx = tid + 256 * u;
      if (!g.a_trans) {
        int m = idx / (KT / 4), k4 = idx % (KT / 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) As(buf)[(4 * k4 + c) * LDA_S + m] = ra[u][c];
      } else {
        int k = idx / (TM / 4), m4 = idx % (TM / 4);
        *reinterpret_cast<floatx4*>(As(buf) + k * LDA_S + 4 * m4) = ra[u];
      }
    }
#pragma unroll
    for (int u = 0; u < NVB; ++u) {
      int idx = tid + 256 * u;
      if (!g.b_trans) {
        int k = idx / (TN / 4), n4 = idx % (TN / 4);
        *reinterpret_cast<floatx4*>(Bs(buf) + k * LDB_S + 4 * n4) = rb[u];
      } else {
        int n = idx / (KT / 4), k4 = idx % (KT / 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) Bs(buf)[(4 * k4 + c) * LDB_S + n] = rb[u][c];
      }
    }
  };

  if (k_lo < k_hi) {
    load_tile(k_lo);
    store_tile(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = k_lo; k0 < k_hi; k0 += KT) {
      const bool more = k0 + KT < k_hi;
      if (more) load_tile(k0 + KT);
      const float* as = As(buf);
      const float* bs = Bs(buf);
#pragma unroll
      for (int kk = 0; kk < KT / 2; ++kk) {
        const int kr = 2 * kk + (lane >> 5);
        float a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = as[kr * LDA_S + wm + 32 * i + (lane & 31)];
#pragma unroll
        for (int j = 0; j < NB; ++j) b[j] = bs[kr * LDB_S + wn + 32 * j + (lane & 31)];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (more) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // ---- epilogue: lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] ----
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < g.M && col < g.N) {
          float* p = g.C + (int64_t)row * g.ldc + col;
          float out = g.alpha * acc[i][j][v];
          if (g.beta != 0.f) out = __builtin_fmaf(g.beta, *p, out);
          *p = out;
        }
      }
    }
}

template <int TM, int TN, int KT>
int64_t tiles_of(const GemmArgs& g) {
  return (g.M <= 0 || g.N <= 0) ? 0 : (int64_t)((g.M + TM - 1) / TM) * ((g.N + TN - 1) / TN);
}

template <int TM, int TN, int KT>
void launch_tile(const GemmArgs& g0, const GemmArgs* g1, hipStream_t s) {
  constexpr size_t smem = (size_t)2 * KT * ((TM + PAD) + (TN + PAD)) * sizeof(float);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)gemm_f32_kernel<TM, TN, KT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)smem);
    attr = true;
  }
  GemmPair pr;
  pr.g[0] = g0;
  pr.g[1] = g1 ? *g1 : g0;
  const int64_t t0 = tiles_of<TM, TN, KT>(g0);
  const int64_t t1 = g1 ? tiles_of<TM, TN, KT>(*g1) : 0;
  pr.tiles0 = (int)t0;
  if (t0 + t1 == 0) return;
  hipLaunchKernelGGL((gemm_f32_kernel<TM, TN, KT>), dim3((unsigned)(t0 + t1)), dim3(256), smem, s, pr);
}

void launch_dispatch(const GemmArgs& g0, const GemmArgs* g1, hipStream_t s) {
  // 128 x 128 tiles when that already gives enough workgroups, else 64 x 64.
  const int64_t t128 = tiles_of<128, 128, 32>(g0) + (g1 ? tiles_of<128, 128, 32>(*g1) : 0);
  if (t128 >= 480) {
    launch_tile<128, 128, 32>(g0, g1, s);
  } else {
    launch_tile<64, 64, 32>(g0, g1, s);
  }
}

}  // namespace

void launch_gemm_f32(const GemmArgs& g, hipStream_t s) { launch_dispatch(g, nullptr, s); }

void launch_gemm_f32_pair(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s) {
  launch_dispatch(g0, &g1, s);
}

}  // namespace gptq
