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

#include <algorithm>
#include <type_traits>

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

// Output tile of workgroup `bid` (tiles of TM x TN).  With upper_only (a
// square problem, TM == TN) only the tiles on and above the diagonal are
// numbered, row by row.  Otherwise a triangular operand gives tiles K-ranges
// of different lengths (see the kernels' k_lo / k_hi), and the tiles are
// numbered longest first along the index that sets the length: the
// dispatcher hands consecutive workgroups to different CUs, so each CU gets
// a mix of long and short tiles instead of one CU getting all the long ones.
GPTQ_DEV void tile_of(const GemmArgs& g, int bid, int TM, int TN, int& bm, int& bn) {
  const int tm = (g.M + TM - 1) / TM, tn = (g.N + TN - 1) / TN;
  if (g.upper_only) {
    int r = 0;
    while (r < tm - 1 && bid >= tn - r) {
      bid -= tn - r;
      ++r;
    }
    bm = r;
    bn = r + bid;
  } else if (g.b_mask != MASK_NONE && g.a_mask == MASK_NONE) {
    const int sl = bid / tm;
    bm = bid % tm;
    bn = g.b_mask == MASK_LOWER ? sl : tn - 1 - sl;   // LOWER: k >= n - off, long for small n
  } else {
    const int sl = bid / tn;
    bn = bid % tn;
    bm = g.a_mask == MASK_LOWER ? tm - 1 - sl : sl;   // UPPER: k >= m - off, long for small m
  }
}

struct GemmPair {
  GemmArgs g[2];
  int tiles0;   // tiles of g[0]; workgroups from here on belong to g[1]
};

// C = alpha * acc (+ beta * C) for one wave's MB x NB blocks of 32 x 32 at
// (r0, c0); lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] of a block.
// When the blocks lie wholly inside C all their old values are loaded before
// any is used (one memory round trip, not one per element); otherwise each
// element is bounds-tested.
template <int MB, int NB>
GPTQ_DEV void store_acc(const GemmArgs& g, const floatx16 (&acc)[MB][NB], int r0, int c0, int lane) {
  auto at = [&](int i, int j, int v) {
    return g.C + (int64_t)(r0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * g.ldc + c0 + 32 * j +
           (lane & 31);
  };
  if (r0 + 32 * MB <= g.M && c0 + 32 * NB <= g.N) {
    float old[MB][NB][16];
    if (g.beta != 0.f) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) old[i][j][v] = *at(i, j, v);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float out = g.alpha * acc[i][j][v];
          if (g.beta != 0.f) out = __builtin_fmaf(g.beta, old[i][j][v], out);
          *at(i, j, v) = out;
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = c0 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < g.M && col < g.N) {
          float out = g.alpha * acc[i][j][v];
          if (g.beta != 0.f) out = __builtin_fmaf(g.beta, *at(i, j, v), out);
          *at(i, j, v) = out;
        }
      }
    }
}

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
  int bm, bn;
  tile_of(g, bid, TM, TN, bm, bn);
  const int m0 = bm * TM, n0 = bn * TN;

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

  store_acc<MB, NB>(g, acc, m0 + wm, n0 + wn, lane);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// The same product with the operands carried from memory straight into LDS
// by buffer loads that write LDS (16 bytes per lane), one K-step ahead, when
// both operands are 16-byte aligned with ld % 4 == 0 (and ld < 2^22).  The
// LDS tiles are plain copies of the operand rows as they lie in memory --
// A[m][k] rows (a_trans == 0) or A^T [k][m] rows, B[k][n] rows (b_trans == 0)
// or B^T [n][k] rows -- and each MFMA operand is read with the matching
// strides.  On the K-steps that cross a triangle's diagonal or the end of K
// the workgroup first overwrites the masked elements (and those with
// k >= K) of the landed tiles with zeros in LDS; the MFMA loop itself has a
// single body, so the accumulators stay in the AGPRs across steps.  Rows past
// the end of an operand load zeros from the descriptor bounds, and columns
// past M or N only reach outputs that are not stored.  The operands and their
// order are those of gemm_f32_kernel, so both kernels give the same bits.
GPTQ_DEV int kswz(int r) { return (r >> 1) & 7; }

// The K-loop of gemm_f32_dma_kernel (a device function, so that the
// LDS-direct loads are compiled for the device only).
template <int TM, int TN, int KT>
GPTQ_DEV void gemm_steps_dma(const GemmArgs& g, int m0, int n0, int k_lo, int k_hi, int wm, int wn,
                             floatx16 (&acc)[TM / 64][TN / 64]) {
  constexpr int MB = TM / 64, NB = TN / 64;
  constexpr int ABYTES = TM * KT * 4, BBYTES = TN * KT * 4, BUF = ABYTES + BBYTES;
  constexpr int NIA = ABYTES / 4096, NIB = BBYTES / 4096;  // load instructions per wave and step
  static_assert(NIA * 4096 == ABYTES && NIB * 4096 == BBYTES, "whole load instructions");
  static_assert(KT == 32, "rows along k are 8 chunks");
  extern __shared__ __attribute__((aligned(16))) float gemm_smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool ak = !g.a_trans, bk = g.b_trans != 0;  // rows run along k
  const int rowa = ak ? KT * 4 : TM * 4, rowb = bk ? KT * 4 : TN * 4;  // bytes per LDS row
  // Byte offset (from the step's tile origin in memory) of the chunk each
  // lane carries: LDS byte I * 1024 + 16 lane is row byte / row_bytes,
  // 16-byte position p of it.  Rows along k (8 chunks) hold chunk c at
  // position c ^ kswz(row), so that the 32 rows an operand read touches at
  // one k spread over 16 banks; rows along m or n are read contiguously and
  // are not swizzled.
  int offa[NIA], offb[NIB];
#pragma unroll
  for (int q = 0; q < NIA; ++q) {
    const int byte = (wave * NIA + q) * 1024 + 16 * lane, r = byte / rowa, p = (byte % rowa) >> 4;
    offa[q] = r * (int)g.lda * 4 + 16 * (ak ? p ^ kswz(r) : p);
  }
#pragma unroll
  for (int q = 0; q < NIB; ++q) {
    const int byte = (wave * NIB + q) * 1024 + 16 * lane, r = byte / rowb, p = (byte % rowb) >> 4;
    offb[q] = r * (int)g.ldb * 4 + 16 * (bk ? p ^ kswz(r) : p);
  }
  lds_u8* lbase = (lds_u8*)gemm_smem;  // generic to LDS address space
  auto dma = [&](int k0, int b) {
    // tile origin, rows that exist from it, and its column offset in a row
    const float* ab = ak ? g.A + (int64_t)m0 * g.lda + k0 : g.A + (int64_t)k0 * g.lda + m0;
    const int ar = ak ? min(g.M - m0, TM) : min(g.K - k0, KT), ac = ak ? k0 : m0;
    const float* bb = bk ? g.B + (int64_t)n0 * g.ldb + k0 : g.B + (int64_t)k0 * g.ldb + n0;
    const int br = bk ? min(g.N - n0, TN) : min(g.K - k0, KT), bc = bk ? k0 : n0;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ab, (short)0, (int)((int64_t)ar * g.lda * 4 - (int64_t)ac * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)bb, (short)0, (int)((int64_t)br * g.ldb * 4 - (int64_t)bc * 4), 0x00020000);
#pragma unroll
    for (int q = 0; q < NIA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lbase + b * BUF + (wave * NIA + q) * 1024, 16, offa[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < NIB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lbase + b * BUF + ABYTES + (wave * NIB + q) * 1024, 16, offb[q],
                                               0, 0, 0);
  };

  if (k_lo < k_hi) {
    dma(k_lo, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = k_lo; k0 < k_hi; k0 += KT) {
      if (k0 + KT < k_hi) dma(k0 + KT, buf ^ 1);
      const float* as = gemm_smem + buf * (BUF / 4);
      const float* bs = as + ABYTES / 4;
      // Masks and the K tail only matter on steps that cross a triangle's
      // diagonal or the end of K (a uniform test); those steps zero the
      // masked elements of this buffer first, the others read plainly.
      bool plain = k0 + KT <= g.K;
      if (g.a_mask == MASK_UPPER) plain = plain && k0 + g.a_off >= m0 + TM - 1;
      if (g.a_mask == MASK_LOWER) plain = plain && m0 + g.a_off >= k0 + KT - 1;
      if (g.b_mask == MASK_UPPER) plain = plain && n0 + g.b_off >= k0 + KT - 1;
      if (g.b_mask == MASK_LOWER) plain = plain && k0 + g.b_off >= n0 + TN - 1;
      if (!plain) {
        float* aw = gemm_smem + buf * (BUF / 4);
        float* bw = aw + ABYTES / 4;
        // LDS element e of a tile: rows along k hold chunk c of row r at
        // position c ^ kswz(r); rows along m or n are contiguous.
#pragma unroll
        for (int q = 0; q < TM * KT / 256; ++q) {
          const int e = (int)threadIdx.x + 256 * q;
          int m, k;
          if (ak) {
            m = e / KT;
            const int w = e % KT;
            k = ((((w >> 2) ^ kswz(m))) << 2) | (w & 3);
          } else {
            k = e / TM;
            m = e % TM;
          }
          if (!(k0 + k < g.K && keep_a(g.a_mask, g.a_off, m0 + m, k0 + k))) aw[e] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < TN * KT / 256; ++q) {
          const int e = (int)threadIdx.x + 256 * q;
          int n, k;
          if (bk) {
            n = e / KT;
            const int w = e % KT;
            k = ((((w >> 2) ^ kswz(n))) << 2) | (w & 3);
          } else {
            k = e / TN;
            n = e % TN;
          }
          if (!(k0 + k < g.K && keep_b(g.b_mask, g.b_off, k0 + k, n0 + n))) bw[e] = 0.f;
        }
        __syncthreads();
      }
      // Operands of pair kk + 1 are read from LDS while the MFMAs of pair kk
      // run (two register sets); the scheduling groups keep that order.
      float a[2][MB], b[2][NB];
      auto rd = [&](int kk, int sl) {
        const int k = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int m = wm + 32 * i + (lane & 31);
          a[sl][i] = ak ? as[m * KT + ((((k >> 2) ^ kswz(m))) << 2) + (k & 3)] : as[k * TM + m];
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = wn + 32 * j + (lane & 31);
          b[sl][j] = bk ? bs[n * KT + ((((k >> 2) ^ kswz(n))) << 2) + (k & 3)] : bs[k * TN + n];
        }
      };
      rd(0, 0);
#pragma unroll
      for (int kk = 0; kk < KT / 2; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < KT / 2) rd(kk + 1, cur ^ 1);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (MB + NB), 0);   // LDS reads of pairs 0 and 1
#pragma unroll
      for (int kk = 0; kk < KT / 2; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, MB * NB, 0);        // MFMAs of pair kk
        if (kk + 2 < KT / 2) __builtin_amdgcn_sched_group_barrier(0x100, MB + NB, 0);   // reads of kk + 2
      }
      // step k0 + KT has landed (own loads) in every wave (barrier); buffer
      // buf is free for the step after it
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      buf ^= 1;
    }
  }

}

template <int TM, int TN, int KT>
__global__ __launch_bounds__(256) void gemm_f32_dma_kernel(GemmPair pr) {
  constexpr int WM = TM / 2, WN = TN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;

  const bool second = (int)blockIdx.x >= pr.tiles0;
  const GemmArgs& g = second ? pr.g[1] : pr.g[0];
  const int bid = second ? (int)blockIdx.x - pr.tiles0 : (int)blockIdx.x;
  int bm, bn;
  tile_of(g, bid, TM, TN, bm, bn);
  const int m0 = bm * TM, n0 = bn * TN;

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

  gemm_steps_dma<TM, TN, KT>(g, m0, n0, k_lo, k_hi, wm, wn, acc);

  store_acc<MB, NB>(g, acc, m0 + wm, n0 + wn, lane);
}

// Small products (few 64 x 64 tiles, K <= 512): 32 x 32 output tiles, the
// workgroup's 4 waves split K four ways and load all their operands straight
// into registers at once (one memory latency instead of one per K-step), then
// the four partial tiles are summed through LDS in wave order.
//
// v_mfma_f32_32x32x2_f32 takes A[m][k0], B[k0][n] from lanes 0..31 and
// A[m][k1], B[k1][n] from lanes 32..63 for one pair (k0, k1) per step; the sum
// over k does not depend on which k values share a step, so the wave's K range
// is split into two contiguous halves (lanes 0..31 the first, 32..63 the
// second), which makes each lane's values of a row-contiguous operand
// contiguous in memory.
constexpr int SK_MAX = 64;   // values per lane per operand (K <= 512)

GPTQ_DEV float ld_a(const GemmArgs& g, int m, int k) {
  if (m >= g.M || k >= g.K || !keep_a(g.a_mask, g.a_off, m, k)) return 0.f;
  return g.a_trans ? g.A[(int64_t)k * g.lda + m] : g.A[(int64_t)m * g.lda + k];
}
GPTQ_DEV float ld_b(const GemmArgs& g, int k, int n) {
  if (n >= g.N || k >= g.K || !keep_b(g.b_mask, g.b_off, k, n)) return 0.f;
  return g.b_trans ? g.B[(int64_t)n * g.ldb + k] : g.B[(int64_t)k * g.ldb + n];
}

__global__ __launch_bounds__(256) void gemm_f32_small_kernel(GemmPair pr) {
  const bool second = (int)blockIdx.x >= pr.tiles0;
  const GemmArgs& g = second ? pr.g[1] : pr.g[0];
  const int bid = second ? (int)blockIdx.x - pr.tiles0 : (int)blockIdx.x;
  int bm, bn;
  tile_of(g, bid, 32, 32, bm, bn);
  const int m0 = bm * 32, n0 = bn * 32;
  __shared__ floatx16 red[3][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, h = lane >> 5;
  // K range of this wave: [kw, kw + kq), half h: [kh, kh + kq/2); kq % 8 == 0
  const int kq = (((g.K + 3) / 4) + 7) / 8 * 8;
  const int half = kq / 2;
  const int kh = wave * kq + h * half;
  const int m = m0 + li, n = n0 + li;

  float a[SK_MAX], b[SK_MAX];
  const bool a_vec = !g.a_trans && ((g.lda & 3) == 0) && ((reinterpret_cast<uintptr_t>(g.A) & 15) == 0);
  const bool b_vec = g.b_trans && ((g.ldb & 3) == 0) && ((reinterpret_cast<uintptr_t>(g.B) & 15) == 0);
#pragma unroll
  for (int s = 0; s < SK_MAX; s += 4) {
    if (s < half) {
      const int k = kh + s;
      if (a_vec && m < g.M && k + 3 < g.K) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(g.A + (int64_t)m * g.lda + k);
#pragma unroll
        for (int c = 0; c < 4; ++c) a[s + c] = keep_a(g.a_mask, g.a_off, m, k + c) ? v[c] : 0.f;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) a[s + c] = ld_a(g, m, k + c);
      }
      if (b_vec && n < g.N && k + 3 < g.K) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(g.B + (int64_t)n * g.ldb + k);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[s + c] = keep_b(g.b_mask, g.b_off, k + c, n) ? v[c] : 0.f;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) b[s + c] = ld_b(g, k + c, n);
      }
    }
  }
  floatx16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int s = 0; s < SK_MAX; ++s)
    if (s < half) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);

  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += red[w][lane];
  floatx16 tile[1][1];
  tile[0][0] = acc;
  store_acc<1, 1>(g, tile, m0, n0, lane);
}

// Workgroups of a problem: every tile, or with upper_only (M == N, square
// tiles) the tiles on and above the diagonal only.
template <int TM, int TN, int KT>
int64_t tiles_of(const GemmArgs& g) {
  static_assert(TM == TN, "upper_only numbering assumes square tiles");
  if (g.M <= 0 || g.N <= 0) return 0;
  const int64_t tm = (g.M + TM - 1) / TM, tn = (g.N + TN - 1) / TN;
  return g.upper_only ? tm * (tm + 1) / 2 : tm * tn;
}

// Operands the LDS-direct kernel can take: 16-byte aligned, rows of a whole
// number of 16-byte chunks, and every byte offset inside a tile's rows below
// 2^31 (ld < 2^22 floats).
bool dma_ok(const GemmArgs& g) {
  auto ok = [](const float* p, int64_t ld) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && (ld & 3) == 0 && ld < (int64_t(1) << 22);
  };
  return ok(g.A, g.lda) && ok(g.B, g.ldb);
}

template <int TM, int TN, int KT>
void launch_tile(const GemmArgs& g0, const GemmArgs* g1, hipStream_t s) {
  GemmPair pr;
  pr.g[0] = g0;
  pr.g[1] = g1 ? *g1 : g0;
  const int64_t t0 = tiles_of<TM, TN, KT>(g0);
  const int64_t t1 = g1 ? tiles_of<TM, TN, KT>(*g1) : 0;
  pr.tiles0 = (int)t0;
  if (t0 + t1 == 0) return;
  if (dma_ok(g0) && (!g1 || dma_ok(*g1))) {
    constexpr size_t smem = (size_t)2 * KT * (TM + TN) * sizeof(float);
    // set once per instantiation; a function-local static is initialised
    // exactly once even when several host threads launch concurrently
    static const bool attr = [&] {
      (void)hipFuncSetAttribute((const void*)gemm_f32_dma_kernel<TM, TN, KT>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((gemm_f32_dma_kernel<TM, TN, KT>), dim3((unsigned)(t0 + t1)), dim3(256), smem, s, pr);
    return;
  }
  constexpr size_t smem = (size_t)2 * KT * ((TM + PAD) + (TN + PAD)) * sizeof(float);
  static const bool attr = [&] {   // once, thread-safe (function-local static)
    (void)hipFuncSetAttribute((const void*)gemm_f32_kernel<TM, TN, KT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)smem);
    return true;
  }();
  (void)attr;
  hipLaunchKernelGGL((gemm_f32_kernel<TM, TN, KT>), dim3((unsigned)(t0 + t1)), dim3(256), smem, s, pr);
}

void launch_dispatch(const GemmArgs& g0, const GemmArgs* g1, hipStream_t s) {
  // Problems too small to fill the chip with 64 x 64 tiles (and K <= 512) go
  // to the small-product kernel.
  const int64_t t128 = tiles_of<128, 128, 32>(g0) + (g1 ? tiles_of<128, 128, 32>(*g1) : 0);
  const int64_t t64 = tiles_of<64, 64, 32>(g0) + (g1 ? tiles_of<64, 64, 32>(*g1) : 0);
  const int kmax = std::max(g0.K, g1 ? g1->K : 0);
  if (t64 < 256 && kmax <= 8 * SK_MAX) {
    GemmPair pr;
    pr.g[0] = g0;
    pr.g[1] = g1 ? *g1 : g0;
    const int64_t t0 = tiles_of<32, 32, 32>(g0);
    const int64_t t1 = g1 ? tiles_of<32, 32, 32>(*g1) : 0;
    pr.tiles0 = (int)t0;
    if (t0 + t1 > 0) hipLaunchKernelGGL(gemm_f32_small_kernel, dim3((unsigned)(t0 + t1)), dim3(256), 0, s, pr);
    return;
  }
  // Tile size from the rounds of workgroups the 256 CUs run: a CU's time
  // follows the most tiles any CU gets, ceil(tiles / 256).  128 x 128 tiles
  // do a quarter of the work of four 64 x 64 tiles at about 10 % less cost
  // per flop, but leave more of the last round idle; they are taken when
  // their rounds, in 64 x 64 units, cost no more than 1.1 times the 64 x 64
  // rounds, and not when every CU would hold a single tile (one wave per
  // SIMD, nothing to hide the LDS and memory latency).
  const int64_t r128 = (t128 + 255) / 256, r64 = (t64 + 255) / 256;
  if (r128 >= 2 && 40 * r128 <= 11 * r64) {
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
