// Hessian accumulation H += 2 X^T X on the gfx950 matrix cores.
//
// "GPTQ, with the code open", section "Measuring damage where it matters":
// H = 2 X X^T with X holding the calibration inputs (features x tokens).  In
// memory X is token-major [N, d], so the contraction runs over the strided
// axis: H[i][j] = 2 sum_t X[t][i] X[t][j].  bf16/fp16 products are exact in
// fp32 and the sums are fp32 (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Work split: 256 x 256 output tiles of the upper triangle, times `splits`
// contiguous token ranges.  Each workgroup streams its token range in K-steps
// of 64; its waves hold blocks of the tile as 32 x 32 MFMA blocks with the
// accumulators in AGPRs (8 waves of 128 x 64 on the LDS-direct path, two per
// SIMD so that one wave's operand reads overlap the other's MFMAs; 4 waves of
// 128 x 128 on the register path).  X arrives feature-contiguous (token rows), while an MFMA
// operand wants 8 consecutive tokens of one feature.  Two data paths:
//  * interior tiles (both 256-feature slabs inside [0, d), X 16-byte aligned,
//    ldx % 8 == 0, ldx < 2^24): buffer loads that write LDS directly carry each
//    K-step's token rows of both slabs into LDS one step ahead of the MFMAs
//    (no registers, no transposes in the ALU); the operands are read back with
//    the LDS transpose read ds_read_b64_tr_b16, which hands each lane four
//    consecutive tokens of one feature.  LDS rows are 512 bytes (one token, 256
//    features) with 16-byte chunk c stored at chunk position c ^ ((row & 3) << 2),
//    so the 16 lanes of a transpose read hit distinct banks;
//  * edge tiles and unaligned X: each thread loads an 8-token x 8-feature patch
//    of each slab through a bounds-checked loader, transposes it in registers
//    with v_perm_b32, and writes eight 16-byte token-contiguous rows into LDS
//    (128-byte rows, chunks XOR-swizzled by the row index), two K-steps ahead.
// Both paths read the same products and add them in the same order, so the
// result does not depend on which one a tile takes.
// With one split the tile is added straight into H; otherwise each workgroup
// writes its partial tile to the workspace and a second kernel sums the
// partials of every tile in split order (deterministic, no floating-point
// atomics) and adds twice the sum into H.  Work items (split, tile) are
// numbered split-major with the tiles of a split in super-tile order; the
// dispatcher deals workgroups round-robin to the eight XCDs, so within every
// 256 workgroups XCD x is handed the 32 consecutive work items 32x .. 32x+31:
// the tiles resident on one XCD share row and column slabs in its L2, and all
// XCDs work on the same one or two token ranges, which stay in the memory-side
// cache.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int TILE = 256;
constexpr int KSTEP = 64;
constexpr int ROWB = KSTEP * 2;  // bytes per LDS row (64 x 16-bit)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) v4s lds_v4s;

GPTQ_DEV int swz(int f) { return (f ^ (f >> 3)) & 7; }

constexpr int SUPER = 4;  // tiles per super-tile edge in the compact tile order

// The t-th upper-triangle tile (bi <= bj) in super-tile order: super-tiles of
// SUPER x SUPER tiles are visited row by row over the upper triangle, and the
// tiles inside each one row by row, so consecutive t share row/column slabs.
GPTQ_DEV void tile_coords(int t, int nt, int& bi, int& bj) {
  const int ns = (nt + SUPER - 1) / SUPER;
  for (int si = 0; si < ns; ++si) {
    for (int sj = si; sj < ns; ++sj) {
      const int r0 = si * SUPER, r1 = min(nt, r0 + SUPER);
      const int c0 = sj * SUPER, c1 = min(nt, c0 + SUPER);
      int cnt = 0;
      for (int r = r0; r < r1; ++r) cnt += max(0, c1 - max(c0, r));
      if (t < cnt) {
        for (int r = r0; r < r1; ++r) {
          const int n = max(0, c1 - max(c0, r));
          if (t < n) {
            bi = r;
            bj = max(c0, r) + t;
            return;
          }
          t -= n;
        }
      }
      t -= cnt;
    }
  }
  bi = bj = 0;  // not reached for t < tiles
}

// Load the 8 x 8 patch (tokens t0..t0+7, features f0..f0+7) as eight rows of
// 4 dwords (two 16-bit features each).  Out-of-range entries are zero.  VEC:
// X is 16-byte aligned with ldx % 8 == 0, so a full row of the patch is one
// 16-byte load; otherwise 16-bit loads.
template <bool VEC>
GPTQ_DEV void load_patch(const uint16_t* X, int64_t ldx, int64_t t0, int64_t t_end, int f0, int d,
                         u32x4 v[8]) {
  const bool full_f = f0 + 8 <= d;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + i;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (t < t_end) {
      const uint16_t* p = X + t * ldx + f0;
      if (VEC && full_f) {
        r = *reinterpret_cast<const u32x4*>(p);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) h[c] = (f0 + c < d) ? (uint32_t)p[c] : 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) r[w] = h[2 * w] | (h[2 * w + 1] << 16);
      }
    }
    v[i] = r;
  }
}

template <int DT>
GPTQ_DEV floatx16 mfma16(u32x4 a, u32x4 b, floatx16 c) {
  if constexpr (DT == 1) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// The K-loop of one tile over tokens [t_beg, t_end) through the
// bounds-checked loader (edge tiles, unaligned X).
//
// Software pipeline over K-steps of 64 tokens: at the start of step s the
// registers hold the raw patches of step s+1.  They are transposed into the
// LDS buffer that step s's MFMAs do not read, and the loads of step s+2 are
// issued into the freed registers, before step s's MFMAs (LDS buffer s&1).
// MFMA operands of the next 16-token sub-step are read from LDS while the
// current sub-step's MFMAs run.
template <int DT, bool VEC, bool DIAG>
GPTQ_DEV void syrk_steps(const uint16_t* __restrict__ X, int64_t ldx, int64_t t_beg, int64_t t_end, int d,
                         int fi0, int fj0, bool compute_lower, int wm, int wn, unsigned char* smem,
                         floatx16 (&acc)[4][4]) {
  constexpr bool diag = DIAG;
  const bool compute = !DIAG || compute_lower;
  auto a_buf = [&](int b) { return smem + b * (TILE * ROWB); };
  auto b_buf = [&](int b) { return smem + (2 + b) * (TILE * ROWB); };
  const int tid = threadIdx.x, lane = tid & 63;
  // Loader role: every thread carries one 8-token x 8-feature patch of the
  // row slab (A) and one of the column slab (B, not needed on diagonal tiles).
  const int tb = tid >> 5, fb = tid & 31;
  u32x4 ra0[8], rb0[8];
  const int64_t nsteps = (t_end - t_beg + KSTEP - 1) / KSTEP;

  auto fetch = [&](int64_t st, u32x4 (&ra)[8], u32x4 (&rb)[8]) {
    const int64_t t0 = t_beg + st * KSTEP + tb * 8;
    load_patch<VEC>(X, ldx, t0, t_end, fi0 + fb * 8, d, ra);
    if (!diag) load_patch<VEC>(X, ldx, t0, t_end, fj0 + fb * 8, d, rb);
  };
  // Transpose feature rows m0 .. m0+3 of a patch and write them to LDS.
  auto stage4 = [&](unsigned char* lds, const u32x4 (&rg)[8], int m0) {
#pragma unroll
    for (int m = m0; m < m0 + 4; ++m) {
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = __builtin_amdgcn_perm(rg[2 * u + 1][m >> 1], rg[2 * u][m >> 1], sel);
      const int f = fb * 8 + m;
      *reinterpret_cast<u32x4*>(lds + f * ROWB + ((tb ^ swz(f)) * 16)) = o;
    }
  };
  auto stage = [&](int buf, const u32x4 (&ra)[8], const u32x4 (&rb)[8]) {
    stage4(a_buf(buf), ra, 0);
    stage4(a_buf(buf), ra, 4);
    if (!diag) {
      stage4(b_buf(buf), rb, 0);
      stage4(b_buf(buf), rb, 4);
    }
  };
  u32x4 fa[2][4], fbm[2][4];
  auto frags = [&](const unsigned char* as, const unsigned char* bs, int kk, u32x4 (&a)[4], u32x4 (&b)[4]) {
    const int chunk_id = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = wm + 32 * i + (lane & 31);
      a[i] = *reinterpret_cast<const u32x4*>(as + f * ROWB + ((chunk_id ^ swz(f)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = wn + 32 * j + (lane & 31);
      b[j] = *reinterpret_cast<const u32x4*>(bs + f * ROWB + ((chunk_id ^ swz(f)) * 16));
    }
  };
  auto mfmas = [&](const u32x4 (&a)[4], const u32x4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<DT>(a[i], b[j], acc[i][j]);
  };
  // K-step st from LDS buffer buf; (na, nb) hold the raw patches of step
  // st+1: they are transposed into the other buffer and then refilled with
  // the loads of step st+2.
  auto step = [&](int64_t st, int buf, u32x4 (&na)[8], u32x4 (&nb)[8]) {
    const unsigned char* as = a_buf(buf);
    const unsigned char* bs = diag ? a_buf(buf) : b_buf(buf);
    if (compute) {
      frags(as, bs, 0, fa[0], fbm[0]);
      frags(as, bs, 1, fa[1], fbm[1]);
    }
    if (st + 1 < nsteps) stage(buf ^ 1, na, nb);
    if (st + 2 < nsteps) fetch(st + 2, na, nb);
    if (compute) {
      mfmas(fa[0], fbm[0]);
      frags(as, bs, 2, fa[0], fbm[0]);
      mfmas(fa[1], fbm[1]);
      frags(as, bs, 3, fa[1], fbm[1]);
      mfmas(fa[0], fbm[0]);
      mfmas(fa[1], fbm[1]);
    }
    __syncthreads();
  };
  if (nsteps > 0) {
    fetch(0, ra0, rb0);
    stage(0, ra0, rb0);
    if (nsteps > 1) fetch(1, ra0, rb0);
    __syncthreads();
    for (int64_t st = 0; st < nsteps; ++st) step(st, (int)(st & 1), ra0, rb0);
  }
}

// The K-loop of one interior tile (see the header): K-step st's token rows
// of both slabs are carried into LDS buffer st & 1 by buffer loads that write
// LDS, issued before step st-1's MFMAs; one wait and one barrier per step.
// LDS buffer b holds slab A at b * 64 KiB and slab B 32 KiB after it, each 64
// token rows of 512 bytes.
GPTQ_DEV int dsw(int r) { return (r & 3) << 2; }

constexpr int DMA_WAVES = 8;   // waves of the LDS-direct kernel: 2 x 4 blocks of 128 x 64
constexpr int DMA_NB = 2;      // 32-column MFMA blocks per wave

template <int DT, bool DIAG>
GPTQ_DEV void syrk_steps_dma(const uint16_t* __restrict__ X, int64_t ldx, int64_t t_beg, int64_t t_end,
                             int fi0, int fj0, bool compute, int wm, int wn, unsigned char* smem,
                             floatx16 (&acc)[4][DMA_NB]) {
  constexpr int SLAB = KSTEP * 512, BUF = 2 * SLAB;
  // Each load instruction of a wave moves two token rows of one slab (32
  // lanes x 16 bytes each); a wave issues 4 per slab and step.
  constexpr int NI = KSTEP / 2 / DMA_WAVES;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  lds_u8* lbase = (lds_u8*)smem;  // generic to LDS address space
  const int64_t nsteps = (t_end - t_beg + KSTEP - 1) / KSTEP;
  auto dma = [&](int64_t st, int b) {
    // One descriptor per K-step (wave-uniform): base at the step's first
    // token row, records up to t_end, so rows past t_end load zeros.  With
    // ldx < 2^24 every offset of the step fits the 32-bit VGPR offset.
    const int64_t ts = t_beg + st * KSTEP;
    const int64_t nrec = min((t_end - ts) * ldx * 2, (int64_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(X + ts * ldx), (short)0, (int)nrec, 0x00020000);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int I = wave * NI + q;
      const int r = 2 * I + (lane >> 5), c = (lane & 31) ^ dsw(r);
      const int ro = r * (int)ldx * 2;
      // lane l of the instruction lands at LDS base + 16 l: row r, position
      // lane & 31, which holds chunk c of the row.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lbase + b * BUF + I * 1024, 16, ro + (fi0 + 8 * c) * 2, 0, 0, 0);
      if (!DIAG)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lbase + b * BUF + SLAB + I * 1024, 16,
                                                 ro + (fj0 + 8 * c) * 2, 0, 0, 0);
    }
  };
  // Four 16-bit values of token row r at slab features fo .. fo+3 (fo % 4 == 0)
  // as read by one lane of a transpose read: the 16 lanes of a group that read
  // rows r0 + (i >> 2), features fo0 + 4 (i & 3), receive, lane i, the values
  // of feature fo0 + i % 16 ... at the four rows r0 .. r0+3.
  auto tr = [&](const lds_u8* slab, int r, int fo) {
    const int off = r * 512 + ((((fo >> 3) ^ dsw(r))) << 4) + ((fo & 7) >> 2) * 8;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(slab + off));
  };
  // The 32x32x16 MFMA operand of lane (G = lane >> 4, j = lane & 15) is feature
  // base_f + 16 (G & 1) + j at tokens 16 kk + 8 (G >> 1) .. +7: two transpose
  // reads of four tokens each.
  const int G = lane >> 4, j = lane & 15;
  auto frag = [&](const lds_u8* slab, int base_f, int kk) {
    const int row0 = 16 * kk + 8 * (G >> 1) + (j >> 2);
    const int fo = base_f + 16 * (G & 1) + 4 * (j & 3);
    const v4s lo = tr(slab, row0, fo), hi = tr(slab, row0 + 4, fo);
    u32x4 v;
    v[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    v[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    v[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    v[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return v;
  };
  u32x4 fa[2][4], fb[2][DMA_NB];
  auto frags = [&](int b, int kk, u32x4 (&a)[4], u32x4 (&bb)[DMA_NB]) {
    const lds_u8* sa = lbase + b * BUF;
    const lds_u8* sb = DIAG ? sa : sa + SLAB;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(sa, wm + 32 * i, kk);
#pragma unroll
    for (int jj = 0; jj < DMA_NB; ++jj) bb[jj] = frag(sb, wn + 32 * jj, kk);
  };
  auto mfmas = [&](const u32x4 (&a)[4], const u32x4 (&bb)[DMA_NB]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < DMA_NB; ++jj) acc[i][jj] = mfma16<DT>(a[i], bb[jj], acc[i][jj]);
  };
  if (nsteps <= 0) return;
  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; ++st) {
    const int b = (int)(st & 1);
    if (st + 1 < nsteps) dma(st + 1, b ^ 1);
    if (compute) {
#pragma unroll
      for (int kk = 0; kk < KSTEP / 16; kk += 2) {
        frags(b, kk, fa[0], fb[0]);
        frags(b, kk + 1, fa[1], fb[1]);
        mfmas(fa[0], fb[0]);
        mfmas(fa[1], fb[1]);
      }
    }
    // step st+1 has landed (own loads), in every wave (barrier); buffer b is
    // free for step st+2.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// Work item of workgroup b.  Workgroup b runs on XCD b % 8; within each full
// run of 256 workgroups it takes work item 32 (b % 8) + (b % 256) / 8 of that
// run (a bijection).
GPTQ_DEV int work_item(int b, int items) {
  if (b < (items & ~255)) b = (b & ~255) | ((b & 7) << 5) | ((b & 255) >> 3);
  return b;
}

// Epilogue of one wave's MB x NBW MFMA blocks at (wm, wn) of tile (fi0, fj0).
// Lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] per block.  With one
// split the tile is added into H, else written as the split's partial tile.
template <int NBW>
GPTQ_DEV void syrk_epilogue(const floatx16 (&acc)[4][NBW], bool compute, int wm, int wn, int fi0, int fj0, int d,
                            float* __restrict__ H, float* __restrict__ part, int split, int tiles, int tile) {
  const int lane = threadIdx.x & 63;
  if (part == nullptr) {
    if (!compute) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int gj = fj0 + wn + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gi = fi0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (gi < d && gj < d) {
            float* p = H + (int64_t)gi * d + gj;
            *p = __builtin_fmaf(2.0f, acc[i][j][v], *p);
          }
        }
      }
  } else {
    float* pt = part + ((int64_t)split * tiles + tile) * (TILE * TILE);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int c = wn + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          pt[r * TILE + c] = compute ? acc[i][j][v] : 0.f;
        }
      }
  }
}

// Interior tiles with 16-byte aligned X, ldx % 8 == 0 and ldx < 2^24: the
// LDS-direct loop with 8 waves (2 per SIMD, so one wave's operand reads
// overlap the other's matrix-core work), each a 128 x 64 block of the tile.
// Work items whose tile is not interior are left to syrk16_kernel.
template <int DT>
__global__ __launch_bounds__(512, 1) void syrk16_dma_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                             int64_t n_tok, int d, int nt, int64_t chunk,
                                                             float* __restrict__ H, float* __restrict__ part,
                                                             int tiles, int splits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int w = work_item((int)blockIdx.x, tiles * splits);
  const int split = w / tiles, tile = w % tiles;
  int bi, bj;
  tile_coords(tile, nt, bi, bj);
  const int fi0 = bi * TILE, fj0 = bj * TILE;
  if (fi0 + TILE > d || fj0 + TILE > d) return;   // an edge tile: syrk16_kernel's
  const bool diag = bi == bj;
  const int64_t t_beg = (int64_t)split * chunk;
  const int64_t t_end = min(n_tok, t_beg + chunk);
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  // On a diagonal tile the blocks strictly below the diagonal mirror ones
  // above it and are not computed.
  const bool compute = !(diag && wn + 64 <= wm);
  floatx16 acc[4][DMA_NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < DMA_NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (diag) syrk_steps_dma<DT, true>(X, ldx, t_beg, t_end, fi0, fj0, compute, wm, wn, smem, acc);
  else syrk_steps_dma<DT, false>(X, ldx, t_beg, t_end, fi0, fj0, compute, wm, wn, smem, acc);
  syrk_epilogue<DMA_NB>(acc, compute, wm, wn, fi0, fj0, d, H, part, split, tiles, tile);
}

// The register path (edge tiles, or X without the alignment of the
// LDS-direct path): 4 waves, each a 128 x 128 block of the tile.  With
// skip_interior the interior tiles are left to syrk16_dma_kernel.
template <int DT, bool VEC>
__global__ __launch_bounds__(256, 1) void syrk16_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                         int64_t n_tok, int d, int nt,
                                                         int64_t chunk, float* __restrict__ H,
                                                         float* __restrict__ part, int tiles,
                                                         int splits, int skip_interior) {
  // LDS: A buffers 0/1 then B buffers 0/1, TILE rows of ROWB bytes each.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int w = work_item((int)blockIdx.x, tiles * splits);
  const int split = w / tiles, tile = w % tiles;
  int bi, bj;
  tile_coords(tile, nt, bi, bj);
  const bool diag = bi == bj;
  const int fi0 = bi * TILE, fj0 = bj * TILE;
  if (skip_interior && fi0 + TILE <= d && fj0 + TILE <= d) return;
  const int64_t t_beg = (int64_t)split * chunk;
  const int64_t t_end = min(n_tok, t_beg + chunk);

  // 4 waves as 2 x 2 blocks of 128 x 128 (4 x 4 MFMA blocks of 32 x 32 each,
  // accumulators in the AGPR half of the register file).  On a diagonal tile
  // the lower-left block mirrors the upper-right one and is not computed.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const bool compute = !(diag && wm > wn);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (diag) syrk_steps<DT, VEC, true>(X, ldx, t_beg, t_end, d, fi0, fj0, compute, wm, wn, smem, acc);
  else syrk_steps<DT, VEC, false>(X, ldx, t_beg, t_end, d, fi0, fj0, compute, wm, wn, smem, acc);
  syrk_epilogue<4>(acc, compute, wm, wn, fi0, fj0, d, H, part, split, tiles, tile);
}

// H[i][j] += 2 * sum over splits of the partial tiles, in split order.  One
// thread per 4 consecutive columns of a tile row; the partial loads are
// issued together before any is summed.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part, float* H, int d,
                                                              int nt, int tiles, int splits) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index over all tiles
  constexpr int Q = TILE * TILE / 4;
  if (q >= (int64_t)tiles * Q) return;
  const int tile = (int)(q / Q), e4 = (int)(q % Q);
  int bi, bj;
  tile_coords(tile, nt, bi, bj);
  const int r = e4 / (TILE / 4), c = (e4 % (TILE / 4)) * 4;
  const int gi = bi * TILE + r, gj = bj * TILE + c;
  if (gi >= d || gj >= d) return;
  const floatx4* p0 = reinterpret_cast<const floatx4*>(part + (int64_t)tile * (TILE * TILE)) + e4;
  const int64_t stride = (int64_t)tiles * Q;   // one split's partials, in float4
  floatx4 sum = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= splits; k += 8) {
    floatx4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p0 + (k + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; k < splits; ++k) sum += __builtin_nontemporal_load(p0 + k * stride);
  float* hp = H + (int64_t)gi * d + gj;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (gj + u < d) hp[u] = __builtin_fmaf(2.0f, sum[u], hp[u]);
}

}  // namespace

SyrkPlan plan_syrk(int64_t d, int64_t n_tok) {
  SyrkPlan p;
  p.tile = TILE;
  const int nt = (int)((d + TILE - 1) / TILE);
  p.tiles = nt * (nt + 1) / 2;
  const int64_t steps = (n_tok + KSTEP - 1) / KSTEP;
  // Enough workgroups to cover the 256 CUs evenly, each with >= 16 K-steps.
  // Each split adds a round trip of partial tiles through memory: a small
  // charge per split while the tiles are few (the partials are small next to
  // the work), a larger one from 1024 tiles on, and at most 16384 partial
  // tiles (4 GiB) in all.
  int best = 1;
  if (p.tiles < 4096) {
    double best_eff = -1.0;
    const double per_split = p.tiles < 1024 ? 0.002 : 0.01;
    for (int s = 1; s <= 64; ++s) {
      if (s > 1 && steps / s < 16) break;
      if (s > 1 && (int64_t)p.tiles * s > 16384) break;
      const int64_t wgs = (int64_t)p.tiles * s;
      const int64_t waves = (wgs + 255) / 256;
      const double eff = (double)wgs / (double)(waves * 256);
      const double score = eff - (wgs < 512 ? 0.5 : 0.0) - per_split * s;
      if (score > best_eff) {
        best_eff = score;
        best = s;
      }
    }
  }
  p.splits = best;
  p.chunk = ((steps + best - 1) / best) * KSTEP;
  return p;
}

size_t syrk_workspace_bytes(const SyrkPlan& p) {
  if (p.splits <= 1) return 0;
  // partial tiles
  return (size_t)p.splits * (size_t)p.tiles * TILE * TILE * sizeof(float);
}

void launch_syrk16(float* H, int64_t d, const void* X, int dtype, int64_t n_tok, int64_t ldx,
                   const SyrkPlan& p, float* ws, hipStream_t s) {
  const int nt = (int)((d + TILE - 1) / TILE);
  const size_t shmem = 4 * TILE * ROWB;  // 128 KiB: A and B, double buffered
  static const bool attr_set = [&] {   // once, thread-safe (function-local static)
    const void* fns[] = {(const void*)syrk16_kernel<1, true>, (const void*)syrk16_kernel<2, true>,
                         (const void*)syrk16_kernel<1, false>, (const void*)syrk16_kernel<2, false>,
                         (const void*)syrk16_dma_kernel<1>, (const void*)syrk16_dma_kernel<2>};
    for (const void* f : fns) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    return true;
  }();
  (void)attr_set;
  dim3 grid((unsigned)(p.tiles * p.splits));
  float* part = p.splits > 1 ? ws : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && (ldx % 8 == 0) && ldx < (int64_t(1) << 24);
  const bool edges = d % TILE != 0;   // tiles reaching past d take the register path
  const uint16_t* Xh = reinterpret_cast<const uint16_t*>(X);
  // Interior tiles of aligned X: the 8-wave LDS-direct kernel; the rest (or
  // everything, for X without that alignment): the register-path kernel.
  // Each (split, tile) is computed by exactly one of the two, and both add
  // the same products in the same order.
  if (vec) {
    if (dtype == 1)
      hipLaunchKernelGGL((syrk16_dma_kernel<1>), grid, dim3(64 * DMA_WAVES), shmem, s, Xh, ldx, n_tok, (int)d, nt,
                         p.chunk, H, part, p.tiles, p.splits);
    else
      hipLaunchKernelGGL((syrk16_dma_kernel<2>), grid, dim3(64 * DMA_WAVES), shmem, s, Xh, ldx, n_tok, (int)d, nt,
                         p.chunk, H, part, p.tiles, p.splits);
  }
  if (!vec || edges) {
#define GPTQ_SYRK_LAUNCH(DT, V)                                                                        \
  hipLaunchKernelGGL((syrk16_kernel<DT, V>), grid, dim3(256), shmem, s, Xh, ldx, n_tok, (int)d, nt, \
                     p.chunk, H, part, p.tiles, p.splits, vec ? 1 : 0)
    if (dtype == 1) {
      if (vec) GPTQ_SYRK_LAUNCH(1, true); else GPTQ_SYRK_LAUNCH(1, false);
    } else {
      if (vec) GPTQ_SYRK_LAUNCH(2, true); else GPTQ_SYRK_LAUNCH(2, false);
    }
#undef GPTQ_SYRK_LAUNCH
  }
  if (p.splits > 1) {
    const int64_t n4 = (int64_t)p.tiles * (TILE * TILE / 4);
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const float*)part, H, (int)d, nt, p.tiles, p.splits);
  }
}

}  // namespace gptq
