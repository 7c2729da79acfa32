// Hessian accumulation H += 2 X^T X on the gfx950 matrix cores.
//
// "GPTQ, with the code open", section "Measuring damage where it matters":
// H = 2 X X^T with X holding the calibration inputs (features x tokens).  In
// memory X is token-major [N, d], so the contraction runs over the strided
// axis: H[i][j] = 2 sum_t X[t][i] X[t][j].  bf16/fp16 products are exact in
// fp32 and the sums are fp32 (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Work split: 256 x 256 output tiles of the upper triangle, times `splits`
// contiguous token ranges.  Each workgroup (4 waves, each a 128 x 128 quarter
// of the tile as 4 x 4 MFMA blocks) streams its token range in K-steps of 64.
// A K-step of X arrives feature-contiguous; each thread loads an 8-token x
// 8-feature patch (eight 16-byte loads), transposes it in registers with
// v_perm_b32, and writes eight 16-byte token-contiguous rows into LDS, so
// every MFMA operand is a single 16-byte LDS read.  LDS rows are 128 bytes
// (64 tokens) with the 16-byte chunks XOR-swizzled by the row index, which
// keeps both the transposed writes and the MFMA reads free of bank conflicts.
// With one split the tile is added straight into H; otherwise partial tiles
// go to the workspace and the last workgroup of each tile to finish (an
// integer arrival counter) sums them in split order -- deterministic, no
// floating-point atomics -- and adds 2x the sum into H.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int TILE = 256;
constexpr int KSTEP = 64;
constexpr int ROWB = KSTEP * 2;  // bytes per LDS row (64 x 16-bit)

GPTQ_DEV int swz(int f) { return (f ^ (f >> 3)) & 7; }

GPTQ_DEV void tile_coords(int t, int nt, int& bi, int& bj) {
  int rem = t;
  bi = 0;
  while (rem >= nt - bi) {
    rem -= nt - bi;
    ++bi;
  }
  bj = bi + rem;
}

// Load the 8 x 8 patch (tokens t0..t0+7, features f0..f0+7) as eight rows of
// 4 dwords (two 16-bit features each).  Out-of-range entries are zero.
GPTQ_DEV void load_patch(const uint16_t* X, int64_t ldx, int64_t t0, int64_t t_end, int f0, int d,
                         u32x4 v[8]) {
  const bool full_f = f0 + 8 <= d;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + i;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (t < t_end) {
      const uint16_t* p = X + t * ldx + f0;
      if (full_f) {
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

// Transpose the patch: o[m] holds feature m for tokens 0..7 (two per dword).
GPTQ_DEV void transpose_patch(const u32x4 v[8], u32x4 o[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      o[m][u] = __builtin_amdgcn_perm(v[2 * u + 1][m >> 1], v[2 * u][m >> 1], sel);
  }
}

GPTQ_DEV void store_patch(unsigned char* lds, int fb, int tb, const u32x4 o[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int f = fb * 8 + m;
    const int chunk = tb ^ swz(f);
    *reinterpret_cast<u32x4*>(lds + f * ROWB + chunk * 16) = o[m];
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

template <int DT>
__global__ __launch_bounds__(256, 1) void syrk16_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                         int64_t n_tok, int d, int nt,
                                                         int64_t chunk, float* __restrict__ H,
                                                         float* __restrict__ part, int tiles,
                                                         int splits, int* __restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // LDS: A buffers 0/1 then B buffers 0/1, TILE rows of ROWB bytes each.
  auto a_buf = [&](int b) { return smem + b * (TILE * ROWB); };
  auto b_buf = [&](int b) { return smem + (2 + b) * (TILE * ROWB); };

  int bi, bj;
  tile_coords(blockIdx.x, nt, bi, bj);
  const bool diag = bi == bj;
  const int fi0 = bi * TILE, fj0 = bj * TILE;
  const int64_t t_beg = (int64_t)blockIdx.y * chunk;
  const int64_t t_end = min(n_tok, t_beg + chunk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int tb = tid >> 5, fb = tid & 31;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  u32x4 va[8], vb[8], o[8];
  auto fetch = [&](int64_t t0) {
    load_patch(X, ldx, t0 + tb * 8, t_end, fi0 + fb * 8, d, va);
    if (!diag) load_patch(X, ldx, t0 + tb * 8, t_end, fj0 + fb * 8, d, vb);
  };
  auto stage = [&](int buf) {
    transpose_patch(va, o);
    store_patch(a_buf(buf), fb, tb, o);
    if (!diag) {
      transpose_patch(vb, o);
      store_patch(b_buf(buf), fb, tb, o);
    }
  };

  if (t_beg < t_end) {
    fetch(t_beg);
    stage(0);
    __syncthreads();
    int buf = 0;
    for (int64_t t0 = t_beg; t0 < t_end; t0 += KSTEP) {
      const bool more = t0 + KSTEP < t_end;
      if (more) fetch(t0 + KSTEP);
      const unsigned char* as = a_buf(buf);
      const unsigned char* bs = diag ? a_buf(buf) : b_buf(buf);
#pragma unroll
      for (int kk = 0; kk < KSTEP / 16; ++kk) {
        const int chunk_id = 2 * kk + (lane >> 5);
        u32x4 a[4], b[4];
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
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<DT>(a[i], b[j], acc[i][j]);
      }
      if (more) stage(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // Epilogue.  Lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] per block.
  if (part == nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
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
    float* pt = part + ((int64_t)blockIdx.y * tiles + blockIdx.x) * (TILE * TILE);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = wn + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          pt[r * TILE + c] = acc[i][j][v];
        }
      }
    // The last of the tile's `splits` workgroups to finish sums all partials
    // in split order (deterministic) and adds twice the sum into H.
    __shared__ int last;
    __threadfence();
    __syncthreads();
    if (tid == 0) last = (atomicAdd(&counters[blockIdx.x], 1) == splits - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();
    const float* p0 = part + (int64_t)blockIdx.x * (TILE * TILE);
    for (int e4 = tid; e4 < TILE * TILE / 4; e4 += 256) {
      const int r = e4 / (TILE / 4), c = (e4 % (TILE / 4)) * 4;
      floatx4 sum = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < splits; ++k)
        sum += __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(p0 + (int64_t)k * tiles * (TILE * TILE) + r * TILE + c));
      const int gi = fi0 + r, gj = fj0 + c;
      if (gi < d) {
        float* hp = H + (int64_t)gi * d + gj;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (gj + q < d) hp[q] = __builtin_fmaf(2.0f, sum[q], hp[q]);
      }
    }
    if (tid == 0) counters[blockIdx.x] = 0;
  }
}

__global__ void zero_counters_kernel(int* counters, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) counters[i] = 0;
}

}  // namespace

SyrkPlan plan_syrk(int64_t d, int64_t n_tok) {
  SyrkPlan p;
  p.tile = TILE;
  const int nt = (int)((d + TILE - 1) / TILE);
  p.tiles = nt * (nt + 1) / 2;
  const int64_t steps = (n_tok + KSTEP - 1) / KSTEP;
  // Enough workgroups to cover the 256 CUs evenly, each with >= 16 K-steps.
  int best = 1;
  if (p.tiles < 1024) {
    double best_eff = -1.0;
    for (int s = 1; s <= 64; ++s) {
      if (s > 1 && steps / s < 16) break;
      const int64_t wgs = (int64_t)p.tiles * s;
      const int64_t waves = (wgs + 255) / 256;
      const double eff = (double)wgs / (double)(waves * 256);
      const double score = eff - (wgs < 512 ? 0.5 : 0.0) - 0.002 * s;
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
  // partial tiles, then one arrival counter per tile
  return (size_t)p.splits * (size_t)p.tiles * TILE * TILE * sizeof(float) + (size_t)p.tiles * sizeof(int);
}

void launch_syrk16(float* H, int64_t d, const void* X, int dtype, int64_t n_tok, int64_t ldx,
                   const SyrkPlan& p, float* ws, hipStream_t s) {
  const int nt = (int)((d + TILE - 1) / TILE);
  const size_t shmem = 4 * TILE * ROWB;  // 128 KiB: A and B, double buffered
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)syrk16_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    hipFuncSetAttribute((const void*)syrk16_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    attr_set = true;
  }
  dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  float* part = p.splits > 1 ? ws : nullptr;
  int* counters = nullptr;
  if (p.splits > 1) {
    counters = reinterpret_cast<int*>(ws + (size_t)p.splits * p.tiles * TILE * TILE);
    hipLaunchKernelGGL(zero_counters_kernel, dim3((p.tiles + 255) / 256), dim3(256), 0, s, counters, p.tiles);
  }
  if (dtype == 1)
    hipLaunchKernelGGL(syrk16_kernel<1>, grid, dim3(256), shmem, s, (const uint16_t*)X, ldx, n_tok,
                       (int)d, nt, p.chunk, H, part, p.tiles, p.splits, counters);
  else
    hipLaunchKernelGGL(syrk16_kernel<2>, grid, dim3(256), shmem, s, (const uint16_t*)X, ldx, n_tok,
                       (int)d, nt, p.chunk, H, part, p.tiles, p.splits, counters);
}

}  // namespace gptq
