// GPTQ column loop on gfx950 ("GPTQ, with the code open", sections "What
// quantization is, and why anyone bothers", "The repair rule", "From one
// repair to a whole model" and "Paper vs. code").
//
// Per layer:
//   init   : cast W to an fp32 working copy in processing order (columns
//            gathered through perm, dead inputs zeroed); per-row rulers are
//            fitted here, on the original weights, before that zeroing.
//   blocks : for each block of B <= 128 columns
//     chain  (block_kernel): for every row in parallel and the block's columns
//            in order: quantize on the row's ruler, record the code, spread the
//            error err = w - w_hat over the block's later columns with row j of
//            V = U / U_jj (the block's B x B corner, staged in LDS), keep the
//            scaled error e = err / U_jj;
//     defer  (fp32 matrix-core GEMM): W[:, i2:] -= E * U[i1:i2, i2:].
//   The deferral is two-level: inside a super-block of 4 blocks the product
//   for the rest of the super-block follows each block, and the product for
//   every later column follows the super-block (K = 4B).  Every column still
//   receives every repair before its own turn, so the values are those of the
//   plain loop up to rounding order, while the trailing columns are read and
//   written 4x less often.
// Group rulers are fitted when the loop reaches a group's first column, on
// the current values of its columns.
//
// Row mapping: L consecutive lanes own one row; lane p holds block columns
// p, p + L, p + 2L, ... in registers, so column j belongs to lane j % L, slot
// j / L.  The owner's error is broadcast to the row's other lanes with one DPP
// move (quad_perm for L = 4, row_newbcast for L = 16).  The per-column
// dependency chain is thereby five instructions: multiply by 1/scale, round,
// clamp, one FMA for the error, the broadcast (plus the FMA repairing the next
// column); codes, errors and the check of the fast decisions are recomputed
// once per block from the values the columns had at their turn.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int BMAX = 128;

// Min-max ruler ("What quantization is"), IEEE fp32 throughout.  Asymmetric:
// the range stretched to include 0, scale = (max - min) / (2^b - 1), zero =
// rne(-min / scale).  Symmetric: the range [-m, m], m = max(|min|, |max|),
// scale = 2m / (2^b - 1), zero = the middle tick (maxq + 1) / 2.  An all-zero
// range uses [-1, 1].
GPTQ_DEV void fit_ruler(float mn, float mx, float maxq, bool sym, float& scale, float& zero) {
  float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
  if (sym) {
    const float m = fmaxf(-lo, hi);
    lo = -m;
    hi = m;
  }
  if (lo == 0.f && hi == 0.f) {
    lo = -1.f;
    hi = 1.f;
  }
  scale = __fdiv_rn(hi - lo, maxq);
  zero = sym ? 0.5f * (maxq + 1.f) : rne(__fdiv_rn(-lo, scale));
}

// perm comes from device memory; an index outside [0, c) (a caller bug) is
// clamped so that no access leaves the arrays.
GPTQ_DEV int64_t clamp_col(int32_t v, int64_t c) { return v < 0 ? 0 : (v >= c ? c - 1 : (int64_t)v); }

GPTQ_DEV float load_w(const void* W, int wt, int64_t idx) {
  if (wt == 0) return reinterpret_cast<const float*>(W)[idx];
  const uint16_t h = reinterpret_cast<const uint16_t*>(W)[idx];
  if (wt == 1) return __uint_as_float((uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

// Eight consecutive weights of a row as fp32 (16-byte aligned, 16-bit types:
// one 16-byte load; fp32: two).
GPTQ_DEV void load_w8(const void* W, int wt, int64_t idx, float (&v)[8]) {
  if (wt == 0) {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(W) + idx);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(W) + idx + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = lo[e];
      v[4 + e] = hi[e];
    }
    return;
  }
  const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(W) + idx);
  const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = (uint16_t)(w4[e] & 0xFFFFu), h1 = (uint16_t)(w4[e] >> 16);
    if (wt == 1) {
      v[2 * e] = __uint_as_float((uint32_t)h0 << 16);
      v[2 * e + 1] = __uint_as_float((uint32_t)h1 << 16);
    } else {
      v[2 * e] = (float)__builtin_bit_cast(_Float16, h0);
      v[2 * e + 1] = (float)__builtin_bit_cast(_Float16, h1);
    }
  }
}

// One workgroup per row: gather/cast into processing order, zero dead inputs,
// per-row ruler on the original row.  MODE 0: one weight per thread and step.
// MODE 1 (no permutation, c % 8 == 0, rows of W 16-byte aligned) and MODE 2
// (a permutation 16-byte aligned, c % 8 == 0): eight consecutive processing
// columns per thread and step, stored with 16-byte stores; MODE 1 reads W
// with 16-byte loads, MODE 2 reads the permutation with 16-byte loads and
// gathers the eight weights independently, or loads them as one vector when
// they are eight consecutive columns of 16-byte aligned rows (wvec).
template <int MODE>
__global__ __launch_bounds__(256) void init_kernel(QuantArgs a, float* Wp, int wvec) {
  const int64_t row = blockIdx.x;
  const int64_t c = a.c;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  if constexpr (MODE != 0) {
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < c; k += 8 * 256) {
      float v[8];
      int64_t src[8];
      if constexpr (MODE == 1) {
        load_w8(a.W, a.wt, row * a.ldw + k, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) src[e] = k + e;
      } else {
        const int4 p0 = *reinterpret_cast<const int4*>(a.perm + k);
        const int4 p1 = *reinterpret_cast<const int4*>(a.perm + k + 4);
        const int32_t pr[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        // eight consecutive source columns (the identity permutation
        // everywhere) starting at a multiple of 8: one vector load
        bool run = wvec != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          src[e] = clamp_col(pr[e], c);
          run = run && src[e] == src[0] + e;
        }
        if (run && (src[0] & 7) == 0) {
          load_w8(a.W, a.wt, row * a.ldw + src[0], v);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = load_w(a.W, a.wt, row * a.ldw + src[e]);
        }
      }
      floatx4 o[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn = fminf(mn, v[e]);
        mx = fmaxf(mx, v[e]);
        o[e >> 2][e & 3] = (a.dead && a.dead[src[e]]) ? 0.f : v[e];
      }
      *reinterpret_cast<floatx4*>(Wp + row * c + k) = o[0];
      *reinterpret_cast<floatx4*>(Wp + row * c + k + 4) = o[1];
    }
  } else {
    for (int64_t k = threadIdx.x; k < c; k += 256) {
      const int64_t src = a.perm ? clamp_col(a.perm[k], c) : k;
      const float v = load_w(a.W, a.wt, row * a.ldw + src);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
      const bool dk = a.dead && a.dead[src];
      Wp[row * c + k] = dk ? 0.f : v;
    }
  }
  if (a.groupsize <= 0) {
    __shared__ float smn[256], smx[256];
    smn[threadIdx.x] = mn;
    smx[threadIdx.x] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) {
        smn[threadIdx.x] = fminf(smn[threadIdx.x], smn[threadIdx.x + w]);
        smx[threadIdx.x] = fmaxf(smx[threadIdx.x], smx[threadIdx.x + w]);
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      float scale, zero;
      fit_ruler(smn[0], smx[0], (float)((1 << a.bits) - 1), a.sym != 0, scale, zero);
      a.scales[row] = scale;
      a.zeros[row] = (int32_t)zero;
    }
  }
  if (threadIdx.x == 0 && a.row_loss) a.row_loss[row] = 0.f;
}

__global__ void gidx_kernel(const int32_t* perm, int64_t c, int64_t g, int32_t* g_idx) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= c) return;
  const int64_t orig = perm ? clamp_col(perm[k], c) : k;
  g_idx[orig] = g > 0 ? (int32_t)(k / g) : 0;
}

template <int L>
GPTQ_DEV float bcast(float v, int src) {
  const int iv = __float_as_int(v);
  int r;
  if constexpr (L == 4) {
    switch (src) {
      case 0: r = __builtin_amdgcn_mov_dpp(iv, 0x00, 0xF, 0xF, false); break;
      case 1: r = __builtin_amdgcn_mov_dpp(iv, 0x55, 0xF, 0xF, false); break;
      case 2: r = __builtin_amdgcn_mov_dpp(iv, 0xAA, 0xF, 0xF, false); break;
      default: r = __builtin_amdgcn_mov_dpp(iv, 0xFF, 0xF, 0xF, false); break;
    }
  } else {
    switch (src) {
#define GPTQ_NB(n) \
  case n: r = __builtin_amdgcn_mov_dpp(iv, 0x150 + n, 0xF, 0xF, true); break;
      GPTQ_NB(0) GPTQ_NB(1) GPTQ_NB(2) GPTQ_NB(3) GPTQ_NB(4) GPTQ_NB(5) GPTQ_NB(6) GPTQ_NB(7)
      GPTQ_NB(8) GPTQ_NB(9) GPTQ_NB(10) GPTQ_NB(11) GPTQ_NB(12) GPTQ_NB(13) GPTQ_NB(14)
      default: r = __builtin_amdgcn_mov_dpp(iv, 0x150 + 15, 0xF, 0xF, true); break;
#undef GPTQ_NB
    }
  }
  return __int_as_float(r);
}

// Butterfly over the L lanes of a row (DPP within a 16-lane row).
template <int L>
GPTQ_DEV float row_min(float v) {
  v = fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (L == 16) {
    v = fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  }
  return v;
}
template <int L>
GPTQ_DEV float row_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (L == 16) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  }
  return v;
}
template <int L>
GPTQ_DEV float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (L == 16) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  }
  return v;
}

struct BlockArgs {
  float* Wp;      // r x c working copy (processing order)
  float* E;       // scaled errors of this block: E[row * lde + k], k = 0 .. Bw - 1
  int64_t lde;
  const float* U; // c x c
  int64_t r, c, i1;
  int Bw;
  int bits;
  int sym;
  int64_t groupsize;
  const int32_t* perm;
  uint8_t* codes;
  float* scales;
  int32_t* zeros;
  float* W_hat;
  float* row_loss;
  int64_t n_groups;
  int vec_u;      // U is 16-byte aligned and c % 4 == 0
};

// Fit the ruler of the group starting at block column j on the current
// values of its columns (registers for the part inside the block, the working
// copy for the part beyond it).
template <int L, int S>
GPTQ_DEV void fit_group(const float (&w)[S], int p, int j, int Bw, int64_t g, int64_t i1, int64_t c,
                        const float* Wrow, bool valid, float maxq, bool sym, float& scale, float& zero) {
  const int64_t gend = min(i1 + j + g, c);
  float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
  for (int m = 0; m < S; ++m) {
    const int64_t col = i1 + p + L * m;
    if (col >= i1 + j && col < gend && p + L * m < Bw) {
      mn = fminf(mn, w[m]);
      mx = fmaxf(mx, w[m]);
    }
  }
  if (gend > i1 + Bw && valid) {
    for (int64_t col = i1 + Bw + p; col < gend; col += L) {
      const float v = Wrow[col];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
  mn = row_min<L>(mn);
  mx = row_max<L>(mx);
  fit_ruler(mn, mx, maxq, sym, scale, zero);
}

// Stage V[j][k] = U[i1 + j][i1 + k] / U[i1 + j][i1 + j] for k > j (0 on and
// left of the diagonal and past Bw) row-major in LDS, and invd[j] = 1 / U_jj.
// With the repairs written as w_k -= err_j * V[j][k], err_j = w_j - w_hat_j,
// the division by the diagonal leaves the column-to-column dependency chain,
// and the zero diagonal leaves each column's register holding the value it
// had when its turn came.
GPTQ_DEV void stage_block(const BlockArgs& a, float* Vl, float* invd, bool full) {
  const int tid = threadIdx.x;
  const int Bw = a.Bw;
  const int64_t i1 = a.i1, c = a.c;
  if (full && a.vec_u) {
    // thread t, load u: row j = t / 32 + 8 u, columns 4 (t % 32) .. +3
    floatx4 v[16];
    const float* ub = a.U + (i1 + (tid >> 5)) * c + i1 + (tid & 31) * 4;
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const floatx4*>(ub + (int64_t)(8 * u) * c);
    if (tid < BMAX) invd[tid] = __fdiv_rn(1.0f, a.U[(i1 + tid) * c + (i1 + tid)]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e4 = tid + 256 * u, j = e4 >> 5, k = (e4 & 31) * 4;
      const float sj = invd[j];
      floatx4 o;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) o[cc] = (k + cc > j) ? v[u][cc] * sj : 0.f;
      *reinterpret_cast<floatx4*>(Vl + j * BMAX + k) = o;
    }
  } else {
    if (tid < BMAX) invd[tid] = tid < Bw ? __fdiv_rn(1.0f, a.U[(i1 + tid) * c + (i1 + tid)]) : 0.f;
    __syncthreads();
    for (int e = tid; e < BMAX * BMAX; e += 256) {
      const int j = e / BMAX, k = e % BMAX;
      float v = 0.f;
      if (j < Bw && k < Bw && k > j) v = a.U[(i1 + j) * c + (i1 + k)] * invd[j];
      Vl[e] = v;
    }
  }
  __syncthreads();
}

// The tick offset dq = q - zero of the value x: clamp(rne(t) + zero, 0, maxq)
// - zero = med3(rne(t), -zero, maxq - zero), zero being a whole number, with
// t = x / scale correctly rounded (EXACT) or t = x * (1/scale).
template <bool EXACT>
GPTQ_DEV float tick(float x, float scale, float y, float lo, float hi) {
  float t;
  if constexpr (EXACT) {
    t = div_by_recip(x, scale, y);
    t = __builtin_fmaf(__builtin_fmaf(-t, scale, x), y, t);
  } else {
    t = __fmul_rn(x, y);
  }
  return __builtin_amdgcn_fmed3f(rne(t), lo, hi);
}

// True when t = x * (1/scale) lies within 2^-21 |t| of a half-integer, where
// the correctly rounded quotient x / scale (|t - x/scale| < 2^-22.4 |t|) might
// round to the other neighbour.
GPTQ_DEV bool near_half(float x, float y) {
  const float t = __fmul_rn(x, y);
  const float d = __fsub_rn(t, rne(t));
  return fabsf(d) >= __builtin_fmaf(-fabsf(t), 0x1p-21f, 0.5f);
}

// Ruler of the block's first column: per row (read), fitted here (group
// starting at the block), or continued from an earlier block (read).
template <int L, int S>
GPTQ_DEV void block_ruler(const BlockArgs& a, const float (&w)[S], int p, int64_t row, bool valid, int Bw,
                          const float* Wrow, float& scale, float& zero) {
  const int64_t g = a.groupsize, i1 = a.i1;
  const float maxq = (float)((1 << a.bits) - 1);
  if (g <= 0) {
    if (valid) {
      scale = a.scales[row * a.n_groups];
      zero = (float)a.zeros[row * a.n_groups];
    }
  } else if (i1 % g == 0) {
    fit_group<L, S>(w, p, 0, Bw, g, i1, a.c, Wrow, valid, maxq, a.sym != 0, scale, zero);
    if (valid && p == 0) {
      a.scales[row * a.n_groups + i1 / g] = scale;
      a.zeros[row * a.n_groups + i1 / g] = (int32_t)zero;
    }
  } else if (valid) {
    // A group longer than the block continues here: its ruler was fitted (and
    // stored) by the block holding the group's first column.
    scale = a.scales[row * a.n_groups + i1 / g];
    zero = (float)a.zeros[row * a.n_groups + i1 / g];
  }
}

// The block's columns in order, for the L lanes of each row (see the file
// header for the lane mapping).  On return w[m] holds, for every column of
// the block, its value when its turn came (V's zero diagonal leaves it
// alone afterwards).  With MIDG != 0 the ruler changes inside the block, so
// the tick offset, w_hat and error of each column are recorded as they are
// taken, and the fast pass's doubtful decisions are collected per step;
// otherwise everything is recomputed from w after the loop.  EXACT == false
// decides with t = x * (1/scale); an unflagged fast pass is bitwise the exact
// pass, because every later value depends on the decision only.
template <int L, int MIDG, bool FULL, bool EXACT>
GPTQ_DEV bool run_chain(const BlockArgs& a, const float* Vl, int p, int64_t row, bool valid,
                        const float* Wrow, float (&w)[BMAX / L], float (&qreg)[BMAX / L],
                        float (&ereg)[BMAX / L], float (&whreg)[BMAX / L], float& scale, float& zero) {
  constexpr int S = BMAX / L;
  const int Bw = FULL ? BMAX : a.Bw;
  const int64_t i1 = a.i1, c = a.c;
  const float maxq = (float)((1 << a.bits) - 1);
  const int64_t g = a.groupsize;
  block_ruler<L, S>(a, w, p, row, valid, Bw, Wrow, scale, zero);
  float y = __fdiv_rn(1.0f, scale);
  float lo = -zero, hi = maxq - zero;
  uint64_t bad = 0;
  int next_group = MIDG != 0 ? (int)g : BMAX;
  // Lanes of the rows' owners of block column j: lane j % L of every row.
  constexpr uint64_t OWN0 = L == 16 ? 0x0001000100010001ull : 0x1111111111111111ull;

  // Rows of V are read two steps ahead into a ring of registers; the
  // scheduling barrier at the end of each step keeps the compiler from
  // hoisting every read of the unrolled loop to the top (and spilling).
  float vb[3][S];
  const float* vcol = Vl + p;
  auto fetch = [&](int jj, float (&dst)[S]) {
#pragma unroll
    for (int m = 0; m < S; ++m)
      if (m >= jj / L) dst[m] = vcol[jj * BMAX + L * m];
  };
  fetch(0, vb[0]);
  fetch(1, vb[1]);

#pragma clang loop unroll(full)
  for (int j = 0; j < BMAX; ++j) {
    if (j + 2 < BMAX) fetch(j + 2, vb[(j + 2) % 3]);
    // A short block runs all BMAX steps: its missing columns hold 0 in w and
    // in V, quantize to an error of exactly 0 and are never stored.
    const int mj = j / L, pj = j % L;
    // A refit can happen at step j only where a group may start: with
    // MIDG == 32 at multiples of 32, so the refit code exists at those steps
    // only (with any width it is copied into every step of the unrolled loop,
    // far beyond the instruction cache).  j is a constant in each unrolled
    // step, so the test folds away.
    const bool can_refit = MIDG == 32 ? (j > 0 && j % 32 == 0) : (MIDG != 0 && j > 0);
    if (can_refit) {
      if (j == next_group && (FULL || j < Bw)) {
        fit_group<L, S>(w, p, j, Bw, g, i1, c, Wrow, valid, maxq, a.sym != 0, scale, zero);
        y = __fdiv_rn(1.0f, scale);
        lo = -zero;
        hi = maxq - zero;
        if (valid && p == 0) {
          const int64_t gi = (i1 + j) / g;
          a.scales[row * a.n_groups + gi] = scale;
          a.zeros[row * a.n_groups + gi] = (int32_t)zero;
        }
        next_group += (int)g;
      }
    }
    const float x = w[mj];
    const float dq = tick<EXACT>(x, scale, y, lo, hi);
    const float err = __builtin_fmaf(-scale, dq, x);   // w - scale * (q - zero)
    if constexpr (MIDG != 0) {
      const bool own = (p == pj);
      qreg[mj] = own ? dq + zero : qreg[mj];
      whreg[mj] = own ? __fmul_rn(scale, dq) : whreg[mj];
      ereg[mj] = own ? err : ereg[mj];
      if constexpr (!EXACT) {
        bad |= __ballot(near_half(x, y)) & (OWN0 << pj);
        asm volatile("" : "+s"(bad));
      }
      // Materialise this step's records here: left alone, the compiler sinks
      // every step's selects past the loop and keeps all operands live.
      asm volatile("" : "+v"(qreg[mj]), "+v"(ereg[mj]), "+v"(whreg[mj]));
    }
    // Repair every later column of the block: w_k -= err * V[j][k].
    const float eb = bcast<L>(err, pj);
#pragma unroll
    for (int m = 0; m < S; ++m) {
      if (m >= mj) w[m] = __builtin_fmaf(-eb, vb[j % 3][m], w[m]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return bad != 0;
}

// MIDG: groups shorter than the block also start inside it (32: their width
// is a multiple of 32; -1: any width; 0: none).  FULL: the
// block has all BMAX columns.
// One block's columns for this thread's row (V and invd staged): the chain
// (fast decisions; repeated exactly from the block's starting values w0 when
// any decision of the wave is doubtful), then codes, w_hat and scaled errors
// e = (w - w_hat) / U_jj, stored at the original columns, E in row-major
// block order, and the row's loss.  w ends holding each column's value at its
// turn; ereg the scaled errors.
template <int L, int MIDG, bool FULL>
GPTQ_DEV void block_columns(const BlockArgs& a, const float* Vl, const float* invd, int p, int64_t row, bool valid,
                            const float* Wrow, float (&w)[BMAX / L], const float (&w0)[BMAX / L],
                            float (&ereg)[BMAX / L]) {
  constexpr int S = BMAX / L;
  const int Bw = FULL ? BMAX : a.Bw;
  const int64_t i1 = a.i1, c = a.c;
  const float maxq = (float)((1 << a.bits) - 1);
  float qreg[S], whreg[S];
#pragma unroll
  for (int m = 0; m < S; ++m) qreg[m] = ereg[m] = whreg[m] = 0.f;
  float scale = 1.f, zero = 0.f;
  bool bad = run_chain<L, MIDG, FULL, false>(a, Vl, p, row, valid, Wrow, w, qreg, ereg, whreg, scale, zero);
  if constexpr (MIDG == 0) {
    const float y = __fdiv_rn(1.0f, scale);
#pragma unroll
    for (int m = 0; m < S; ++m) bad = bad || near_half(w[m], y);
  }
  const bool exact = __ballot(bad) != 0;   // wave-uniform
  if (exact) {                              // repeat this wave's rows exactly
#pragma unroll
    for (int m = 0; m < S; ++m) w[m] = w0[m];
    run_chain<L, MIDG, FULL, true>(a, Vl, p, row, valid, Wrow, w, qreg, ereg, whreg, scale, zero);
  }
  if constexpr (MIDG == 0) {
    // Codes, w_hat and errors from the values the columns had at their turn.
    const float y = __fdiv_rn(1.0f, scale);
    const float lo = -zero, hi = maxq - zero;
#pragma unroll
    for (int m = 0; m < S; ++m) {
      const float dq = exact ? tick<true>(w[m], scale, y, lo, hi) : tick<false>(w[m], scale, y, lo, hi);
      qreg[m] = dq + zero;
      whreg[m] = __fmul_rn(scale, dq);
      ereg[m] = __builtin_fmaf(-scale, dq, w[m]);
    }
  }

  float loss = 0.f;
#pragma unroll
  for (int m = 0; m < S; ++m) {
    const int col = p + L * m;
    if (col < Bw) {
      ereg[m] *= invd[col];                      // e = (w - w_hat) / U_jj
      loss = __builtin_fmaf(0.5f * ereg[m], ereg[m], loss);
    }
  }
  loss = row_sum<L>(loss);
  if (!valid) return;
#pragma unroll
  for (int m = 0; m < S; ++m) {
    const int col = p + L * m;
    if (col < Bw) {
      const int64_t pk = i1 + col;
      const int64_t orig = a.perm ? clamp_col(a.perm[pk], c) : pk;
      a.codes[row * c + orig] = (uint8_t)(int)qreg[m];
      if (a.W_hat) a.W_hat[row * c + orig] = whreg[m];
      a.E[row * a.lde + col] = ereg[m];
    }
  }
  if (p == 0 && a.row_loss) a.row_loss[row] += loss;
}

template <int L, int MIDG, bool FULL>
__global__ __launch_bounds__(256) void block_kernel(BlockArgs a) {
  constexpr int S = BMAX / L;          // slots per lane
  constexpr int ROWS = 256 / L;        // rows per workgroup
  __shared__ __attribute__((aligned(16))) float Vl[BMAX * BMAX];
  __shared__ float invd[BMAX];

  const int tid = threadIdx.x;
  const int p = tid % L;
  const int64_t row = (int64_t)blockIdx.x * ROWS + tid / L;
  const bool valid = row < a.r;
  const int Bw = FULL ? BMAX : a.Bw;
  const float* Wrow = a.Wp + (valid ? row : 0) * a.c;

  float w[S], w0[S], ereg[S];
#pragma unroll
  for (int m = 0; m < S; ++m) {
    const int col = p + L * m;
    w[m] = w0[m] = (valid && col < Bw) ? Wrow[a.i1 + col] : 0.f;
  }
  stage_block(a, Vl, invd, FULL);
  block_columns<L, MIDG, FULL>(a, Vl, invd, p, row, valid, Wrow, w, w0, ereg);
}

// A super-block of SB_BLOCKS full blocks in one launch (16 lanes per row, 16
// rows per workgroup; one ruler per row, groups of one block, or with MIDG ==
// 32 groups of 32 or 64 columns, which start and end inside a block): the row's
// 512 columns stay in registers from the first block to the last.  After
// each block, its scaled errors E (16 rows x 128, through LDS) update the
// super-block's later blocks on the matrix cores,
//     W[:, k'] -= E_k U[block k, block k'],
// with v_mfma_f32_16x16x4f32 (M = the 16 rows, N = 128, K = 128; each wave
// two 16-column tiles), the product going back to the rows' lanes through
// LDS.  The E of all blocks is also stored for the deferred product beyond
// the super-block.
//
// Every 128 x 128 tile of U the workgroup needs -- the next update's tile of
// U, or the next block's corner -- is loaded into registers one phase ahead
// (16 float4 per thread, all in flight at once) and written to the one LDS
// tile buffer when its phase comes, so the loads of the first update run
// under the chain and each later load under the previous phase.
constexpr int SB_BLOCKS = (int)kSuperBlocks;
constexpr int EPAD = BMAX + 4;   // LDS row stride of the E and product tiles
constexpr int TPAD = BMAX + 4;   // LDS row stride of a tile of U in an update (4 rows of an
                                 // MFMA operand read land on different banks)

// Thread t's share of the 128 x 128 tile of U at (i0, j0): rows t / 32 + 8u,
// columns 4 (t % 32) .. +3 (U 16-byte aligned, c % 4 == 0), and for t < 128
// the diagonal U[i0 + t][i0 + t] (used when the tile is a block's corner).
struct TileRegs {
  floatx4 v[16];
  float dg;
};

GPTQ_DEV void tile_issue(const float* U, int64_t c, int64_t i0, int64_t j0, TileRegs& t) {
  const int tid = threadIdx.x;
  const float* ub = U + (i0 + (tid >> 5)) * c + j0 + (tid & 31) * 4;
#pragma unroll
  for (int u = 0; u < 16; ++u) t.v[u] = *reinterpret_cast<const floatx4*>(ub + (int64_t)(8 * u) * c);
  t.dg = tid < BMAX ? U[(i0 + tid) * c + (i0 + tid)] : 1.f;
}

// The tile as it is (row-major 128 x 128, row stride TPAD), for an update.
GPTQ_DEV void tile_commit_raw(const TileRegs& t, float* Tl) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e4 = tid + 256 * u;
    *reinterpret_cast<floatx4*>(Tl + (e4 >> 5) * TPAD + (e4 & 31) * 4) = t.v[u];
  }
}

// The tile as a block's V = U / diag(U), zero on and left of the diagonal
// (the layout stage_block writes), and invd = 1 / U_jj.
GPTQ_DEV void tile_commit_corner(const TileRegs& t, float* Vl, float* invd) {
  const int tid = threadIdx.x;
  if (tid < BMAX) invd[tid] = __fdiv_rn(1.0f, t.dg);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e4 = tid + 256 * u, j = e4 >> 5, k = (e4 & 31) * 4;
    const float sj = invd[j];
    floatx4 o;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) o[cc] = (k + cc > j) ? t.v[u][cc] * sj : 0.f;
    *reinterpret_cast<floatx4*>(Vl + j * BMAX + k) = o;
  }
  __syncthreads();
}

template <int MIDG>
__global__ __launch_bounds__(256) void superblock_kernel(BlockArgs a, int64_t s1) {
  constexpr int L = 16, S = BMAX / L, ROWS = 16;
  __shared__ __attribute__((aligned(16))) float Vl[BMAX * TPAD];   // a block's V, or a tile of U
  __shared__ float invd[BMAX];
  // The scaled errors of the block just done, and then, once every thread
  // holds its operands from them (the barrier after the first tile commit),
  // the products E_k U[k, k'] for one later block k' at a time: one buffer.
  __shared__ float Et[ROWS * EPAD];
  float* const Pt = Et;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = tid % L, rl = tid / L;
  const int64_t row = (int64_t)blockIdx.x * ROWS + rl;
  const bool valid = row < a.r;
  const int64_t c = a.c;
  const float* Wrow = a.Wp + (valid ? row : 0) * c;

  TileRegs tr;
  tile_issue(a.U, c, s1, s1, tr);   // the first block's corner
  float wsb[SB_BLOCKS][S];
#pragma unroll
  for (int kb = 0; kb < SB_BLOCKS; ++kb)
#pragma unroll
    for (int m = 0; m < S; ++m) wsb[kb][m] = valid ? Wrow[s1 + BMAX * kb + p + L * m] : 0.f;
  tile_commit_corner(tr, Vl, invd);

  float* E0 = a.E;
#pragma unroll
  for (int kb = 0; kb < SB_BLOCKS; ++kb) {
    BlockArgs b = a;
    b.i1 = s1 + BMAX * kb;
    b.Bw = BMAX;
    b.E = E0 + BMAX * kb;
    // the first update's tile of U, in flight during the chain
    if (kb + 1 < SB_BLOCKS) tile_issue(a.U, c, b.i1, b.i1 + BMAX, tr);
    float w[S], ereg[S];
#pragma unroll
    for (int m = 0; m < S; ++m) w[m] = wsb[kb][m];
    block_columns<16, MIDG, true>(b, Vl, invd, p, row, valid, Wrow, w, wsb[kb], ereg);
    if (kb + 1 < SB_BLOCKS) {
#pragma unroll
      for (int m = 0; m < S; ++m) Et[rl * EPAD + p + L * m] = ereg[m];   // 0 on rows past r
      __syncthreads();   // E complete; every wave is done with V
      // A operand for every later block: lane l gives E[l % 16][4 s + l / 16].
      float ea[BMAX / 4];
#pragma unroll
      for (int s4 = 0; s4 < BMAX / 4; ++s4) ea[s4] = Et[(lane & 15) * EPAD + 4 * s4 + (lane >> 4)];
#pragma unroll
      for (int kb2 = kb + 1; kb2 < SB_BLOCKS; ++kb2) {
        tile_commit_raw(tr, Vl);   // U[block kb, block kb2]
        // next phase's tile: the next update's, or the next block's corner
        if (kb2 + 1 < SB_BLOCKS) tile_issue(a.U, c, b.i1, s1 + BMAX * (kb2 + 1), tr);
        else tile_issue(a.U, c, b.i1 + BMAX, b.i1 + BMAX, tr);
        __syncthreads();
        // wave w: columns 32 w .. 32 w + 31 of block kb2 (two 16-column tiles)
        const float* Ut = Vl + (lane >> 4) * TPAD + 32 * wave + (lane & 15);
        floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < BMAX / 4; ++s4) {
          d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[s4], Ut[4 * s4 * TPAD], d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[s4], Ut[4 * s4 * TPAD + 16], d1, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 4 * (lane >> 4) + v;
          Pt[i * EPAD + 32 * wave + (lane & 15)] = d0[v];
          Pt[i * EPAD + 32 * wave + 16 + (lane & 15)] = d1[v];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < S; ++m) wsb[kb2][m] -= Pt[rl * EPAD + p + L * m];
      }
      tile_commit_corner(tr, Vl, invd);   // the next block's V (barriers inside)
    }
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

constexpr int64_t SUPER_BLOCKS = kSuperBlocks;

namespace {

// Columns whose repairs are applied at once before the deferred product:
// SUPER_BLOCKS blocks when that keeps every group inside one super-block or
// starting at a super-block start (so a group's ruler always sees fully
// repaired values), else one block.
int64_t super_block(int64_t B, int64_t g) {
  const int64_t sb = SUPER_BLOCKS * B;
  if (g <= 0 || sb % g == 0 || g % sb == 0) return sb;
  return B;
}

void gemm_update(hipStream_t s, int64_t r, int64_t c, const float* E, int64_t lde, int K, const float* U,
                 int64_t k0, int64_t n0, int64_t n1, float* Wp) {
  // Wp[:, n0:n1] -= E[:, 0:K] * U[k0:k0+K, n0:n1], E row-major with row stride lde
  GemmArgs gm;
  gm.M = (int)r;
  gm.N = (int)(n1 - n0);
  gm.K = K;
  gm.A = E;
  gm.lda = lde;
  gm.a_trans = 0;
  gm.a_mask = MASK_NONE;
  gm.a_off = 0;
  gm.B = U + k0 * c + n0;
  gm.ldb = c;
  gm.b_trans = 0;
  gm.b_mask = MASK_NONE;
  gm.b_off = 0;
  gm.C = Wp + n0;
  gm.ldc = c;
  gm.alpha = -1.f;
  gm.beta = 1.f;
  gm.upper_only = 0;
  launch_gemm_f32(gm, s);
}

}  // namespace

void launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t r = a.r, c = a.c;
  float* Wp = reinterpret_cast<float*>(a.ws);
  // E: r x SB row-major, the scaled errors of the current super-block
  float* E = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + align256((size_t)r * c * sizeof(float)));
  const int wbytes = a.wt == 0 ? 4 : 2;
  // rows of W 16-byte aligned: eight consecutive columns starting at a
  // multiple of 8 are one 16- or 32-byte load
  const bool rows16 = (reinterpret_cast<uintptr_t>(a.W) & 15) == 0 && (a.ldw * wbytes) % 16 == 0;
  const bool vec_w = a.perm == nullptr && c % 8 == 0 && rows16;
  const bool vec_p = a.perm != nullptr && c % 8 == 0 && (reinterpret_cast<uintptr_t>(a.perm) & 15) == 0;
  const int wv = rows16 ? 1 : 0;
  if (vec_w) hipLaunchKernelGGL((init_kernel<1>), dim3((unsigned)r), dim3(256), 0, s, a, Wp, wv);
  else if (vec_p) hipLaunchKernelGGL((init_kernel<2>), dim3((unsigned)r), dim3(256), 0, s, a, Wp, wv);
  else hipLaunchKernelGGL((init_kernel<0>), dim3((unsigned)r), dim3(256), 0, s, a, Wp, wv);
  hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)((c + 255) / 256)), dim3(256), 0, s, a.perm, c,
                     a.groupsize, a.g_idx);
  BlockArgs b;
  b.Wp = Wp;
  b.U = a.U;
  b.r = r;
  b.c = c;
  b.bits = a.bits;
  b.sym = a.sym;
  b.groupsize = a.groupsize;
  b.perm = a.perm;
  b.codes = a.codes;
  b.scales = a.scales;
  b.zeros = a.zeros;
  b.W_hat = a.W_hat;
  b.row_loss = a.row_loss;
  b.n_groups = a.groupsize > 0 ? (c + a.groupsize - 1) / a.groupsize : 1;
  b.vec_u = ((c & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.U) & 15) == 0);
  const int64_t B = a.blocksize;
  const int64_t SB = super_block(B, a.groupsize);
  b.lde = SB;
  // 16 lanes per row when there are enough rows to fill the chip that way.
  const bool wide = r * 16 >= 256 * 64;
  // groups shorter than the block: width a multiple of 32 (32), any (-1)
  const int midg = !(a.groupsize > 0 && a.groupsize < B) ? 0 : (a.groupsize % 32 == 0) ? 32 : -1;
  const dim3 g16((unsigned)((r + 15) / 16)), g4((unsigned)((r + 63) / 64));
  // Whole super-blocks of four full blocks, with 16 lanes per row and rulers
  // per row or per block, run as one launch each.
  // Groups of 32 or 64 lie inside a block, so their rulers are fitted from
  // the registers of the block at hand (MIDG == 32).
  const bool sb_ok = wide && B == BMAX && SB == SB_BLOCKS * BMAX && b.vec_u &&
                     (a.groupsize <= 0 || a.groupsize == BMAX || a.groupsize == 32 || a.groupsize == 64);
  for (int64_t s1 = 0; s1 < c; s1 += SB) {
    const int64_t s2 = std::min(s1 + SB, c);
    if (sb_ok && s2 - s1 == SB) {
      b.i1 = s1;
      b.Bw = BMAX;
      b.E = E;
      if (midg == 32) hipLaunchKernelGGL((superblock_kernel<32>), g16, dim3(256), 0, s, b, s1);
      else hipLaunchKernelGGL((superblock_kernel<0>), g16, dim3(256), 0, s, b, s1);
      if (s2 < c) gemm_update(s, r, c, E, SB, (int)(s2 - s1), a.U, s1, s2, c, Wp);
      continue;
    }
    for (int64_t i1 = s1; i1 < s2; i1 += B) {
      const int Bw = (int)std::min<int64_t>(B, s2 - i1);
      const int64_t i2 = i1 + Bw;
      b.i1 = i1;
      b.Bw = Bw;
      b.E = E + (i1 - s1);
      const bool full = Bw == BMAX;
#define GPTQ_BLOCK(LL, MID, FU, G) hipLaunchKernelGGL((block_kernel<LL, MID, FU>), G, dim3(256), 0, s, b)
#define GPTQ_BLOCK_F(LL, MID, G) \
  do { if (full) GPTQ_BLOCK(LL, MID, true, G); else GPTQ_BLOCK(LL, MID, false, G); } while (0)
      // Widths that are multiples of 32 have their own variant in the
      // 16-lane kernel (layers of 1024 rows and more); otherwise any width.
      if (wide) {
        if (midg == 0) GPTQ_BLOCK_F(16, 0, g16);
        else if (midg == 32) GPTQ_BLOCK_F(16, 32, g16);
        else GPTQ_BLOCK_F(16, -1, g16);
      } else {
        if (midg == 0) GPTQ_BLOCK_F(4, 0, g4);
        else GPTQ_BLOCK_F(4, -1, g4);
      }
#undef GPTQ_BLOCK_F
#undef GPTQ_BLOCK
      // repairs of this block's errors to the rest of the super-block, at once
      if (i2 < s2) gemm_update(s, r, c, b.E, SB, Bw, a.U, i1, i2, s2, Wp);
    }
    // repairs of the whole super-block to every later column, deferred to here
    if (s2 < c) gemm_update(s, r, c, E, SB, (int)(s2 - s1), a.U, s1, s2, c, Wp);
  }
}

}  // namespace gptq
