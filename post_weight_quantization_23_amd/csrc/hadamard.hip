// Hadamard pre-rotation of rows: out[i, :] = A[i, :] * blockdiag(H_b / sqrt(b)).
// The page "Post-Training Quantization: Calibration, GPTQ and Why Rotations
// Help", sections "Rotations: making outliers disappear" and "Why do Hadamard
// rotations help quantization?": a Hadamard matrix scaled to a rotation
// spreads a lone large activation over all entries, and rotating a layer's
// inputs while applying the inverse rotation to its weights leaves the
// product unchanged.  H_b is Sylvester's (symmetric, so the rotation is its
// own inverse); b is a power of two dividing the row length.
//
// Design (HBM-bound: one read and one write of every element):
//   * One workgroup of 256 threads transforms a tile of 256 E elements
//     (E = 16, or 32 for b = 8192): 4096 / b whole blocks, or one block.
//     Thread t owns tile elements t + 256 k, so every load and store of a
//     wave touches consecutive elements, whatever the block size.
//   * The butterflies over index bits 8 and up (in-block) run on the thread's
//     own registers straight after the loads; the bits below 8 go through
//     LDS in passes of four bits (radix-16 in registers per pass), with one
//     padding word per 16 so the strided passes are free of bank conflicts.
//   * fp32 arithmetic; the result is scaled by b^-1/2 and rounded once (RNE)
//     to the output type.
//   * Rows whose starts are 16-byte aligned take the vector path below (each
//     thread moves runs of 8 consecutive elements with 16-byte accesses);
//     the element-wise path above serves any other layout.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

GPTQ_DEV float load_elem(const void* base, int64_t off, int dt) {
  if (dt == 0) return static_cast<const float*>(base)[off];
  const uint16_t b = static_cast<const uint16_t*>(base)[off];
  if (dt == 1) return __uint_as_float((uint32_t)b << 16);
  return (float)__builtin_bit_cast(_Float16, b);
}

// fp32 -> bf16 with round-to-nearest-even (NaN kept quiet).
GPTQ_DEV uint16_t to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

GPTQ_DEV void store_elem(void* base, int64_t off, int dt, float v) {
  if (dt == 0) static_cast<float*>(base)[off] = v;
  else if (dt == 1) static_cast<uint16_t*>(base)[off] = to_bf16(v);
  else static_cast<uint16_t*>(base)[off] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

GPTQ_DEV int lds_pos(int i) { return i + (i >> 4); }

struct FwhtArgs {
  const void* A;
  int64_t lda;
  void* out;
  int64_t ldo;
  int64_t nblocks;   // rows * (d / b)
  int64_t bpr;       // blocks per row
  int at, ot;        // 0 f32, 1 bf16, 2 f16
  float scale;       // b^-1/2
};

template <int LOGB, int E>
__global__ __launch_bounds__(256) void fwht_kernel(FwhtArgs a) {
  constexpr int B = 1 << LOGB;
  constexpr int N = 256 * E;
  constexpr int TB = N / B;           // blocks per tile
  static_assert(N >= B, "a tile holds whole blocks");
  __shared__ float lds[N + N / 16];
  const int t = threadIdx.x;
  const int64_t blk0 = (int64_t)blockIdx.x * TB;

  // ---- loads: element t + 256 k of the tile; its block and in-block index
  float v[E];
  int64_t in_off[E], out_off[E];
  bool ok[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int i = t + 256 * k;
    const int64_t gb = blk0 + (i >> LOGB);
    ok[k] = gb < a.nblocks;
    // block -> (row, block of the row); block counts fit 31 bits (host check)
    const uint32_t g32 = ok[k] ? (uint32_t)gb : 0u;
    const uint32_t row = a.bpr == 1 ? g32 : g32 / (uint32_t)a.bpr;
    const int64_t col = (int64_t)(g32 - row * (uint32_t)a.bpr) * B + (i & (B - 1));
    in_off[k] = (int64_t)row * a.lda + col;
    out_off[k] = (int64_t)row * a.ldo + col;
  }
#pragma unroll
  for (int k = 0; k < E; ++k) v[k] = ok[k] ? load_elem(a.A, in_off[k], a.at) : 0.f;

  // ---- in-block bits 8 .. LOGB-1 live in k: butterflies in registers
  if constexpr (LOGB > 8) {
#pragma unroll
    for (int h = 0; h < LOGB - 8; ++h) {
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (!(k & (1 << h))) {
          const float x = v[k], y = v[k | (1 << h)];
          v[k] = x + y;
          v[k | (1 << h)] = x - y;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < E; ++k) lds[lds_pos(t + 256 * k)] = v[k];
  __syncthreads();

  // ---- bits 0 .. min(LOGB, 8)-1 through LDS, four bits per pass
  constexpr int LOW = LOGB < 8 ? LOGB : 8;
#pragma unroll
  for (int s = 0; s < LOW; s += 4) {
    const int q = (LOW - s) < 4 ? (LOW - s) : 4;
    const int nk = 1 << q;
    const int groups_per_thread = N / nk / 256;
    for (int u = 0; u < groups_per_thread; ++u) {
      const int g = t + 256 * u;
      const int low = g & ((1 << s) - 1), high = g >> s;
      const int base = low + (high << (s + q));
      float w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < nk) w[k] = lds[lds_pos(base + (k << s))];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < q) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            if (k < nk && !(k & (1 << h))) {
              const float x = w[k], y = w[k | (1 << h)];
              w[k] = x + y;
              w[k | (1 << h)] = x - y;
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < nk) lds[lds_pos(base + (k << s))] = w[k];
    }
    __syncthreads();
  }

  // ---- scale, round once, store
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const float r = lds[lds_pos(t + 256 * k)] * a.scale;
    if (ok[k]) store_elem(a.out, out_off[k], a.ot, r);
  }
}

// ---- vector path (16-byte aligned rows): thread t owns runs of 8
// consecutive elements, tile element i = (e & 7) + 8 t + 2048 (e >> 3) for its
// register e.  Index bits 0..2 and 11.. are in registers; bits 3..10 go
// through LDS in passes of up to four bits.  LDS padding: 4 words per 64 (keeps
// 16-byte runs aligned and staggers the strided passes across banks).
GPTQ_DEV int vpos(int i) { return i + ((i >> 6) << 2); }

GPTQ_DEV void load8(const void* base, int64_t off, int dt, float (&x)[8]) {
  if (dt == 0) {
    const floatx4* p = reinterpret_cast<const floatx4*>(static_cast<const float*>(base) + off);
    const floatx4 a = p[0], b = p[1];
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3]; x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    return;
  }
  const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = w[j];
    if (dt == 1) {
      x[2 * j] = __uint_as_float(u << 16);
      x[2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
    } else {
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
  }
}

GPTQ_DEV void store8(void* base, int64_t off, int dt, const float (&x)[8]) {
  if (dt == 0) {
    floatx4* p = reinterpret_cast<floatx4*>(static_cast<float*>(base) + off);
    p[0] = floatx4{x[0], x[1], x[2], x[3]};
    p[1] = floatx4{x[4], x[5], x[6], x[7]};
    return;
  }
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t lo, hi;
    if (dt == 1) {
      lo = to_bf16(x[2 * j]);
      hi = to_bf16(x[2 * j + 1]);
    } else {
      lo = __builtin_bit_cast(uint16_t, (_Float16)x[2 * j]);
      hi = __builtin_bit_cast(uint16_t, (_Float16)x[2 * j + 1]);
    }
    w[j] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off) = w;
}

template <int LOGB, int E>
__global__ __launch_bounds__(256) void fwht_vec_kernel(FwhtArgs a) {
  constexpr int B = 1 << LOGB;
  constexpr int N = 256 * E;
  constexpr int TB = N / B;
  constexpr int R = E / 8;            // runs of 8 per thread
  static_assert(N >= B && B >= 32, "a tile holds whole blocks of at least 32");
  __shared__ __align__(16) float lds[N + N / 16];
  const int t = threadIdx.x;
  const int64_t blk0 = (int64_t)blockIdx.x * TB;

  float v[R][8];
  int64_t in_off[R], out_off[R];
  bool ok[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int i = 8 * t + 2048 * u;
    const int64_t gb = blk0 + (i >> LOGB);
    ok[u] = gb < a.nblocks;
    const uint32_t g32 = ok[u] ? (uint32_t)gb : 0u;
    const uint32_t row = a.bpr == 1 ? g32 : g32 / (uint32_t)a.bpr;
    const int64_t col = (int64_t)(g32 - row * (uint32_t)a.bpr) * B + (i & (B - 1));
    in_off[u] = (int64_t)row * a.lda + col;
    out_off[u] = (int64_t)row * a.ldo + col;
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (ok[u]) {
      load8(a.A, in_off[u], a.at, v[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u][j] = 0.f;
    }
  }
  // bits 0..2 (within a run)
#pragma unroll
  for (int h = 0; h < 3; ++h) {
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!(j & (1 << h))) {
          const float x = v[u][j], y = v[u][j | (1 << h)];
          v[u][j] = x + y;
          v[u][j | (1 << h)] = x - y;
        }
  }
  // bits 11.. (across runs), in-block only
  if constexpr (LOGB > 11) {
#pragma unroll
    for (int h = 0; h < LOGB - 11; ++h) {
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (!(u & (1 << h))) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = v[u][j], y = v[u | (1 << h)][j];
            v[u][j] = x + y;
            v[u | (1 << h)][j] = x - y;
          }
        }
    }
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    floatx4* p = reinterpret_cast<floatx4*>(&lds[vpos(8 * t + 2048 * u)]);
    p[0] = floatx4{v[u][0], v[u][1], v[u][2], v[u][3]};
    p[1] = floatx4{v[u][4], v[u][5], v[u][6], v[u][7]};
  }
  __syncthreads();

  // bits 3 .. min(LOGB, 11)-1 through LDS
  constexpr int HI = LOGB < 11 ? LOGB : 11;
#pragma unroll
  for (int s = 3; s < HI; s += 4) {
    const int q = (HI - s) < 4 ? (HI - s) : 4;
    const int nk = 1 << q;
    const int groups_per_thread = N / nk / 256;
    for (int u = 0; u < groups_per_thread; ++u) {
      const int g = t + 256 * u;
      const int low = g & ((1 << s) - 1), high = g >> s;
      const int base = low + (high << (s + q));
      float w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < nk) w[k] = lds[vpos(base + (k << s))];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < q) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            if (k < nk && !(k & (1 << h))) {
              const float x = w[k], y = w[k | (1 << h)];
              w[k] = x + y;
              w[k | (1 << h)] = x - y;
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < nk) lds[vpos(base + (k << s))] = w[k];
    }
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < R; ++u) {
    const floatx4* p = reinterpret_cast<const floatx4*>(&lds[vpos(8 * t + 2048 * u)]);
    const floatx4 lo = p[0], hi = p[1];
    float r[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] *= a.scale;
    if (ok[u]) store8(a.out, out_off[u], a.ot, r);
  }
}

}  // namespace

void launch_hadamard(const void* A, int at, int64_t lda, int64_t rows, int64_t d, int64_t block, void* out,
                     int ot, int64_t ldo, hipStream_t s) {
  int logb = 0;
  while ((1LL << logb) < block) ++logb;
  FwhtArgs a;
  a.A = A;
  a.lda = lda;
  a.out = out;
  a.ldo = ldo;
  a.bpr = d / block;
  a.nblocks = rows * a.bpr;
  a.at = at;
  a.ot = ot;
  a.scale = (float)(1.0 / __builtin_sqrt((double)block));
  const int E = logb == 13 ? 32 : 16;
  const int64_t tb = (256LL * E) / block;
  const unsigned grid = (unsigned)((a.nblocks + tb - 1) / tb);
  // 16-byte runs when every row start is 16-byte aligned in both buffers
  const size_t ea = at == 0 ? 4 : 2, eo = ot == 0 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0) &&
                   ((lda * (int64_t)ea) % 16 == 0) && ((ldo * (int64_t)eo) % 16 == 0);
  switch (logb) {
#define GPTQ_FWHT_CASE(L)                                                                             \
  case L:                                                                                             \
    if (vec) hipLaunchKernelGGL((fwht_vec_kernel<L, (L == 13 ? 32 : 16)>), dim3(grid), dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((fwht_kernel<L, (L == 13 ? 32 : 16)>), dim3(grid), dim3(256), 0, s, a);         \
    break;
    GPTQ_FWHT_CASE(5)
    GPTQ_FWHT_CASE(6)
    GPTQ_FWHT_CASE(7)
    GPTQ_FWHT_CASE(8)
    GPTQ_FWHT_CASE(9)
    GPTQ_FWHT_CASE(10)
    GPTQ_FWHT_CASE(11)
    GPTQ_FWHT_CASE(12)
    GPTQ_FWHT_CASE(13)
#undef GPTQ_FWHT_CASE
    default:
      break;
  }
}

}  // namespace gptq
