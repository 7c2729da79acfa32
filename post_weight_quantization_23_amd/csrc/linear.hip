// Forward pass of a quantized linear layer over the calibration tokens:
//     Y[t, i] = act( sum_k X[t, k] * round16(W_hat[i, k]) )
// The page "What is GPTQ" (queryfeedz glossary), section "How it works":
// layers are processed one at a time and the next layer is calibrated on the
// quantized outputs of the previous one.  This kernel produces those outputs:
// the dequantized weights W_hat (fp32, as the quantizer writes them) are
// rounded once to the activations' 16-bit type (the model's own precision),
// products are exact in fp32 and sums are fp32 (MFMA), and the result is
// rounded once to the output type.  A gated epilogue fuses the MLP's
// silu(gate) * up: the up projection's sum is rounded to the 16-bit type, then
// multiplied by silu of the gate output (read from memory) in fp32 and
// rounded once more.
//
// Layout and tiling: X token-major [n_tok, d] and W_hat [r, d] are both
// contiguous along the contraction axis, so no transpose is needed: a
// workgroup of 4 waves computes a 256 x 256 tile (each wave 128 x 128 as
// 4 x 4 v_mfma_f32_32x32x16 blocks, accumulators in AGPRs) over K-steps of
// 64, with each 16-byte run of 8 K-values written to an LDS row of 128 bytes
// whose chunks are XOR-swizzled by the row (conflict-free MFMA operand reads).
// W_hat is read as fp32 and rounded on its way into LDS.  Two LDS buffers:
// the loads of step s+2 are in flight while step s computes, and the first
// MFMA operands of a step are read before the next step is staged.  Consecutive
// workgroups share the same X rows (the larger operand), which the caches
// then serve to all the column tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int LT = 256;      // tile edge
constexpr int LK = 64;       // K-step
constexpr int LROWB = LK * 2;

GPTQ_DEV int lswz(int f) { return (f ^ (f >> 3)) & 7; }

template <int DT>
GPTQ_DEV floatx16 lmfma(u32x4 a, u32x4 b, floatx16 c) {
  if constexpr (DT == 1) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
GPTQ_DEV uint32_t bf16_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int DT>
GPTQ_DEV uint32_t to16(float v) {
  if constexpr (DT == 1) return bf16_bits(v);
  else return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

template <int DT>
GPTQ_DEV float from16(uint16_t b) {
  if constexpr (DT == 1) return __uint_as_float((uint32_t)b << 16);
  else return (float)__builtin_bit_cast(_Float16, b);
}

struct LinArgs {
  const uint16_t* X;
  int64_t ldx;
  const float* W;
  int64_t ldw;
  const uint16_t* G;   // gate output (gated mode)
  int64_t ldg;
  void* Y;
  int64_t ldy;
  int64_t M;           // tokens
  int N;               // output features
  int K;               // input features (multiple of 64)
  int yt;              // 0 f32, 1 bf16, 2 f16
  int act;             // 0 none, 1 silu(G) * round16(acc)
  int ntn;             // column tiles
};

template <int DT, int ACT, int YT>
GPTQ_DEV void store_out(const LinArgs& a, int64_t gm, int gn, float y, float g) {
  if constexpr (ACT == 1) {
    const float u = from16<DT>((uint16_t)to16<DT>(y));
    // silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (a few
    // ulp of fp32, far below the 16-bit rounding that follows)
    y = __fdividef(g, 1.0f + __expf(-g)) * u;
  }
  if constexpr (YT == 0) static_cast<float*>(a.Y)[gm * a.ldy + gn] = y;
  else if constexpr (YT == 1) static_cast<uint16_t*>(a.Y)[gm * a.ldy + gn] = (uint16_t)bf16_bits(y);
  else static_cast<uint16_t*>(a.Y)[gm * a.ldy + gn] = __builtin_bit_cast(uint16_t, (_Float16)y);
}

// Template arguments: activation type (1 bf16, 2 f16), epilogue (0 plain,
// 1 gated), output type (0 f32, 1 bf16, 2 f16).
template <int DT, int ACT, int YT>
__global__ __launch_bounds__(256, 1) void linear_kernel(LinArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lsm[];
  auto a_buf = [&](int b) { return lsm + b * (LT * LROWB); };
  auto b_buf = [&](int b) { return lsm + (2 + b) * (LT * LROWB); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)(blockIdx.x / a.ntn) * LT;
  const int n0 = (int)(blockIdx.x % a.ntn) * LT;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;

  // loader role: 8 chunks of 8 K-values per operand; chunk c = tid + 256 i
  // covers row c / 8, K-offset 8 (c % 8) of the step
  u32x4 ra[8];
  floatx4 rb[16];
  auto fetch = [&](int st) {
    const int k0 = st * LK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      const int64_t gm = m0 + row;
      ra[i] = gm < a.M ? *reinterpret_cast<const u32x4*>(a.X + gm * a.ldx + k0 + 8 * kc) : u32x4{0u, 0u, 0u, 0u};
      const int gn = n0 + row;
      if (gn < a.N) {
        const floatx4* p = reinterpret_cast<const floatx4*>(a.W + (int64_t)gn * a.ldw + k0 + 8 * kc);
        rb[2 * i] = p[0];
        rb[2 * i + 1] = p[1];
      } else {
        rb[2 * i] = floatx4{0.f, 0.f, 0.f, 0.f};
        rb[2 * i + 1] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(a_buf(buf) + row * LROWB + ((kc ^ lswz(row)) * 16)) = ra[i];
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        w[2 * u] = to16<DT>(rb[2 * i + u][0]) | (to16<DT>(rb[2 * i + u][1]) << 16);
        w[2 * u + 1] = to16<DT>(rb[2 * i + u][2]) | (to16<DT>(rb[2 * i + u][3]) << 16);
      }
      *reinterpret_cast<u32x4*>(b_buf(buf) + row * LROWB + ((kc ^ lswz(row)) * 16)) = w;
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nsteps = a.K / LK;
  fetch(0);
  stage(0);
  if (nsteps > 1) fetch(1);
  __syncthreads();
  u32x4 fa[2][4], fb[2][4];
  auto frags = [&](const unsigned char* as, const unsigned char* bs, int kk, u32x4 (&xa)[4], u32x4 (&xb)[4]) {
    const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = wm + 32 * i + (lane & 31);
      xa[i] = *reinterpret_cast<const u32x4*>(as + f * LROWB + ((chunk ^ lswz(f)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = wn + 32 * j + (lane & 31);
      xb[j] = *reinterpret_cast<const u32x4*>(bs + f * LROWB + ((chunk ^ lswz(f)) * 16));
    }
  };
  auto mfmas = [&](const u32x4 (&xa)[4], const u32x4 (&xb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = lmfma<DT>(xa[i], xb[j], acc[i][j]);
  };
  // Step st computes from LDS buffer st & 1.  The first two sub-steps'
  // operands are read before the next step's words are written to the other
  // buffer and the loads of step st+2 issued, so the MFMAs start at once;
  // the later operands are read while earlier MFMAs run.
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const unsigned char* as = a_buf(buf);
    const unsigned char* bs = b_buf(buf);
    frags(as, bs, 0, fa[0], fb[0]);
    frags(as, bs, 1, fa[1], fb[1]);
    if (st + 1 < nsteps) stage(buf ^ 1);
    if (st + 2 < nsteps) fetch(st + 2);
    mfmas(fa[0], fb[0]);
    frags(as, bs, 2, fa[0], fb[0]);
    mfmas(fa[1], fb[1]);
    frags(as, bs, 3, fa[1], fb[1]);
    mfmas(fa[0], fb[0]);
    mfmas(fa[1], fb[1]);
    __syncthreads();
  }

  // Epilogue through LDS, one 32-row strip of each wave's 128 x 128 block at a
  // time (16 KiB per wave): the accumulators are written with static indices
  // (lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32 x 32
  // block), then read back row-major so that consecutive lanes store
  // consecutive columns.
  float* ep = reinterpret_cast<float*>(lsm) + wave * (32 * 128);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ep[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * 128 + 32 * j + (lane & 31)] = acc[i][j][v];
    __syncthreads();
    // 32 outputs per lane at a time; their gate values are all requested
    // before any is used
#pragma unroll 1
    for (int c = 0; c < 2; ++c) {
      float gv[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int idx = (32 * c + e) * 64 + lane, row = idx >> 7, col = idx & 127;
        const int64_t gm = m0 + wm + 32 * i + row;
        const int gn = n0 + wn + col;
        gv[e] = (ACT == 1 && gm < a.M && gn < a.N) ? from16<DT>(a.G[gm * a.ldg + gn]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int idx = (32 * c + e) * 64 + lane, row = idx >> 7, col = idx & 127;
        const int64_t gm = m0 + wm + 32 * i + row;
        const int gn = n0 + wn + col;
        if (gm < a.M && gn < a.N) store_out<DT, ACT, YT>(a, gm, gn, ep[idx], gv[e]);
      }
    }
  }
}

}  // namespace

void launch_linear(const void* X, int xt, int64_t n_tok, int64_t d, int64_t ldx, const float* W, int64_t r,
                   int64_t ldw, int act, const void* G, int64_t ldg, void* Y, int yt, int64_t ldy, hipStream_t s) {
  LinArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.ldx = ldx;
  a.W = W;
  a.ldw = ldw;
  a.G = static_cast<const uint16_t*>(G);
  a.ldg = ldg;
  a.Y = Y;
  a.ldy = ldy;
  a.M = n_tok;
  a.N = (int)r;
  a.K = (int)d;
  a.yt = yt;
  a.act = act;
  a.ntn = (int)((r + LT - 1) / LT);
  const int64_t ntm = (n_tok + LT - 1) / LT;
  const size_t lds = 4 * LT * LROWB;
  const dim3 grid((unsigned)(ntm * a.ntn));
  // 128 KiB of dynamic LDS: A and B, double buffered
#define GPTQ_LIN(D_, A_, Y_)                                                                          \
  do {                                                                                                \
    static bool set = false;                                                                          \
    if (!set) {                                                                                       \
      (void)hipFuncSetAttribute((const void*)linear_kernel<D_, A_, Y_>,                               \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                \
      set = true;                                                                                     \
    }                                                                                                 \
    hipLaunchKernelGGL((linear_kernel<D_, A_, Y_>), grid, dim3(256), lds, s, a);                     \
  } while (0)
#define GPTQ_LIN_Y(D_, A_)               \
  do {                                   \
    if (yt == 0) GPTQ_LIN(D_, A_, 0);    \
    else if (yt == 1) GPTQ_LIN(D_, A_, 1); \
    else GPTQ_LIN(D_, A_, 2);            \
  } while (0)
  if (xt == 1) {
    if (act == 1) GPTQ_LIN_Y(1, 1); else GPTQ_LIN_Y(1, 0);
  } else {
    if (act == 1) GPTQ_LIN_Y(2, 1); else GPTQ_LIN_Y(2, 0);
  }
#undef GPTQ_LIN_Y
#undef GPTQ_LIN
}

}  // namespace gptq
