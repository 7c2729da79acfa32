// Forward pass of a quantized linear layer over the calibration tokens:
//     Y[t, i] = act( sum_k X[t, k] * round16(W_hat[i, k]) )
// The page "What is GPTQ" (queryfeedz glossary), section "How it works":
// layers are processed in sequence, each calibrated on what the already-
// quantized layers before it produce.  This kernel produces those inputs:
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
// workgroup computes a 256 x 256 tile (8 waves of 128 x 64 as 4 x 2
// v_mfma_f32_32x32x16 blocks when the weights are already 16-bit, else 4
// waves of 128 x 128 as 4 x 4 blocks, accumulators in AGPRs) over K-steps of
// 64, with each 16-byte run of 8 K-values written to an LDS row of 128 bytes
// whose chunks are XOR-swizzled by the row (conflict-free MFMA operand reads).
// Two ways in for W_hat.  Given as fp32 (the quantizer's output), it is read
// into registers, rounded, and written to LDS next to the X tile, with the
// loads two K-steps ahead.  Given already rounded to the 16-bit type (one
// pass of round16_kernel), both operands go from memory straight into LDS with
// buffer loads that write LDS (each lane fetches the 16-byte chunk that
// belongs at its LDS position, so the swizzle costs nothing), one K-step
// ahead, and no registers or ALU work sit between memory and the MFMA
// operands.  Both paths feed the MFMAs the same values in the same order.
//
// Tile order: work items are numbered in panels of 4 token tiles, walking the
// 4 token tiles of a panel for each output-column tile in turn.  The
// dispatcher deals workgroups round-robin to the eight XCDs, so within every
// 256 workgroups XCD x takes the 32 consecutive items 32x .. 32x+31: about 4
// token tiles x 8 column tiles, whose X and W slabs its L2 shares; all XCDs
// work on the same few token tiles, and W streams once per panel.
#include <type_traits>

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
  const float* W;      // fp32 weights (W16 == nullptr)
  const uint16_t* W16; // weights already rounded to the 16-bit type
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
  int ntm;             // token tiles
  int yvec;            // Y rows start on 16 (fp32) / 8 (16-bit) bytes: vector stores
  int gvec;            // G rows start on 8 bytes: vector loads
  int ntn;             // column tiles
};

// The output value before its final rounding: the sum itself, or
// silu(g) * round16(sum) in the gated mode.
template <int DT, int ACT>
GPTQ_DEV float out_value(float y, float g) {
  if constexpr (ACT == 1) {
    const float u = from16<DT>((uint16_t)to16<DT>(y));
    // silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (a few
    // ulp of fp32, far below the 16-bit rounding that follows)
    return __fdividef(g, 1.0f + __expf(-g)) * u;
  } else {
    return y;
  }
}

template <int YT>
GPTQ_DEV void store1(const LinArgs& a, int64_t gm, int gn, float y) {
  if constexpr (YT == 0) static_cast<float*>(a.Y)[gm * a.ldy + gn] = y;
  else if constexpr (YT == 1) static_cast<uint16_t*>(a.Y)[gm * a.ldy + gn] = (uint16_t)bf16_bits(y);
  else static_cast<uint16_t*>(a.Y)[gm * a.ldy + gn] = __builtin_bit_cast(uint16_t, (_Float16)y);
}

// Four consecutive outputs of row gm from column gn (all inside the output).
template <int YT>
GPTQ_DEV void store4(const LinArgs& a, int64_t gm, int gn, const float (&y)[4]) {
  if (a.yvec) {
    if constexpr (YT == 0) {
      *reinterpret_cast<floatx4*>(static_cast<float*>(a.Y) + gm * a.ldy + gn) = floatx4{y[0], y[1], y[2], y[3]};
    } else {
      uint2 o;
      o.x = to16<YT>(y[0]) | (to16<YT>(y[1]) << 16);
      o.y = to16<YT>(y[2]) | (to16<YT>(y[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.Y) + gm * a.ldy + gn) = o;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) store1<YT>(a, gm, gn + e, y[e]);
  }
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Work item of workgroup b: see the tile order in the header.
GPTQ_DEV void lin_tile(int b, int ntm, int ntn, int64_t& tm, int& tn) {
  int w = b;
  if (w < ((ntm * ntn) & ~255)) w = (w & ~255) | ((w & 7) << 5) | ((w & 255) >> 3);
  const int p = w / (4 * ntn);
  const int h = min(4, ntm - 4 * p);
  const int j = w - p * 4 * ntn;
  tn = j / h;
  tm = 4 * p + j % h;
}

// K-loop with both operands 16-bit: K-step st's rows (256 of X, 256 of W, 64
// K-values = 128 bytes each) are carried into LDS buffer st & 1 by buffer
// loads that write LDS, issued before step st-1's MFMAs; one wait and one
// barrier per step.  An instruction of a wave moves 8 rows (64 lanes x 16
// bytes, lane l to LDS base + 16 l); lane l fetches chunk (l & 7) ^ lswz(row)
// of its row, so chunk c of row f lands at position c ^ lswz(f), where the
// operand reads expect it.  Rows past the end of X or W fall outside the
// descriptors' records and load zeros.
// NQ: load instructions per wave and operand (8 rows each; 32 per operand
// and step over the workgroup's waves); NB: 32-column MFMA blocks per wave.
template <int DT, int NQ, int NB>
GPTQ_DEV void lin_steps_dma(const LinArgs& a, int64_t m0, int n0, int wm, int wn, unsigned char* smem,
                            floatx16 (&acc)[4][NB]) {
  constexpr int SLAB = LT * LROWB, BUF = 2 * SLAB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  lds_u8* lbase = (lds_u8*)smem;  // generic to LDS address space
  const int nsteps = a.K / LK;
  // byte offsets of the lane's chunks inside a K-step (ldx, ldw < 2^22)
  static_assert(NQ <= 8, "at most 8 load instructions per wave");
  int offx[8], offw[8];   // the first NQ are used
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int row = 8 * (wave * NQ + q) + (lane >> 3), c = (lane & 7) ^ lswz(row);
    offx[q] = row * (int)a.ldx * 2 + 16 * c;
    offw[q] = row * (int)a.ldw * 2 + 16 * c;
  }
  const int64_t xrec = min(a.M - m0, (int64_t)LT) * a.ldx * 2;
  const int64_t wrec = (int64_t)min(a.N - n0, LT) * a.ldw * 2;
  auto dma = [&](int st, int b) {
    const int k0 = st * LK;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.X + m0 * a.ldx + k0), (short)0, (int)(xrec - 2 * k0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W16 + (int64_t)n0 * a.ldw + k0), (short)0, (int)(wrec - 2 * k0), 0x00020000);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int I = wave * NQ + q;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lbase + b * BUF + I * 1024, 16, offx[q], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lbase + b * BUF + SLAB + I * 1024, 16, offw[q], 0, 0, 0);
    }
  };
  u32x4 fa[2][4], fb[2][NB];
  auto frags = [&](const unsigned char* as, const unsigned char* bs, int kk, u32x4 (&xa)[4], u32x4 (&xb)[NB]) {
    const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = wm + 32 * i + (lane & 31);
      xa[i] = *reinterpret_cast<const u32x4*>(as + f * LROWB + ((chunk ^ lswz(f)) * 16));
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int f = wn + 32 * j + (lane & 31);
      xb[j] = *reinterpret_cast<const u32x4*>(bs + f * LROWB + ((chunk ^ lswz(f)) * 16));
    }
  };
  auto mfmas = [&](const u32x4 (&xa)[4], const u32x4 (&xb)[NB]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = lmfma<DT>(xa[i], xb[j], acc[i][j]);
  };
  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int b = st & 1;
    if (st + 1 < nsteps) dma(st + 1, b ^ 1);
    const unsigned char* as = smem + b * BUF;
    const unsigned char* bs = as + SLAB;
#pragma unroll
    for (int kk = 0; kk < LK / 16; kk += 2) {
      frags(as, bs, kk, fa[0], fb[0]);
      frags(as, bs, kk + 1, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      mfmas(fa[1], fb[1]);
    }
    // step st+1 has landed (own loads) in every wave (barrier); buffer b is
    // free for step st+2
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// K-loop with fp32 weights: each thread loads 8 chunks of 8 K-values of each
// operand into registers, the weights are rounded to the 16-bit type, and the
// chunks are written to the swizzled LDS rows; the loads of step s+2 are in
// flight while step s computes.
template <int DT>
GPTQ_DEV void lin_steps_f32(const LinArgs& a, int64_t m0, int n0, int wm, int wn, unsigned char* lsm,
                            floatx16 (&acc)[4][4]) {
  auto a_buf = [&](int b) { return lsm + b * (LT * LROWB); };
  auto b_buf = [&](int b) { return lsm + (2 + b) * (LT * LROWB); };
  const int tid = threadIdx.x, lane = tid & 63;
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
}

// Template arguments: activation type (1 bf16, 2 f16), epilogue (0 plain,
// 1 gated), output type (0 f32, 1 bf16, 2 f16), weights already 16-bit.
// With 16-bit weights the workgroup is 8 waves of 128 x 64 (two per SIMD, so
// one wave's operand reads overlap the other's MFMAs); with fp32 weights 4
// waves of 128 x 128 (the register staging needs the registers).
template <int DT, int ACT, int YT, bool W16>
__global__ __launch_bounds__(W16 ? 512 : 256, 1) void linear_kernel(LinArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lsm[];
  constexpr int NW = W16 ? 8 : 4;        // waves
  constexpr int NB = W16 ? 2 : 4;        // 32-column MFMA blocks per wave
  constexpr int WN = 32 * NB;            // columns per wave
  constexpr int LPR = 8 * NB;            // epilogue lanes per row (4 columns each)
  constexpr int RPP = 64 / LPR;          // epilogue rows per pass
  constexpr int PASSES = 32 / RPP;       // passes per 32-row strip

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t tm;
  int tn;
  lin_tile((int)blockIdx.x, a.ntm, a.ntn, tm, tn);
  const int64_t m0 = tm * LT;
  const int n0 = tn * LT;
  const int wm = (wave / (NW / 2)) * 128, wn = (wave % (NW / 2)) * WN;

  floatx16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if constexpr (W16) lin_steps_dma<DT, 32 / NW, NB>(a, m0, n0, wm, wn, lsm, acc);
  else lin_steps_f32<DT>(a, m0, n0, wm, wn, lsm, acc);

  // Epilogue through LDS, one 32-row strip of each wave's 128 x WN block at a
  // time (32 x WN floats per wave): the accumulators are written with static
  // indices (lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each
  // 32 x 32 block), then read back four consecutive columns at a time: lane l
  // takes columns 4 (l % LPR) .. +3 of rows RPP k + l / LPR, so each row is
  // written by LPR lanes in one contiguous run.  In the gated mode the gate
  // values of strip i+1 (eight-byte loads) are requested before strip i is
  // processed, and those of strip 0 before the first barrier.
  float* ep = reinterpret_cast<float*>(lsm) + wave * (32 * WN);
  const int cq = lane % LPR, rh = lane / LPR;
  const int gn = n0 + wn + 4 * cq;
  const bool full4 = gn + 4 <= a.N;
  uint2 gq[2][PASSES];
  auto load_gate = [&](int i, uint2 (&g)[PASSES]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int64_t gm = m0 + wm + 32 * i + RPP * k + rh;
      const uint16_t* gp = a.G + gm * a.ldg + gn;
      if (gm < a.M && full4 && a.gvec) {
        g[k] = *reinterpret_cast<const uint2*>(gp);
      } else {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (gm < a.M && gn + e < a.N) ? (uint32_t)gp[e] : 0u;
        g[k].x = h[0] | (h[1] << 16);
        g[k].y = h[2] | (h[3] << 16);
      }
    }
  };
  // one strip; the strip index is a compile-time constant so that the
  // accumulators stay in registers
  auto strip = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    if constexpr (ACT == 1 && i + 1 < 4) load_gate(i + 1, gq[(i + 1) & 1]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ep[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * WN + 32 * j + (lane & 31)] = acc[i][j][v];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int r = RPP * k + rh;
      const int64_t gm = m0 + wm + 32 * i + r;
      const floatx4 v = *reinterpret_cast<const floatx4*>(ep + r * WN + 4 * cq);
      float g[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (ACT == 1) {
        const uint2 w = gq[i & 1][k];
        g[0] = from16<DT>((uint16_t)(w.x & 0xFFFFu));
        g[1] = from16<DT>((uint16_t)(w.x >> 16));
        g[2] = from16<DT>((uint16_t)(w.y & 0xFFFFu));
        g[3] = from16<DT>((uint16_t)(w.y >> 16));
      }
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = out_value<DT, ACT>(v[e], g[e]);
      if (gm < a.M) {
        if (full4) {
          store4<YT>(a, gm, gn, y);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < a.N) store1<YT>(a, gm, gn + e, y[e]);
        }
      }
    }
  };
  if constexpr (ACT == 1) load_gate(0, gq[0]);
  strip(std::integral_constant<int, 0>{});
  strip(std::integral_constant<int, 1>{});
  strip(std::integral_constant<int, 2>{});
  strip(std::integral_constant<int, 3>{});
}

// dst = round16(src) element-wise (round-to-nearest-even; bf16 keeps NaN
// quiet, fp16 saturates to infinity as the conversion instruction does).  One
// thread per 4 consecutive elements of a row; rows whose starts are 16-byte
// aligned (src) and 8-byte aligned (dst) use vector accesses.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void round16_kernel(const float* __restrict__ src, int64_t lds,
                                                      uint16_t* __restrict__ dst, int64_t ldd, int64_t rows,
                                                      int64_t cols) {
  const int64_t q4 = (cols + 3) / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * q4) return;
  const int64_t row = t / q4, c0 = (t - row * q4) * 4;
  const float* sp = src + row * lds + c0;
  uint16_t* dp = dst + row * ldd + c0;
  if (VEC && c0 + 4 <= cols) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(sp);
    uint2 o;
    o.x = to16<DT>(v[0]) | (to16<DT>(v[1]) << 16);
    o.y = to16<DT>(v[2]) | (to16<DT>(v[3]) << 16);
    *reinterpret_cast<uint2*>(dp) = o;
  } else {
    for (int e = 0; e < 4 && c0 + e < cols; ++e) dp[e] = (uint16_t)to16<DT>(sp[e]);
  }
}

}  // namespace

void launch_round16(const float* src, int64_t rows, int64_t cols, int64_t lds, int dt, void* dst, int64_t ldd,
                    hipStream_t s) {
  const int64_t n = rows * ((cols + 3) / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && lds % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 8 == 0 && ldd % 4 == 0;
  uint16_t* d16 = static_cast<uint16_t*>(dst);
  if (dt == 1) {
    if (vec) hipLaunchKernelGGL((round16_kernel<1, true>), grid, dim3(256), 0, s, src, lds, d16, ldd, rows, cols);
    else hipLaunchKernelGGL((round16_kernel<1, false>), grid, dim3(256), 0, s, src, lds, d16, ldd, rows, cols);
  } else {
    if (vec) hipLaunchKernelGGL((round16_kernel<2, true>), grid, dim3(256), 0, s, src, lds, d16, ldd, rows, cols);
    else hipLaunchKernelGGL((round16_kernel<2, false>), grid, dim3(256), 0, s, src, lds, d16, ldd, rows, cols);
  }
}

void launch_linear(const void* X, int xt, int64_t n_tok, int64_t d, int64_t ldx, const void* W, bool w16,
                   int64_t r, int64_t ldw, int act, const void* G, int64_t ldg, void* Y, int yt, int64_t ldy,
                   hipStream_t s) {
  LinArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.ldx = ldx;
  a.W = w16 ? nullptr : static_cast<const float*>(W);
  a.W16 = w16 ? static_cast<const uint16_t*>(W) : nullptr;
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
  a.ntm = (int)((n_tok + LT - 1) / LT);
  const size_t ysz = yt == 0 ? 4 : 2;
  a.yvec = reinterpret_cast<uintptr_t>(Y) % (4 * ysz) == 0 && ldy % 4 == 0;
  a.gvec = G != nullptr && reinterpret_cast<uintptr_t>(G) % 8 == 0 && ldg % 4 == 0;
  a.ntn = (int)((r + LT - 1) / LT);
  const size_t lds = 4 * LT * LROWB;
  const dim3 grid((unsigned)((int64_t)a.ntm * a.ntn));
  // 128 KiB of dynamic LDS: A and B, double buffered
#define GPTQ_LIN(D_, A_, Y_, W_)                                                                      \
  do {                                                                                                \
    static const bool set = [&] { /* once, thread-safe (function-local static) */                     \
      (void)hipFuncSetAttribute((const void*)linear_kernel<D_, A_, Y_, W_>,                           \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                \
      return true;                                                                                    \
    }();                                                                                              \
    (void)set;                                                                                        \
    hipLaunchKernelGGL((linear_kernel<D_, A_, Y_, W_>), grid, dim3((W_) ? 512 : 256), lds, s, a);    \
  } while (0)
#define GPTQ_LIN_W(D_, A_, Y_)                  \
  do {                                          \
    if (w16) GPTQ_LIN(D_, A_, Y_, true);        \
    else GPTQ_LIN(D_, A_, Y_, false);           \
  } while (0)
#define GPTQ_LIN_Y(D_, A_)                   \
  do {                                       \
    if (yt == 0) GPTQ_LIN_W(D_, A_, 0);      \
    else if (yt == 1) GPTQ_LIN_W(D_, A_, 1); \
    else GPTQ_LIN_W(D_, A_, 2);              \
  } while (0)
  if (xt == 1) {
    if (act == 1) GPTQ_LIN_Y(1, 1); else GPTQ_LIN_Y(1, 0);
  } else {
    if (act == 1) GPTQ_LIN_Y(2, 1); else GPTQ_LIN_Y(2, 0);
  }
#undef GPTQ_LIN_Y
#undef GPTQ_LIN_W
#undef GPTQ_LIN
}

}  // namespace gptq
