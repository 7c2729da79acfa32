// Dequantize-on-the-fly matrix-vector product over packed codes, batch 1:
//     y[i] = sum_j scale[i, g(j)] * (q[i, j] - zero[i, g(j)]) * x[j]
// The pages: "GPTQ, with the code open", section "What quantization is, and
// why anyone bothers" -- a generated token reads every weight once, so the
// stored tick indices are turned back into scale * (tick - zero) inside the
// product and the smaller words become a faster read.  The page "Post-training
// quantization", section "Weight-only and weight-and-activation", names the
// regime: four-bit (or three-bit) weights, sixteen-bit activations.
//
// Design (HBM-bound streaming, one pass over the packed words):
//   * A "chunk" is 32 consecutive packed columns: 16 bytes at 4 bits, 12 bytes
//     at 3 bits.  Lane l of a wave owns chunks l, l + 64 S, l + 128 S, ... of
//     its column slice for every row it visits, so one wave-wide load reads
//     64 consecutive chunks of a row (1 KiB at 4 bits) and the lane's slice of
//     x stays in registers across all rows.
//   * Codes become fp16 values with two bit operations and one packed add:
//     a field of the packed word masked into bits p .. p+b-1 of a 16-bit half
//     and OR-ed with the exponent of 1024 reads as 1024 + q 2^p, and
//     subtracting 1024 leaves q 2^p exactly.  Two such halves meet a pair of
//     x values pre-scaled by 2^(16-p-e) in one v_dot2_f32_f16: the products
//     q x 2^(16-e) are exact and the sums are fp32.  (The codes are kept out
//     of fp16's subnormal range on purpose: the dot instruction's products
//     with subnormal inputs are not exact.)  Each 8-code block takes two
//     32-bit windows of the packed stream and two masks per window; the
//     pairing (8m+t, 8m+t+4) is the same for both widths, only the field
//     positions differ.
//   * x (bf16 or fp16) is rescaled per chunk by a power of two chosen from the
//     chunk's largest |x| so that every pre-scaled value fits fp16; bf16 and
//     fp16 significands fit fp16's, so the conversion is exact for every value
//     within 2^-29 of the chunk maximum (smaller ones fall on fp16's subnormal
//     grid, where they contribute below 2^-29 of the chunk maximum each).
//   * The zero point is taken out once per chunk: sum q x - zero * sum x, with
//     sum x of the chunk computed once in fp32.
//   * Rows are visited four at a time; the four partial sums of a wave are
//     folded with a transposed butterfly (each exchange halves the values per
//     lane) and, when a row's columns are split over S waves of the
//     workgroup, summed across waves through LDS in wave order once per
//     epoch of 16 quads (the waves are not held together on every quad).
//     Two row quads are in flight per wave: the words of the next quad are
//     loaded before the current one is used.
//   * act-order layers are handled by packing their codes in the order the
//     columns were quantized (groups are then contiguous) and gathering x
//     through that permutation once per lane.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxNch = 3;     // chunks per lane (register budget)
constexpr int kRows = 4;       // rows per wave visit

struct GemvArgs {
  const uint32_t* packed;
  int64_t ldw;            // words per row
  const float* scales;
  const int32_t* zeros;
  int64_t ldg;            // groups per row (row stride of scales / zeros)
  const int32_t* perm;    // nullable: packed column j holds original column perm[j]
  const uint16_t* x;      // bf16 or fp16 bits
  float* y;
  int r, c, nch;          // rows, columns, 32-column chunks
  int cpg;                // chunks per group (>= nch: one group per row)
  int S;                  // waves sharing one row (column split)
  int G;                  // wave groups per workgroup
  int nquads;             // ceil(r / 4)
  int f16x;               // x is fp16 (else bf16)
};

// Field positions (p of the low half, p of the high half) of the two masks.
template <int BITS>
struct Fields;
template <>
struct Fields<4> {
  static constexpr uint32_t M1 = 0x000F000Fu, M2 = 0x00F000F0u;
  static constexpr int P1LO = 0, P1HI = 0, P2LO = 4, P2HI = 4;
};
template <>
struct Fields<3> {
  static constexpr uint32_t M1 = 0x00070070u, M2 = 0x00380380u;
  static constexpr int P1LO = 4, P1HI = 0, P2LO = 7, P2HI = 3;
};

template <int BITS>
struct Words;
template <>
struct Words<4> {
  uint32_t w[4];
};
template <>
struct Words<3> {
  uint32_t w[3];
};

// Bits s .. s+31 of the 64-bit value hi:lo (v_alignbit_b32).
GPTQ_DEV uint32_t window(uint32_t hi, uint32_t lo, uint32_t s) { return __builtin_amdgcn_alignbit(hi, lo, s); }

// The two 32-bit windows (A, B) of 8-code block m of a chunk.
//   4 bits: A = word m, B = word m >> 8.
//   3 bits: block m spans stream bits 24m .. 24m+23; A starts at bit 24m - 4,
//           B at bit 24m + 2 of the 96-bit little-endian stream.
template <int BITS>
GPTQ_DEV void windows(const Words<BITS>& v, int m, uint32_t& A, uint32_t& B);
template <>
GPTQ_DEV void windows<4>(const Words<4>& v, int m, uint32_t& A, uint32_t& B) {
  A = v.w[m];
  B = v.w[m] >> 8;
}
template <>
GPTQ_DEV void windows<3>(const Words<3>& v, int m, uint32_t& A, uint32_t& B) {
  if (m == 0) {
    A = v.w[0] << 4;
    B = v.w[0] >> 2;
  } else if (m == 1) {
    A = window(v.w[1], v.w[0], 20);
    B = window(v.w[1], v.w[0], 26);
  } else if (m == 2) {
    A = window(v.w[2], v.w[1], 12);
    B = window(v.w[2], v.w[1], 18);
  } else {
    A = v.w[2] >> 4;
    B = v.w[2] >> 10;
  }
}

GPTQ_DEV float dot2(uint32_t codes, half2_t x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, codes), x, acc, false);
}

template <int BITS>
GPTQ_DEV Words<BITS> load_words(const uint32_t* __restrict__ p) {
  Words<BITS> v;
  if constexpr (BITS == 4) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(p);
    v.w[0] = t[0]; v.w[1] = t[1]; v.w[2] = t[2]; v.w[3] = t[3];
  } else {
    v.w[0] = p[0]; v.w[1] = p[1]; v.w[2] = p[2];
  }
  return v;
}

template <int BITS>
struct RowBuf {
  Words<BITS> w[kRows][kMaxNch];
  float s[kRows][kMaxNch];
  int z[kRows][kMaxNch];
};

// Words and rulers of rows 4 quad .. 4 quad + 3 for this lane's chunks.  Rows
// past the end and the quads of idle wave groups read row r-1 (results are
// dropped); a lane's chunks past the end read the last chunk, and their
// contribution is zero because their x values are zero and their scale is
// replaced by 0.  No branches, so every load is issued back to back.
template <int BITS, int NCH>
GPTQ_DEV void load_quad(const GemvArgs& a, int quad, const int (&jc)[kMaxNch], const int (&grp)[kMaxNch],
                        const bool (&jv)[kMaxNch], RowBuf<BITS>& b) {
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int row = __builtin_amdgcn_readfirstlane(min(quad * kRows + i, a.r - 1));
    const uint32_t* prow = a.packed + (int64_t)row * a.ldw;
    const float* srow = a.scales + (int64_t)row * a.ldg;
    const int32_t* zrow = a.zeros + (int64_t)row * a.ldg;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      // 32-bit unsigned offsets from a wave-uniform row base (global_load with saddr)
      const uint32_t wo = (uint32_t)jc[k] * (4u * BITS), go = (uint32_t)grp[k] * 4u;
      b.w[i][k] = load_words<BITS>(reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(prow) + wo));
      const float sc = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(srow) + go);
      b.s[i][k] = jv[k] ? sc : 0.f;
      b.z[i][k] = *reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(zrow) + go);
    }
  }
}

// Field under mask M of window W as the fp16 pair (q_lo 2^p_lo, q_hi 2^p_hi):
// exponent of 1024 OR-ed in, 1024 subtracted (exact: the result has at most
// 11 significant bits).
// `magic` is 0x64006400 held in a VGPR, so that mask-and-or is one
// v_and_or_b32 (its other constant, the mask, takes the one scalar operand).
GPTQ_DEV uint32_t code_pair(uint32_t W, uint32_t M, uint32_t magic) {
  const half2_t h = __builtin_bit_cast(half2_t, (W & M) | magic);
  const half2_t k = {(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, h - k);
}

// sum_j q_j x_j over one chunk, in units of 2^(e - 16) (see the x prologue).
template <int BITS>
GPTQ_DEV float chunk_dot(const Words<BITS>& v, const uint32_t (&xp)[16], uint32_t magic) {
  using F = Fields<BITS>;
  float d = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t A, B;
    windows<BITS>(v, m, A, B);
    d = dot2(code_pair(A, F::M1, magic), __builtin_bit_cast(half2_t, xp[4 * m + 0]), d);
    d = dot2(code_pair(A, F::M2, magic), __builtin_bit_cast(half2_t, xp[4 * m + 1]), d);
    d = dot2(code_pair(B, F::M1, magic), __builtin_bit_cast(half2_t, xp[4 * m + 2]), d);
    d = dot2(code_pair(B, F::M2, magic), __builtin_bit_cast(half2_t, xp[4 * m + 3]), d);
  }
  return d;
}

// DPP lane exchange (row_mask and bank_mask all on, bound_ctrl off).
template <int CTRL>
GPTQ_DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kRowRor4 = 0x124;  // row_ror:4 (rotate within 16 lanes)
constexpr int kRowRor8 = 0x128;  // row_ror:8

// Four row sums spread over the wave -> lane i (i < 4) holds row i's total.
// Transposed butterfly: the first two exchanges (within lane quads) halve the
// values per lane, so lane l ends with row l & 3; the rest adds the 16 lanes
// of each residue class (rotations within rows of 16, then across rows).
GPTQ_DEV float fold4(float v0, float v1, float v2, float v3, int lane) {
  const bool b0 = lane & 1;
  float ka = b0 ? v1 : v0, kb = b0 ? v3 : v2;
  const float sa = b0 ? v0 : v1, sb = b0 ? v2 : v3;
  ka += dpp<kQuadXor1>(sa);
  kb += dpp<kQuadXor1>(sb);
  const bool b1 = lane & 2;
  float k = b1 ? kb : ka;
  const float s = b1 ? ka : kb;
  k += dpp<kQuadXor2>(s);
  k += dpp<kRowRor4>(k);
  k += dpp<kRowRor8>(k);
  k += __shfl_xor(k, 16);
  k += __shfl_xor(k, 32);
  return k;
}

// ---- activation prologue ------------------------------------------------
// Raw activations of chunk j (32 16-bit values, two per dword).
GPTQ_DEV void load_x_raw(const GemvArgs& a, int j, bool valid, uint32_t (&v)[16]) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0u;
    return;
  }
  const int64_t c0 = (int64_t)j * 32;
  if (a.perm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s0 = min(max(a.perm[c0 + 2 * i], 0), a.c - 1);
      const int s1 = min(max(a.perm[c0 + 2 * i + 1], 0), a.c - 1);
      v[i] = (uint32_t)a.x[s0] | ((uint32_t)a.x[s1] << 16);
    }
  } else {
    const u32x4* px = reinterpret_cast<const u32x4*>(a.x + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 t = px[q];
      v[4 * q + 0] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
    }
  }
}

// Pre-scaled fp16 pairs of one chunk, its scaled sum and exponent:
//   e  = frexp exponent of max |x| (every |x| < 2^e);
//   xp = pairs (x_{8m+t} 2^(16-p_lo-e), x_{8m+t+4} 2^(16-p_hi-e)), fp16;
//   sx = sum_j x_j 2^(16-e) (fp32 sum of the unscaled values, then the exact
//        power-of-two scaling).
template <int BITS, bool F16X>
GPTQ_DEV void x_prep(const uint32_t (&v)[16], uint32_t (&xp)[16], float& sx, int& ex) {
  using F = Fields<BITS>;
  float xf[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (F16X) {
      xf[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] & 0xFFFFu));
      xf[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] >> 16));
    } else {
      xf[2 * i] = __uint_as_float(v[i] << 16);
      xf[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  float mx = 0.f, sum = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    mx = fmaxf(mx, fabsf(xf[i]));
    sum += xf[i];
  }
  const int e1 = __builtin_amdgcn_frexp_expf(mx);
  ex = e1;
  sx = __builtin_ldexpf(sum, 16 - e1);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int plo = (t & 1) ? F::P2LO : F::P1LO;
      const int phi = (t & 1) ? F::P2HI : F::P1HI;
      const float lo = __builtin_ldexpf(xf[8 * m + t], 16 - plo - e1);
      const float hi = __builtin_ldexpf(xf[8 * m + t + 4], 16 - phi - e1);
      xp[4 * m + t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
  }
}

// Template arguments: code width, chunks per lane, fp16 (else bf16)
// activations, and whether the workgroup's waves share one activation
// prologue through LDS (several wave groups reading the same chunks).
template <int BITS, int NCH, bool F16X, bool SHARE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NCH == 1 ? 4 : (NCH == 2 ? 3 : 2))))
void dq_gemv_kernel(GemvArgs a) {
  // Row sums of the column slices, kept for an epoch of row quads and summed
  // across the slices' waves once per epoch (one pair of barriers per epoch).
  constexpr int kEpoch = 16;
  __shared__ float red[8][kEpoch][4];   // [wave][quad of the epoch][row]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int g = wave / a.S, sl = wave - g * a.S;

  // ---- chunk ownership of this lane (jc: clamped index, jv: in range)
  int jc[kMaxNch], grp[kMaxNch];
  bool jv[kMaxNch];
#pragma unroll
  for (int k = 0; k < kMaxNch; ++k) {
    const int j = sl * 64 + lane + k * 64 * a.S;
    jv[k] = j < a.nch;
    jc[k] = jv[k] ? j : a.nch - 1;
    grp[k] = jc[k] / a.cpg;
  }

  int quad = blockIdx.x * a.G + g;
  const int qstride = gridDim.x * a.G;
  const int iters = (a.nquads - (int)blockIdx.x * a.G + qstride - 1) / qstride;
  RowBuf<BITS> bufA, bufB;

  // ---- activations go out first, then the first rows' words; the prologue
  //      runs while the words are in flight
  uint32_t xp[NCH][16];
  float sx[NCH];
  int ex[NCH];
  if constexpr (SHARE) {
    // tasks (slice, k) = t % S, t / S; wave w prepares tasks w and w + waves
    constexpr int kMaxTasks = 2 * kMaxNch;
    __shared__ uint32_t xl[kMaxTasks][18][64];
    const int ntask = a.S * NCH;
    uint32_t raw[2][16];
    bool mine[2];
    int tj[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wave + u * waves;
      mine[u] = t < ntask;
      const int tsl = mine[u] ? t % a.S : 0, tk = mine[u] ? t / a.S : 0;
      tj[u] = tsl * 64 + lane + tk * 64 * a.S;
      load_x_raw(a, tj[u], mine[u] && tj[u] < a.nch, raw[u]);
    }
    load_quad<BITS, NCH>(a, quad, jc, grp, jv, bufA);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (mine[u]) {
        uint32_t p[16];
        float s;
        int e;
        x_prep<BITS, F16X>(raw[u], p, s, e);
        const int t = wave + u * waves;
#pragma unroll
        for (int i = 0; i < 16; ++i) xl[t][i][lane] = p[i];
        xl[t][16][lane] = __float_as_uint(s);
        xl[t][17][lane] = (uint32_t)e;
      }
    }
    if (iters > 1) load_quad<BITS, NCH>(a, quad + qstride, jc, grp, jv, bufB);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int t = k * a.S + sl;
#pragma unroll
      for (int i = 0; i < 16; ++i) xp[k][i] = xl[t][i][lane];
      sx[k] = __uint_as_float(xl[t][16][lane]);
      ex[k] = (int)xl[t][17][lane];
    }
  } else {
    uint32_t raw[NCH][16];
#pragma unroll
    for (int k = 0; k < NCH; ++k) load_x_raw(a, sl * 64 + lane + k * 64 * a.S, jv[k], raw[k]);
    load_quad<BITS, NCH>(a, quad, jc, grp, jv, bufA);
    if (iters > 1) load_quad<BITS, NCH>(a, quad + qstride, jc, grp, jv, bufB);
#pragma unroll
    for (int k = 0; k < NCH; ++k) x_prep<BITS, F16X>(raw[k], xp[k], sx[k], ex[k]);
  }

  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  auto compute = [&](const RowBuf<BITS>& b) {
    float acc[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const float d = chunk_dot<BITS>(b.w[i][k], xp[k], magic);
        const float t = __builtin_fmaf(-(float)b.z[i][k], sx[k], d);
        // scale first, then undo the chunk's power of two: no intermediate
        // overflow for activations near the top of bf16's range
        s += __builtin_ldexpf(t * b.s[i][k], ex[k] - 16);
      }
      acc[i] = s;
    }
    return fold4(acc[0], acc[1], acc[2], acc[3], lane);
  };
  const int quad0 = quad;
  auto emit = [&](float tot, int it) {
    const int qd = quad0 + it * qstride;
    if (a.S == 1) {
      const int row = qd * kRows + lane;
      if (lane < kRows && qd < a.nquads && row < a.r) a.y[row] = tot;
    } else if (lane < kRows) {
      red[wave][it % kEpoch][lane] = tot;
    }
  };
  // Sum the slices of the epoch's quads it0 .. it0 + n - 1: lane = 4 quad + row.
  auto flush = [&](int it0, int n) {
    __syncthreads();
    const int e = lane >> 2, rr = lane & 3;
    if (sl == 0 && e < n) {
      float tot = red[wave][e][rr];
      for (int w = 1; w < a.S; ++w) tot += red[wave + w][e][rr];
      const int qd = quad0 + (it0 + e) * qstride;
      const int row = qd * kRows + rr;
      if (qd < a.nquads && row < a.r) a.y[row] = tot;
    }
    __syncthreads();
  };

  // two row quads in flight: while one is folded the next one's words land
  for (int it = 0; it < iters; it += 2) {
    emit(compute(bufA), it);
    if (it + 2 < iters) load_quad<BITS, NCH>(a, quad0 + (it + 2) * qstride, jc, grp, jv, bufA);
    if (it + 1 < iters) emit(compute(bufB), it + 1);
    if (it + 3 < iters) load_quad<BITS, NCH>(a, quad0 + (it + 3) * qstride, jc, grp, jv, bufB);
    if (a.S > 1) {
      const int done = min(it + 2, iters);
      if (done % kEpoch == 0 || done == iters) {
        const int it0 = (done - 1) / kEpoch * kEpoch;
        flush(it0, done - it0);
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

// Launch shape from the row length: one chunk per lane when a wave covers
// the row, else two chunks per lane over as many waves as needed (up to 8),
// else three.  (Measured on the Llama-7B and OPT-175B layer shapes: two
// chunks per lane balance register use against the per-row fold.)
GemvPlan plan_gemv(int64_t c) {
  GemvPlan p{};
  const int64_t nch = c / 32;
  if (nch <= 64) {
    p.S = 1;
    p.nch_lane = 1;
  } else if (nch <= 8 * 64 * 2) {
    p.S = (int)((nch + 127) / 128);
    p.nch_lane = 2;
  } else if (nch <= 8 * 64 * kMaxNch) {
    p.S = (int)((nch + 64 * kMaxNch - 1) / (64 * kMaxNch));
    p.nch_lane = kMaxNch;
  }
  return p;
}

void launch_dequant_gemv(const uint32_t* packed, int64_t r, int64_t c, int bits, int64_t ld_words,
                         const float* scales, const int32_t* zeros, int64_t ld_groups, int64_t groupsize,
                         const int32_t* perm, const void* x, int x_f16, float* y, hipStream_t s) {
  if (c == 0) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((r + 255) / 256)), dim3(256), 0, s, y, r);
    return;
  }
  const GemvPlan p = plan_gemv(c);
  GemvArgs a;
  a.packed = packed;
  a.ldw = ld_words;
  a.scales = scales;
  a.zeros = zeros;
  a.ldg = ld_groups;
  a.perm = perm;
  a.x = static_cast<const uint16_t*>(x);
  a.y = y;
  a.r = (int)r;
  a.c = (int)c;
  a.nch = (int)(c / 32);
  a.cpg = (groupsize > 0 && groupsize < c) ? (int)(groupsize / 32) : a.nch;
  a.S = p.S;
  a.G = p.S >= 4 ? 1 : 4 / p.S;
  const int waves = a.S * a.G;
  a.nquads = (int)((r + kRows - 1) / kRows);
  a.f16x = x_f16;
  // Balanced persistent grid: at most `cap` workgroups (as many as the
  // register budget keeps resident on every CU at once), every workgroup
  // visiting the same number of row quads give or take one.  Waves per SIMD
  // the register budget allows:
  // ~100 VGPRs with one chunk per lane, ~165 with two, ~235 with three.
  const int64_t tasks = (a.nquads + a.G - 1) / a.G;
  const int per_simd = p.nch_lane == 1 ? 4 : (p.nch_lane == 2 ? 3 : 2);
  const int per_cu = (4 * per_simd) / waves > 0 ? (4 * per_simd) / waves : 1;
  const int64_t cap = (int64_t)device_cus() * per_cu;
  const int64_t rounds = (tasks + cap - 1) / cap;
  const unsigned grid = (unsigned)((tasks + rounds - 1) / rounds);
  const dim3 block(64 * waves);
  const bool share = a.G > 1;
#define GPTQ_GEMV_LAUNCH(B_, N_)                                                                  \
  do {                                                                                            \
    if (x_f16) {                                                                                  \
      if (share) hipLaunchKernelGGL((dq_gemv_kernel<B_, N_, true, true>), dim3(grid), block, 0, s, a);   \
      else hipLaunchKernelGGL((dq_gemv_kernel<B_, N_, true, false>), dim3(grid), block, 0, s, a);        \
    } else {                                                                                      \
      if (share) hipLaunchKernelGGL((dq_gemv_kernel<B_, N_, false, true>), dim3(grid), block, 0, s, a);  \
      else hipLaunchKernelGGL((dq_gemv_kernel<B_, N_, false, false>), dim3(grid), block, 0, s, a);       \
    }                                                                                             \
  } while (0)
  if (bits == 4) {
    if (p.nch_lane == 1) GPTQ_GEMV_LAUNCH(4, 1);
    else if (p.nch_lane == 2) GPTQ_GEMV_LAUNCH(4, 2);
    else GPTQ_GEMV_LAUNCH(4, 3);
  } else {
    if (p.nch_lane == 1) GPTQ_GEMV_LAUNCH(3, 1);
    else if (p.nch_lane == 2) GPTQ_GEMV_LAUNCH(3, 2);
    else GPTQ_GEMV_LAUNCH(3, 3);
  }
#undef GPTQ_GEMV_LAUNCH
}

}  // namespace gptq
