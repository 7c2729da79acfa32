// Packing of tick indices into 32-bit words (the pages store one tick index
// per weight -- "GPTQ, with the code open", "What quantization is, and why
// anyone bothers"; the word layout is this library's own):
//   4 bits: 8 codes per word, code k of the word in bits 4k .. 4k+3;
//   3 bits: 32 codes per 3 words, code k in bits 3k .. 3k+2 of the
//           little-endian 96-bit value.
// Streaming kernel: each thread turns one 8-byte (4-bit) or 32-byte (3-bit)
// run of codes into one or three words.  With a column permutation (act-order
// layers packed in the order their columns were quantized, so that groups are
// contiguous for the dequantizing product) each thread gathers its codes byte
// by byte instead.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

__global__ __launch_bounds__(256) void pack4_kernel(const uint8_t* __restrict__ codes, int64_t r,
                                                    int64_t c, uint32_t* __restrict__ out,
                                                    int64_t ldw) {
  const int64_t wpr = c / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * wpr) return;
  const int64_t row = idx / wpr, wd = idx % wpr;
  const uint2 v = *reinterpret_cast<const uint2*>(codes + row * c + wd * 8);
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w |= ((v.x >> (8 * k)) & 0xFu) << (4 * k);
    w |= ((v.y >> (8 * k)) & 0xFu) << (4 * (k + 4));
  }
  out[row * ldw + wd] = w;
}

// 4-bit, 32 codes per thread: two 16-byte loads, one 16-byte store of four
// words (rows of codes and of words 16-byte aligned, c % 32 == 0).
__global__ __launch_bounds__(256) void pack4x4_kernel(const uint8_t* __restrict__ codes, int64_t r,
                                                      int64_t c, uint32_t* __restrict__ out, int64_t ldw) {
  const int64_t qpr = c / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * qpr) return;
  const int64_t row = idx / qpr, qd = idx % qpr;
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + row * c + qd * 32);
  const u32x4 a = __builtin_nontemporal_load(src), b = __builtin_nontemporal_load(src + 1);
  const uint32_t in[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 o;
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    const uint32_t x = in[2 * wd], y = in[2 * wd + 1];
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w |= ((x >> (8 * k)) & 0xFu) << (4 * k);
      w |= ((y >> (8 * k)) & 0xFu) << (4 * (k + 4));
    }
    o[wd] = w;
  }
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + row * ldw + qd * 4));
}

__global__ __launch_bounds__(256) void pack3_kernel(const uint8_t* __restrict__ codes, int64_t r,
                                                    int64_t c, uint32_t* __restrict__ out,
                                                    int64_t ldw) {
  const int64_t gpr = c / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * gpr) return;
  const int64_t row = idx / gpr, grp = idx % gpr;
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + row * c + grp * 32);
  const u32x4 a = src[0], b = src[1];
  uint32_t byte4[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint64_t lo = 0, hi = 0;  // 96-bit accumulator: lo = bits 0..63, hi = bits 64..95
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint64_t v = (byte4[k >> 2] >> (8 * (k & 3))) & 0x7u;
    const int sh = 3 * k;
    if (sh + 3 <= 64) {
      lo |= v << sh;
    } else if (sh >= 64) {
      hi |= v << (sh - 64);
    } else {
      lo |= v << sh;
      hi |= v >> (64 - sh);
    }
  }
  uint32_t* o = out + row * ldw + grp * 3;
  o[0] = (uint32_t)lo;
  o[1] = (uint32_t)(lo >> 32);
  o[2] = (uint32_t)hi;
}

// Packed column j takes the code of original column perm[j]; one thread per
// 32 packed columns (one 4-bit quad of words or one 3-bit triple).
__global__ __launch_bounds__(256) void pack_perm_kernel(const uint8_t* __restrict__ codes, int64_t r,
                                                        int64_t c, int bits,
                                                        const int32_t* __restrict__ perm,
                                                        uint32_t* __restrict__ out, int64_t ldw) {
  const int64_t nch = (c + 31) / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * nch) return;
  const int64_t row = idx / nch, ch = idx % nch;
  const uint8_t* src = codes + row * c;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  const int n = (int)min((int64_t)32, c - ch * 32);
  for (int k = 0; k < n; ++k) {
    const int64_t col = min(max((int64_t)perm[ch * 32 + k], (int64_t)0), c - 1);  // entries outside 0..c-1 clamp
    const uint32_t v = (uint32_t)src[col] & mask;
    const int bit = bits * k;
    w[bit >> 5] |= v << (bit & 31);
    if ((bit & 31) + bits > 32) w[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
  }
  uint32_t* o = out + row * ldw + ch * bits;
  const int nw = (n * bits + 31) / 32;
  for (int t = 0; t < nw; ++t) o[t] = w[t];
}

}  // namespace

void launch_pack(const uint8_t* codes, int64_t r, int64_t c, int bits, const int32_t* perm,
                 uint32_t* packed, int64_t ld_words, hipStream_t s) {
  if (perm) {
    const int64_t n = r * ((c + 31) / 32);
    hipLaunchKernelGGL(pack_perm_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, r, c,
                       bits, perm, packed, ld_words);
    return;
  }
  const bool wide = (c % 32 == 0) && (ld_words % 4 == 0) && (reinterpret_cast<uintptr_t>(packed) % 16 == 0);
  if (bits == 4 && wide) {
    const int64_t n = r * (c / 32);
    hipLaunchKernelGGL(pack4x4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, r, c,
                       packed, ld_words);
  } else if (bits == 4) {
    const int64_t n = r * (c / 8);
    hipLaunchKernelGGL(pack4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, r, c,
                       packed, ld_words);
  } else {
    const int64_t n = r * (c / 32);
    hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, r, c,
                       packed, ld_words);
  }
}

}  // namespace gptq
