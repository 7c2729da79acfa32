// Shared device-side helpers for the gfx950 GPTQ kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GPTQ_DEV __device__ __forceinline__

namespace gptq {

// Host-side launch helpers report failures through this.
struct LaunchError {
  hipError_t err;
};

// fp32 helpers whose rounding is fixed (no contraction by the compiler).
GPTQ_DEV float mul_rn(float a, float b) { return __fmul_rn(a, b); }
GPTQ_DEV float div_rn(float a, float b) { return __fdiv_rn(a, b); }
GPTQ_DEV float fma_rn(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// Correctly rounded a / b from y = RN(1/b): q0 = RN(a*y), r = a - b*q0 (exact
// with an FMA), q1 = RN(q0 + r*y).  Markstein's theorem (Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", 1990) gives
// q1 = RN(a/b) when y is the correctly rounded reciprocal and no underflow or
// overflow occurs.
GPTQ_DEV float div_by_recip(float a, float b, float y) {
  float q0 = __fmul_rn(a, y);
  float r = __builtin_fmaf(-q0, b, a);
  return __builtin_fmaf(r, y, q0);
}

GPTQ_DEV float rne(float x) { return __builtin_rintf(x); }

}  // namespace gptq
