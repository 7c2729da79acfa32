// Host-side argument validation of the C ABI (include/gptq.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.
//
// Every call below must be rejected by the host checks before anything is
// enqueued (the kernels' launch functions are replaced by stubs that abort),
// including sizes at the limits of int64_t, where a careless product of
// sizes would overflow.  Built and run by tests/test_boundary_cpu.py.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "gptq.h"
#include "kernels.hpp"

namespace gptq {
// Launches never happen in this driver: every call fails validation first.
[[noreturn]] static void launched(const char* fn) {
  std::fprintf(stderr, "validation let a call through to %s\n", fn);
  std::abort();
}
void launch_quantize(const QuantArgs&, hipStream_t) { launched("launch_quantize"); }
void launch_linear(const void*, int, int64_t, int64_t, int64_t, const void*, bool, int64_t, int64_t, int, const void*,
                   int64_t, void*, int, int64_t, hipStream_t) {
  launched("launch_linear");
}
void launch_round16(const float*, int64_t, int64_t, int64_t, int, void*, int64_t, hipStream_t) {
  launched("launch_round16");
}
}  // namespace gptq

static int failures = 0;
static void expect(const char* what, gptq_status got, gptq_status want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, gptq_last_error());
    ++failures;
  }
  (void)gptq_status_string(got);
}

int main() {
  const int64_t BIG = std::numeric_limits<int64_t>::max();
  void* A = reinterpret_cast<void*>(uintptr_t(0x10000));      // never dereferenced
  void* B = reinterpret_cast<void*>(uintptr_t(0x40000000));
  size_t sz = 0;

  // workspace queries at and beyond the limits
  expect("hws ok", gptq_hessian_workspace_size(4096, 262144, GPTQ_BF16, &sz), GPTQ_OK);
  expect("hws big d", gptq_hessian_workspace_size(BIG, 1, GPTQ_BF16, &sz), GPTQ_EUNSUPPORTED);
  expect("hws big n", gptq_hessian_workspace_size(16, BIG, GPTQ_BF16, &sz), GPTQ_EUNSUPPORTED);
  expect("hws neg", gptq_hessian_workspace_size(-1, 1, GPTQ_BF16, &sz), GPTQ_EINVAL);
  expect("pws big", gptq_prepare_workspace_size(BIG, 0, &sz), GPTQ_EUNSUPPORTED);
  expect("pws max", gptq_prepare_workspace_size(65535, 1, &sz), GPTQ_OK);
  expect("qws big", gptq_quantize_layer_workspace_size(BIG, BIG, 128, &sz), GPTQ_EUNSUPPORTED);
  expect("qws ok", gptq_quantize_layer_workspace_size(12288, 49152, 128, &sz), GPTQ_OK);

  // Hessian
  float* H = static_cast<float*>(A);
  expect("h big d", gptq_hessian_accumulate(H, BIG, A, GPTQ_BF16, 8, BIG, nullptr, 0, nullptr), GPTQ_EUNSUPPORTED);
  expect("h big n", gptq_hessian_accumulate(H, 64, A, GPTQ_BF16, BIG, 64, nullptr, 0, nullptr), GPTQ_EUNSUPPORTED);
  expect("h ldx", gptq_hessian_accumulate(H, 64, A, GPTQ_BF16, 8, 32, nullptr, 0, nullptr), GPTQ_ESHAPE);
  expect("h ws", gptq_hessian_accumulate(H, 4096, A, GPTQ_BF16, 262144, 4096, nullptr, 0, nullptr),
         GPTQ_EWORKSPACE);
  expect("h dtype", gptq_hessian_accumulate(H, 64, A, (gptq_dtype)7, 8, 64, nullptr, 0, nullptr), GPTQ_EDTYPE);

  // prepare and its allocation-free variant
  int32_t* I = static_cast<int32_t*>(A);
  uint8_t* U8 = static_cast<uint8_t*>(A);
  expect("p big", gptq_prepare(H, BIG, 0.01f, 0, I, U8, I, B, 0, nullptr), GPTQ_EUNSUPPORTED);
  expect("p nan damp", gptq_prepare(H, 64, std::numeric_limits<float>::quiet_NaN(), 0, I, U8, I, B, 0, nullptr),
         GPTQ_EINVAL);
  expect("p ws", gptq_prepare(H, 64, 0.01f, 0, I, U8, I, nullptr, 0, nullptr), GPTQ_EWORKSPACE);
  expect("pn big", gptq_prepare_noalloc(H, BIG, 0.01f, 0, I, U8, I, nullptr), GPTQ_EUNSUPPORTED);
  expect("pn 4097", gptq_prepare_noalloc(H, 4097, 0.01f, 0, I, U8, I, nullptr), GPTQ_EUNSUPPORTED);
  expect("pn perm", gptq_prepare_noalloc(H, 64, 0.01f, 1, nullptr, U8, I, nullptr), GPTQ_EINVAL);

  // quantize
  expect("q big", gptq_quantize_layer(A, GPTQ_BF16, BIG, BIG, BIG, H, nullptr, nullptr, 4, 0, 128, 128, U8, H, I, I,
                                      nullptr, nullptr, B, 1 << 20, nullptr), GPTQ_EUNSUPPORTED);
  expect("q rows", gptq_quantize_layer(A, GPTQ_BF16, int64_t(1) << 24, 256, 256, H, nullptr, nullptr, 4, 0, 128, 128,
                                       U8, H, I, I, nullptr, nullptr, B, 1 << 20, nullptr), GPTQ_EUNSUPPORTED);
  expect("q ws", gptq_quantize_layer(A, GPTQ_BF16, 64, 256, 256, H, nullptr, nullptr, 4, 0, 128, 128, U8, H, I, I,
                                     nullptr, nullptr, nullptr, 0, nullptr), GPTQ_EWORKSPACE);
  expect("q bits", gptq_quantize_layer(A, GPTQ_BF16, 64, 256, 256, H, nullptr, nullptr, 5, 0, 128, 128, U8, H, I, I,
                                       nullptr, nullptr, B, 1 << 20, nullptr), GPTQ_EUNSUPPORTED);

  // pack, GEMV, rotation, forward, rounding
  uint32_t* W32 = static_cast<uint32_t*>(A);
  expect("pk big", gptq_pack(U8, BIG, BIG - (BIG % 32), 4, nullptr, W32, BIG, nullptr), GPTQ_EUNSUPPORTED);
  expect("pk ld", gptq_pack(U8, 4, 64, 4, nullptr, W32, 2, nullptr), GPTQ_ESHAPE);
  expect("gv big", gptq_dequant_gemv(W32, BIG, 64, 4, 8, H, I, 1, 128, nullptr, A, GPTQ_BF16, H, nullptr),
         GPTQ_EUNSUPPORTED);
  expect("gv c", gptq_dequant_gemv(W32, 4, 49184, 4, 6148, H, I, 1, -1, nullptr, A, GPTQ_BF16, H, nullptr),
         GPTQ_EUNSUPPORTED);
  expect("hr big", gptq_hadamard_rotate(A, GPTQ_BF16, BIG, 4096, 4096, 0, B, GPTQ_BF16, 4096, nullptr),
         GPTQ_EUNSUPPORTED);
  expect("hr ld", gptq_hadamard_rotate(A, GPTQ_BF16, 4, 4096, 100, 0, B, GPTQ_BF16, 4096, nullptr), GPTQ_ESHAPE);
  expect("lf big", gptq_linear_forward(A, GPTQ_BF16, BIG, 256, 256, B, GPTQ_F32, BIG, 256, 0, nullptr, 0, B,
                                       GPTQ_BF16, BIG, nullptr), GPTQ_EUNSUPPORTED);
  expect("lf d", gptq_linear_forward(A, GPTQ_BF16, 8, 100, 100, B, GPTQ_F32, 8, 100, 0, nullptr, 0, B, GPTQ_BF16, 8,
                                     nullptr), GPTQ_EUNSUPPORTED);
  expect("r16 big", gptq_round16(H, BIG, BIG, BIG, GPTQ_BF16, B, BIG, nullptr), GPTQ_EUNSUPPORTED);
  expect("r16 overlap", gptq_round16(H, 4, 64, 64, GPTQ_BF16, reinterpret_cast<char*>(A) + 64, 64, nullptr),
         GPTQ_EINVAL);
  // leading dimensions whose extents overflow 64 bits
  expect("hr huge ld", gptq_hadamard_rotate(A, GPTQ_BF16, 1 << 20, 4096, BIG / 2, 0, B, GPTQ_BF16, 4096, nullptr),
         GPTQ_EUNSUPPORTED);
  expect("r16 huge ld", gptq_round16(H, 1 << 20, 64, BIG / 2, GPTQ_BF16, B, 64, nullptr), GPTQ_EUNSUPPORTED);
  expect("lf huge ld", gptq_linear_forward(A, GPTQ_BF16, 1 << 20, 256, 256, B, GPTQ_F32, 64, 256, 0, nullptr, 0, B,
                                           GPTQ_BF16, BIG / 4, nullptr), GPTQ_EUNSUPPORTED);
  // enumeration values outside the lists
  expect("status string", (gptq_status_string((gptq_status)1234)[0] != 0) ? GPTQ_OK : GPTQ_EINVAL, GPTQ_OK);
  expect("bad dtype", gptq_round16(H, 4, 64, 64, (gptq_dtype)-5, B, 64, nullptr), GPTQ_EINVAL);


  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("all validation checks passed under the sanitizers\n");
  return 0;
}
