// Workspace sizes of the host-side plans that the C ABI's validation needs
// without any kernel (kept apart from the kernels so that the argument
// checks can be built and tested on their own).
#include "kernels.hpp"

namespace gptq {

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t quantize_workspace_bytes(int64_t r, int64_t c, int64_t blocksize) {
  const int64_t B = blocksize > 0 ? blocksize : 1;
  return align256((size_t)r * c * sizeof(float)) + align256((size_t)kSuperBlocks * B * r * sizeof(float));
}

}  // namespace gptq
