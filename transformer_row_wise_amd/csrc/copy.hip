// The 16-byte copy used as the bandwidth ceiling and to calibrate the byte counters, and
// the NRM_FORCE_PATH test override.
#include <cstdlib>
#include <cstring>

#include "launch.hpp"

namespace nrm {

int forced_path() {
  const char* s = std::getenv("NRM_FORCE_PATH");
  if (!s) return PATH_AUTO;
  if (!std::strcmp(s, "wave")) return PATH_WAVE;
  if (!std::strcmp(s, "block")) return PATH_BLOCK;
  if (!std::strcmp(s, "rowblock")) return PATH_ROWBLOCK;
  if (!std::strcmp(s, "chunked")) return PATH_CHUNKED;
  if (!std::strcmp(s, "scalar")) return PATH_SCALAR;
  return PATH_AUTO;
}

constexpr int64_t kMaxCopyGrid = 0x7fffffff;

// ---------------------------------------------------------------- 16-byte copy

// One 16-byte chunk per thread, non-temporal load and store: the fastest plain copy
// measured on MI355X (~6.45 TB/s counting both directions; four chunks per thread without
// the streaming hint reach ~5.6 TB/s).
__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) st16_nt(dst + i, ld16_nt(src + i));
}

hipError_t launch_copy16(const void* src, void* dst, int64_t n16, hipStream_t stream) {
  const int64_t blocks = (n16 + 255) / 256;
  if (blocks > kMaxCopyGrid) return hipErrorInvalidValue;
  copy16_kernel<<<(unsigned)blocks, 256, 0, stream>>>((const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace nrm
