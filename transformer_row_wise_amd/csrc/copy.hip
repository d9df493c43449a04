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
  if (!std::strcmp(s, "chunked")) return PATH_CHUNKED;
  if (!std::strcmp(s, "scalar")) return PATH_SCALAR;
  return PATH_AUTO;
}

constexpr int64_t kMaxCopyGrid = 0x7fffffff;

// ---------------------------------------------------------------- 16-byte copy

__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  // Four 16-byte chunks per thread, 256 threads: a block moves 16 KiB.
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = base + k * 256;
    if (i < n) v[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = base + k * 256;
    if (i < n) dst[i] = v[k];
  }
}

hipError_t launch_copy16(const void* src, void* dst, int64_t n16, hipStream_t stream) {
  const int64_t blocks = (n16 + 1023) / 1024;
  if (blocks > kMaxCopyGrid) return hipErrorInvalidValue;
  copy16_kernel<<<(unsigned)blocks, 256, 0, stream>>>((const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace nrm
