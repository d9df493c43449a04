// The 16-byte copies used as bandwidth ceilings (one stream into one, and two into two) and
// to calibrate the byte counters, and the NRM_FORCE_PATH test override.
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

// Two streams copied into two, one 16-byte chunk of each per thread, 512 threads per block,
// non-temporal: the residual add-RMSNorm's byte pattern (two inputs in, two outputs out)
// without arithmetic, in the fastest shape measured for that pattern on MI355X. The launch
// reserves 58 KB of LDS per block (unused), which caps residency at two blocks (16 waves)
// per compute unit: 82% of 8 TB/s over four rotating buffer sets, against 76-78% at three or
// four blocks per CU and 78% at one. Two chunks of each array per thread, 256- or 1024-thread
// blocks, or a barrier between the loads and the stores at four blocks per CU stay at 74-79%.
constexpr size_t kCopy2Lds = 58000;
__global__ void __launch_bounds__(512)
copy16x2_kernel(const u32x4* s1, const u32x4* s2, u32x4* d1, u32x4* d2, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x;
  if (i < n) {
    const u32x4 a = ld16_nt(s1 + i), b = ld16_nt(s2 + i);
    st16_nt(d1 + i, a);
    st16_nt(d2 + i, b);
  }
}

hipError_t launch_copy16x2(const void* s1, const void* s2, void* d1, void* d2, int64_t n16,
                           hipStream_t stream) {
  const int64_t blocks = (n16 + 511) / 512;
  if (blocks > kMaxCopyGrid) return hipErrorInvalidValue;
  copy16x2_kernel<<<(unsigned)blocks, 512, kCopy2Lds, stream>>>((const u32x4*)s1, (const u32x4*)s2,
                                                                (u32x4*)d1, (u32x4*)d2, n16);
  return hipGetLastError();
}

}  // namespace nrm
