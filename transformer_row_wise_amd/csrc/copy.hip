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

// The same pattern with a row kernel's work unit: each 512-thread block copies one unit of NV
// 16-byte chunks per thread of each source (chunks t, t + 512, ...: a unit of 8 KB * NV per
// array, as row_block holds a row), and a barrier after the loads keeps every store of the
// block waiting until its whole unit has arrived, as a row's outputs wait for its statistic.
// That is add-RMSNorm's memory traffic in row_block's shape without its arithmetic.
template <int NV>
__global__ void __launch_bounds__(512)
copy16x2_row_kernel(const u32x4* s1, const u32x4* s2, u32x4* d1, u32x4* d2) {
  const int64_t base = (int64_t)blockIdx.x * 512 * NV + threadIdx.x;
  u32x4 a[NV], b[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    a[k] = ld16_nt(s1 + base + k * 512);
    b[k] = ld16_nt(s2 + base + k * 512);
  }
  // The loaded values are inputs of this empty statement, so the loads have completed before
  // the barrier.
#pragma unroll
  for (int k = 0; k < NV; ++k) __asm__ volatile("" ::"v"(a[k]), "v"(b[k]) : "memory");
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    st16_nt(d1 + base + k * 512, a[k]);
    st16_nt(d2 + base + k * 512, b[k]);
  }
}

hipError_t launch_copy16x2_row(const void* s1, const void* s2, void* d1, void* d2, int64_t n16,
                               int nv, hipStream_t stream) {
  const int64_t unit = 512 * (int64_t)nv;
  if (nv < 1 || n16 % unit) return hipErrorInvalidValue;
  const int64_t blocks = n16 / unit;
  if (blocks > kMaxCopyGrid) return hipErrorInvalidValue;
  const u32x4 *a = (const u32x4*)s1, *b = (const u32x4*)s2;
  u32x4 *c = (u32x4*)d1, *d = (u32x4*)d2;
  switch (nv) {
    case 1: copy16x2_row_kernel<1><<<(unsigned)blocks, 512, 0, stream>>>(a, b, c, d); break;
    case 2: copy16x2_row_kernel<2><<<(unsigned)blocks, 512, 0, stream>>>(a, b, c, d); break;
    case 4: copy16x2_row_kernel<4><<<(unsigned)blocks, 512, 0, stream>>>(a, b, c, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
