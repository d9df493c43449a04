// Internal interface between the C-ABI layer (api.hip) and the kernel launchers.
#pragma once

#include "common.hpp"
#include "row_kernels.hpp"

namespace nrm {

// Kernel-shape override for tests, from the environment variable NRM_FORCE_PATH:
// "wave" (one wave per row), "block" (one 512-thread block per row), "rowblock" (one block
// of up to 1024 threads per row, the default shape), "chunked" (looping kernel, 16-byte chunks), "scalar" (looping kernel
// element by element; for NormRope: the generic kernel). Unset or anything else: automatic
// choice. A forced shape that cannot hold the row falls back to the automatic choice.
enum ForcePath : int { PATH_AUTO = 0, PATH_WAVE, PATH_BLOCK, PATH_ROWBLOCK, PATH_CHUNKED, PATH_SCALAR };
int forced_path();
inline bool force_generic_path() { return forced_path() == PATH_SCALAR; }

template <bool BF16, int OP>
hipError_t launch_row(const RowArgs& a, bool aligned16, hipStream_t stream);

hipError_t launch_copy16(const void* src, void* dst, int64_t n16, hipStream_t stream);
hipError_t launch_copy16x2(const void* s1, const void* s2, void* d1, void* d2, int64_t n16,
                           hipStream_t stream);
hipError_t launch_copy16x2_row(const void* s1, const void* s2, void* d1, void* d2, int64_t n16,
                               int nv, hipStream_t stream);

}  // namespace nrm
