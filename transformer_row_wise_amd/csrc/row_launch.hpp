// Kernel-shape choice and launch of the row kernels (RMSNorm, add-RMSNorm, LayerNorm).
//
// For a row of n = hidden / VEC 16-byte chunks (VEC = 8 bf16 or 4 fp32):
//   n <= 64 * NV      one wave per row, NV chunks per lane (hidden <= 8192 for bf16 and fp32)
//   n <= 512 * NV     one 512-thread block per row (hidden <= 65536 bf16 / 32768 fp32)
//   otherwise, or when hidden or a base address is not 16-byte granular: the looping
//   kernel (16-byte chunks, or single elements).
// NV is rounded up to the next instantiated size; lanes whose chunk index passes the row
// end skip it. Each op instantiates this in its own translation unit.
#pragma once

#include "launch.hpp"

namespace nrm {

namespace {

constexpr int64_t kMaxGrid = 0x7fffffff;

template <bool BF16, int OP, int NV>
hipError_t go_wave(const RowArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 3) / 4;
  row_regs<BF16, OP, NV, 1><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int NV>
hipError_t go_block(const RowArgs& a, hipStream_t stream) {
  row_regs<BF16, OP, NV, 8><<<(unsigned)a.rows, 512, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int V>
hipError_t go_chunked(const RowArgs& a, hipStream_t stream) {
  const int64_t blocks = a.rows < 1048576 ? a.rows : 1048576;
  row_chunked<BF16, OP, V><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

// One wave per row: chunks per lane needed -> instantiated NV (0: does not fit).
template <bool BF16, int OP>
hipError_t try_wave(const RowArgs& a, int per_lane, hipStream_t stream, bool* done) {
  *done = true;
  if constexpr (BF16) {  // hidden <= 8192
    switch (per_lane) {
      case 1: return go_wave<BF16, OP, 1>(a, stream);
      case 2: return go_wave<BF16, OP, 2>(a, stream);
      case 3: case 4: return go_wave<BF16, OP, 4>(a, stream);
      case 5: case 6: return go_wave<BF16, OP, 6>(a, stream);
      case 7: case 8: return go_wave<BF16, OP, 8>(a, stream);
      case 9: case 10: return go_wave<BF16, OP, 10>(a, stream);
      case 11: case 12: return go_wave<BF16, OP, 12>(a, stream);
      case 13: case 14: case 15: case 16: return go_wave<BF16, OP, 16>(a, stream);
      default: break;
    }
  } else {  // hidden <= 8192
    switch (per_lane) {
      case 1: return go_wave<BF16, OP, 1>(a, stream);
      case 2: return go_wave<BF16, OP, 2>(a, stream);
      case 3: case 4: return go_wave<BF16, OP, 4>(a, stream);
      case 5: case 6: case 7: case 8: return go_wave<BF16, OP, 8>(a, stream);
      case 9: case 10: case 11: case 12: return go_wave<BF16, OP, 12>(a, stream);
      case 13: case 14: case 15: case 16: return go_wave<BF16, OP, 16>(a, stream);
      case 17: case 18: case 19: case 20: return go_wave<BF16, OP, 20>(a, stream);
      case 21: case 22: case 23: case 24: return go_wave<BF16, OP, 24>(a, stream);
      default:
        if (per_lane <= 32) return go_wave<BF16, OP, 32>(a, stream);
        break;
    }
  }
  *done = false;
  return hipSuccess;
}

template <bool BF16, int OP>
hipError_t try_block(const RowArgs& a, int per_thread, hipStream_t stream, bool* done) {
  *done = true;
  switch (per_thread) {
    case 1: return go_block<BF16, OP, 1>(a, stream);
    case 2: return go_block<BF16, OP, 2>(a, stream);
    case 3: case 4: return go_block<BF16, OP, 4>(a, stream);
    case 5: case 6: case 7: case 8: return go_block<BF16, OP, 8>(a, stream);
    default:
      if (per_thread <= 16) return go_block<BF16, OP, 16>(a, stream);
      break;
  }
  *done = false;
  return hipSuccess;
}

}  // namespace

template <bool BF16, int OP>
hipError_t launch_row(const RowArgs& a, bool aligned16, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  const int path = forced_path();
  const bool vec = aligned16 && a.hidden % V == 0 && path != PATH_SCALAR;
  if (!vec) return go_chunked<BF16, OP, 1>(a, stream);
  const int64_t n = a.hidden / V;
  bool done = false;
  hipError_t err = hipSuccess;
  if (path == PATH_AUTO || path == PATH_WAVE) {
    if ((a.rows + 3) / 4 <= kMaxGrid) {
      err = try_wave<BF16, OP>(a, (int)((n + 63) / 64), stream, &done);
      if (done) return err;
    }
  }
  if (path != PATH_CHUNKED && a.rows <= kMaxGrid) {
    err = try_block<BF16, OP>(a, (int)((n + 511) / 512), stream, &done);
    if (done) return err;
  }
  return go_chunked<BF16, OP, V>(a, stream);
}

}  // namespace nrm
