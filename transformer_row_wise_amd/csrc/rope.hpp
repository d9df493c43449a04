// Internal interface of the rotary-embedding kernels (NormRope, Rope, and the positions form
// on query and key rows).
#pragma once

#include "launch.hpp"

namespace nrm {

// The kernels see a grid of rows indexed by (bh, l): l in [0, L) selects the position and bh
// in [0, BH) a row at that position. Rows bh < BH1 belong to tensor A (x -> out), the others
// to tensor B (x2 -> out2, row bh - BH1). Row addresses, in rows of D elements:
//   A input  bh * x_sbh  + l * x_sl              B input  b * x2_sbh + l * x2_sl
//   A output bh * o_sbh  + (o_row0 + l) * o_sl   B output b * o2_sbh + l * o2_sl
// [B, H, L, D] (NormRope, Rope): BH = B * H, x_sbh = L, x_sl = 1; the output rows are L or
// a cache of cache_len rows per (b, h) starting at o_row0 = offset.
// [T, H, D] query and key rows with a positions array: L = T, x_sbh = 1, x_sl = H.
struct RopeArgs {
  const void* x;
  const void* w;          // NormRope scale, or null (= 1); unused without normalisation
  void* out;
  const void* x2;         // second tensor, or null (BH1 == BH)
  void* out2;
  int64_t BH;             // rows per position (both tensors)
  int64_t BH1;            // rows per position of tensor A
  int64_t L;              // positions
  int64_t x_sbh, x_sl, o_sbh, o_sl, o_row0;
  int64_t x2_sbh, x2_sl, o2_sbh, o2_sl;
  int D;
  int dims;
  int normalize;
  float eps;
  int traditional;
  float base;
  float scale;
  int64_t offset;         // position of l = 0 when there is no positions array
  int forward;
  const float* freqs;     // [dims / 2] divisors of the position (theta_i = 1 / freqs[i]), or null
  const void* positions;  // [L] int32 or int64 positions, or null (position = offset + l)
  int pos_i64;
  float mscale;           // factor on the rotated features
  int w_f32;
  int iters;              // filled in by the launcher
  int pb;                 // positions per block of the multi-position kernel, by the launcher
  double log2_base;       // log2(base), filled in by the launcher
};

template <bool BF16>
hipError_t launch_norm_rope(const RopeArgs& a, bool aligned16, hipStream_t stream);

}  // namespace nrm
