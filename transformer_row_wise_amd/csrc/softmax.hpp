// Internal interface of the softmax-family kernels.
#pragma once

#include <algorithm>

#include "launch.hpp"

namespace nrm {

enum SmOp : int { SM_SOFTMAX = 0, SM_CAUSAL = 1, SM_LSE = 2, SM_CE = 3, SM_CE_VJP = 4 };

struct SmArgs {
  const void* x;          // [rows, n] scores / logits
  void* out;              // [rows, n] (Softmax, CausalSoftmax, gradient) or [rows] (LogSumExp)
  const void* targets;    // CE: [rows] int32 or int64 target columns
  int tgt_i64;
  const float* g;         // CE gradient: [rows] cotangent of the loss
  float* loss;            // CE: [rows] fp32 loss
  int64_t rows;           // rows (all leading axes)
  int64_t n;              // columns (the last axis), < 2^31
  int64_t causal_R;       // CAUSAL: length of the second-to-last axis (a multiple of causal_rows)
  int64_t causal_rows;    // CAUSAL: rows per block
  int team;               // filled in by the launcher
};

template <bool BF16, int OP>
hipError_t launch_softmax(const SmArgs& a, bool aligned16, hipStream_t stream);

}  // namespace nrm
