// residual add-RMSNorm: kernel instantiations (see row_kernels.hpp and row_launch.hpp).
#include "row_launch.hpp"

namespace nrm {

template hipError_t launch_row<true, OP_ADD_RMS>(const RowArgs&, bool, hipStream_t);
template hipError_t launch_row<false, OP_ADD_RMS>(const RowArgs&, bool, hipStream_t);

}  // namespace nrm
