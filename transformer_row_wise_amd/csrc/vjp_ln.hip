// LayerNorm backward: kernel instantiations (see vjp.hpp and vjp_launch.hpp).
#include "vjp_launch.hpp"

namespace nrm {

template hipError_t launch_vjp<true, VJP_LN>(const VjpArgs&, void*, void*, bool, hipStream_t);
template hipError_t launch_vjp<false, VJP_LN>(const VjpArgs&, void*, void*, bool, hipStream_t);

}  // namespace nrm
