// MALA backward kernels (in progress).
#include "mala_common.hpp"

namespace mala {
hipError_t launch_bwd(const mala_problem&, const BwdParams&, hipStream_t, bool* supported) {
  *supported = false;
  return hipSuccess;
}
}  // namespace mala
