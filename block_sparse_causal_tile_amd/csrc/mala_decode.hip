// MALA decode kernels (in progress).
#include "mala_common.hpp"

namespace mala {
hipError_t launch_decode(const mala_problem&, const DecodeParams&, hipStream_t, bool* supported) {
  *supported = false;
  return hipSuccess;
}
}  // namespace mala
