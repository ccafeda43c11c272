#include "fattn_launch.h"
namespace fattn {
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const float*,
                           const void*, void*, void*, void*, float*, float*, int, int, int, int,
                           bool, float, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fattn
