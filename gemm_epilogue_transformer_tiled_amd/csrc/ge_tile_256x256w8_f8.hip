// Instances of the fused kernel for the 256x256 tile with two waves per SIMD, fp8-e4m3 operands (B
// laid out [N][K]).
#include "ge_kernel_impl.h"

namespace ge {

hipError_t launch_tile_256x256w8_f8(int act, bool fp8_out, const Params& p, hipStream_t stream) {
  return launch_tile_pp8<T256W8>(act, fp8_out, p, stream);
}

}  // namespace ge
