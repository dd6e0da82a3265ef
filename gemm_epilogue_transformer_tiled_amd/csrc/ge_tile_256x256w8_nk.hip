// Instances of the fused kernel for the 256x256 tile with two waves per SIMD, B laid out [N][K].
#include "ge_kernel_impl.h"

namespace ge {

hipError_t launch_tile_256x256w8_nk(int act, bool fp8_out, const Params& p, hipStream_t stream) {
  return launch_tile_pp<T256W8, true>(act, fp8_out, p, stream);
}

}  // namespace ge
