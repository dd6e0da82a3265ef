// Instances of the fused kernel for the 256x256 tile with two waves per SIMD, B laid out [K][N].
#include "ge_kernel_impl.h"

namespace ge {

hipError_t launch_tile_256x256w8_kn(int act, bool fp8_out, const Params& p, hipStream_t stream) {
  return launch_tile_pp<T256W8, false>(act, fp8_out, p, stream);
}

}  // namespace ge
