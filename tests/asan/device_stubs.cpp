// Stand-ins for the library's device-side entry points, so that the C-ABI's host code links
// without the kernels for the sanitizer build.  Each reports hipErrorNotSupported; the fuzzer
// never reaches them (without a gfx950 device no plan is created, so nothing is launched).
#include "../../gemm_epilogue_transformer_tiled_amd/csrc/ge_internal.h"

namespace ge {

hipError_t launch_fused(TileKind, int, bool, const Params&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_amax_zero(uint32_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_zero_words(uint32_t*, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  return hipErrorNotSupported;
}

}  // namespace ge
