// Dispatch of the fused kernel instances (one translation unit per tile shape) and the
// zero-fill kernel for AMAX on empty problems.
#include <hip/hip_runtime.h>

#include "ge_internal.h"

namespace ge {
namespace {

__global__ void zero_words_kernel(uint32_t* p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void amax_zero_kernel(uint32_t* amax) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *amax = 0u;
}

}  // namespace

hipError_t launch_fused(TileKind kind, int act, bool fp8_out, const Params& p, hipStream_t stream) {
  if (two_wave_tile(kind)) {
    if (p.flags & F_IN_FP8)
      return kind == TILE_256x256_2W ? launch_tile_256x256w8_f8(act, fp8_out, p, stream)
                                     : launch_tile_256x128w8_pair_f8(act, fp8_out, p, stream);
    if (p.flags & F_B_NK)
      return kind == TILE_256x256_2W ? launch_tile_256x256w8_nk(act, fp8_out, p, stream)
                                     : launch_tile_256x128w8_pair_nk(act, fp8_out, p, stream);
    return kind == TILE_256x256_2W ? launch_tile_256x256w8_kn(act, fp8_out, p, stream)
                                   : launch_tile_256x128w8_pair_kn(act, fp8_out, p, stream);
  }
  if (p.flags & F_IN_FP8) {
    switch (kind) {
      case TILE_256x256: return launch_tile_256x256_f8(act, fp8_out, p, stream);
      case TILE_256x128_PAIR: return launch_tile_256x128_pair_f8(act, fp8_out, p, stream);
      case TILE_128x128: return launch_tile_128x128_f8(act, fp8_out, p, stream);
      case TILE_64x64: return launch_tile_64x64_f8(act, fp8_out, p, stream);
      case TILE_128x128_PAIR: return launch_tile_128x128_pair_f8(act, fp8_out, p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (kind) {
    case TILE_256x256: return (p.flags & F_B_NK) ? launch_tile_256x256_nk(act, fp8_out, p, stream)
                                     : launch_tile_256x256_kn(act, fp8_out, p, stream);
    case TILE_256x128_PAIR: return (p.flags & F_B_NK) ? launch_tile_256x128_pair_nk(act, fp8_out, p, stream)
                                     : launch_tile_256x128_pair_kn(act, fp8_out, p, stream);
    case TILE_128x128: return (p.flags & F_B_NK) ? launch_tile_128x128_nk(act, fp8_out, p, stream)
                                     : launch_tile_128x128_kn(act, fp8_out, p, stream);
    case TILE_64x64: return (p.flags & F_B_NK) ? launch_tile_64x64_nk(act, fp8_out, p, stream)
                                     : launch_tile_64x64_kn(act, fp8_out, p, stream);
    case TILE_128x128_PAIR: return (p.flags & F_B_NK) ? launch_tile_128x128_pair_nk(act, fp8_out, p, stream)
                                     : launch_tile_128x128_pair_kn(act, fp8_out, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero_words(uint32_t* p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 65535 ? blocks : 65535)), dim3(256), 0, stream, p,
                     count);
  return hipGetLastError();
}

hipError_t launch_amax_zero(uint32_t* amax, hipStream_t stream) {
  hipLaunchKernelGGL(amax_zero_kernel, dim3(1), dim3(64), 0, stream, amax);
  return hipGetLastError();
}

}  // namespace ge
