// The 16x16x32 bf16 form of the matrix-core probe in baselines.hip: the same random bf16
// operand sets (four per source, chain i taking sets (i % 4, i / 4)), 16 independent chains of
// v_mfma_f32_16x16x32_bf16 per wave.  Built with -mllvm -amdgpu-mfma-vgpr-form (build.py): with
// the accumulators in AGPRs the compiler copies every 4-register accumulator between AGPRs on
// each iteration, which would put accumulator moves in the loop and understate the instruction;
// in VGPR form the loop holds the 16 instructions and the loop counter only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_probe16(float* sink, int iters) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)(((float)(probe_hash(t * 64 + s * 8 + i) & 0xFFFF) - 32768.0f) / 16384.0f);
      b[s][i] = (__bf16)(((float)(probe_hash(t * 64 + 32 + s * 8 + i) & 0xFFFF) - 32768.0f) / 16384.0f);
    }
  f32x4_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i % 4], b[i / 4], acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

void ge_launch_probe_mfma16(float* sink, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe16, dim3((unsigned)workgroups), dim3(256), 0, stream, sink, iters);
}
