// Unfused comparator kernels and calibration probes (libge_baselines.so).
//
// The comparators run the epilogue the way the pages describe it before fusion: one kernel per
// operation, each reading its bf16 input(s) from HBM and writing a bf16 (or fp8) result back
// ("Optimising GPU kernels with TileLang", fused-epilogue paragraph; superoptimizer write-up,
// sections 7 and 9; CODA news item, "How CODA works"; cuDNN tutorial, AMAX node).  They are
// plain streaming kernels -- 16-byte vector accesses, grid-stride loops -- so that the unfused
// sequence is measured at its own memory roofline, not handicapped.
//
// The probes measure what this GPU sustains: back-to-back matrix-core instructions on register
// data, and a streaming device copy.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/ge_baselines.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 256 * 16;     // 16 workgroups per CU, grid-stride beyond

__device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t to_bf(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);          // round to nearest even
}
__device__ __forceinline__ uint32_t pack(float a, float b) {
  bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Activations in their textbook forms (GELU: tanh approximation).
__device__ __forceinline__ float act_fn(int act, float t) {
  switch (act) {
    case 1: return fmaxf(t, 0.0f);
    case 2: return 0.5f * t * (1.0f + tanhf(0.7978845608028654f * (t + 0.044715f * t * t * t)));
    case 3: return t / (1.0f + expf(-t));
    default: return t;
  }
}

// Derivatives of the activations above at z.
__device__ __forceinline__ float act_grad_fn(int act, float z) {
  switch (act) {
    case 1: return z > 0.0f ? 1.0f : 0.0f;
    case 2: {
      const float c = 0.7978845608028654f;
      const float th = tanhf(c * (z + 0.044715f * z * z * z));
      return 0.5f * (1.0f + th) + 0.5f * z * (1.0f - th * th) * c * (1.0f + 3.0f * 0.044715f * z * z);
    }
    case 3: {
      const float sg = 1.0f / (1.0f + expf(-z));
      return sg * (1.0f + z * (1.0f - sg));
    }
    default: return 1.0f;
  }
}

int64_t blocks_for(int64_t items) {
  int64_t b = (items + kThreads - 1) / kThreads;
  return b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b);
}

int launched() {
  if (hipGetLastError() != hipSuccess) return 2;
  return 0;
}

// ---- elementwise: OP maps 8 inputs (as fp32) at element index i0 to 8 outputs ----
// Vectors of 8 bf16 cover [0, n - n % 8); the tail is handled element by element.
template <class F>
__global__ __launch_bounds__(kThreads) void map1(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                 int64_t n, F f) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nv; v += stride) {
    const u32x4_t w = *(const u32x4_t*)(x + 8 * v);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack(f(8 * v + 2 * j, lo(w[j])), f(8 * v + 2 * j + 1, hi(w[j])));
    *(u32x4_t*)(y + 8 * v) = o;
  }
  if (blockIdx.x == 0)
    for (int64_t i = 8 * nv + threadIdx.x; i < n; i += kThreads) y[i] = to_bf(f(i, bf(x[i])));
}

template <class F>
__global__ __launch_bounds__(kThreads) void map2(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                 uint16_t* __restrict__ y, int64_t n, F f) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nv; v += stride) {
    const u32x4_t wa = *(const u32x4_t*)(a + 8 * v);
    const u32x4_t wb = *(const u32x4_t*)(b + 8 * v);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack(f(lo(wa[j]), lo(wb[j])), f(hi(wa[j]), hi(wb[j])));
    *(u32x4_t*)(y + 8 * v) = o;
  }
  if (blockIdx.x == 0)
    for (int64_t i = 8 * nv + threadIdx.x; i < n; i += kThreads) y[i] = to_bf(f(bf(a[i]), bf(b[i])));
}

struct Scale {
  float alpha;
  __device__ float operator()(int64_t, float v) const { return alpha * v; }
};
struct Act {
  int act;
  __device__ float operator()(int64_t, float v) const { return act_fn(act, v); }
};
struct ActMul {
  int act;
  __device__ float operator()(float g, float u) const { return act_fn(act, g) * u; }
};
struct ActGrad {
  int act;
  __device__ float operator()(float x, float z) const { return x * act_grad_fn(act, z); }
};
struct Add {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// ---- row / column broadcasts: rows x cols with cols % 8 == 0, so a vector stays in one row ----
// (vector indices and column counts fit 32 bits; the host checks).
__global__ __launch_bounds__(kThreads) void bias_col_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, uint32_t nv, uint32_t cv) {
  for (uint32_t v = blockIdx.x * kThreads + threadIdx.x; v < nv; v += gridDim.x * kThreads) {
    const uint32_t c = v % cv;
    const u32x4_t w = *(const u32x4_t*)(x + 8 * (int64_t)v);
    const u32x4_t b = *(const u32x4_t*)(bias + 8 * (int64_t)c);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack(lo(w[j]) + lo(b[j]), hi(w[j]) + hi(b[j]));
    *(u32x4_t*)(y + 8 * (int64_t)v) = o;
  }
}

__global__ __launch_bounds__(kThreads) void row_scale_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ s,
                                                             uint16_t* __restrict__ y, uint32_t nv, uint32_t cv) {
  for (uint32_t v = blockIdx.x * kThreads + threadIdx.x; v < nv; v += gridDim.x * kThreads) {
    const float r = s[v / cv];
    const u32x4_t w = *(const u32x4_t*)(x + 8 * (int64_t)v);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack(lo(w[j]) * r, hi(w[j]) * r);
    *(u32x4_t*)(y + 8 * (int64_t)v) = o;
  }
}

// ---- column sums: one thread per column, rows added in order ----
__global__ __launch_bounds__(kThreads) void col_sum_kernel(const uint16_t* __restrict__ x, float* __restrict__ out,
                                                           int64_t rows, int64_t cols) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= cols) return;
  float acc = 0.0f;
  for (int64_t r = 0; r < rows; ++r) acc += bf(x[r * cols + c]);
  out[c] = acc;
}

// ---- row statistic: one workgroup per row ----
__global__ __launch_bounds__(kThreads) void row_rms_kernel(const uint16_t* __restrict__ x, float* __restrict__ s,
                                                           int64_t cols, float eps) {
  __shared__ float part[kThreads / 64];
  const uint16_t* row = x + (int64_t)blockIdx.x * cols;
  float acc = 0.0f;
  const int64_t nv = (cols % 8 == 0) ? cols / 8 : 0;
  for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
    const u32x4_t w = *(const u32x4_t*)(row + 8 * v);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += lo(w[j]) * lo(w[j]) + hi(w[j]) * hi(w[j]);
  }
  for (int64_t i = 8 * nv + threadIdx.x; i < cols; i += kThreads) acc += bf(row[i]) * bf(row[i]);
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < kThreads / 64; ++w) t += part[w];
    s[blockIdx.x] = 1.0f / sqrtf(t / (float)cols + eps);
  }
}

// ---- AMAX: |x| maxima on the fp32 bit patterns, one atomic per workgroup ----
__global__ void zero_u32(uint32_t* p) {
  if (threadIdx.x == 0) *p = 0u;
}

__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                        uint32_t* __restrict__ out) {
  __shared__ uint32_t part[kThreads / 64];
  uint32_t m = 0;
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nv; v += stride) {
    const u32x4_t w = *(const u32x4_t*)(x + 8 * v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = max(m, (w[j] << 16) & 0x7FFF0000u);
      m = max(m, w[j] & 0x7FFF0000u);
    }
  }
  if (blockIdx.x == 0)
    for (int64_t i = 8 * nv + threadIdx.x; i < n; i += kThreads) m = max(m, ((uint32_t)x[i] << 16) & 0x7FFF0000u);
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) m = max(m, part[w]);
    atomicMax(out, max(m, part[0]));
  }
}

// ---- fp8 quantiser ----
__global__ __launch_bounds__(kThreads) void quant_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ y,
                                                         int64_t n, float scale) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto q = [&](float v) { return fminf(fmaxf(v * scale, -448.0f), 448.0f); };
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nv; v += stride) {
    const u32x4_t w = *(const u32x4_t*)(x + 8 * v);
    int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(q(lo(w[0])), q(hi(w[0])), 0, false);
    p0 = __builtin_amdgcn_cvt_pk_fp8_f32(q(lo(w[1])), q(hi(w[1])), p0, true);
    int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(q(lo(w[2])), q(hi(w[2])), 0, false);
    p1 = __builtin_amdgcn_cvt_pk_fp8_f32(q(lo(w[3])), q(hi(w[3])), p1, true);
    *(uint2*)(y + 8 * v) = make_uint2((unsigned)p0, (unsigned)p1);
  }
  if (blockIdx.x == 0)
    for (int64_t i = 8 * nv + threadIdx.x; i < n; i += kThreads) {
      const float v = q(bf(x[i]));
      y[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFF);
    }
}

// ---- probes ----
// Operand values for the matrix-core probe: random bf16 in [-2, 2) from a hash of (thread, set,
// element), so that, as in a GEMM's inner loop, consecutive instructions see unrelated bits.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_probe(float* sink, int iters) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)(((float)(probe_hash(t * 64 + s * 8 + i) & 0xFFFF) - 32768.0f) / 16384.0f);
      b[s][i] = (__bf16)(((float)(probe_hash(t * 64 + 32 + s * 8 + i) & 0xFFFF) - 32768.0f) / 16384.0f);
    }
  f32x16_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
    // chain i takes operand sets (i % 4, i / 4): every instruction's operands differ from the last
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 4], b[i / 4], acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The fp8 form of the same probe: v_mfma_f32_32x32x64_f8f6f4, the instruction of the
// fp8-operand mainloop, on random e4m3 codes (no NaN code; four 32-byte sets per source, 8
// chains: each instruction is 64 cycles, so 8 keep the matrix core fed; operand sets
// (i % 4, (i / 2) % 4), so consecutive instructions differ in at least one source).  The
// 16x16x32 bf16 form lives in probe_mfma16.hip, which needs its own compiler flags.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256) void mfma_probe_f8(float* sink, int iters) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  i32x8_t a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t wa = probe_hash(t * 64 + k * 8 + i), wb = probe_hash(t * 64 + 32 + k * 8 + i);
      // e4m3 NaN is S.1111.111: clear the lowest bit of any byte that would be one
      wa &= ~((((wa & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7);
      wb &= ~((((wb & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7);
      a[k][i] = (int)wa;
      b[k][i] = (int)wb;
    }
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i % 4], b[(i / 2) % 4], acc[i], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One fp8 matrix-core instruction per wave on caller-given register contents: lane l of wave w
// takes 32 bytes of e4m3 codes from src0 and from src1 at byte (64 w + l) * 32 and 16 fp32
// accumulator values from c at float (64 w + l) * 16, runs v_mfma_f32_32x32x64_f8f6f4 (e4m3 for
// both sources, no block scales) and writes the 16 result values to d at the same place.  This
// shows how the instruction sums its 64 products into the accumulator.
__global__ __launch_bounds__(64) void mfma_f8_probe(const i32x8_t* __restrict__ s0, const i32x8_t* __restrict__ s1,
                                                    const f32x16_t* __restrict__ c, f32x16_t* __restrict__ d) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(s0[i], s1[i], c[i], 0, 0, 0, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding (gfx9
// encoding: vmcnt[3:0] and [15:14]; expcnt and lgkmcnt at their maxima, i.e. not waited for).
constexpr int probe_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// L2 -> LDS probe: the mainloops' operand path alone.  Each wave of a 256-thread workgroup
// issues direct global->LDS buffer loads (16 bytes per lane, 1 KB per instruction) from a
// buffer small enough to stay in L2 into the workgroup's 64 KB of LDS, eight per round with
// up to sixteen in flight, and nothing else.  Source offsets stay inside the buffer (the
// resource's extent); LDS destinations stay inside the array.
__global__ __launch_bounds__(256) void lds_load_probe(const unsigned char* __restrict__ src, int src_kb,
                                                      float* __restrict__ sink, int iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char buf[65536];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src), (short)0, src_kb * 1024, 0x00020000);
  uint32_t kb = (uint32_t)(blockIdx.x * 37 + wave * 8) % (uint32_t)src_kb;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t off = ((kb + (uint32_t)t) % (uint32_t)src_kb) * 1024u + (uint32_t)lane * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + (wave * 8 + t) * 2048 + (it & 1) * 1024), 16, off, 0,
          0, 0);
    }
    kb = (kb + 32u) % (uint32_t)src_kb;
    __builtin_amdgcn_s_waitcnt(probe_vmcnt(8));      // the previous round's eight have landed
  }
  __builtin_amdgcn_s_waitcnt(probe_vmcnt(0));
  __syncthreads();
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)buf[threadIdx.x * 4];
}

// LDS read probe: the mainloops' fragment reads alone.  A 512-thread workgroup (two waves per
// SIMD, as in the two-wave instances) holds 96 KB of LDS, so one runs per CU.  Each wave reads
// its own 12 KB with ds_read_b128 (16 bytes per lane, lanes on consecutive 16-byte chunks, so
// no bank conflicts), eight reads of 1 KB per round at a base that moves with the round, and
// folds the words into two registers with byte dot products (two VALU operations per read,
// half of what the SIMDs issue at 256 bytes per clock per CU).  Wave 0 records the shader-clock counter (s_memtime) and the
// constant-rate counter (s_memrealtime) around the loop, barriers on both sides.
__global__ __launch_bounds__(512) void lds_read_probe(uint32_t* __restrict__ sink, uint64_t* __restrict__ clocks,
                                                      int iters) {
  __shared__ __attribute__((aligned(1024))) uint32_t buf[24576];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < 24576; i += 512) buf[i] = probe_hash((uint32_t)i + blockIdx.x * 24576u);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t a0 = 0, a1 = 0;
  // byte offsets: wave * 12288 + lane * 16 + (it % 4) * 1024 + r * 1024 <= wave * 12288 + 12272
  const unsigned char* wbase = (const unsigned char*)buf + wave * 12288 + lane * 16;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");    // every round reads LDS anew (no reuse across rounds)
    const unsigned char* q = wbase + (it & 3) * 1024;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x4_t v = *(const u32x4_t*)(q + r * 1024);
      a0 = __builtin_amdgcn_udot4(v[0], v[1], a0, false);
      a1 = __builtin_amdgcn_udot4(v[2], v[3], a1, false);
    }
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * 512 + tid] = a0 ^ a1;
  if (tid == 0) {
    clocks[2 * (int64_t)blockIdx.x] = t1 - t0;
    clocks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                        int64_t nv) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nv; v += stride) dst[v] = src[v];
}

template <class K, class... Args>
int launch(K kernel, int64_t blocks, hipStream_t s, Args... args) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, args...);
  return launched();
}

}  // namespace

// probe_mfma16.hip: launches the 16x16x32 bf16 form of the matrix-core probe.
void ge_launch_probe_mfma16(float* sink, int workgroups, int iters, hipStream_t stream);

extern "C" {

int ge_unfused_scale(const uint16_t* x, uint16_t* y, int64_t n, float alpha, void* stream) {
  if (n < 0 || (n > 0 && (!x || !y))) return 1;
  if (n == 0) return 0;
  return launch(map1<Scale>, blocks_for(n / 8 + 1), (hipStream_t)stream, x, y, n, Scale{alpha});
}

int ge_unfused_bias_col(const uint16_t* x, const uint16_t* bias, uint16_t* y, int64_t rows, int64_t cols,
                        void* stream) {
  if (rows < 0 || cols < 0 || cols % 8 != 0 || (rows * cols > 0 && (!x || !y || !bias))) return 1;
  const int64_t nv = rows * cols / 8;
  if (nv >= (int64_t)1 << 32) return 1;
  if (nv == 0) return 0;
  return launch(bias_col_kernel, blocks_for(nv), (hipStream_t)stream, x, bias, y, (uint32_t)nv,
                (uint32_t)(cols / 8));
}

int ge_unfused_act(const uint16_t* x, uint16_t* y, int64_t n, int act, void* stream) {
  if (n < 0 || act < 0 || act > 3 || (n > 0 && (!x || !y))) return 1;
  if (n == 0) return 0;
  return launch(map1<Act>, blocks_for(n / 8 + 1), (hipStream_t)stream, x, y, n, Act{act});
}

int ge_unfused_act_mul(const uint16_t* g, const uint16_t* u, uint16_t* y, int64_t n, int act, void* stream) {
  if (n < 0 || act < 0 || act > 3 || (n > 0 && (!g || !u || !y))) return 1;
  if (n == 0) return 0;
  return launch(map2<ActMul>, blocks_for(n / 8 + 1), (hipStream_t)stream, g, u, y, n, ActMul{act});
}

int ge_unfused_row_rms(const uint16_t* x, float* s, int64_t rows, int64_t cols, float eps, void* stream) {
  if (rows < 0 || cols <= 0 || rows > 0x7FFFFFFF || (rows > 0 && (!x || !s))) return 1;
  if (rows == 0) return 0;
  return launch(row_rms_kernel, rows, (hipStream_t)stream, x, s, cols, eps);
}

int ge_unfused_row_scale(const uint16_t* x, const float* s, uint16_t* y, int64_t rows, int64_t cols,
                         void* stream) {
  if (rows < 0 || cols < 0 || cols % 8 != 0 || (rows * cols > 0 && (!x || !y || !s))) return 1;
  const int64_t nv = rows * cols / 8;
  if (nv >= (int64_t)1 << 32) return 1;
  if (nv == 0) return 0;
  return launch(row_scale_kernel, blocks_for(nv), (hipStream_t)stream, x, s, y, (uint32_t)nv,
                (uint32_t)(cols / 8));
}

int ge_unfused_act_grad(const uint16_t* x, const uint16_t* z, uint16_t* y, int64_t n, int act, void* stream) {
  if (n < 0 || act < 0 || act > 3 || (n > 0 && (!x || !z || !y))) return 1;
  if (n == 0) return 0;
  return launch(map2<ActGrad>, blocks_for(n / 8 + 1), (hipStream_t)stream, x, z, y, n, ActGrad{act});
}

int ge_unfused_col_sum(const uint16_t* x, float* out, int64_t rows, int64_t cols, void* stream) {
  if (rows < 0 || cols < 0 || (cols > 0 && !out) || (rows * cols > 0 && !x)) return 1;
  if (cols == 0) return 0;
  return launch(col_sum_kernel, (cols + kThreads - 1) / kThreads, (hipStream_t)stream, x, out, rows, cols);
}

int ge_unfused_add(const uint16_t* x, const uint16_t* r, uint16_t* y, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !r || !y))) return 1;
  if (n == 0) return 0;
  return launch(map2<Add>, blocks_for(n / 8 + 1), (hipStream_t)stream, x, r, y, n, Add{});
}

int ge_unfused_amax(const uint16_t* x, int64_t n, float* amax, void* stream) {
  if (n < 0 || !amax || (n > 0 && !x)) return 1;
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint32_t*)amax);
  if (launched()) return 2;
  if (n == 0) return 0;
  return launch(amax_kernel, blocks_for(n / 8 + 1), (hipStream_t)stream, x, n, (uint32_t*)amax);
}

int ge_unfused_quant_fp8(const uint16_t* x, uint8_t* y, int64_t n, float scale, void* stream) {
  if (n < 0 || (n > 0 && (!x || !y))) return 1;
  if (n == 0) return 0;
  return launch(quant_kernel, blocks_for(n / 8 + 1), (hipStream_t)stream, x, y, n, scale);
}

int ge_probe_mfma(float* sink, int workgroups, int iters, void* stream) {
  if (!sink || workgroups <= 0 || iters < 0) return 1;
  hipLaunchKernelGGL(mfma_probe, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters);
  return launched();
}

int ge_probe_mfma_variant(float* sink, int workgroups, int iters, int variant, void* stream) {
  if (!sink || workgroups <= 0 || iters < 0) return 1;
  if (variant == 0) {
    hipLaunchKernelGGL(mfma_probe, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters);
  } else if (variant == 1) {
    ge_launch_probe_mfma16(sink, workgroups, iters, (hipStream_t)stream);
  } else if (variant == 2) {
    hipLaunchKernelGGL(mfma_probe_f8, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters);
  } else {
    return 1;
  }
  return launched();
}

int ge_probe_mfma_f8(const uint8_t* src0, const uint8_t* src1, const float* c, float* d, int waves, void* stream) {
  if (waves < 0 || (waves > 0 && (!src0 || !src1 || !c || !d))) return 1;
  if ((((uintptr_t)src0) | ((uintptr_t)src1) | ((uintptr_t)c) | ((uintptr_t)d)) & 63u) return 1;
  if (waves == 0) return 0;
  hipLaunchKernelGGL(mfma_f8_probe, dim3((unsigned)waves), dim3(64), 0, (hipStream_t)stream, (const i32x8_t*)src0,
                     (const i32x8_t*)src1, (const f32x16_t*)c, (f32x16_t*)d);
  return launched();
}

int ge_probe_lds_load(const void* src, int src_kb, float* sink, int workgroups, int iters, void* stream) {
  if (!src || !sink || src_kb < 8 || src_kb > (1 << 20) || workgroups <= 0 || iters < 0) return 1;
  hipLaunchKernelGGL(lds_load_probe, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const unsigned char*>(src), src_kb, sink, iters);
  return launched();
}

int ge_probe_lds_read(uint32_t* sink, uint64_t* clocks, int workgroups, int iters, void* stream) {
  if (!sink || !clocks || workgroups <= 0 || iters < 0) return 1;
  hipLaunchKernelGGL(lds_read_probe, dim3((unsigned)workgroups), dim3(512), 0, (hipStream_t)stream, sink, clocks,
                     iters);
  return launched();
}

int ge_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || (bytes > 0 && (!src || !dst))) return 1;
  if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15u) return 1;
  if (bytes == 0) return 0;
  const int64_t nv = bytes / 16;
  return launch(copy_kernel, blocks_for(nv), (hipStream_t)stream, (const u32x4_t*)src, (u32x4_t*)dst, nv);
}

}  // extern "C"
