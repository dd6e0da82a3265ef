// Fused bf16 GEMM + register-resident epilogue for MI355X (gfx950, CDNA4).
//
// What is computed (pages as titled): the tiled GEMM whose output tile stays in
// register fragments while the epilogue runs, then one store ("Optimising GPU
// kernels with TileLang", tiled-matmul and fused-epilogue paragraphs;
// superoptimizer write-up, section 8); the epilogue primitives of the CODA news
// item ("How CODA works"): scale, per-row scale, column bias, activation or the
// pairwise SwiGLU gate (superoptimizer write-up, section 7), residual
// accumulation, the AMAX reduction of the cuDNN tutorial's batched-matmul
// paragraph, and bf16 / OCP fp8-e4m3 writers.  The RMS row statistic of the
// superoptimizer write-up's section 9 is gathered from the A operand while it
// is staged, so no separate scale kernel or round trip of S is needed.
//
// Mainloop design (per workgroup of 4 waves):
//   * A tile [BM x 64] and B tile [64 x BN] (two B tiles when pairwise) per K
//     step, loaded from HBM with 16-byte buffer loads.  Out-of-range rows,
//     columns and K chunks are given an offset past the buffer extent, so the
//     hardware returns zeros (and drops stores) -- ragged tails need no branches.
//   * B is row-major [K, N] (N contiguous), but the matrix core wants K packed
//     inside each lane's registers for both operands.  Each thread loads an
//     8(k) x 8(n) block of B and transposes it in registers with byte permutes,
//     so LDS holds B as [n][k] exactly like A's [m][k].
//   * LDS rows are 128 bytes (64 bf16 of K); the eight 16-byte chunks of row r
//     are XOR-swizzled by (r ^ r>>3) & 7 so fragment reads and transposed
//     writes hit distinct banks.  Two LDS stages: the next tile is fetched into
//     registers while the matrix cores work on the current stage, then written
//     to the other stage; one barrier per K step.
//   * v_mfma_f32_32x32x16_bf16 with the operands swapped (B fragment as the
//     first source) so that each lane's accumulators hold four consecutive
//     output columns of one output row: the epilogue then loads bias/residual
//     and stores Y with 8-byte (bf16) or 4-byte (fp8) vector accesses.
//   * Workgroup ids are remapped so each XCD (own L2) receives a contiguous run
//     of tiles, which are then walked in groups of 8 tile-rows for L2 reuse.
#include "ge_internal.h"

namespace ge {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;                   // K depth of one LDS stage
constexpr int kRowBytes = kBK * 2;        // one staged row: 128 bytes
constexpr uint32_t kOOB = 0x80000000u;    // offset past every buffer extent
constexpr int kXCDs = 8;                  // MI355X: 8 accelerator dies, each with its own L2
constexpr int kGroupM = 8;                // tile-rows walked together for L2 reuse
constexpr float kLog2e = 1.4426950408889634f;
// GELU tanh form as t * sigmoid(2u), u = sqrt(2/pi) (t + 0.044715 t^3):
// sigmoid(2u) = 1 / (1 + 2^(-2 log2(e) u)).
constexpr float kGeluC = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;

template <int BM_, int BN_, bool PAIR_, int WPE_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool PAIR = PAIR_;
  static constexpr int WPE = WPE_;                   // waves per SIMD the kernel is built for
  static constexpr int WAVES = 4, NT = 256;          // 2 x 2 waves
  static constexpr int WM = BM / 2, WN = BN / 2;     // per-wave output tile
  static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int NB = PAIR ? 2 : 1;            // B operands
  static constexpr int A_CHUNKS = BM * 8 / NT;       // 16-byte chunks of A per thread per stage
  static constexpr int B_UNITS_TOTAL = BN * NB;      // 8x8 transpose units per stage
  static constexpr int B_UNITS = (B_UNITS_TOTAL + NT - 1) / NT;
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 2x2 waves of 32x32 blocks");
  static_assert(A_CHUNKS >= 1 && BM * 8 % NT == 0, "A staging must divide evenly");
};

using T256 = Tile<256, 256, false, 1>;
using T256P = Tile<256, 128, true, 1>;
using T128 = Tile<128, 128, false, 2>;
using T64 = Tile<64, 64, false, 2>;
using T128P = Tile<128, 128, true, 1>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // raw buffer: stride 0, num_records = extent in bytes (< 2^31, checked on the host)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row ^ (row >> 3)) & 7u; }

__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t h = {(__bf16)a, (__bf16)b};   // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <int ACT>
__device__ __forceinline__ float activate(float t) {
  if constexpr (ACT == ACT_RELU) {
    return fmaxf(t, 0.0f);
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float e = __builtin_amdgcn_exp2f(kGeluC * (t + kGeluCubic * t * t * t));
    return t * __builtin_amdgcn_rcpf(1.0f + e);
  } else if constexpr (ACT == ACT_SILU) {
    const float e = __builtin_amdgcn_exp2f(-kLog2e * t);
    return t * __builtin_amdgcn_rcpf(1.0f + e);
  } else {
    return t;
  }
}

// Workgroup id -> (batch, tile row, tile column).
__device__ __forceinline__ void tile_coords(int wg, const Params& p, int& b, int& tm, int& tn) {
  const int per_batch = p.tiles_m * p.tiles_n;
  const int total = per_batch * p.batch;
  // XCD-aware remap: hardware deals consecutive ids round-robin over the 8 XCDs;
  // give each XCD a contiguous run of tiles instead.
  const int xcd = wg % kXCDs, local = wg / kXCDs;
  const int per_xcd = (total + kXCDs - 1) / kXCDs;
  int tall = total % kXCDs;
  if (tall == 0) tall = kXCDs;
  const int id = xcd < tall ? xcd * per_xcd + local
                            : tall * per_xcd + (xcd - tall) * (per_xcd - 1) + local;
  b = id / per_batch;
  const int r = id - b * per_batch;
  const int group_span = kGroupM * p.tiles_n;
  const int g = r / group_span;
  const int first_m = g * kGroupM;
  const int gsize = min(p.tiles_m - first_m, kGroupM);
  const int in_g = r - g * group_span;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

template <class T, int ACT, bool FP8, bool ROWSTAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(T::WPE, T::WPE)))
void fused_gemm_epilogue(Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];
  __shared__ float row_ss[ROWSTAT ? T::BM : 1];
  __shared__ uint32_t wave_amax[T::WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave & 1, wave_n = wave >> 1;

  int b, tm, tn;
  tile_coords(blockIdx.x, p, b, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- buffer resources (extent = last byte this tile may touch, so a bad offset reads 0) ----
  const uint16_t* a_base = p.A + b * p.sa + (int64_t)m0 * p.lda;
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(a_base, ((int64_t)(M - 1 - m0) * p.lda + K) * 2);
  const uint16_t* b_base = p.B + b * p.sb + n0;
  const int64_t b_ext = K > 0 ? ((int64_t)(K - 1) * p.ldb + (N - n0)) * 2 : 0;
  const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(b_base, b_ext);
  __amdgpu_buffer_rsrc_t b2_rs = b_rs;
  if constexpr (T::PAIR) b2_rs = make_rsrc(p.B2 + b * p.sb + n0, b_ext);

  // ---- per-thread staging assignment ----
  // A: chunk q = tid + i*NT -> row q/8, 16-byte K-chunk q%8
  // B: unit u = tid + i*NT -> operand u/BN, column block (u%BN)%(BN/8), K group (u%BN)/(BN/8)
  u32x4_t a_stage[T::A_CHUNKS];
  u32x4_t b_stage[T::B_UNITS][8];
  float ss_part[ROWSTAT ? T::A_CHUNKS : 1];
  if constexpr (ROWSTAT) {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) ss_part[i] = 0.0f;
  }

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) {
      const int q = tid + i * T::NT;
      const int r = q >> 3, c = q & 7;
      const bool ok = (m0 + r < M) && (k0 + c * 8 < K);
      const uint32_t off = ok ? (uint32_t)(((int64_t)r * p.lda + k0 + c * 8) * 2) : kOOB;
      a_stage[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T::B_UNITS; ++i) {
      const int u = tid + i * T::NT;
      if (T::B_UNITS_TOTAL % T::NT == 0 || u < T::B_UNITS_TOTAL) {
        const int op = u / T::BN, uu = u % T::BN;
        const int nb = uu % (T::BN / 8), kg = uu / (T::BN / 8);
        const bool col_ok = n0 + nb * 8 < N;
        const __amdgpu_buffer_rsrc_t rs = (T::PAIR && op == 1) ? b2_rs : b_rs;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + kg * 8 + j;
          const bool ok = col_ok && k < K;
          const uint32_t off = ok ? (uint32_t)(((int64_t)k * p.ldb + nb * 8) * 2) : kOOB;
          b_stage[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
      }
    }
  };

  auto store_stage = [&](unsigned char* stage) {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) {
      const int q = tid + i * T::NT;
      const int r = q >> 3, c = q & 7;
      *(u32x4_t*)(stage + lds_off(r, c)) = a_stage[i];
      if constexpr (ROWSTAT) {
        float s = ss_part[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(a_stage[i][w]), hi = bf16_hi(a_stage[i][w]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        }
        ss_part[i] = s;
      }
    }
#pragma unroll
    for (int i = 0; i < T::B_UNITS; ++i) {
      const int u = tid + i * T::NT;
      if (T::B_UNITS_TOTAL % T::NT == 0 || u < T::B_UNITS_TOTAL) {
        const int op = u / T::BN, uu = u % T::BN;
        const int nb = uu % (T::BN / 8), kg = uu / (T::BN / 8);
        unsigned char* bs = stage + T::A_BYTES + op * T::B_BYTES;
        // 8x8 bf16 transpose: out[c] = column n = nb*8+c, K = kg*8 .. kg*8+7
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t o;
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            o[pr] = __builtin_amdgcn_perm(b_stage[i][2 * pr + 1][c >> 1], b_stage[i][2 * pr][c >> 1], sel);
          }
          *(u32x4_t*)(bs + lds_off(nb * 8 + c, kg)) = o;
        }
      }
    }
  };

  f32x16_t acc[T::FN][T::FM];
  f32x16_t acc2[T::PAIR ? T::FN : 1][T::PAIR ? T::FM : 1];
#pragma unroll
  for (int i = 0; i < T::FN; ++i)
#pragma unroll
    for (int j = 0; j < T::FM; ++j) {
      acc[i][j] = f32x16_t{};
      if constexpr (T::PAIR) acc2[i][j] = f32x16_t{};
    }

  const int nk = (K + kBK - 1) / kBK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wm0 = wave_m * T::WM, wn0 = wave_n * T::WN;

  if (nk > 0) {
    load_stage(0);
    store_stage(smem);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    unsigned char* cur = smem + (kt & 1) * T::STAGE;
    const bool more = kt + 1 < nk;
    if (more) load_stage((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = 2 * ks + lhalf;
      bf16x8_t af[T::FM], bfr[T::FN], bfr2[T::PAIR ? T::FN : 1];
#pragma unroll
      for (int j = 0; j < T::FM; ++j)
        af[j] = *(const bf16x8_t*)(cur + lds_off(wm0 + 32 * j + lrow, chunk));
#pragma unroll
      for (int i = 0; i < T::FN; ++i) {
        bfr[i] = *(const bf16x8_t*)(cur + T::A_BYTES + lds_off(wn0 + 32 * i + lrow, chunk));
        if constexpr (T::PAIR)
          bfr2[i] = *(const bf16x8_t*)(cur + T::A_BYTES + T::B_BYTES + lds_off(wn0 + 32 * i + lrow, chunk));
      }
#pragma unroll
      for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[i], af[j], acc[i][j], 0, 0, 0);
          if constexpr (T::PAIR)
            acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr2[i], af[j], acc2[i][j], 0, 0, 0);
        }
    }
    if (more) store_stage(smem + ((kt + 1) & 1) * T::STAGE);
    __syncthreads();
  }

  // ---- RMS row statistic: reduce the 8 lanes that share a row, park it in LDS ----
  if constexpr (ROWSTAT) {
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) {
      float s = ss_part[i];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      const int q = tid + i * T::NT;
      if ((q & 7) == 0) row_ss[q >> 3] = s;
    }
    __syncthreads();
  }

  // ---- epilogue on the register tile ----
  const uint32_t flags = p.flags;
  const float alpha = (flags & F_SCALE) ? p.alpha : 1.0f;
  const float inv_k = K > 0 ? 1.0f / (float)K : 0.0f;

  // bias for this lane's columns: n = wn0 + 32i + 8g + 4*lhalf + e
  float bias_v[T::FN][4][4];
  if (flags & F_BIAS) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bias + n0, (int64_t)(N - n0) * 2);
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn0 + 32 * i + 8 * g + 4 * lhalf;
        const uint32_t off = (n0 + nl < N) ? (uint32_t)(nl * 2) : kOOB;
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
        bias_v[i][g][0] = bf16_lo(w[0]);
        bias_v[i][g][1] = bf16_hi(w[0]);
        bias_v[i][g][2] = bf16_lo(w[1]);
        bias_v[i][g][3] = bf16_hi(w[1]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias_v[i][g][e] = 0.0f;
  }

  const int esize = FP8 ? 1 : 2;
  void* y_base = (unsigned char*)p.Y + (b * p.sy + (int64_t)m0 * p.ldy + n0) * esize;
  const __amdgpu_buffer_rsrc_t y_rs =
      make_rsrc(y_base, ((int64_t)(M - 1 - m0) * p.ldy + (N - n0)) * esize);
  __amdgpu_buffer_rsrc_t r_rs = y_rs;
  if (flags & F_RESIDUAL)
    r_rs = make_rsrc(p.R + b * p.sr + (int64_t)m0 * p.ldr + n0, ((int64_t)(M - 1 - m0) * p.ldr + (N - n0)) * 2);

  uint32_t amax_bits = 0;
#pragma unroll
  for (int j = 0; j < T::FM; ++j) {
    const int ml = wm0 + 32 * j + lrow;
    const bool m_ok = m0 + ml < M;
    float rscale = alpha;
    if constexpr (ROWSTAT) {
      if (flags & F_ROW_RMS) rscale *= __builtin_amdgcn_rsqf(row_ss[ml] * inv_k + p.eps);
    }
    if (flags & F_ROW_SCALE) rscale *= m_ok ? p.row_scale[(int64_t)b * M + m0 + ml] : 0.0f;
#pragma unroll
    for (int i = 0; i < T::FN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn0 + 32 * i + 8 * g + 4 * lhalf;
        const bool ok = m_ok && (n0 + nl < N);
        float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (flags & F_RESIDUAL) {
          const uint32_t roff = ok ? (uint32_t)(((int64_t)ml * p.ldr + nl) * 2) : kOOB;
          const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r_rs, roff, 0, 0);
          res[0] = bf16_lo(w[0]);
          res[1] = bf16_hi(w[0]);
          res[2] = bf16_lo(w[1]);
          res[3] = bf16_hi(w[1]);
        }
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float t = acc[i][j][4 * g + e] * rscale + bias_v[i][g][e];
          if constexpr (T::PAIR) {
            const float up = acc2[i][j][4 * g + e] * rscale;
            y[e] = activate<ACT>(t) * up;
          } else {
            y[e] = activate<ACT>(t);
          }
          y[e] += res[e];
          const uint32_t mag = __float_as_uint(y[e]) & 0x7FFFFFFFu;
          amax_bits = (ok && mag > amax_bits) ? mag : amax_bits;
        }
        const uint32_t yoff = ok ? (uint32_t)(((int64_t)ml * p.ldy + nl) * esize) : kOOB;
        if constexpr (FP8) {
          const float qs = p.qscale;
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = fminf(fmaxf(y[e] * qs, -448.0f), 448.0f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], w, true);
          __builtin_amdgcn_raw_buffer_store_b32((unsigned)w, y_rs, yoff, 0, 0);
        } else {
          u32x2_t w;
          w[0] = pack_bf16x2(y[0], y[1]);
          w[1] = pack_bf16x2(y[2], y[3]);
          __builtin_amdgcn_raw_buffer_store_b64(w, y_rs, yoff, 0, 0);
        }
      }
    }
  }

  // ---- AMAX: wave max on the |y| bit patterns (integer max keeps NaN), one atomic per
  // workgroup into the workspace slot; the last workgroup to finish publishes the result
  // and leaves the workspace zeroed for the next run.  Non-negative floats order like
  // their bit patterns, so unsigned max is float max.
  if (flags & F_AMAX) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)amax_bits, off);
      amax_bits = o > amax_bits ? o : amax_bits;
    }
    if (lane == 0) wave_amax[wave] = amax_bits;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = wave_amax[0];
#pragma unroll
      for (int w = 1; w < T::WAVES; ++w) m = wave_amax[w] > m ? wave_amax[w] : m;
      __hip_atomic_fetch_max(&p.ws[0], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t total = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n * (uint32_t)p.batch;
      const uint32_t ticket = __hip_atomic_fetch_add(&p.ws[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (ticket == total - 1) {
        const uint32_t v = __hip_atomic_load(&p.ws[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.amax, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.ws[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.ws[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__global__ void amax_zero_kernel(uint32_t* amax) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *amax = 0u;
}

template <class T>
constexpr TileInfo info_of() {
  return TileInfo{T::BM, T::BN, T::NT, T::WAVES, T::PAIR, T::LDS};
}

template <class T, int ACT, bool FP8>
hipError_t launch_t(const Params& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  if (grid <= 0) return hipSuccess;
  if (p.flags & F_ROW_RMS)
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, FP8, true>), dim3((unsigned)grid), dim3(T::NT), 0, s, p);
  else
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, FP8, false>), dim3((unsigned)grid), dim3(T::NT), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_tile(int act, bool fp8, const Params& p, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return fp8 ? launch_t<T, ACT_NONE, true>(p, s) : launch_t<T, ACT_NONE, false>(p, s);
    case ACT_RELU: return fp8 ? launch_t<T, ACT_RELU, true>(p, s) : launch_t<T, ACT_RELU, false>(p, s);
    case ACT_GELU_TANH:
      return fp8 ? launch_t<T, ACT_GELU_TANH, true>(p, s) : launch_t<T, ACT_GELU_TANH, false>(p, s);
    case ACT_SILU: return fp8 ? launch_t<T, ACT_SILU, true>(p, s) : launch_t<T, ACT_SILU, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

TileInfo tile_info(TileKind kind) {
  switch (kind) {
    case TILE_256x256: return info_of<T256>();
    case TILE_256x128_PAIR: return info_of<T256P>();
    case TILE_128x128: return info_of<T128>();
    case TILE_64x64: return info_of<T64>();
    case TILE_128x128_PAIR: return info_of<T128P>();
    default: return TileInfo{0, 0, 0, 0, false, 0};
  }
}

hipError_t launch_fused(TileKind kind, int act, bool fp8_out, const Params& p, hipStream_t stream) {
  switch (kind) {
    case TILE_256x256: return launch_tile<T256>(act, fp8_out, p, stream);
    case TILE_256x128_PAIR: return launch_tile<T256P>(act, fp8_out, p, stream);
    case TILE_128x128: return launch_tile<T128>(act, fp8_out, p, stream);
    case TILE_64x64: return launch_tile<T64>(act, fp8_out, p, stream);
    case TILE_128x128_PAIR: return launch_tile<T128P>(act, fp8_out, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_amax_zero(uint32_t* amax, hipStream_t stream) {
  hipLaunchKernelGGL(amax_zero_kernel, dim3(1), dim3(64), 0, stream, amax);
  return hipGetLastError();
}

}  // namespace ge
