// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ge {

// Epilogue flags decided at run time (uniform per launch).
enum : uint32_t {
  F_SCALE = 1u << 0,
  F_ROW_SCALE = 1u << 1,   // caller-supplied fp32 row_scale[batch][M]
  F_ROW_RMS = 1u << 2,     // in-kernel 1/sqrt(mean(A^2)+eps)
  F_BIAS = 1u << 3,
  F_RESIDUAL = 1u << 4,
  F_AMAX = 1u << 5,
  F_B_NK = 1u << 6,      // B and B2 given as [batch][N][K] (K contiguous)
};

enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_SILU = 3 };

// Kernel instances (tile shapes).  Each is MI355X-specific: 4 waves of 64 lanes.
enum TileKind : int {
  TILE_256x256 = 0,      // 2x2 waves, 128x128 per wave
  TILE_256x128_PAIR = 1, // pairwise: two B operands, 2x2 waves, 128x64 x2 accumulators per wave
  TILE_128x128 = 2,      // 2x2 waves, 64x64 per wave
  TILE_64x64 = 3,        // 2x2 waves, 32x32 per wave
  TILE_128x128_PAIR = 4, // pairwise, 2x2 waves, 64x64 x2 per wave
  TILE_KIND_COUNT = 5
};

struct Params {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* B2;
  const uint16_t* bias;
  const float* row_scale;
  const uint16_t* R;
  void* Y;
  uint32_t* amax;          // fp32 AMAX viewed as its bit pattern
  uint32_t* ws;            // AMAX workspace (layout below); counters are zero between runs
  int64_t lda, ldb, ldy, ldr;
  int64_t sa, sb, sy, sr;  // batch strides in elements
  int32_t M, N, K, batch;
  int32_t tiles_m, tiles_n;
  float alpha, qscale, eps;
  uint32_t flags;
};

struct TileInfo {
  int bm, bn, threads, waves;
  bool pair;
  int lds_bytes;
};

TileInfo tile_info(TileKind kind);

// Per-tile instance sets (ge_tile_*.hip).
hipError_t launch_tile_256x256_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x256_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
TileInfo tile_info_256x256();
hipError_t launch_tile_256x128_pair_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128_pair_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
TileInfo tile_info_256x128_pair();
hipError_t launch_tile_128x128_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
TileInfo tile_info_128x128();
hipError_t launch_tile_64x64_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_64x64_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
TileInfo tile_info_64x64();
hipError_t launch_tile_128x128_pair_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_pair_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
TileInfo tile_info_128x128_pair();

// Enqueues the fused kernel.  `act` in Act, `fp8_out` selects the E4M3 writer.
hipError_t launch_fused(TileKind kind, int act, bool fp8_out, const Params& p, hipStream_t stream);

// Enqueues a one-thread kernel that writes 0 to *amax (empty problems only).
hipError_t launch_amax_zero(uint32_t* amax, hipStream_t stream);

// AMAX workspace layout (32-bit words): eight dispatch-group ticket counters and one top
// counter, each on its own 256-byte line, then one partial-maximum slot per workgroup.
constexpr uint32_t kAmaxGroups = 8;
constexpr uint32_t kAmaxCounterStride = 64;
constexpr uint32_t kAmaxSlot0 = 1024;
constexpr uint32_t kAmaxFlatGrid = 64;   // up to this many workgroups take one ticket each on the top counter
inline size_t amax_workspace_bytes(int64_t workgroups) { return 4 * ((size_t)kAmaxSlot0 + (size_t)workgroups); }

}  // namespace ge
