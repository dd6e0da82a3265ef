// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Reference build: GE_SERIAL_PIPELINE=1 compiles every instance with a mainloop that overlaps
// nothing (each two-step slot is loaded, waited for and read between two full barriers).  The
// tiles, waves, MFMAs, their operands and their order are those of the pipelined build, so
// its results are bit-identical to it; a difference means a synchronisation mistake in the
// pipelined mainloop.
#ifndef GE_SERIAL_PIPELINE
#define GE_SERIAL_PIPELINE 0
#endif

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
  F_ACT_GRAD = 1u << 7,  // y = t * act'(Z) instead of act(t)
  F_COL_SUM = 1u << 8,   // column sums of y over rows and batches
  F_IN_FP8 = 1u << 9,    // A and B hold fp8-e4m3 codes (B given [N][K])
  F_RS_SHARE = 1u << 10, // two-wave F_ROW_RMS: tiles of one tile row share the row statistic
};

enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_SILU = 3 };

// Kernel instances (tile shapes).  Each is MI355X-specific: 4 or 8 waves of 64 lanes.
enum TileKind : int {
  TILE_256x256 = 0,      // 2x2 waves, 128x128 per wave
  TILE_256x128_PAIR = 1, // pairwise: two B operands, 2x2 waves, 128x64 x2 accumulators per wave
  TILE_128x128 = 2,      // 2x2 waves, 64x64 per wave
  TILE_64x64 = 3,        // 2x2 waves, 32x32 per wave
  TILE_128x128_PAIR = 4, // pairwise, 2x2 waves, 64x64 x2 per wave
  TILE_256x256_2W = 5,   // two waves per SIMD: 2x4 waves, 128x64 per wave
  TILE_256x128_PAIR_2W = 6, // two waves per SIMD, pairwise: 2x4 waves, 128x32 x2 per wave
  TILE_KIND_COUNT = 7
};

// The two-wave instances need K to be a multiple of two steps (64 bf16 or 128 fp8 values).
inline bool two_wave_tile(TileKind k) { return k == TILE_256x256_2W || k == TILE_256x128_PAIR_2W; }

struct Params {
  const uint16_t* A;       // bf16 elements, or fp8 codes (bytes) with F_IN_FP8
  const uint16_t* B;
  const uint16_t* B2;
  const uint16_t* bias;
  const float* row_scale;
  const uint16_t* R;
  void* Y;
  uint32_t* amax;          // fp32 AMAX viewed as its bit pattern
  uint32_t* ws;            // AMAX workspace (layout below); counters are zero between runs
  const uint16_t* Z;       // ACT_GRAD: saved pre-activation, bf16
  float* col_sum;          // COL_SUM output [N]
  uint32_t* cs_ctr;        // COL_SUM ticket counters, one per column tile (stride kColSumCtrStride)
  float* cs_part;          // COL_SUM partials [batch * tiles_m][N]
  uint32_t* rs_ctr;        // F_RS_SHARE: per tile row, a published flag and a ticket counter
                           // (stride kRowStatCtrStride words)
  float* rs_val;           // F_RS_SHARE: per tile row, the published sums of squares [BM]
  int64_t ldz, sz;
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
hipError_t launch_tile_256x128_pair_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128_pair_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_64x64_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_64x64_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_pair_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_pair_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x256w8_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128w8_pair_kn(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x256w8_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128w8_pair_nk(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x256w8_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128w8_pair_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
// fp8-e4m3 operands, B laid out [N][K]
hipError_t launch_tile_256x256_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_256x128_pair_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_64x64_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);
hipError_t launch_tile_128x128_pair_f8(int act, bool fp8_out, const Params& p, hipStream_t stream);

// Enqueues the fused kernel.  `act` in Act, `fp8_out` selects the E4M3 writer.
hipError_t launch_fused(TileKind kind, int act, bool fp8_out, const Params& p, hipStream_t stream);

// Enqueues a one-thread kernel that writes 0 to *amax (empty problems only).
hipError_t launch_amax_zero(uint32_t* amax, hipStream_t stream);

// Enqueues a kernel that writes `count` zero words at p (COL_SUM of an empty problem).
hipError_t launch_zero_words(uint32_t* p, int64_t count, hipStream_t stream);

// AMAX workspace layout (32-bit words): eight dispatch-group ticket counters and one top
// counter, each on its own 256-byte line, then one partial-maximum slot per workgroup.
constexpr uint32_t kAmaxGroups = 8;
constexpr uint32_t kAmaxCounterStride = 64;
constexpr uint32_t kAmaxSlot0 = 1024;
constexpr uint32_t kAmaxFlatGrid = 64;
constexpr uint32_t kColSumCtrStride = 16;   // 64 bytes between column-tile counters
constexpr uint32_t kRowStatCtrStride = 16;  // 64 bytes between tile-row flag/counter pairs
inline size_t round64(size_t w) { return (w + 63) / 64 * 64; }
// Workspace words: [AMAX region][COL_SUM counters][row-statistic flags and counters]
// [COL_SUM partials][row-statistic sums], each region 256-byte aligned and present only when
// the plan uses it.  Everything before the COL_SUM partials is a counter that is zero between
// runs.
struct WsLayout {
  size_t cs_ctr, rs_ctr, cs_part, rs_val;   // word offsets
  size_t counters;                          // words that hold counters (from word 0)
  size_t total;                             // words in all
};
inline WsLayout ws_layout(bool amax, bool colsum, bool rs_share, int64_t workgroups, int64_t tiles_n,
                          int64_t rows, int64_t n, int64_t bm) {
  WsLayout l;
  l.cs_ctr = amax ? round64((size_t)kAmaxSlot0 + (size_t)workgroups) : 0;
  l.rs_ctr = colsum ? round64(l.cs_ctr + (size_t)tiles_n * kColSumCtrStride) : l.cs_ctr;
  l.cs_part = rs_share ? round64(l.rs_ctr + (size_t)rows * kRowStatCtrStride) : l.rs_ctr;
  l.counters = (colsum || rs_share) ? l.cs_part : (amax ? (size_t)kAmaxSlot0 : 0);
  l.rs_val = colsum ? round64(l.cs_part + (size_t)rows * (size_t)n) : l.cs_part;
  if (rs_share)
    l.total = l.rs_val + (size_t)rows * (size_t)bm;
  else if (colsum)
    l.total = l.cs_part + (size_t)rows * (size_t)n;
  else
    l.total = amax ? (size_t)kAmaxSlot0 + (size_t)workgroups : 0;
  return l;
}

// Device address of the static scratch array behind gemm_epilogue_run_noalloc on the current
// device (looked up once per device).
hipError_t noalloc_scratch(void** out);

}  // namespace ge
