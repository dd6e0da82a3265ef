// Tile shapes of the fused kernel instances: LDS layout and load counts, as compile-time
// constants.  No device code, so host-only builds (the C-ABI's validation, its sanitizer
// build) read the same figures the kernels are compiled with.
#pragma once

#include "ge_internal.h"

namespace ge {

// WAVES_ = 4: one wave per SIMD, 2 x 2 waves over the tile, each wave runs the whole K loop
// with its loads, fragment reads and MFMAs interleaved.  WAVES_ = 8: two waves per SIMD
// (2 x 4 over the tile); the waves 0-3 and 4-7 form two groups, one wave of each on every
// SIMD, that alternate between a memory phase (direct loads, fragment reads) and a matrix
// phase (MFMAs only), so each SIMD's matrix core is fed by one wave while the other waits.
template <int BM_, int BN_, bool PAIR_, int WPE_, int WAVES_ = 4>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool PAIR = PAIR_;
  static constexpr int WPE = WPE_;                   // waves per SIMD the kernel is built for
  static constexpr int WAVES = WAVES_, NT = 64 * WAVES_;
  static constexpr int WGN = WAVES / 2;              // wave grid: 2 x WGN
  static constexpr int WM = BM / 2, WN = BN / WGN;   // per-wave output tile
  static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int NB = PAIR ? 2 : 1;            // B operands
  // Pipeline: K steps of BK = 32.  B tiles ([BK][BN] per operand) go through a ring of
  // NS = 4 LDS stages; A tiles are staged two steps at a time ([BM][64], 128-byte rows, so
  // every fetched cache line is used whole) in two slots.  The tiles of step k+2 are
  // fetched while step k computes.
  static constexpr int BK = 32, NS = 4, PD = 2;
  static constexpr int GROUPS = BK / 16;             // 16-deep MFMA groups per step
  static constexpr int A_ROWB = 128;                 // one A row: 64 K values
  static constexpr int A_CHUNKS = A_ROWB / 16;
  static constexpr int A_SLOT = BM * A_ROWB;         // two steps of A
  static constexpr int B_ROWB = BN * 2;              // bytes per staged B row
  static constexpr int B_CHUNKS = B_ROWB / 16;       // 16-byte chunks per B row
  static constexpr int B_BYTES = BK * B_ROWB;        // one B operand, one step
  static constexpr int B_STAGE = NB * B_BYTES;
  // Epilogue: each wave stages a 32-row block of fp32 rows (WN + 4 floats) in LDS; half of
  // the waves share each A slot, which is sized to hold them.
  static constexpr int EP_LD = WN + 4;
  static constexpr int EP_WAVE_BYTES = 32 * EP_LD * 4;
  static constexpr int EP_PER_SLOT = WAVES / 2;
  static constexpr int A_ALLOC = A_SLOT > EP_PER_SLOT * EP_WAVE_BYTES ? A_SLOT : EP_PER_SLOT * EP_WAVE_BYTES;
  static constexpr int LDS = 2 * A_ALLOC + NS * B_STAGE;
  // Direct global->LDS loads: one instruction moves 1 KB (64 lanes x 16 bytes).
  static constexpr int A_ROWS_PER_LOAD = 1024 / A_ROWB;
  static constexpr int A_LOADS = A_SLOT / 1024 / WAVES;            // per wave per A slot
  static constexpr int B_ROWS_PER_LOAD = 1024 / B_ROWB;
  static constexpr int B_LOADS_PER_OP = BK / B_ROWS_PER_LOAD;     // per operand per step
  static constexpr int B_LOADS = NB * B_LOADS_PER_OP / WAVES;     // per wave per step
  static_assert(WAVES == 4 || WAVES == 8, "one or two waves per SIMD");
  static_assert(BM % 64 == 0 && BN % (32 * WGN) == 0, "tile must split into 2 x WGN waves of 32x32 blocks");
  static_assert(A_LOADS >= 1 && A_SLOT % (1024 * WAVES) == 0, "A loads must divide over the waves");
  static_assert(B_LOADS >= 1 && (NB * B_LOADS_PER_OP) % WAVES == 0, "B loads must divide over the waves");
  static_assert(B_LOADS_PER_OP % B_LOADS == 0 || B_LOADS % B_LOADS_PER_OP == 0, "one operand per load");
  static_assert(A_LOADS + B_LOADS < 64, "vmcnt range");
  static_assert(LDS + 1024 + 64 <= 160 * 1024, "LDS budget of one workgroup");
};

using T256 = Tile<256, 256, false, 1>;
using T256P = Tile<256, 128, true, 1>;
using T128 = Tile<128, 128, false, 2>;
using T64 = Tile<64, 64, false, 2>;
using T128P = Tile<128, 128, true, 1>;
using T256W8 = Tile<256, 256, false, 2, 8>;     // 128 x 64 per wave
using T256PW8 = Tile<256, 128, true, 2, 8>;     // 128 x 32 (x2: gate, up) per wave

template <class T>
constexpr TileInfo info_of() {
  return TileInfo{T::BM, T::BN, T::NT, T::WAVES, T::PAIR, T::LDS};
}

}  // namespace ge
