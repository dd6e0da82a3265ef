#pragma once
// Fused bf16 GEMM + register-resident epilogue for MI355X (gfx950, CDNA4): kernel templates.
//
// Included by one translation unit per tile shape (ge_tile_*.hip), so the instances compile
// in parallel; ge_kernels.hip holds the dispatch.
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
// Mainloop design (one-wave instances: a workgroup of 4 waves, 2 x 2 over the output tile,
// one wave per SIMD; the two-wave instances below differ in how the waves take turns):
//   * Operands reach LDS with direct global->LDS buffer loads (16 bytes per lane, 1 KB per
//     instruction, no register staging).  Out-of-range rows, columns and K chunks are
//     given an offset past the buffer extent, so the hardware returns zeros -- ragged
//     tails need no branches.
//   * K advances in steps of 32.  A ([M, K], K contiguous) is staged two steps at a time
//     as [BM][64] with 128-byte rows, so every cache line fetched from L2 is used whole
//     and fetched once; B ([K, N], N contiguous) is staged per step as [32][BN], row-major
//     as it sits in memory.  Two A slots and a ring of four B stages let the loads of
//     step k+2 run while step k computes; one barrier per step.
//   * 16-byte chunks are XOR-swizzled within each LDS row so that fragment reads are free
//     of bank conflicts while the direct loads still write whole 1-KB blocks.
//   * A fragments are plain 16-byte LDS reads; B fragments (K packed inside each lane, as
//     the matrix core wants) come from transposing LDS reads (ds_read_b64_tr_b16).
//   * v_mfma_f32_32x32x16_bf16 with the operands swapped (B fragment as the first source)
//     so that each lane's accumulators hold four consecutive output columns of one output
//     row.  The epilogue stages each 32-row block through LDS once so that bias/residual
//     loads and Y stores cover whole rows.
//   * Workgroup ids are remapped so each XCD (own L2) receives a contiguous run of tiles,
//     which are then walked in groups of 8 tile-rows for L2 reuse.
//   * Two-wave instances (8 waves, 2 x 4 over a 256-row tile, two per SIMD): the same LDS
//     stages and slots, but the waves form two groups of four that alternate a memory phase
//     (this step's fragment reads, later steps' loads, waits) and a matrix phase (MFMAs only,
//     at raised priority), one phase apart, so one wave per SIMD keeps the matrix core busy
//     while the other waits on memory; the row statistic comes from the staged A slots, and
//     a tile that starts after another tile of its tile row has published it reads it instead.
//     With bf16 operands they multiply with v_mfma_f32_16x16x32_bf16 (one instruction per
//     16x16 block and 32-deep step: half the accumulator traffic per flop of 32x32x16).
#include <type_traits>
#include <utility>

#include "ge_internal.h"
#include "ge_tiles.h"

namespace ge {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf16_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u;    // offset past every buffer extent
constexpr int kXCDs = 8;                  // MI355X: 8 accelerator dies, each with its own L2
constexpr int kGroupM = 8;                // tile-rows walked together for L2 reuse
// s_waitcnt immediate for "vector memory count 0" with the other counters left free
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kVmcnt0 = vmcnt_imm(0);
// Same, with the LDS counter (lgkmcnt) also drained to zero.
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }
constexpr float kLog2e = 1.4426950408889634f;
// GELU tanh form as t * sigmoid(2u), u = sqrt(2/pi) (t + 0.044715 t^3):
// sigmoid(2u) = 1 / (1 + 2^(-2 log2(e) u)).
constexpr float kGeluC = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;


__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // raw buffer: stride 0, num_records = extent in bytes (< 2^31, checked on the host)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Step resources are built at kernel scope, between the (host-device) step lambdas.

// A rows are 128 bytes (eight 16-byte chunks).  Chunk c of row r lives at chunk
// c ^ swz_a(r).  The swizzle uses only r mod 32, so it is the same for every 32-row MFMA
// block; 16 consecutive rows read at one logical chunk land on distinct banks for both
// 128-byte and 256-byte LDS cycles (even rows take all eight chunks, odd rows too).
__device__ __forceinline__ uint32_t swz_a(uint32_t row) {
  return (row & 7u) ^ ((row >> 3) & 3u);
}

// B rows ([k][n], 2*BN bytes).  Chunk c of row k lives at chunk c ^ swz_b(k).  A
// 16-lane transpose read touches rows k..k+3 (k % 4 == 0) and one pair of chunks;
// the XOR pattern {0, 4, 10, 14} sends those four pairs to four different pairs of
// every aligned group of four (distinct banks for 128-byte LDS cycles) and the two
// 16-lane groups of a half-wave to complementary halves (256-byte cycles).
template <int CHUNKS>
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
  const uint32_t q = k & 3u;
  return ((q << 2) | ((q >> 1) << 1)) & (uint32_t)(CHUNKS - 1);
}
// The same for the 16x16x32 fragments, whose two 16-lane groups of a half-wave read rows
// k..k+3 and k+8..k+11 of the same columns: rows with bit 3 set also flip chunk bit 3, which
// sends the second group's four chunk pairs to the complement of the first group's in every
// aligned group of sixteen chunks (256 bytes).
template <int CHUNKS>
__device__ __forceinline__ uint32_t swz_b16(uint32_t k) {
  return swz_b<CHUNKS>(k) ^ (k & 8u);
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

// Derivative of activate<ACT> at z, for the backward activation-gradient epilogue.  With
// s = sigmoid(2u), u = sqrt(2/pi)(z + 0.044715 z^3): GELU' = s + 2 sqrt(2/pi) z s(1-s)
// (1 + 3*0.044715 z^2); SiLU' = s(1 + z(1-s)) with s = sigmoid(z); ReLU' = [z > 0].
template <int ACT>
__device__ __forceinline__ float activate_grad(float z) {
  if constexpr (ACT == ACT_RELU) {
    return z > 0.0f ? 1.0f : 0.0f;
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kGeluC * (z + kGeluCubic * z * z * z)));
    return s + 2.0f * 0.7978845608028654f * z * s * (1.0f - s) * (1.0f + 3.0f * kGeluCubic * z * z);
  } else if constexpr (ACT == ACT_SILU) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
    return s * (1.0f + z * (1.0f - s));
  } else {
    return 1.0f;
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

// Scheduling recipe for one 16-deep MFMA group of MF instructions: after MFMA m come
// ceil(NL / MF) of the step's NL direct loads (VMEM = 0x010, while any remain) and, for
// m < RD, one of the next group's fragment reads (DS read = 0x100); MFMA = 0x008.
template <int MF, int NL, int RD, int M = 0>
__device__ __forceinline__ void sched_group() {
  if constexpr (M < MF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int per = (NL + MF - 1) / MF;
    constexpr int left = NL - M * per;
    constexpr int n = left < per ? left : per;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x010, n, 0);
    if constexpr (M < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    sched_group<MF, NL, RD, M + 1>();
  }
}

// The same for the fp8 mainloop, whose fragment reads outnumber its MFMAs: after MFMA m come
// ceil(NL / MF) loads and ceil(RD / MF) fragment reads while any remain.
template <int MF, int NL, int RD, int M = 0>
__device__ __forceinline__ void sched_group8() {
  if constexpr (M < MF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int per = (NL + MF - 1) / MF;
    constexpr int left = NL - M * per;
    constexpr int n = left < per ? left : per;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x010, n, 0);
    constexpr int rper = (RD + MF - 1) / MF;
    constexpr int rleft = RD - M * rper;
    constexpr int rn = rleft < rper ? rleft : rper;
    if constexpr (rn > 0) __builtin_amdgcn_sched_group_barrier(0x100, rn, 0);
    sched_group8<MF, NL, RD, M + 1>();
  }
}

// KMASK: K is not a multiple of two steps (64 bf16 or 128 fp8 values), so one A slot straddles
// K and needs per-lane masking.
// BNK: B (and B2) are given as [N][K] (K contiguous) -- for instance W when the product is
// dY @ W^T of a backward pass -- and are staged exactly like A: two steps at a time as
// [BN][64] with 128-byte rows, fragments by plain 16-byte LDS reads.
// GRAD: the activation-gradient epilogue y = t * act'(Z) replaces y = act(t) (non-pairwise).
// F8IN: A and B hold OCP fp8-e4m3 codes (B given [N][K]); the mainloop runs
// v_mfma_f32_32x32x64_f8f6f4, K advancing 64 values (64 bytes) per step, so the same LDS
// slots of 128-byte rows hold two steps and every byte offset is what it is for bf16.  The
// dequantisation factors of delayed scaling (1 / (scale_A * scale_B)) are the epilogue's
// alpha; everything after the accumulator is shared with the bf16 path.
template <class T, int ACT, bool GRAD, bool FP8, bool ROWSTAT, bool KMASK, bool BNK, bool F8IN = false>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::WPE, T::WPE)))
void fused_gemm_epilogue(Params p) {
  constexpr bool PP = T::WAVES == 8;              // two waves per SIMD, alternating phases
  // Two-wave bf16 instances multiply with v_mfma_f32_16x16x32_bf16: half the accumulator bytes
  // per flop of the 32x32x16 form, which under the power limit runs the matrix cores faster
  // (measured +2.5 to +3.7 % on every bf16 workload against the same loop on 32x32x16).
  constexpr bool MF16 = PP && !F8IN;
  static_assert(!PP || !KMASK, "the two-wave instances: K a multiple of two steps");
  constexpr int ES = F8IN ? 1 : 2;                // bytes per operand element
  constexpr int BKE = F8IN ? 64 : T::BK;          // K values per step (64 bytes of a row)
  constexpr uint32_t EPC = 16 / ES;               // K values per 16-byte chunk
  static_assert(!F8IN || (BNK && !ROWSTAT && !GRAD), "fp8 operands: B given [N][K], no row statistic");
  // The LDS stages and slots are distinct arrays, so the compiler can tell that the direct
  // loads filling one never alias the fragment reads of another.
  __shared__ __attribute__((aligned(1024))) unsigned char aslot0[T::A_ALLOC];
  __shared__ __attribute__((aligned(1024))) unsigned char aslot1[T::A_ALLOC];
  // B buffers: [N][K] layout -- two slots of two steps each; [K][N] -- a ring of four stages.
  constexpr int BNK_SLOT = T::NB * T::BN * T::A_ROWB;
  constexpr int B_BUF = BNK ? BNK_SLOT : T::B_STAGE;
  constexpr int B_BUF23 = BNK ? 16 : T::B_STAGE;
  constexpr int BL = BNK ? BNK_SLOT / 1024 / T::WAVES : T::B_LOADS;   // B loads per wave per fill
  static_assert(!BNK || (BL >= 1 && BNK_SLOT % (1024 * T::WAVES) == 0), "B slot loads divide over the waves");
  static_assert(2 * T::A_ALLOC + 2 * B_BUF + 2 * B_BUF23 + 4096 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char bstage0[B_BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char bstage1[B_BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char bstage2[B_BUF23];
  __shared__ __attribute__((aligned(1024))) unsigned char bstage3[B_BUF23];
  __shared__ float row_ss[ROWSTAT ? (PP ? 2 : 1) * T::BM : 1];   // two-wave: one half per wave group
  __shared__ uint32_t wave_amax[T::WAVES];
  __shared__ uint32_t rs_have;                    // row statistic already published for this tile row
  __shared__ __attribute__((aligned(256))) unsigned char pf_sink[T::WAVES * 256];   // L2 prefetch target
  static_assert(T::NS == 4, "four B stage arrays");
  // B buffer of step s ([K][N]: its stage; [N][K]: its slot), A slot of step s (two
  // consecutive steps share a slot).
  auto bstage = [&](auto s_c) -> unsigned char* {
    constexpr int S = decltype(s_c)::value % T::NS;
    if constexpr (BNK) {
      if constexpr (S / 2 == 0) return bstage0;
      else return bstage1;
    } else {
      if constexpr (S == 0) return bstage0;
      else if constexpr (S == 1) return bstage1;
      else if constexpr (S == 2) return bstage2;
      else return bstage3;
    }
  };
  auto aslot = [&](auto s_c) -> unsigned char* {
    constexpr int S = decltype(s_c)::value % T::NS;
    if constexpr (S / 2 == 0) return aslot0;
    else return aslot1;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave & 1, wave_n = wave >> 1;

  int b, tm, tn;
  tile_coords(blockIdx.x, p, b, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- buffer resources (extent = last byte this tile may touch; an offset past it reads 0) ----
  // The K position of a step is carried by the resource: its base moves to column (A) or row
  // (B) k0 and its extent shrinks by the same amount, so per-lane offsets stay fixed for the
  // whole loop (no vector instructions for addressing).  A step entirely outside [0, K) gets
  // an empty resource, which reads zeros.
  const unsigned char* a_base = (const unsigned char*)p.A + (b * p.sa + (int64_t)m0 * p.lda) * ES;
  const int64_t a_ext = ((int64_t)(M - 1 - m0) * p.lda + K) * ES;
  // [K][N]: the tile's columns start at n0; [N][K]: its rows start at n0 (like A's at m0)
  const int64_t b_ofs = BNK ? (int64_t)n0 * p.ldb : (int64_t)n0;
  const unsigned char* b_base = (const unsigned char*)p.B + (b * p.sb + b_ofs) * ES;
  const unsigned char* b2_base = T::PAIR ? (const unsigned char*)p.B2 + (b * p.sb + b_ofs) * ES : b_base;
  const int64_t b_ext = BNK ? ((int64_t)(N - 1 - n0) * p.ldb + K) * ES
                            : (K > 0 ? ((int64_t)(K - 1) * p.ldb + (N - n0)) * 2 : 0);
  __amdgpu_buffer_rsrc_t b_rs0 = make_rsrc(b_base, b_ext), b2_rs0 = b_rs0;   // ragged K, [N][K]
  if constexpr (T::PAIR) b2_rs0 = make_rsrc(b2_base, b_ext);
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(a_base, a_ext);       // ragged K: fixed resource

  // ---- direct global->LDS loads: per-lane source offsets, fixed for the whole K loop ----
  // A load t of this wave fills slot rows 8u .. 8u+7 (1 KB), u = wave * A_LOADS + t:
  // lane -> row 8u + lane/8, physical chunk lane%8, so it fetches logical chunk
  // (lane%8) ^ swz_a(row) = a_x ^ (u & 3), i.e. K columns 8 * that chunk of the slot's 64.
  // Rows past M fall outside the resource extent (lda >= K).  With K a multiple of 64 every
  // slot is wholly inside or outside [0, K); otherwise chunks outside [0, K) get the
  // out-of-range offset, per lane, with k0 added to the offset instead of the resource.
  static_assert(T::A_ROWS_PER_LOAD == 8 && T::A_CHUNKS == 8, "one 128-byte row per 8 lanes");
  const uint32_t lda2 = (uint32_t)p.lda * (uint32_t)ES, ldb2 = (uint32_t)p.ldb * (uint32_t)ES;   // row pitch, bytes
  const uint32_t a_x = (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t a_row = (uint32_t)(lane >> 3) * lda2;
  uint32_t a_voff[T::A_LOADS];
#pragma unroll
  for (int t = 0; t < T::A_LOADS; ++t) {
    const uint32_t u = (uint32_t)(wave * T::A_LOADS + t);
    a_voff[t] = a_row + u * 8u * lda2 + (a_x ^ (u & 3u)) * 16u;
  }
  // B load t fills B_ROWS_PER_LOAD rows of one operand: lane -> row lane/B_CHUNKS (within
  // the load), physical chunk lane%B_CHUNKS, logical chunk ^ swz_b(row).  Rows past K fall
  // outside the extent; a column block past N gets the out-of-range offset.
  // [N][K]: B load t (u = wave * BL + t over the operands) fills slot rows 8r .. 8r+7 of
  // operand u / (BN/8), r = u % (BN/8), with A's lane mapping and swizzle; rows past N fall
  // outside the extent (ldb >= K).
  uint32_t b_voff[BL];
#pragma unroll
  for (int t = 0; t < BL; ++t) {
    if constexpr (BNK) {
      const uint32_t r = (uint32_t)(wave * BL + t) % (uint32_t)(T::BN / 8);
      b_voff[t] = (uint32_t)(lane >> 3) * ldb2 + r * 8u * ldb2 + (a_x ^ (r & 3u)) * 16u;
    } else {
      const int blk = (wave * T::B_LOADS + t) % T::B_LOADS_PER_OP;
      const uint32_t row = (uint32_t)blk * T::B_ROWS_PER_LOAD + (uint32_t)(lane / T::B_CHUNKS);
      const uint32_t lchunk = (uint32_t)(lane % T::B_CHUNKS) ^ (MF16 ? swz_b16<T::B_CHUNKS>(row) : swz_b<T::B_CHUNKS>(row));
      b_voff[t] = (n0 + (int)lchunk * 8 < N) ? row * ldb2 + lchunk * 16u : kOOB;
    }
  }

  // ---- L2 prefetch ----
  // On even steps each wave also issues one 4-byte load per lane for A and for B (or B2) of the
  // slot four steps ahead, one lane per 128-byte line, so those lines wait in the XCD's L2 when
  // the real loads of that slot are issued two steps later.  Only one of the tiles sharing a
  // slice prefetches it (A: tile columns 0 mod 4, B: tile rows 0 mod 8), so the L2 sees each
  // line about once.  The loads go to a dummy LDS area; they complete in order with the others
  // and the barrier waits below let them stay in flight.  Tiles that do not prefetch a slice
  // give the loads out-of-range offsets: they return without a memory access.  (Prefetching
  // every slice from every tile that uses it cost 1.5-6 %; one prefetcher per slice gains up
  // to 8 %: the operand lines otherwise reach L2 only when the real loads ask for them, a
  // fabric round trip of 1.5-2.5 us under load against two steps of prefetch.)
  // Only the one-wave bf16 [N][K] instances prefetch (measured: it pays there, a loss
  // elsewhere; the two-wave loop hides the loads' latency itself, and a prefetch cost it 6-7 %).
  constexpr bool L2PF = BNK && !F8IN && !PP;
  constexpr int PF = L2PF ? 2 : 0;                     // prefetch loads per wave per even step
  const uint32_t pf_a_off = ((tn & 3) == 0 && tid < T::BM) ? (uint32_t)tid * lda2 : kOOB;
  constexpr int PF_T = T::NT / T::NB;                  // threads per operand
  const int pf_t = tid % PF_T;
  const bool pf_b2 = T::PAIR && tid >= PF_T;           // wave-uniform
  uint32_t pf_b_off = kOOB;
  if ((tm & 7) == 0) {
    if constexpr (BNK) {
      pf_b_off = pf_t < T::BN ? (uint32_t)pf_t * ldb2 : kOOB;
    } else {
      constexpr int LPB = T::BN / 64;
      const int row = pf_t / LPB, line = pf_t % LPB;
      pf_b_off = row < 2 * BKE ? (uint32_t)row * ldb2 + (uint32_t)line * 128u : kOOB;
    }
  }

  // Resources of the step starting at K column/row k0 (a multiple of the step, so a B step --
  // and, with K a multiple of two steps, an A slot -- is wholly inside or outside [0, K)): the base is
  // clamped into range and an out-of-range step gets extent 0.  Byte offsets fit 32 bits:
  // every extent is checked below 2^31 on the host.  Scalar, branch-free code.
#define GE_KCLAMP(k0) ((k0) < 0 ? 0 : ((k0) > K ? K : (k0)))
#define GE_KLIVE(k0) (((k0) >= 0) & ((k0) < K))
#define GE_A_RS(k0) \
  make_rsrc(a_base + (uint32_t)GE_KCLAMP(k0) * (uint32_t)ES, GE_KLIVE(k0) ? a_ext - ES * (int64_t)GE_KCLAMP(k0) : 0)
#define GE_B_RS(base, k0) \
  make_rsrc((base) + (uint32_t)GE_KCLAMP(k0) * (BNK ? (uint32_t)ES : ldb2), \
            GE_KLIVE(k0) ? b_ext - (int64_t)((uint32_t)GE_KCLAMP(k0) * (BNK ? (uint32_t)ES : ldb2)) : 0)

  // A slot for steps k0/BK and k0/BK + 1; k0 may be negative (leading all-zero steps).
  // K a multiple of 64: `rs` is the step's resource and the offsets are fixed.  Otherwise the
  // fixed resource a_rs, with k0 in the offset and one unsigned compare per chunk sending
  // every chunk outside [0, K) out of range.
  __amdgpu_buffer_rsrc_t ars = a_rs, brs = a_rs, b2rs = a_rs;      // the step being filled
  auto issue_a = [&](int k0, unsigned char* slot) {
#pragma unroll
    for (int t = 0; t < T::A_LOADS; ++t) {
      uint32_t off = a_voff[t];
      if constexpr (KMASK) {
        const uint32_t u = (uint32_t)(wave * T::A_LOADS + t);          // wave-uniform
        const uint32_t c = a_x ^ (u & 3u);
        off = ((uint32_t)(k0 + (int)(c * EPC)) < (uint32_t)K) ? off + (uint32_t)k0 * (uint32_t)ES : kOOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ars, (__attribute__((address_space(3))) void*)(slot + (wave * T::A_LOADS + t) * 1024), 16, off, 0, 0, 0);
    }
  };
  // B stage of one step from its resources (rows past K fall outside the shrunk extent).
  auto issue_b = [&](unsigned char* st, int k0) {
    if constexpr (BNK) {
#pragma unroll
      for (int t = 0; t < BL; ++t) {
        const uint32_t u = (uint32_t)(wave * BL + t);                  // wave-uniform
        const uint32_t op = u / (uint32_t)(T::BN / 8), r = u % (uint32_t)(T::BN / 8);
        uint32_t off = b_voff[t];
        if constexpr (KMASK) {
          const uint32_t c = a_x ^ (r & 3u);
          off = ((uint32_t)(k0 + (int)(c * EPC)) < (uint32_t)K) ? off + (uint32_t)k0 * (uint32_t)ES : kOOB;
        }
        unsigned char* dst = st + op * (T::BN * T::A_ROWB) + r * 1024;
        if (T::PAIR && op == 1)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b2rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
      }
      return;
    }
    (void)k0;
#pragma unroll
    for (int t = 0; t < T::B_LOADS; ++t) {
      const int gblk = wave * T::B_LOADS + t;           // wave-uniform
      const int op = gblk / T::B_LOADS_PER_OP;
      const int blk = gblk % T::B_LOADS_PER_OP;
      unsigned char* dst = st + op * T::B_BYTES + blk * 1024;
      // (a local copy: a captured array element passed straight to the builtin makes the
      // host pass drop the launch stub)
      const uint32_t off = b_voff[t];
      if (T::PAIR && op == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b2rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    }
  };

  // L2 prefetch of the slot at K position k0 (two steps: 2 * BKE K values)
  auto prefetch_l2 = [&](int k0) {
    if constexpr (!L2PF) return;
    auto* dst = (__attribute__((address_space(3))) void*)(pf_sink + wave * 256);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(GE_A_RS(k0), dst, 4, pf_a_off, 0, 0, 0);
    const unsigned char* bb = pf_b2 ? b2_base : b_base;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(GE_B_RS(bb, k0), dst, 4, pf_b_off, 0, 0, 0);
  };

  // ---- fragment addressing ----
  // A (second MFMA source): for group g of the step in slot half h, lane reads row
  // wm0 + 32j + lane%32, logical chunk 4h + 2g + lane/32 (eight consecutive K); the swizzle
  // depends on lane%32 only, so j is an immediate offset.
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wm0 = wave_m * T::WM, wn0 = wave_n * T::WN;
  uint32_t a_frag[2 * T::GROUPS];
#pragma unroll
  for (int hg = 0; hg < 2 * T::GROUPS; ++hg)
    a_frag[hg] = (uint32_t)(wm0 + lrow) * T::A_ROWB + (((uint32_t)(2 * hg + lhalf) ^ swz_a(lrow)) << 4);
  // B (first MFMA source) through 16-lane transpose reads: in each group of 16 lanes, lane s
  // points at row k0 + s/4 and columns nb + 4(s%4) .. +3, and receives column nb + s of rows
  // k0 .. k0+3.  Two reads (rows +0..3, +4..7) give the eight K values of A's lane layout.
  const int grp = lane >> 4, sl = lane & 15;
  const uint32_t kl = (uint32_t)(8 * (grp >> 1) + (sl >> 2));            // row within the 16-K slice
  uint32_t b_frag[T::NB][T::FN];
#pragma unroll
  for (int op = 0; op < T::NB; ++op)
#pragma unroll
    for (int i = 0; i < T::FN; ++i) {
      const uint32_t ncol = (uint32_t)(wn0 + 32 * i + 16 * (grp & 1) + 4 * (sl & 3));
      const uint32_t lchunk = ncol >> 3;
      b_frag[op][i] = (uint32_t)(op * T::B_BYTES) + kl * T::B_ROWB +
                      ((lchunk ^ swz_b<T::B_CHUNKS>(kl)) << 4) + (ncol & 7u) * 2u;
    }
  // [N][K]: like A -- lane reads slot row wn0 + 32i + lane%32 of operand op, logical chunk
  // 4h + 2g + lane/32; i and op are immediate offsets.
  uint32_t bnk_frag[2 * T::GROUPS];
#pragma unroll
  for (int hg = 0; hg < 2 * T::GROUPS; ++hg)
    bnk_frag[hg] = (uint32_t)(wn0 + lrow) * T::A_ROWB + (((uint32_t)(2 * hg + lhalf) ^ swz_a(lrow)) << 4);

  // 16x16x32 fragments: a lane holds eight consecutive K of one row (A, [N][K] B) or column
  // ([K][N] B): row/column lane % 16 of the block, K 8 * (lane / 16) .. +7 of the step, i.e.
  // logical chunk 4h + lane / 16 of a slot row.  swz_a depends on the row mod 32, so 16-row
  // blocks of even and odd index have a base address each; further 32 rows are immediate
  // offsets.  [K][N] B: in each 16-lane group q, lane s points at rows 8q + s/4 (and + 4) and
  // columns nb + 4(s%4) .. +3, and receives column nb + s.
  constexpr int FN16 = MF16 ? T::WN / 16 : 1, FM16 = MF16 ? T::WM / 16 : 1;
  const uint32_t l16 = (uint32_t)(lane & 15), q16 = (uint32_t)(lane >> 4);
  uint32_t a16[2][2], bnk16[2][2];          // [slot half][16-row block parity]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const uint32_t r = 16u * (uint32_t)par + l16, c = ((4u * (uint32_t)h + q16) ^ swz_a(r)) << 4;
      a16[h][par] = ((uint32_t)wm0 + r) * T::A_ROWB + c;
      bnk16[h][par] = ((uint32_t)wn0 + r) * T::A_ROWB + c;
    }
  uint32_t b16[T::NB][FN16];
#pragma unroll
  for (int op = 0; op < T::NB; ++op)
#pragma unroll
    for (int i = 0; i < FN16; ++i) {
      const uint32_t k16 = 8u * q16 + (l16 >> 2);
      const uint32_t ncol = (uint32_t)(wn0 + 16 * i) + 4u * (l16 & 3u);
      b16[op][i] = (uint32_t)(op * T::B_BYTES) + k16 * T::B_ROWB +
                   (((ncol >> 3) ^ swz_b16<T::B_CHUNKS>(k16)) << 4) + (ncol & 7u) * 2u;
    }

  constexpr int AFN = MF16 ? 1 : T::FN, AFM = MF16 ? 1 : T::FM;
  f32x16_t acc[AFN][AFM];
  f32x16_t acc2[T::PAIR ? AFN : 1][T::PAIR ? AFM : 1];
#pragma unroll
  for (int i = 0; i < AFN; ++i)
#pragma unroll
    for (int j = 0; j < AFM; ++j) {
      acc[i][j] = f32x16_t{};
      if constexpr (T::PAIR) acc2[i][j] = f32x16_t{};
    }
  // 16x16x32 accumulators: block (i, j) of the wave's tile, lane holds row 16j + lane % 16,
  // columns 16i + 4 (lane / 16) .. +3
  f32x4_t c16[FN16][FM16];
  f32x4_t c16b[T::PAIR ? FN16 : 1][T::PAIR ? FM16 : 1];
#pragma unroll
  for (int i = 0; i < FN16; ++i)
#pragma unroll
    for (int j = 0; j < FM16; ++j) {
      c16[i][j] = f32x4_t{};
      if constexpr (T::PAIR) c16b[i][j] = f32x4_t{};
    }
  // RMS statistic from the A fragments (one-wave instances): waves with wave_n == 0 own the
  // first half of the wave's 32-row blocks, wave_n == 1 the second half (all of them when
  // FM == 1 and wave_n == 0).  The two-wave instances take it from the A slots instead.
  constexpr int SS_J = T::FM > 1 ? T::FM / 2 : 1;
  float ss[SS_J];
#pragma unroll
  for (int j = 0; j < SS_J; ++j) ss[j] = 0.0f;
  const bool ss_owner = T::FM > 1 || wave_n == 0;
  const int ss_j0 = T::FM > 1 ? wave_n * SS_J : 0;

  struct Frags {
    bf16x8_t a[T::FM];
    bf16x8_t b[T::NB][T::FN];
  };
  typedef __attribute__((address_space(3))) v4bf16_t lds_v4bf16;
  auto read_frags = [&](const unsigned char* as, const unsigned char* bs, int h, int g, Frags& f) {
#pragma unroll
    for (int j = 0; j < T::FM; ++j)
      f.a[j] = *(const bf16x8_t*)(as + a_frag[h * T::GROUPS + g] + j * 32 * T::A_ROWB);
    if constexpr (BNK) {
#pragma unroll
      for (int op = 0; op < T::NB; ++op)
#pragma unroll
        for (int i = 0; i < T::FN; ++i)
          f.b[op][i] = *(const bf16x8_t*)(bs + bnk_frag[h * T::GROUPS + g] + op * T::BN * T::A_ROWB +
                                          i * 32 * T::A_ROWB);
      return;
    }
#pragma unroll
    for (int op = 0; op < T::NB; ++op)
#pragma unroll
      for (int i = 0; i < T::FN; ++i) {
        const unsigned char* q = bs + b_frag[op][i] + 16 * g * T::B_ROWB;
        const v4bf16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(q));
        const v4bf16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(q + 4 * T::B_ROWB));
        f.b[op][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  auto mfmas = [&](const auto& f) {
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
      for (int j = 0; j < T::FM; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[0][i], f.a[j], acc[i][j], 0, 0, 0);
        if constexpr (T::PAIR)
          acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[T::NB - 1][i], f.a[j], acc2[i][j], 0, 0, 0);
      }
    if constexpr (ROWSTAT && !PP) {
      if (ss_owner) {
#pragma unroll
        for (int j = 0; j < SS_J; ++j) {
          const bf16x8_t v = (T::FM > 1 && wave_n == 1) ? f.a[(T::FM > 1 ? SS_J : 0) + j] : f.a[j];
          const bf16x2_t p0 = __builtin_shufflevector(v, v, 0, 1), p1 = __builtin_shufflevector(v, v, 2, 3);
          const bf16x2_t p2 = __builtin_shufflevector(v, v, 4, 5), p3 = __builtin_shufflevector(v, v, 6, 7);
          ss[j] = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, ss[j], false);
          ss[j] = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, ss[j], false);
          ss[j] = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss[j], false);
          ss[j] = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, ss[j], false);
        }
      }
    }
  };
  struct Frags16 {
    bf16x8_t a[FM16];
    bf16x8_t b[T::NB][FN16];
  };
  // one 32-deep step (slot half h) of 16x16x32 fragments
  auto read_frags16 = [&](const unsigned char* as, const unsigned char* bs, int h, Frags16& f) {
#pragma unroll
    for (int j = 0; j < FM16; ++j)
      f.a[j] = *(const bf16x8_t*)(as + a16[h][j & 1] + (j >> 1) * 32 * T::A_ROWB);
    if constexpr (BNK) {
#pragma unroll
      for (int op = 0; op < T::NB; ++op)
#pragma unroll
        for (int i = 0; i < FN16; ++i)
          f.b[op][i] = *(const bf16x8_t*)(bs + bnk16[h][i & 1] + (i >> 1) * 32 * T::A_ROWB + op * T::BN * T::A_ROWB);
      return;
    }
#pragma unroll
    for (int op = 0; op < T::NB; ++op)
#pragma unroll
      for (int i = 0; i < FN16; ++i) {
        const unsigned char* q = bs + b16[op][i];
        const v4bf16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(q));
        const v4bf16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(q + 4 * T::B_ROWB));
        f.b[op][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  auto mfmas16 = [&](const auto& f) {
#pragma unroll
    for (int i = 0; i < FN16; ++i)
#pragma unroll
      for (int j = 0; j < FM16; ++j) {
        c16[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[0][i], f.a[j], c16[i][j], 0, 0, 0);
        if constexpr (T::PAIR)
          c16b[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[T::NB - 1][i], f.a[j], c16b[i][j], 0, 0, 0);
      }
  };
  constexpr int READS_PER_GROUP = T::FM + 2 * T::NB * T::FN;
  constexpr int MFMAS_PER_GROUP = T::FM * T::FN * T::NB;
  // One K step s (tile kt), entered with the fragments of its first group in f0:
  //   * start the direct loads of step kt+2 -- its B stage, and on even steps the A slot of
  //     steps kt+2 and kt+3.  Both were freed before the previous barrier: the B stage held
  //     step kt-2, the A slot steps kt-2 and kt-1, whose last fragment reads (issued before
  //     the previous barrier) were waited for there;
  //   * run group 0 with group 1's fragments in flight;
  //   * wait until step kt+1 has landed: on an even step every load but this step's; on an
  //     odd step every load but this step's B loads (the A slot of kt+1 came with the
  //     previous step's loads), and also this wave's LDS reads of the A slot, which the
  //     next step refills;
  //   * meet the other waves at the barrier, then run group 1 while the first fragments of
  //     step kt+1 are read -- the matrix cores stay busy across the barrier.
  // Loads are issued even past the last step: those offsets are all out of range, so they
  // only write zeros into stages whose reads are discarded (no branch in the loop body).
  Frags f0, f1;
  auto k_step = [&](auto s_c, int kt) {
    constexpr int S = decltype(s_c)::value;
    constexpr bool EVEN = S % 2 == 0;
    using Cur = std::integral_constant<int, S>;
    using Next = std::integral_constant<int, S + 1>;
    using Fill = std::integral_constant<int, S + 2>;
    // [K][N]: B every step; [N][K]: B with A, on even steps only
    constexpr int B_NOW = BNK ? (EVEN ? BL : 0) : BL;
    if constexpr (!BNK || EVEN) issue_b(bstage(Fill{}), (kt + 2) * BKE);
    if constexpr (EVEN) issue_a((kt + 2) * BKE, aslot(Fill{}));
    if constexpr (EVEN) prefetch_l2((kt + 4) * BKE);
    static_assert(T::GROUPS == 2, "two groups per step");
    read_frags(aslot(Cur{}), bstage(Cur{}), S % 2, 1, f1);
    mfmas(f0);
    sched_group<MFMAS_PER_GROUP, EVEN ? T::A_LOADS + B_NOW + PF : B_NOW, READS_PER_GROUP>();
    // No memory fence: the later loads stay in flight across the barrier, and so do the
    // prefetches of the last even step (issued after that step's real loads).
    if constexpr (EVEN)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(T::A_LOADS + B_NOW + PF));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(B_NOW + PF));
    __builtin_amdgcn_s_barrier();
    read_frags(aslot(Next{}), bstage(Next{}), (S + 1) % 2, 0, f0);
    mfmas(f1);
    sched_group<MFMAS_PER_GROUP, 0, READS_PER_GROUP>();
  };

  // ---- fp8 operands (F8IN) ----
  // One v_mfma_f32_32x32x64_f8f6f4 per 32x32 block and step takes 32 bytes per lane from each
  // operand.  A dot product does not depend on which K position a (lane half, byte) pair
  // stands for, as long as both operands use the same assignment, so each lane reads the two
  // 16-byte chunks that the bf16 path reads for its two 16-deep groups (chunks 4h + lhalf and
  // 4h + 2 + lhalf of the slot row): the same conflict-free LDS pattern.  The step's MFMAs are
  // split into two halves over the B fragments (operand, column block): the first half runs
  // before the barrier while the rest of this step's B fragments are read, the second half
  // after it while the next step's A fragments and first B fragments are read.  A fragments
  // alternate between two register sets by step parity.
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  constexpr int NQ = T::NB * T::FN;                    // B fragments per step
  constexpr int NQ0 = NQ / 2;                          // consumed before the barrier
  i32x8_t fa8[2][F8IN ? T::FM : 1];
  i32x8_t fb8[F8IN ? NQ : 1];
  auto frag8 = [&](const unsigned char* base, int h) -> i32x8_t {
    const i32x4_t lo = *(const i32x4_t*)(base + a_frag[2 * h]);
    const i32x4_t hi = *(const i32x4_t*)(base + a_frag[2 * h + 1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto read_a8 = [&](const unsigned char* as, int h, i32x8_t* fa) {
#pragma unroll
    for (int j = 0; j < T::FM; ++j) fa[j] = frag8(as + j * 32 * T::A_ROWB, h);
  };
  // B rows start at wn0 + 32i of operand op; bnk_frag equals a_frag shifted by wn0 - wm0 rows
  auto read_b8 = [&](const unsigned char* bs, int h, auto q0_c, auto q1_c) {
    constexpr int Q0 = decltype(q0_c)::value, Q1 = decltype(q1_c)::value;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
      const int op = q / T::FN, i = q % T::FN;
      const unsigned char* base = bs + op * T::BN * T::A_ROWB + i * 32 * T::A_ROWB;
      const i32x4_t lo = *(const i32x4_t*)(base + bnk_frag[2 * h]);
      const i32x4_t hi = *(const i32x4_t*)(base + bnk_frag[2 * h + 1]);
      fb8[q] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto mfma8 = [&](const i32x8_t* fa, auto q0_c, auto q1_c) {
    constexpr int Q0 = decltype(q0_c)::value, Q1 = decltype(q1_c)::value;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
      const int op = q / T::FN, i = q % T::FN;
#pragma unroll
      for (int j = 0; j < T::FM; ++j) {
        // format 0 = fp8 e4m3 for both sources; zero scale operands select the unscaled form
        if (!T::PAIR || op == 0) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[q], fa[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        } else {
          constexpr int P = T::PAIR ? 1 : 0;      // acc2 is [1][1] without the pairwise op
          acc2[P * i][P * j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[q], fa[j], acc2[P * i][P * j],
                                                                                0, 0, 0, 0, 0, 0);
        }
      }
    }
  };
  using Q0c = std::integral_constant<int, 0>;
  using QHc = std::integral_constant<int, NQ0>;
  using QNc = std::integral_constant<int, NQ>;
  // One fp8 step; the loads, waits and barrier are those of k_step ([N][K] B).
  auto k_step8 = [&](auto s_c, int kt) {
    constexpr int S = decltype(s_c)::value;
    constexpr bool EVEN = S % 2 == 0;
    using Cur = std::integral_constant<int, S>;
    using Next = std::integral_constant<int, S + 1>;
    using Fill = std::integral_constant<int, S + 2>;
    constexpr int B_NOW = EVEN ? BL : 0;
    if constexpr (EVEN) {
      issue_b(bstage(Fill{}), (kt + 2) * BKE);
      issue_a((kt + 2) * BKE, aslot(Fill{}));
      prefetch_l2((kt + 4) * BKE);
    }
    read_b8(bstage(Cur{}), S % 2, QHc{}, QNc{});
    mfma8(fa8[S % 2], Q0c{}, QHc{});
    sched_group8<T::FM * NQ0, EVEN ? T::A_LOADS + B_NOW + PF : 0, 2 * (NQ - NQ0)>();
    if constexpr (EVEN)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(T::A_LOADS + B_NOW + PF));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(B_NOW + PF));
    __builtin_amdgcn_s_barrier();
    read_a8(aslot(Next{}), (S + 1) % 2, fa8[(S + 1) % 2]);
    read_b8(bstage(Next{}), (S + 1) % 2, Q0c{}, QHc{});
    mfma8(fa8[S % 2], QHc{}, QNc{});
    sched_group8<T::FM * (NQ - NQ0), 0, 2 * (T::FM + NQ0)>();
  };

  // Step count rounded up to a multiple of NS with leading all-zero steps, so the loop
  // always runs whole stage rings, A slots pair steps (0,1) and (2,3) of each ring, and the
  // accumulators have one exit path.
  const int nk = (K + BKE - 1) / BKE;
  const int nsteps = (nk + T::NS - 1) / T::NS * T::NS;
  int kt = nk - nsteps;
  // [N][K] B follows A: slot resources at the slot's first step, fixed ones for ragged K
#define GE_SET_RS(ka, kb)                                                      \
  do {                                                                         \
    if constexpr (!KMASK) ars = GE_A_RS(ka);                                   \
    if constexpr (BNK && KMASK) {                                              \
      brs = b_rs0;                                                             \
      b2rs = b2_rs0;                                                           \
    } else {                                                                   \
      brs = GE_B_RS(b_base, BNK ? (ka) : (kb));                                \
      if constexpr (T::PAIR) b2rs = GE_B_RS(b2_base, BNK ? (ka) : (kb));       \
    }                                                                          \
  } while (0)
  // Row statistic shared along a tile row (two-wave RMS plans, F_RS_SHARE): a tile that finds
  // the row's flag set when it starts reads the published sums after its mainloop instead of
  // squaring its A slots; one that does not computes them (the same values: the same slots in
  // the same order), publishes them and sets the flag.  No tile waits for another.
  const bool rs_share = ROWSTAT && PP && !GE_SERIAL_PIPELINE && (p.flags & F_RS_SHARE) != 0;
  const uint32_t rs_row = (uint32_t)(b * p.tiles_m + tm);
  bool stat_on = true;
  if constexpr (GE_SERIAL_PIPELINE) {
    // ---- reference build: one two-step slot at a time, nothing overlapped ----
    // Load the slot's A and B (B [K][N]: both steps' stages), wait for every load, barrier;
    // read and multiply steps k and k+1 with the pipelined build's fragments, MFMAs and order
    // (and, on the two-wave tiles, square the slot's rows for the row statistic once per slot,
    // as their even steps do); wait for the reads, barrier, so no stage is refilled while a
    // wave still reads it.
    [[maybe_unused]] const int grp = wave >> 2;
    [[maybe_unused]] float ss1 = 0.0f;
    [[maybe_unused]] const uint32_t sq_row = (uint32_t)((wave & 3) * 64 + lane) * T::A_ROWB;
    [[maybe_unused]] const uint32_t sq_c = ((uint32_t)((lane & 15) + ((lane & 15) >> 3)) & 7u) ^ (uint32_t)(4 * grp);
    [[maybe_unused]] Frags16 f16;
    for (int k = kt; k < nk; k += 2) {
      GE_SET_RS(k * BKE, k * BKE);
      issue_a(k * BKE, aslot(S0{}));
      issue_b(bstage(S0{}), k * BKE);
      if constexpr (!BNK) {
        GE_SET_RS(k * BKE, (k + 1) * BKE);
        issue_b(bstage(S1{}), (k + 1) * BKE);
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __builtin_amdgcn_s_barrier();
      if constexpr (PP && ROWSTAT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t v = *(const bf16x8_t*)(aslot(S0{}) + sq_row + ((sq_c ^ (uint32_t)i) << 4));
          const bf16x2_t p0 = __builtin_shufflevector(v, v, 0, 1), p1 = __builtin_shufflevector(v, v, 2, 3);
          const bf16x2_t p2 = __builtin_shufflevector(v, v, 4, 5), p3 = __builtin_shufflevector(v, v, 6, 7);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, ss1, false);
        }
      }
      if constexpr (F8IN) {
        read_a8(aslot(S0{}), 0, fa8[0]);
        read_b8(bstage(S0{}), 0, Q0c{}, QNc{});
        mfma8(fa8[0], Q0c{}, QNc{});
        read_a8(aslot(S0{}), 1, fa8[0]);
        read_b8(bstage(S0{}), 1, Q0c{}, QNc{});
        mfma8(fa8[0], Q0c{}, QNc{});
      } else if constexpr (MF16) {
        read_frags16(aslot(S0{}), bstage(S0{}), 0, f16);
        mfmas16(f16);
        read_frags16(aslot(S1{}), bstage(S1{}), 1, f16);
        mfmas16(f16);
      } else {
        read_frags(aslot(S0{}), bstage(S0{}), 0, 0, f0);
        read_frags(aslot(S0{}), bstage(S0{}), 0, 1, f1);
        mfmas(f0);
        mfmas(f1);
        read_frags(aslot(S1{}), bstage(S1{}), 1, 0, f0);
        read_frags(aslot(S1{}), bstage(S1{}), 1, 1, f1);
        mfmas(f0);
        mfmas(f1);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
      __builtin_amdgcn_s_barrier();
    }
    if constexpr (PP && ROWSTAT) row_ss[grp * T::BM + (wave & 3) * 64 + lane] = ss1;
  } else if constexpr (PP) {
    // ---- two waves per SIMD: a memory phase and a matrix phase per step ----
    // Both groups run this sequence with one barrier between phases; group 1 starts one phase
    // behind group 0, so in every phase one wave of each SIMD issues MFMAs while the other
    // issues loads and fragment reads.  Group 0 reads step j in phase 2j, group 1 in 2j+1.
    //   memory phase of step j: start the direct loads of later steps -- for even j the A
    //     slot of steps j+2 and j+3 (it held steps j-2 and j-1), for odd j the B stages of
    //     steps j+2 and j+3 (they held steps j-2 and j-1, read by both groups before the
    //     previous barrier), so every step moves 32 KB per workgroup; with B given
    //     [N][K], B is staged in two-step slots like A and loaded with it on even steps --
    //     read every fragment of step j; wait for them and for this wave's loads of step j+1
    //     (group 0 reads that step two phases later, and every wave passes the barrier in
    //     between).
    //   matrix phase of step j: the step's MFMAs only, at raised wave priority, so the
    //     partner wave's memory work fills the issue slots the MFMAs leave.
    static_assert(MF16 || F8IN, "two-wave instances: 16x16x32 bf16 or fp8 operands");
    const int grp = wave >> 2;
    Frags16 f16;
    // Step resources: K is a multiple of two steps here, so a step is wholly inside or outside
    // [0, K), and an outside step needs only an empty extent (its base is never used): one
    // unsigned compare instead of the clamps of the general case.
    const uint32_t a_ext32 = (uint32_t)a_ext, b_ext32 = (uint32_t)b_ext;
    auto rs_pp = [&](const unsigned char* base, uint32_t ext, int k0, uint32_t bytes_per_k) {
      const uint32_t off = (uint32_t)k0 * bytes_per_k;
      return make_rsrc(base + off, (uint32_t)k0 < (uint32_t)K ? (int64_t)(ext - off) : 0);
    };
    auto set_rs_pp = [&](int ka, int kb) {
      ars = rs_pp(a_base, a_ext32, ka, ES);
      const int kbb = BNK ? ka : kb;
      const uint32_t bpk = BNK ? (uint32_t)ES : ldb2;
      brs = rs_pp(b_base, b_ext32, kbb, bpk);
      if constexpr (T::PAIR) b2rs = rs_pp(b2_base, b_ext32, kbb, bpk);
    };
    // Row statistic: in the memory phase of each even step j every lane squares half of one
    // row of the A slot of steps j and j+1 (its first use): slot row (wave % 4) * 64 + lane,
    // physical chunks sq_c ^ i (i < 4), where sq_c's bit 2 is the wave group, so the two
    // groups cover the row's eight chunks between them (the sum does not depend on which
    // K a chunk holds).  sq_c = (l + l / 8) % 8, l = lane % 16, gives the 8 (16) lanes one
    // LDS pass serves 8 (16) distinct chunk columns: no bank conflicts.  The loads and
    // v_dot2 run while the other group's MFMAs use the matrix core; the fragments stay as
    // they are.
    static_assert(!ROWSTAT || T::BM == 4 * 64, "one slot row per lane of a wave group");
    float ss1 = 0.0f;
    const uint32_t sq_row = (uint32_t)((wave & 3) * 64 + lane) * T::A_ROWB;
    const uint32_t sq_c = ((uint32_t)((lane & 15) + ((lane & 15) >> 3)) & 7u) ^ (uint32_t)(4 * grp);
    // the tile row's flag: loaded before the prologue's loads, so it lands with them
    uint32_t have = 0;
    if (rs_share && tid == 0)
      have = __hip_atomic_load(p.rs_ctr + rs_row * kRowStatCtrStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    set_rs_pp(kt * BKE, kt * BKE);
    issue_a(kt * BKE, aslot(S0{}));
    issue_b(bstage(S0{}), kt * BKE);
    if constexpr (!BNK) {
      set_rs_pp(kt * BKE, (kt + 1) * BKE);
      issue_b(bstage(S1{}), (kt + 1) * BKE);
      set_rs_pp(kt * BKE, (kt + 2) * BKE);
      issue_b(bstage(S2{}), (kt + 2) * BKE);
    }
    if (rs_share && tid == 0) {
      rs_have = have;
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));       // the LDS store, before the barrier
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(BNK ? 0 : 2 * T::B_LOADS));   // A slot and B of step kt landed
    __builtin_amdgcn_s_barrier();
    if (rs_share) stat_on = __builtin_amdgcn_readfirstlane(rs_have) == 0u;
    if (grp == 1) __builtin_amdgcn_s_barrier();               // one phase behind group 0
    auto mem_phase = [&](auto s_c, int j, auto stat_c) {
      constexpr int S = decltype(s_c)::value;
      constexpr bool EVEN = S % 2 == 0;
      constexpr bool SQ = ROWSTAT && EVEN && decltype(stat_c)::value;    // this step squares its slot
      using Cur = std::integral_constant<int, S>;
      using FillA = std::integral_constant<int, S + 2>;
      using FillB = std::integral_constant<int, S + 3>;
      using FillB2 = std::integral_constant<int, S + 2>;
      // The loads of later steps fill other stages, so they may go before or after this step's
      // fragment reads.  Reads first (the phase waits for them; the loads' issue then overlaps
      // their LDS latency) measured +1 to +4.5 % on B [K][N] and fp8 operands, -1 % on bf16
      // B [N][K] (whose even steps carry all eight loads): loads first there.
      auto issue_loads = [&]() {
        set_rs_pp((j + 2) * BKE, (j + 3) * BKE);
        if constexpr (BNK) {
          if constexpr (EVEN) {
            issue_a((j + 2) * BKE, aslot(FillA{}));
            issue_b(bstage(FillA{}), (j + 2) * BKE);
          }
        } else if constexpr (EVEN) {
          issue_a((j + 2) * BKE, aslot(FillA{}));
        } else {
          // B [K][N]: two one-step stages on odd steps, so that every step moves the same
          // 32 KB (the A slot alone on even steps); one B stage per step with the A slot on
          // top of it on even steps (48 KB, then 16 KB) measured 3-5 % slower
          set_rs_pp((j + 2) * BKE, (j + 2) * BKE);
          issue_b(bstage(FillB2{}), (j + 2) * BKE);
          set_rs_pp((j + 2) * BKE, (j + 3) * BKE);
          issue_b(bstage(FillB{}), (j + 3) * BKE);
        }
      };
      constexpr bool READS_FIRST = !BNK || F8IN;
      if constexpr (!READS_FIRST) issue_loads();
      if constexpr (F8IN) {
        // fp8 operands: one 64-deep step, one register set (the matrix phase uses it whole)
        read_a8(aslot(Cur{}), S % 2, fa8[0]);
        read_b8(bstage(Cur{}), S % 2, Q0c{}, QNc{});
      } else {
        read_frags16(aslot(Cur{}), bstage(Cur{}), S % 2, f16);
      }
      bf16x8_t sq[4];
      if constexpr (SQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sq[i] = *(const bf16x8_t*)(aslot(Cur{}) + sq_row + ((sq_c ^ (uint32_t)i) << 4));
      }
      if constexpr (READS_FIRST) {
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the loads
        issue_loads();
      }
      // loads younger than those of step j+1: even j -- B of step j+2 (issued with B of
      // step j+1 on step j-1) and the A slot of j+2, j+3; odd j -- B of steps j+2, j+3 (the
      // A slot of j+1 came on step j-1, after B of step j+1).  [N][K]: even j -- the A and B
      // slots of j+2, j+3; odd j -- none.
      constexpr int YOUNGER = BNK ? (EVEN ? T::A_LOADS + BL : 0)
                                  : (EVEN ? T::B_LOADS + T::A_LOADS : 2 * T::B_LOADS);
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(YOUNGER));
      if constexpr (SQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t v = sq[i];
          const bf16x2_t p0 = __builtin_shufflevector(v, v, 0, 1), p1 = __builtin_shufflevector(v, v, 2, 3);
          const bf16x2_t p2 = __builtin_shufflevector(v, v, 4, 5), p3 = __builtin_shufflevector(v, v, 6, 7);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss1, false);
          ss1 = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, ss1, false);
        }
        asm volatile("" : "+v"(ss1));      // keep the squares in this phase
      }
      __builtin_amdgcn_s_barrier();
    };
    auto mat_phase = [&]() {
      __builtin_amdgcn_s_setprio(1);
      if constexpr (F8IN) {
        mfma8(fa8[0], Q0c{}, QNc{});
      } else {
        mfmas16(f16);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_s_barrier();
    };
    // the loop with and without the row statistic's squares, each with its own registers
    auto run_loop = [&](auto stat_c) {
      for (; kt < nk; kt += T::NS) {
        mem_phase(S0{}, kt, stat_c);
        mat_phase();
        mem_phase(S1{}, kt + 1, stat_c);
        mat_phase();
        mem_phase(S2{}, kt + 2, stat_c);
        mat_phase();
        mem_phase(S3{}, kt + 3, stat_c);
        mat_phase();
      }
    };
    if constexpr (ROWSTAT) {
      if (stat_on)
        run_loop(std::true_type{});
      else
        run_loop(std::false_type{});
    } else {
      run_loop(std::false_type{});
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();               // matches group 1's last phase
    if constexpr (ROWSTAT) row_ss[grp * T::BM + (wave & 3) * 64 + lane] = ss1;
  } else {
    GE_SET_RS(kt * BKE, kt * BKE);
    issue_a(kt * BKE, aslot(S0{}));
    issue_b(bstage(S0{}), kt * BKE);
    if constexpr (!BNK) {
      GE_SET_RS(kt * BKE, (kt + 1) * BKE);
      issue_b(bstage(S1{}), (kt + 1) * BKE);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(BNK ? 0 : T::B_LOADS));
    __builtin_amdgcn_s_barrier();
    if constexpr (F8IN) {
      read_a8(aslot(S0{}), 0, fa8[0]);
      read_b8(bstage(S0{}), 0, Q0c{}, QHc{});
    } else {
      read_frags(aslot(S0{}), bstage(S0{}), 0, 0, f0);
    }
    auto step = [&](auto s_c, int k) {
      if constexpr (F8IN) k_step8(s_c, k);
      else k_step(s_c, k);
    };
    for (; kt < nk; kt += T::NS) {
      // each step fills the stages of step + 2 (A: on even steps, the slot of steps + 2, + 3)
      GE_SET_RS((kt + 2) * BKE, (kt + 2) * BKE);
      step(S0{}, kt);
      GE_SET_RS((kt + 2) * BKE, (kt + 3) * BKE);
      step(S1{}, kt + 1);
      GE_SET_RS((kt + 4) * BKE, (kt + 4) * BKE);
      step(S2{}, kt + 2);
      GE_SET_RS((kt + 4) * BKE, (kt + 5) * BKE);
      step(S3{}, kt + 3);
    }
  }
#undef GE_SET_RS
#undef GE_B_RS
#undef GE_A_RS
#undef GE_KLIVE
#undef GE_KCLAMP
  __builtin_amdgcn_s_waitcnt(kVmcnt0);                 // trailing zero-tile loads into the stages

  // ---- RMS row statistic: the two lane halves hold different K of the same rows ----
  if constexpr (ROWSTAT) {
    if constexpr (!PP) {
#pragma unroll
      for (int j = 0; j < SS_J; ++j) {
        const float s = ss[j] + __shfl_xor(ss[j], 32);
        if (ss_owner && lhalf == 0) row_ss[wm0 + 32 * (ss_j0 + j) + lrow] = s;
      }
    }
    __syncthreads();
    if (rs_share) {                                      // uniform
      // publish: every sum performed at device scope before the flag (each thread waits for
      // its store, then the barrier); read: the flag was seen set when the tile started, so
      // the sums were performed before it.  The reader keeps the epilogue's sum of the two
      // halves exact by storing the published sum and a zero.
      uint32_t* ctr = p.rs_ctr + rs_row * kRowStatCtrStride;
      uint32_t* val = reinterpret_cast<uint32_t*>(p.rs_val) + rs_row * (uint32_t)T::BM;
      if (stat_on) {
        if (tid < T::BM) {
          const float s = row_ss[tid] + row_ss[T::BM + tid];
          __hip_atomic_store(val + tid, __float_as_uint(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(kVmcnt0);
        }
        __syncthreads();
        if (tid == 0) {
          __hip_atomic_store(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(kVmcnt0);           // flag performed before the ticket
        }
      } else {
        if (tid < T::BM) {
          row_ss[tid] = __uint_as_float(__hip_atomic_load(val + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          row_ss[T::BM + tid] = 0.0f;
        }
        __syncthreads();
      }
      // the tile row's ticket: the last of its tiles_n tiles clears the flag and the counter
      if (tid == 0 &&
          __hip_atomic_fetch_add(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)p.tiles_n - 1u) {
        __hip_atomic_store(ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // ---- epilogue, two phases per 32-row block of the wave's tile ----
  // Phase 1 (registers -> LDS): the per-row linear part t = acc * alpha * s[m] (for the
  // pairwise op the finished product act(t_gate) * t_up) goes to a wave-private fp32
  // block in LDS, rows padded by 16 bytes so the 32 rows written at one column spread
  // over all banks.  Phase 2 (LDS -> HBM): each lane takes 4 consecutive columns of a
  // row, adds the column bias, applies the activation, adds the residual, folds |y|
  // into AMAX (fp32, before rounding), converts and stores; one instruction covers whole
  // rows, so residual loads and output stores are fully coalesced.
  const uint32_t flags = p.flags;
  const bool has_bias = (flags & F_BIAS) != 0;
  const bool has_res = (flags & F_RESIDUAL) != 0;
  static_assert(!(GRAD && T::PAIR), "the activation gradient is not a pairwise epilogue");
  const bool has_cs = (flags & F_COL_SUM) != 0;
  const bool has_rs = (flags & F_ROW_SCALE) != 0;
  const bool has_rms = ROWSTAT && (flags & F_ROW_RMS) != 0;
  const float alpha = (flags & F_SCALE) ? p.alpha : 1.0f;
  const float inv_k = K > 0 ? 1.0f / (float)K : 0.0f;

  constexpr int EP_LD = T::EP_LD;                       // floats per LDS row
  constexpr int LPR = T::WN / 4;                        // phase-2 lanes per row
  constexpr int RPP = 64 / LPR;                         // rows per phase-2 pass
  constexpr int PASSES = 32 / RPP;
  __syncthreads();                                      // every wave is done with the stages
  float* ep = (float*)((wave < T::EP_PER_SLOT ? aslot0 : aslot1) + (wave % T::EP_PER_SLOT) * T::EP_WAVE_BYTES);

  const int p2_row = lane / LPR, p2_col = 4 * (lane % LPR);
  const int gcol = n0 + wn0 + p2_col;
  const bool col_ok = gcol < N;
  float bias4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (has_bias) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bias + n0, (int64_t)(N - n0) * 2);
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(rs, col_ok ? (uint32_t)(gcol - n0) * 2u : kOOB, 0, 0);
    bias4[0] = bf16_lo(w[0]);
    bias4[1] = bf16_hi(w[0]);
    bias4[2] = bf16_lo(w[1]);
    bias4[3] = bf16_hi(w[1]);
  }
  const int esize = FP8 ? 1 : 2;
  void* y_base = (unsigned char*)p.Y + (b * p.sy + (int64_t)m0 * p.ldy + n0) * esize;
  const __amdgpu_buffer_rsrc_t y_rs =
      make_rsrc(y_base, ((int64_t)(M - 1 - m0) * p.ldy + (N - n0)) * esize);
  const __amdgpu_buffer_rsrc_t r_rs =
      has_res ? make_rsrc(p.R + b * p.sr + (int64_t)m0 * p.ldr + n0, ((int64_t)(M - 1 - m0) * p.ldr + (N - n0)) * 2)
              : y_rs;
  const __amdgpu_buffer_rsrc_t z_rs =
      GRAD ? make_rsrc(p.Z + b * p.sz + (int64_t)m0 * p.ldz + n0, ((int64_t)(M - 1 - m0) * p.ldz + (N - n0)) * 2)
               : y_rs;
  const uint32_t ldy_b = (uint32_t)p.ldy * (uint32_t)esize, ldr_b = (uint32_t)p.ldr * 2u;
  const uint32_t ldz_b = (uint32_t)p.ldz * 2u;
  const uint32_t col_y = col_ok ? (uint32_t)(wn0 + p2_col) * (uint32_t)esize : kOOB;
  const uint32_t col_r = col_ok ? (uint32_t)(wn0 + p2_col) * 2u : kOOB;

  uint32_t amax_bits = 0;
  float csum[4] = {0.0f, 0.0f, 0.0f, 0.0f};    // COL_SUM: this lane's four columns
  // Residual rows (and, for the activation gradient, saved pre-activation rows) of a 32-row
  // block, in phase-2 layout, loaded at the start of the block so that phase 1 hides their
  // latency.
  u32x2_t rvb[1][PASSES];
  u32x2_t zvb[GRAD ? PASSES : 1];
  auto load_rows = [&](int j, __amdgpu_buffer_rsrc_t rs, uint32_t ld_b, u32x2_t* rv) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int ml = wm0 + 32 * j + ps * RPP + p2_row;
      const uint32_t off = (m0 + ml < M) ? (uint32_t)ml * ld_b + col_r : kOOB;
      rv[ps] = __builtin_amdgcn_raw_buffer_load_b64(rs, off | (col_r & kOOB), 0, 0);
    }
  };
  auto prefetch = [&](int j) {
    if (has_res) load_rows(j, r_rs, ldr_b, rvb[0]);
    if constexpr (GRAD) load_rows(j, z_rs, ldz_b, zvb);
  };
  // Phase 2 in chunks of PCH passes (bounds the registers the batched LDS reads and the
  // saved pre-activation occupy).
  constexpr int PCH = PASSES < 8 ? PASSES : 8;
  auto phase2 = [&](int j, auto res_c, const u32x2_t* rv) {
    constexpr bool RES = decltype(res_c)::value;
#pragma unroll
    for (int c0 = 0; c0 < PASSES; c0 += PCH) {
    f32x4_t vv[PCH];
#pragma unroll
    for (int q = 0; q < PCH; ++q) vv[q] = *(const f32x4_t*)(ep + ((c0 + q) * RPP + p2_row) * EP_LD + p2_col);
#pragma unroll
    for (int q = 0; q < PCH; ++q) {
      const int ps = c0 + q;
      const int r = ps * RPP + p2_row;
      const int ml = wm0 + 32 * j + r;
      const bool ok = (m0 + ml < M) & col_ok;
      const f32x4_t v = vv[q];
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (T::PAIR) {
          y[e] = v[e];
        } else if constexpr (GRAD) {
          const uint32_t zw = zvb[c0 + q][e >> 1];
          y[e] = (v[e] + bias4[e]) * activate_grad<ACT>((e & 1) ? bf16_hi(zw) : bf16_lo(zw));
        } else {
          y[e] = activate<ACT>(v[e] + bias4[e]);
        }
      }
      if constexpr (RES) {
        y[0] += bf16_lo(rv[ps][0]);
        y[1] += bf16_hi(rv[ps][0]);
        y[2] += bf16_lo(rv[ps][1]);
        y[3] += bf16_hi(rv[ps][1]);
      }
      const uint32_t m01 = max(__float_as_uint(y[0]) & 0x7FFFFFFFu, __float_as_uint(y[1]) & 0x7FFFFFFFu);
      const uint32_t m23 = max(__float_as_uint(y[2]) & 0x7FFFFFFFu, __float_as_uint(y[3]) & 0x7FFFFFFFu);
      amax_bits = ok ? max(amax_bits, max(m01, m23)) : amax_bits;
#pragma unroll
      for (int e = 0; e < 4; ++e) csum[e] += ok ? y[e] : 0.0f;
      const uint32_t yoff = ok ? (uint32_t)ml * ldy_b + col_y : kOOB;
      // Y is written once and not read back here: non-temporal stores (cache policy bit 1, "nt")
      // measured +1 to +4 % over plain stores across the workloads.
      if constexpr (FP8) {
        const float qs = p.qscale;
        float x[4], z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = y[e] * qs;
          z[e] = fminf(fmaxf(x[e], -448.0f), 448.0f);
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], w, true);
        // The clamp sends NaN to -448 (fmaxf returns the number); OCP e4m3 keeps NaN as the
        // code S.1111.111, written here as 0x7F.  Taken only by waves that hold a NaN.
        if ((x[0] != x[0]) | (x[1] != x[1]) | (x[2] != x[2]) | (x[3] != x[3])) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (x[e] != x[e]) w = (w & ~(0xFF << (8 * e))) | (0x7F << (8 * e));
        }
        __builtin_amdgcn_raw_buffer_store_b32((unsigned)w, y_rs, yoff, 0, 2);
      } else {
        u32x2_t w;
        w[0] = pack_bf16x2(y[0], y[1]);
        w[1] = pack_bf16x2(y[2], y[3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, y_rs, yoff, 0, 2);
      }
    }
    }
  };

  // per-row scale of slot row ml: alpha, the RMS factor, the caller's row scale
  auto row_factor = [&](int ml) {
    float rscale = alpha;
    if constexpr (ROWSTAT) {
      float ssq = row_ss[ml];
      if constexpr (PP) ssq += row_ss[T::BM + ml];
      if (has_rms) rscale *= __builtin_amdgcn_rsqf(ssq * inv_k + p.eps);
    }
    if (has_rs) rscale *= (m0 + ml < M) ? p.row_scale[(int64_t)b * M + m0 + ml] : 0.0f;
    return rscale;
  };
  if constexpr (MF16) {
#pragma unroll
    for (int j = 0; j < T::FM; ++j) {
      prefetch(j);
      // phase 1: 16x16 blocks 2j, 2j+1 of each column block; lane's rows 16 par + lane % 16,
      // columns 16i + 4 (lane / 16) + e of the wave's 32-row block
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int r = 16 * par + (int)l16;
        const float rscale = row_factor(wm0 + 32 * j + r);
#pragma unroll
        for (int i = 0; i < FN16; ++i) {
          f32x4_t t;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (T::PAIR) {
              t[e] = activate<ACT>(c16[i][2 * j + par][e] * rscale) * (c16b[i][2 * j + par][e] * rscale);
            } else {
              t[e] = c16[i][2 * j + par][e] * rscale;
            }
          }
          *(f32x4_t*)(ep + r * EP_LD + 16 * i + 4 * (int)q16) = t;
        }
      }
      if (has_res)
        phase2(j, std::integral_constant<bool, true>{}, rvb[0]);
      else
        phase2(j, std::integral_constant<bool, false>{}, rvb[0]);
    }
  } else {
#pragma unroll
  for (int j = 0; j < T::FM; ++j) {
    prefetch(j);
    const int ml = wm0 + 32 * j + lrow;
    float rscale = alpha;
    if constexpr (ROWSTAT) {
      float ssq = row_ss[ml];
      if constexpr (PP) ssq += row_ss[T::BM + ml];
      if (has_rms) rscale *= __builtin_amdgcn_rsqf(ssq * inv_k + p.eps);
    }
    if (has_rs) rscale *= (m0 + ml < M) ? p.row_scale[(int64_t)b * M + m0 + ml] : 0.0f;
    // phase 1: lane's row lrow, columns 32i + 8g + 4*lhalf + e of the wave's block
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (T::PAIR) {
            t[e] = activate<ACT>(acc[i][j][4 * g + e] * rscale) * (acc2[i][j][4 * g + e] * rscale);
          } else {
            t[e] = acc[i][j][4 * g + e] * rscale;
          }
        }
        *(f32x4_t*)(ep + lrow * EP_LD + 32 * i + 8 * g + 4 * lhalf) = t;
      }
    // phase 2 reads what this wave just wrote; a wave's LDS operations complete in order
    if (has_res)
      phase2(j, std::integral_constant<bool, true>{}, rvb[0]);
    else
      phase2(j, std::integral_constant<bool, false>{}, rvb[0]);
  }
  }

  // ---- cross-workgroup reductions: memory ordering ----
  // COL_SUM and AMAX hand values between workgroups through workspace slots and ticket
  // counters, all of them agent-scope atomics with relaxed order.  The order they need comes
  // from how this GPU performs them: an agent-scope atomic store writes through the XCD's L2
  // to the memory side, an agent-scope atomic load or read-modify-write is performed there, and
  // s_waitcnt vmcnt(0) returns once this wave's stores are acknowledged at that level.  Each
  // workgroup waits so between its slot stores and its ticket; the tickets of one counter are
  // performed in one order at the memory side; the workgroup that draws a counter's last
  // ticket issues its slot loads only after that read-modify-write has returned, so it reads
  // every slot stored before any ticket of that counter (and, through a group's last
  // workgroup, of its whole group).  Release/acquire tickets would state the same order in the
  // language's model, but the release writes back every dirty line of the XCD's L2 (the
  // output tiles too, which no reader of the workspace needs) at each workgroup's ticket and
  // costs 1-7% of the kernel's time; the slots need none of it.
  // ---- COL_SUM ----
  // Lanes holding the same four columns (equal lane % LPR) add up their rows; the two waves of
  // a column half (wave_m = 0, 1) meet in LDS; the workgroup stores its partial column sums
  // (device scope) in its [batch * tiles_m] row of the workspace and takes a ticket from its
  // column tile's counter.  The workgroup completing a column tile adds that tile's partials
  // in row-tile order -- a fixed order, so the result does not depend on which workgroup
  // finishes last -- writes col_sum and resets the counter.
  if (has_cs) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) csum[e] += __shfl_xor(csum[e], off);
    __syncthreads();                                    // LDS: epilogue blocks are done with
    float* cs_lds = (float*)aslot0;
    if (wave_m == 1 && lane < LPR)
      *(f32x4_t*)(cs_lds + wn0 + p2_col) = f32x4_t{csum[0], csum[1], csum[2], csum[3]};
    __syncthreads();
    const uint32_t prow = (uint32_t)(b * p.tiles_m + tm);
    if (wave_m == 0 && lane < LPR) {
      const f32x4_t o = *(const f32x4_t*)(cs_lds + wn0 + p2_col);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (gcol + e < N)
          __hip_atomic_store(&p.cs_part[(int64_t)prow * N + gcol + e], csum[e] + o[e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);                // partials performed before the ticket
    __syncthreads();
    const uint32_t rows_of_tiles = (uint32_t)(p.batch * p.tiles_m);
    if (tid == 0) {
      uint32_t* ctr = &p.cs_ctr[(uint32_t)tn * kColSumCtrStride];
      bool last = false;
      if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == rows_of_tiles - 1u) {
        __hip_atomic_exchange(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = true;
      }
      wave_amax[0] = last ? 1u : 0u;
    }
    __syncthreads();
    if (wave_amax[0]) {                                 // uniform: the tile's last workgroup
      static_assert(T::BN <= T::NT, "one thread per column");
      const int n = n0 + tid;
      if (tid < T::BN && n < N) {
        float sum = 0.0f;
        for (uint32_t r = 0; r < rows_of_tiles; ++r)
          sum += __hip_atomic_load(&p.cs_part[(int64_t)r * N + n], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.col_sum[n] = sum;
      }
    }
    __syncthreads();                                    // wave_amax is reused below
  }

  // ---- AMAX ----
  // Wave max on the |y| bit patterns (integer max keeps NaN; non-negative floats order like
  // their bit patterns), then a workgroup max.  Each workgroup stores its partial maximum
  // in its own workspace slot (no contended read-modify-write), waits for the store to be
  // performed at device scope, and takes a ticket from the counter of its dispatch group
  // (workgroup id mod 8 = the XCD it runs on).  The workgroup completing a group takes a
  // ticket from the top counter; the one completing the top counter is last: every slot is
  // in place, it reduces them and publishes *amax.  Grids of at most kAmaxFlatGrid
  // workgroups take their ticket from the top counter directly.  Counters are reset by the
  // workgroup that completes them, so the workspace is zero again when the kernel ends.
  if (flags & F_AMAX) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)amax_bits, off);
      amax_bits = o > amax_bits ? o : amax_bits;
    }
    if (lane == 0) wave_amax[wave] = amax_bits;
    __syncthreads();
    const uint32_t total = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n * (uint32_t)p.batch;
    if (tid == 0) {
      uint32_t m = wave_amax[0];
#pragma unroll
      for (int w = 1; w < T::WAVES; ++w) m = wave_amax[w] > m ? wave_amax[w] : m;
      const uint32_t wg = blockIdx.x;
      __hip_atomic_store(&p.ws[kAmaxSlot0 + wg], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);              // slot performed before the ticket
      const uint32_t grp = wg % kAmaxGroups;
      const uint32_t gsize = (total + kAmaxGroups - 1u - grp) / kAmaxGroups;
      const uint32_t ngroups = total < kAmaxGroups ? total : kAmaxGroups;
      uint32_t* gctr = &p.ws[grp * kAmaxCounterStride];
      uint32_t* tctr = &p.ws[kAmaxGroups * kAmaxCounterStride];
      bool last = false;
      if (total <= kAmaxFlatGrid) {
        // small grids: one ticket on the top counter (saves a round trip on the critical path)
        if (__hip_atomic_fetch_add(tctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1u) {
          __hip_atomic_exchange(tctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = true;
        }
      } else if (__hip_atomic_fetch_add(gctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1u) {
        __hip_atomic_exchange(gctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__hip_atomic_fetch_add(tctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1u) {
          __hip_atomic_exchange(tctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = true;
        }
      }
      wave_amax[0] = last ? 1u : 0u;
    }
    __syncthreads();
    if (wave_amax[0]) {                                  // uniform: the last workgroup
      uint32_t mm = 0;
      for (uint32_t i = (uint32_t)tid; i < total; i += T::NT)
        mm = max(mm, __hip_atomic_load(&p.ws[kAmaxSlot0 + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mm = max(mm, (uint32_t)__shfl_xor((int)mm, off));
      __syncthreads();
      if (lane == 0) wave_amax[wave] = mm;
      __syncthreads();
      if (tid == 0) {
        uint32_t v = wave_amax[0];
#pragma unroll
        for (int w = 1; w < T::WAVES; ++w) v = max(v, wave_amax[w]);
        __hip_atomic_store(p.amax, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}


template <class T, int ACT, bool GRAD, bool FP8, bool ROWSTAT, bool BNK>
void launch_k(const Params& p, hipStream_t s, unsigned grid) {
  if (p.K % 64 != 0)
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, GRAD, FP8, ROWSTAT, true, BNK>), dim3(grid), dim3(T::NT), 0, s, p);
  else
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, GRAD, FP8, ROWSTAT, false, BNK>), dim3(grid), dim3(T::NT), 0, s, p);
}

template <class T, int ACT, bool FP8, bool BNK>
hipError_t launch_t(const Params& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  if (grid <= 0) return hipSuccess;
  if (p.flags & F_ACT_GRAD) {
    // backward epilogue instances: bf16 output, no in-kernel row statistic (checked on the host)
    if constexpr (!T::PAIR && !FP8) {
      if (p.flags & F_ROW_RMS) return hipErrorInvalidValue;
      launch_k<T, ACT, true, false, false, BNK>(p, s, (unsigned)grid);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (p.flags & F_ROW_RMS) {
    launch_k<T, ACT, false, FP8, true, BNK>(p, s, (unsigned)grid);
  } else {
    launch_k<T, ACT, false, FP8, false, BNK>(p, s, (unsigned)grid);
  }
  return hipGetLastError();
}

// fp8 operands (B given [N][K]): forward epilogues only, no in-kernel row statistic (checked
// on the host).  One A slot holds 128 K values, so K % 128 decides the per-lane masking.
template <class T, int ACT, bool FP8>
hipError_t launch_t8(const Params& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  if (grid <= 0) return hipSuccess;
  if (p.flags & (F_ACT_GRAD | F_ROW_RMS)) return hipErrorInvalidValue;
  if (p.K % 128 != 0)
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, false, FP8, false, true, true, true>), dim3((unsigned)grid),
                       dim3(T::NT), 0, s, p);
  else
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, false, FP8, false, false, true, true>), dim3((unsigned)grid),
                       dim3(T::NT), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_tile_f8(int act, bool fp8, const Params& p, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return fp8 ? launch_t8<T, ACT_NONE, true>(p, s) : launch_t8<T, ACT_NONE, false>(p, s);
    case ACT_RELU: return fp8 ? launch_t8<T, ACT_RELU, true>(p, s) : launch_t8<T, ACT_RELU, false>(p, s);
    case ACT_GELU_TANH:
      return fp8 ? launch_t8<T, ACT_GELU_TANH, true>(p, s) : launch_t8<T, ACT_GELU_TANH, false>(p, s);
    case ACT_SILU: return fp8 ? launch_t8<T, ACT_SILU, true>(p, s) : launch_t8<T, ACT_SILU, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Two-wave instances (two waves per SIMD) of one B layout: bf16 operands and K a multiple of
// 64 (checked on the host; anything else is refused here too).
template <class T, int ACT, bool FP8, bool BNK>
hipError_t launch_pp(const Params& p, hipStream_t s) {
  static_assert(T::WAVES == 8, "two-wave tile");
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  if (grid <= 0) return hipSuccess;
  if ((p.flags & F_IN_FP8) || ((p.flags & F_B_NK) != 0) != BNK || p.K % 64 != 0) return hipErrorInvalidValue;
  if (p.flags & F_ACT_GRAD) {
    // backward epilogue instances: bf16 output, no in-kernel row statistic (checked on the host)
    if constexpr (!T::PAIR && !FP8) {
      if (p.flags & F_ROW_RMS) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, true, false, false, false, BNK>), dim3((unsigned)grid),
                         dim3(T::NT), 0, s, p);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (p.flags & F_ROW_RMS) {
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, false, FP8, true, false, BNK>), dim3((unsigned)grid),
                       dim3(T::NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, false, FP8, false, false, BNK>), dim3((unsigned)grid),
                       dim3(T::NT), 0, s, p);
  }
  return hipGetLastError();
}

// Two-wave instances with fp8 operands (B given [N][K]): forward epilogues, no row statistic
// (checked on the host), K a multiple of 128 (one slot: two 64-deep steps).
template <class T, int ACT, bool FP8>
hipError_t launch_pp8(const Params& p, hipStream_t s) {
  static_assert(T::WAVES == 8, "two-wave tile");
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  if (grid <= 0) return hipSuccess;
  if ((p.flags & (F_ACT_GRAD | F_ROW_RMS)) || !(p.flags & F_IN_FP8) || !(p.flags & F_B_NK) || p.K % 128 != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((fused_gemm_epilogue<T, ACT, false, FP8, false, false, true, true>), dim3((unsigned)grid),
                     dim3(T::NT), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_tile_pp8(int act, bool fp8, const Params& p, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return fp8 ? launch_pp8<T, ACT_NONE, true>(p, s) : launch_pp8<T, ACT_NONE, false>(p, s);
    case ACT_RELU: return fp8 ? launch_pp8<T, ACT_RELU, true>(p, s) : launch_pp8<T, ACT_RELU, false>(p, s);
    case ACT_GELU_TANH:
      return fp8 ? launch_pp8<T, ACT_GELU_TANH, true>(p, s) : launch_pp8<T, ACT_GELU_TANH, false>(p, s);
    case ACT_SILU: return fp8 ? launch_pp8<T, ACT_SILU, true>(p, s) : launch_pp8<T, ACT_SILU, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <class T, bool BNK>
hipError_t launch_tile_pp(int act, bool fp8, const Params& p, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return fp8 ? launch_pp<T, ACT_NONE, true, BNK>(p, s) : launch_pp<T, ACT_NONE, false, BNK>(p, s);
    case ACT_RELU: return fp8 ? launch_pp<T, ACT_RELU, true, BNK>(p, s) : launch_pp<T, ACT_RELU, false, BNK>(p, s);
    case ACT_GELU_TANH:
      return fp8 ? launch_pp<T, ACT_GELU_TANH, true, BNK>(p, s) : launch_pp<T, ACT_GELU_TANH, false, BNK>(p, s);
    case ACT_SILU: return fp8 ? launch_pp<T, ACT_SILU, true, BNK>(p, s) : launch_pp<T, ACT_SILU, false, BNK>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// The instances of one tile shape and one B layout (one translation unit each).
template <class T, bool BNK>
hipError_t launch_tile(int act, bool fp8, const Params& p, hipStream_t s) {
  switch (act) {
    case ACT_NONE: return fp8 ? launch_t<T, ACT_NONE, true, BNK>(p, s) : launch_t<T, ACT_NONE, false, BNK>(p, s);
    case ACT_RELU: return fp8 ? launch_t<T, ACT_RELU, true, BNK>(p, s) : launch_t<T, ACT_RELU, false, BNK>(p, s);
    case ACT_GELU_TANH:
      return fp8 ? launch_t<T, ACT_GELU_TANH, true, BNK>(p, s) : launch_t<T, ACT_GELU_TANH, false, BNK>(p, s);
    case ACT_SILU: return fp8 ? launch_t<T, ACT_SILU, true, BNK>(p, s) : launch_t<T, ACT_SILU, false, BNK>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace ge
