// C-ABI of the fused GEMM-epilogue library: validate / create / run / destroy.
//
// The split follows the cuDNN Graph API tutorial's build-then-execute model
// (opening paragraph): a descriptor is checked and turned into a plan once
// (validate, support check, kernel choice), then executed many times against a
// pack of device pointers with host scalars (batched-matmul paragraph: alpha is
// a host scalar).  The op set is the CODA news item's epilogue primitive set
// ("How CODA works").  The handle holds host memory only.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/gemm_epilogue.h"
#include "ge_internal.h"

struct ge_plan {
  ge_desc_t desc;
  ge::TileKind tile;
  int act;            // ge::Act
  bool fp8_out;
  uint32_t flags;     // ge::F_*
  float eps;
  int64_t tiles_m, tiles_n;
};

namespace {

static_assert(GE_TILE_256x256 == ge::TILE_256x256 && GE_TILE_256x128_PAIR == ge::TILE_256x128_PAIR &&
                  GE_TILE_128x128 == ge::TILE_128x128 && GE_TILE_64x64 == ge::TILE_64x64 &&
                  GE_TILE_128x128_PAIR == ge::TILE_128x128_PAIR && GE_TILE_256x256_2W == ge::TILE_256x256_2W &&
                  GE_TILE_256x128_PAIR_2W == ge::TILE_256x128_PAIR_2W && GE_TILE_COUNT == ge::TILE_KIND_COUNT,
              "public tile ids mirror the kernel instances");

constexpr int64_t kMaxExtent = 0x7FFFFFF0;   // buffer extents are 31-bit byte counts

int op_rank(int kind) {
  switch (kind) {
    case GE_OP_SCALE: return 0;
    case GE_OP_ROW_RMS:
    case GE_OP_ROW_SCALE: return 1;
    case GE_OP_BIAS_COL: return 2;
    case GE_OP_ACT:
    case GE_OP_PAIRWISE_ACT_MUL:
    case GE_OP_ACT_GRAD: return 3;
    case GE_OP_RESIDUAL: return 4;
    case GE_OP_COL_SUM: return 5;
    case GE_OP_AMAX: return 6;
    case GE_OP_QUANT_FP8: return 7;
    default: return -1;
  }
}

bool has_op(const ge_desc_t* d, int kind) {
  for (int i = 0; i < d->n_ops; ++i)
    if (d->ops[i].kind == kind) return true;
  return false;
}

const ge_op_t* find_op(const ge_desc_t* d, int kind) {
  for (int i = 0; i < d->n_ops; ++i)
    if (d->ops[i].kind == kind) return &d->ops[i];
  return nullptr;
}

// Bytes from a matrix's base to one past its last element: ((rows-1)*ld + cols) * esize,
// saturating at INT64_MAX (every such extent is then rejected): descriptors come from callers,
// so leading dimensions may be anything non-negative.
int64_t extent_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  if (rows <= 0 || cols <= 0) return 0;
  int64_t e;
  if (__builtin_mul_overflow(rows - 1, ld, &e) || __builtin_add_overflow(e, cols, &e) ||
      __builtin_mul_overflow(e, esize, &e))
    return INT64_MAX;
  return e;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The two-wave instances need K to be a multiple of two steps: 64 (bf16) or 128 (fp8) values.
bool two_wave_ok(const ge_desc_t* d);

ge::TileKind pick_tile(const ge_desc_t* d, bool pair) {
  if (d->tile > 0) return (ge::TileKind)(d->tile - 1);        // validated: matches the chain
  const char* force = std::getenv("GE_FORCE_TILE");
  if (force && *force) {
    const int k = std::atoi(force);
    if (k >= 0 && k < ge::TILE_KIND_COUNT && ge::tile_info((ge::TileKind)k).pair == pair &&
        (!ge::two_wave_tile((ge::TileKind)k) || two_wave_ok(d)))
      return (ge::TileKind)k;
  }
  auto tiles = [&](int bm, int bn) { return ceil_div(d->M, bm) * ceil_div(d->N, bn) * d->batch; };
  // the largest tile that still gives >= 256 workgroups; at 256 x 256 (256 x 128 pairwise) the
  // two-wave instance where it applies (its matrix cores are fed by one wave while the other
  // loads)
  const bool tw = two_wave_ok(d);
  if (pair) {
    if (tiles(256, 128) < 256) return ge::TILE_128x128_PAIR;
    return tw ? ge::TILE_256x128_PAIR_2W : ge::TILE_256x128_PAIR;
  }
  if (tiles(256, 256) >= 256) return tw ? ge::TILE_256x256_2W : ge::TILE_256x256;
  if (tiles(128, 128) >= 128) return ge::TILE_128x128;
  return ge::TILE_64x64;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool two_wave_ok(const ge_desc_t* d) {
  return d->K % (d->a_type == GE_DT_FP8_E4M3 ? 128 : 64) == 0;
}

}  // namespace

extern "C" {

ge_status_t gemm_epilogue_validate(const ge_desc_t* d) {
  if (!d) return GE_ERR_INVALID_ARG;
  if (d->batch < 0 || d->M < 0 || d->N < 0 || d->K < 0) return GE_ERR_INVALID_ARG;
  if (d->n_ops < 0 || d->n_ops > GE_MAX_OPS) return GE_ERR_INVALID_ARG;
  if (d->lda < 0 || d->ldb < 0 || d->ldy < 0 || d->ldr < 0) return GE_ERR_INVALID_ARG;
  if (d->stride_a < 0 || d->stride_b < 0 || d->stride_y < 0 || d->stride_r < 0) return GE_ERR_INVALID_ARG;
  if (d->b_layout != GE_LAYOUT_KN && d->b_layout != GE_LAYOUT_NK) return GE_ERR_INVALID_ARG;
  if (d->tile < 0 || d->tile > GE_TILE_COUNT) return GE_ERR_INVALID_ARG;
  const bool bnk = d->b_layout == GE_LAYOUT_NK;
  // sizes beyond 32 bits are outside the supported set; past this point M + 256 etc. cannot overflow
  const bool huge = d->M > INT32_MAX || d->N > INT32_MAX || d->K > INT32_MAX || d->batch > INT32_MAX;

  // op chain: known kinds, canonical order, each at most once, exclusive pairs
  int last_rank = -1;
  for (int i = 0; i < d->n_ops; ++i) {
    const ge_op_t& op = d->ops[i];
    const int r = op_rank(op.kind);
    if (r < 0) return GE_ERR_INVALID_ARG;
    if (r <= last_rank) return GE_ERR_INVALID_ARG;
    last_rank = r;
    if (op.kind == GE_OP_ACT || op.kind == GE_OP_PAIRWISE_ACT_MUL || op.kind == GE_OP_ACT_GRAD) {
      if (op.act < GE_ACT_NONE || op.act > GE_ACT_SILU) return GE_ERR_INVALID_ARG;
    }
    if (op.kind == GE_OP_ROW_RMS) {
      if (!std::isfinite(op.eps) || op.eps < 0.0f) return GE_ERR_INVALID_ARG;
    }
  }
  const bool pair = has_op(d, GE_OP_PAIRWISE_ACT_MUL);
  const bool quant = has_op(d, GE_OP_QUANT_FP8);
  if (has_op(d, GE_OP_ROW_RMS) && d->K < 1) return GE_ERR_INVALID_ARG;
  // a requested instance must be a pairwise one exactly when the chain is pairwise
  if (d->tile > 0 && ge::tile_info((ge::TileKind)(d->tile - 1)).pair != pair) return GE_ERR_INVALID_ARG;
  const bool two_wave_requested = d->tile > 0 && ge::two_wave_tile((ge::TileKind)(d->tile - 1));

  // dtypes: bf16 operands, or fp8-e4m3 operands with B given [N][K]
  auto known = [](int32_t t) { return t == GE_DT_BF16 || t == GE_DT_FP8_E4M3 || t == GE_DT_FP32; };
  if (!known(d->a_type) || !known(d->b_type)) return GE_ERR_INVALID_ARG;
  const bool f8in = d->a_type == GE_DT_FP8_E4M3;
  if (f8in) {
    if (d->b_type != GE_DT_FP8_E4M3 || !bnk) return GE_ERR_UNSUPPORTED;
    // the fp8 instances run forward epilogues without the in-kernel row statistic
    if (has_op(d, GE_OP_ROW_RMS) || has_op(d, GE_OP_ACT_GRAD)) return GE_ERR_UNSUPPORTED;
  } else if (d->a_type != GE_DT_BF16 || d->b_type != GE_DT_BF16) {
    return GE_ERR_UNSUPPORTED;
  }
  if (d->y_type == GE_DT_FP8_E4M3) {
    if (!quant) return GE_ERR_INVALID_ARG;
  } else if (d->y_type == GE_DT_BF16) {
    if (quant) return GE_ERR_INVALID_ARG;
  } else if (d->y_type == GE_DT_FP32) {
    return GE_ERR_UNSUPPORTED;
  } else {
    return GE_ERR_INVALID_ARG;
  }
  if (pair && has_op(d, GE_OP_BIAS_COL)) return GE_ERR_UNSUPPORTED;
  // the activation-gradient instances write bf16 and take no in-kernel row statistic
  if (has_op(d, GE_OP_ACT_GRAD) && (quant || has_op(d, GE_OP_ROW_RMS))) return GE_ERR_UNSUPPORTED;

  // layout
  const bool res = has_op(d, GE_OP_RESIDUAL);
  const bool grad = has_op(d, GE_OP_ACT_GRAD);
  if (grad && (d->ldz < 0 || d->stride_z < 0)) return GE_ERR_INVALID_ARG;
  if (grad && d->M > 0 && d->ldz < d->N) return GE_ERR_INVALID_ARG;
  if (grad && (d->ldz % 8 || d->stride_z % 8)) return GE_ERR_UNSUPPORTED;
  if (grad && !huge && extent_bytes(d->M + 256, d->N, d->ldz, 2) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  if (d->M > 0 && d->lda < d->K) return GE_ERR_INVALID_ARG;
  if (!bnk && d->K > 0 && d->ldb < d->N) return GE_ERR_INVALID_ARG;
  if (bnk && d->N > 0 && d->ldb < d->K) return GE_ERR_INVALID_ARG;
  if (d->M > 0 && d->ldy < d->N) return GE_ERR_INVALID_ARG;
  if (res && d->M > 0 && d->ldr < d->N) return GE_ERR_INVALID_ARG;
  if (d->batch > 1 && d->stride_y == 0 && d->M > 0 && d->N > 0) return GE_ERR_INVALID_ARG;  // batches would race

  // supported set: 16-byte vector access everywhere (16 fp8 operand values per 16 bytes)
  if (huge) return GE_ERR_UNSUPPORTED;
  if (two_wave_requested && !two_wave_ok(d)) return GE_ERR_UNSUPPORTED;
  if (d->N % 8 || d->K % 8) return GE_ERR_UNSUPPORTED;
  if (f8in && (d->K % 16 || d->lda % 16 || d->ldb % 16 || d->stride_a % 16 || d->stride_b % 16))
    return GE_ERR_UNSUPPORTED;
  if (d->lda % 8 || d->ldb % 8 || d->ldy % 8 || (res && d->ldr % 8)) return GE_ERR_UNSUPPORTED;
  if (d->stride_a % 8 || d->stride_b % 8 || d->stride_y % 8 || (res && d->stride_r % 8))
    return GE_ERR_UNSUPPORTED;
  const int64_t esize = d->y_type == GE_DT_FP8_E4M3 ? 1 : 2;
  // Kernels address each operand with 32-bit byte offsets from a per-tile base and mark
  // masked accesses with an offset of 2^31; every offset a tile can form (one tile and one
  // K step past the end included) must therefore stay below 2^31.
  // (operand element size ae; one A slot spans slot_k K values)
  const int64_t ae = f8in ? 1 : 2, slot_k = f8in ? 128 : 64;
  if (extent_bytes(d->M + 256, d->K + slot_k, d->lda, ae) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  if (!bnk && extent_bytes(d->K + 128, d->N, d->ldb, 2) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  if (bnk && extent_bytes(d->N + 256, d->K + slot_k, d->ldb, ae) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  if (extent_bytes(d->M + 256, d->N, d->ldy, esize) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  if (res && extent_bytes(d->M + 256, d->N, d->ldr, 2) > kMaxExtent) return GE_ERR_UNSUPPORTED;
  // grid: one workgroup per 64x64 tile at most (M, N, batch < 2^31 here: the product of the
  // first two fits, the third factor is checked by division)
  const int64_t tiles64 = ceil_div(d->M, 64) * ceil_div(d->N, 64);
  if (tiles64 > 0 && d->batch > INT32_MAX / tiles64) return GE_ERR_UNSUPPORTED;
  return GE_OK;
}

ge_status_t gemm_epilogue_create(const ge_desc_t* desc, ge_handle_t* out) {
  if (!out) return GE_ERR_INVALID_ARG;
  *out = nullptr;
  const ge_status_t st = gemm_epilogue_validate(desc);
  if (st != GE_OK) return st;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return GE_ERR_DEVICE;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GE_ERR_DEVICE;

  ge_plan* p = new (std::nothrow) ge_plan();
  if (!p) return GE_ERR_HIP;
  p->desc = *desc;
  const bool pair = has_op(desc, GE_OP_PAIRWISE_ACT_MUL);
  p->tile = pick_tile(desc, pair);
  p->fp8_out = desc->y_type == GE_DT_FP8_E4M3;
  p->act = ge::ACT_NONE;
  if (const ge_op_t* a = find_op(desc, GE_OP_ACT)) p->act = a->act;
  if (const ge_op_t* a = find_op(desc, GE_OP_PAIRWISE_ACT_MUL)) p->act = a->act;
  p->flags = 0;
  if (has_op(desc, GE_OP_SCALE)) p->flags |= ge::F_SCALE;
  if (has_op(desc, GE_OP_ROW_SCALE)) p->flags |= ge::F_ROW_SCALE;
  if (const ge_op_t* r = find_op(desc, GE_OP_ROW_RMS)) {
    p->flags |= ge::F_ROW_RMS;
    p->eps = r->eps;
  } else {
    p->eps = 0.0f;
  }
  if (has_op(desc, GE_OP_BIAS_COL)) p->flags |= ge::F_BIAS;
  if (has_op(desc, GE_OP_RESIDUAL)) p->flags |= ge::F_RESIDUAL;
  if (has_op(desc, GE_OP_AMAX)) p->flags |= ge::F_AMAX;
  if (const ge_op_t* g = find_op(desc, GE_OP_ACT_GRAD)) {
    p->flags |= ge::F_ACT_GRAD;
    p->act = g->act;
  }
  if (has_op(desc, GE_OP_COL_SUM)) p->flags |= ge::F_COL_SUM;
  if (desc->b_layout == GE_LAYOUT_NK) p->flags |= ge::F_B_NK;
  if (desc->a_type == GE_DT_FP8_E4M3) p->flags |= ge::F_IN_FP8;
  const ge::TileInfo ti = ge::tile_info(p->tile);
  p->tiles_m = ceil_div(desc->M, ti.bm);
  p->tiles_n = ceil_div(desc->N, ti.bn);
  // two-wave RMS plans with several tile columns: a tile that starts after another tile of its
  // tile row has published the row statistic reads it instead of recomputing it
  if ((p->flags & ge::F_ROW_RMS) && ge::two_wave_tile(p->tile) && p->tiles_n > 1) p->flags |= ge::F_RS_SHARE;
  *out = p;
  return GE_OK;
}

namespace {
ge::WsLayout layout_of(const ge_plan* h) {
  const int64_t wgs = h->tiles_m * h->tiles_n * h->desc.batch;
  return ge::ws_layout((h->flags & ge::F_AMAX) != 0, (h->flags & ge::F_COL_SUM) != 0,
                       (h->flags & ge::F_RS_SHARE) != 0, wgs, h->tiles_n, h->desc.batch * h->tiles_m, h->desc.N,
                       ge::tile_info(h->tile).bm);
}
size_t workspace_bytes(const ge_plan* h) { return 4 * layout_of(h).total; }
}  // namespace

ge_status_t gemm_epilogue_workspace_size(ge_handle_t h, size_t* bytes) {
  if (!h || !bytes) return GE_ERR_INVALID_ARG;
  *bytes = workspace_bytes(h);
  return GE_OK;
}

namespace {

bool empty_problem(const ge_desc_t& d) { return d.batch == 0 || d.M == 0 || d.N == 0; }

// Every pointer the plan's chain needs is present and aligned, and the workspace is large
// enough; nothing is enqueued before this passes.
ge_status_t check_args(const ge_plan* h, const ge_args_t* a) {
  const ge_desc_t& d = h->desc;
  const bool empty = empty_problem(d);
  const uint32_t f = h->flags;

  if (f & ge::F_AMAX) {
    if (!a->amax || !aligned(a->amax, 4)) return GE_ERR_INVALID_ARG;
  }
  if (f & ge::F_COL_SUM) {
    if (d.N > 0 && (!a->col_sum || !aligned(a->col_sum, 4))) return GE_ERR_INVALID_ARG;
  }
  if ((f & (ge::F_AMAX | ge::F_COL_SUM)) && !empty &&
      (!a->workspace || !aligned(a->workspace, 16) || a->workspace_bytes < workspace_bytes(h)))
    return GE_ERR_INVALID_ARG;
  if (!empty) {
    if (!a->Y || !aligned(a->Y, 16)) return GE_ERR_INVALID_ARG;
    if (d.K > 0) {
      if (!a->A || !a->B || !aligned(a->A, 16) || !aligned(a->B, 16)) return GE_ERR_INVALID_ARG;
      if (ge::tile_info(h->tile).pair) {
        if (!a->B2 || !aligned(a->B2, 16)) return GE_ERR_INVALID_ARG;
      }
    }
    if ((f & ge::F_BIAS) && (!a->bias || !aligned(a->bias, 16))) return GE_ERR_INVALID_ARG;
    if ((f & ge::F_ROW_SCALE) && (!a->row_scale || !aligned(a->row_scale, 4))) return GE_ERR_INVALID_ARG;
    if ((f & ge::F_RESIDUAL) && (!a->residual || !aligned(a->residual, 16))) return GE_ERR_INVALID_ARG;
    if ((f & ge::F_ACT_GRAD) && (!a->aux || !aligned(a->aux, 16))) return GE_ERR_INVALID_ARG;
  }

  return GE_OK;
}

// Enqueues the plan's work (arguments already checked).
ge_status_t enqueue(const ge_plan* h, const ge_args_t* a, hipStream_t s) {
  const ge_desc_t& d = h->desc;
  const bool empty = empty_problem(d);
  const uint32_t f = h->flags;

  if (empty) {
    // nothing to reduce: AMAX of no outputs is 0
    if ((f & ge::F_AMAX) && ge::launch_amax_zero(reinterpret_cast<uint32_t*>(a->amax), s) != hipSuccess)
      return GE_ERR_HIP;
    // and the column sums over no rows are 0
    if ((f & ge::F_COL_SUM) && d.N > 0 &&
        ge::launch_zero_words(reinterpret_cast<uint32_t*>(a->col_sum), d.N, s) != hipSuccess)
      return GE_ERR_HIP;
    return GE_OK;
  }

  ge::Params p;
  p.A = static_cast<const uint16_t*>(a->A);
  p.B = static_cast<const uint16_t*>(a->B);
  p.B2 = static_cast<const uint16_t*>(a->B2);
  p.bias = static_cast<const uint16_t*>(a->bias);
  p.row_scale = a->row_scale;
  p.R = static_cast<const uint16_t*>(a->residual);
  p.Y = a->Y;
  p.amax = reinterpret_cast<uint32_t*>(a->amax);
  p.ws = static_cast<uint32_t*>(a->workspace);
  p.Z = static_cast<const uint16_t*>(a->aux);
  p.col_sum = a->col_sum;
  {
    const ge::WsLayout l = layout_of(h);
    p.cs_ctr = (f & ge::F_COL_SUM) ? p.ws + l.cs_ctr : nullptr;
    p.cs_part = (f & ge::F_COL_SUM) ? reinterpret_cast<float*>(p.ws + l.cs_part) : nullptr;
    p.rs_ctr = (f & ge::F_RS_SHARE) ? p.ws + l.rs_ctr : nullptr;
    p.rs_val = (f & ge::F_RS_SHARE) ? reinterpret_cast<float*>(p.ws + l.rs_val) : nullptr;
  }
  p.ldz = d.ldz;
  p.sz = d.stride_z;
  p.lda = d.lda;
  p.ldb = d.ldb;
  p.ldy = d.ldy;
  p.ldr = d.ldr;
  p.sa = d.stride_a;
  p.sb = d.stride_b;
  p.sy = d.stride_y;
  p.sr = d.stride_r;
  p.M = (int32_t)d.M;
  p.N = (int32_t)d.N;
  p.K = (int32_t)d.K;
  p.batch = (int32_t)d.batch;
  p.tiles_m = (int32_t)h->tiles_m;
  p.tiles_n = (int32_t)h->tiles_n;
  p.alpha = a->alpha;
  p.qscale = a->quant_scale;
  p.eps = h->eps;
  p.flags = f;
  if (ge::launch_fused(h->tile, h->act, h->fp8_out, p, s) != hipSuccess) return GE_ERR_HIP;
  return GE_OK;
}

}  // namespace

ge_status_t gemm_epilogue_run(ge_handle_t h, const ge_args_t* a, void* stream) {
  if (!h || !a) return GE_ERR_INVALID_ARG;
  const ge_status_t st = check_args(h, a);
  if (st != GE_OK) return st;
  return enqueue(h, a, reinterpret_cast<hipStream_t>(stream));
}

ge_status_t gemm_epilogue_run_noalloc(ge_handle_t h, const ge_args_t* a, void* stream) {
  if (!h || !a) return GE_ERR_INVALID_ARG;
  const ge_desc_t& d = h->desc;
  const size_t need = workspace_bytes(h);
  const bool uses_scratch = need > 0 && !empty_problem(d);
  if (uses_scratch && need > GE_NOALLOC_SCRATCH_BYTES) return GE_ERR_SCRATCH;
  ge_args_t b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (uses_scratch) {
    void* ptr = nullptr;
    if (ge::noalloc_scratch(&ptr) != hipSuccess || !ptr) return GE_ERR_HIP;
    b.workspace = ptr;
    b.workspace_bytes = need;
  }
  const ge_status_t st = check_args(h, &b);
  if (st != GE_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (uses_scratch) {
    // the array keeps the previous call's contents, possibly another plan's partials where this
    // plan keeps its counters: zero the counters (a kernel, not a memset node)
    const size_t words = layout_of(h).counters;
    if (ge::launch_zero_words(static_cast<uint32_t*>(b.workspace), (int64_t)words, s) != hipSuccess)
      return GE_ERR_HIP;
  }
  return enqueue(h, &b, s);
}

void gemm_epilogue_destroy(ge_handle_t h) { delete h; }

const char* gemm_epilogue_status_string(ge_status_t s) {
  switch (s) {
    case GE_OK: return "GE_OK";
    case GE_ERR_INVALID_ARG: return "GE_ERR_INVALID_ARG: malformed descriptor or argument";
    case GE_ERR_UNSUPPORTED: return "GE_ERR_UNSUPPORTED: outside the supported set";
    case GE_ERR_DEVICE: return "GE_ERR_DEVICE: no gfx950 device is current";
    case GE_ERR_HIP: return "GE_ERR_HIP: a HIP call or kernel launch failed";
    case GE_ERR_SCRATCH: return "GE_ERR_SCRATCH: the plan needs more scratch than GE_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

ge_status_t gemm_epilogue_tile_info(int32_t tile, ge_tile_info_t* info) {
  if (!info || tile < 0 || tile >= GE_TILE_COUNT) return GE_ERR_INVALID_ARG;
  const ge::TileInfo ti = ge::tile_info((ge::TileKind)tile);
  info->bm = ti.bm;
  info->bn = ti.bn;
  info->pairwise = ti.pair ? 1 : 0;
  info->threads = ti.threads;
  info->lds_bytes = ti.lds_bytes;
  return GE_OK;
}

ge_status_t gemm_epilogue_describe(ge_handle_t h, char* buf, size_t len) {
  if (!h || !buf || len == 0) return GE_ERR_INVALID_ARG;
  const ge::TileInfo ti = ge::tile_info(h->tile);
  std::snprintf(buf, len, "tile=%dx%dx64 pair=%d in=%s b=%s threads=%d lds=%d grid=%lld act=%d fp8=%d flags=0x%x%s",
                ti.bm, ti.bn, ti.pair ? 1 : 0, (h->flags & ge::F_IN_FP8) ? "fp8" : "bf16",
                (h->flags & ge::F_B_NK) ? "NK" : "KN", ti.threads, ti.lds_bytes,
                (long long)(h->tiles_m * h->tiles_n * h->desc.batch), h->act, h->fp8_out ? 1 : 0,
                (unsigned)h->flags, GE_SERIAL_PIPELINE ? " pipeline=serial" : "");
  return GE_OK;
}

}  // extern "C"
