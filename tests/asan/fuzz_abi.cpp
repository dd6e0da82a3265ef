// Host-side fuzzing of the C-ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Random descriptors -- sizes, leading dimensions and strides drawn from pools of edge values
// (0, 1, tile multiples, ragged sizes, 2^31 neighbours, INT64 extremes, negatives) and raw
// random bits; op chains with known and unknown kinds, activations and eps values; dtypes and
// layouts in and out of range -- go through gemm_epilogue_validate, which must return one of its
// documented codes and the same code twice.  Every 64th descriptor also goes through
// gemm_epilogue_create (GE_ERR_DEVICE on a host without a gfx950 GPU), and the other host entry
// points get NULL and out-of-range arguments.  Half of the descriptors are a valid workload
// descriptor with one or two fields mutated, so the deeper checks are reached as well.
//
// Usage: fuzz_abi [seed] [iterations]; prints "fuzz ok" and a status histogram.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>

#include "../../include/gemm_epilogue.h"

namespace {

std::mt19937_64 rng;

uint64_t bits() { return rng(); }
int64_t pick(const int64_t* pool, size_t n) { return pool[bits() % n]; }

const int64_t kSizes[] = {0, 1, 7, 8, 16, 31, 32, 63, 64, 65, 128, 200, 256, 264, 300, 1000, 1024,
                          4096, 8192, 11008, 65536, 1 << 20, (1LL << 31) - 8, 1LL << 31, (1LL << 31) + 8,
                          (1LL << 32), INT64_MAX, INT64_MAX - 7, -1, -8, INT64_MIN};

int64_t size_value() {
  switch (bits() % 4) {
    case 0: return static_cast<int64_t>(bits());                   // raw bits, any sign
    case 1: return static_cast<int64_t>(bits() % 20000);           // plausible
    default: return pick(kSizes, sizeof(kSizes) / sizeof(kSizes[0]));
  }
}

int32_t small_enum(int lo, int hi) {
  if (bits() % 8 == 0) return static_cast<int32_t>(bits());       // anything
  return lo + static_cast<int32_t>(bits() % (uint64_t)(hi - lo + 1));
}

float eps_value() {
  const float pool[] = {0.0f, 1e-6f, 1e-5f, -1e-6f, std::numeric_limits<float>::quiet_NaN(),
                        std::numeric_limits<float>::infinity(), -std::numeric_limits<float>::infinity(),
                        std::numeric_limits<float>::denorm_min(), 3.0e38f};
  if (bits() % 4 == 0) {
    uint32_t u = static_cast<uint32_t>(bits());
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  return pool[bits() % (sizeof(pool) / sizeof(pool[0]))];
}

ge_desc_t random_desc() {
  ge_desc_t d;
  std::memset(&d, 0, sizeof d);
  int64_t* f64[] = {&d.batch, &d.M, &d.N, &d.K, &d.lda, &d.ldb, &d.ldy, &d.ldr,
                    &d.stride_a, &d.stride_b, &d.stride_y, &d.stride_r, &d.ldz, &d.stride_z};
  for (int64_t* p : f64) *p = size_value();
  d.a_type = small_enum(-1, 3);
  d.b_type = small_enum(-1, 3);
  d.y_type = small_enum(-1, 3);
  d.b_layout = small_enum(-1, 2);
  d.tile = small_enum(-1, GE_TILE_COUNT + 1);
  const int32_t n_pool[] = {-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 100, INT32_MIN, INT32_MAX};
  d.n_ops = n_pool[bits() % (sizeof(n_pool) / sizeof(n_pool[0]))];
  for (int i = 0; i < GE_MAX_OPS; ++i) {
    d.ops[i].kind = small_enum(-1, 12);
    d.ops[i].act = small_enum(-1, 5);
    d.ops[i].eps = eps_value();
  }
  return d;
}

// The workload chains the library is built for, as valid starting points.
ge_desc_t valid_desc(int which) {
  ge_desc_t d;
  std::memset(&d, 0, sizeof d);
  auto set = [&](int64_t b, int64_t M, int64_t N, int64_t K) {
    d.batch = b; d.M = M; d.N = N; d.K = K;
    d.lda = K; d.ldb = N; d.ldy = N; d.ldr = N; d.ldz = N;
    d.stride_a = M * K; d.stride_b = K * N; d.stride_y = M * N; d.stride_r = M * N; d.stride_z = M * N;
  };
  auto op = [&](int32_t kind, int32_t act = 0, float eps = 0.0f) {
    d.ops[d.n_ops].kind = kind;
    d.ops[d.n_ops].act = act;
    d.ops[d.n_ops].eps = eps;
    ++d.n_ops;
  };
  switch (which % 6) {
    case 0: set(1, 256, 256, 256); op(GE_OP_SCALE); op(GE_OP_BIAS_COL); op(GE_OP_ACT, GE_ACT_GELU_TANH); op(GE_OP_AMAX); break;
    case 1: set(16, 1024, 1024, 1024); op(GE_OP_SCALE); op(GE_OP_BIAS_COL); op(GE_OP_ACT, GE_ACT_RELU); op(GE_OP_AMAX); break;
    case 2: set(1, 8192, 11008, 4096); op(GE_OP_PAIRWISE_ACT_MUL, GE_ACT_SILU); break;
    case 3: set(1, 8192, 4096, 4096); op(GE_OP_ROW_RMS, 0, 1e-6f); op(GE_OP_RESIDUAL); break;
    case 4:
      set(1, 8192, 8192, 8192); op(GE_OP_BIAS_COL); op(GE_OP_ACT, GE_ACT_GELU_TANH); op(GE_OP_AMAX); op(GE_OP_QUANT_FP8);
      d.y_type = GE_DT_FP8_E4M3;
      break;
    default:
      set(1, 8192, 11008, 4096); op(GE_OP_ACT_GRAD, GE_ACT_GELU_TANH); op(GE_OP_COL_SUM);
      d.b_layout = GE_LAYOUT_NK; d.ldb = 4096; d.stride_b = 11008LL * 4096;
      break;
  }
  return d;
}

void mutate(ge_desc_t& d) {
  const ge_desc_t r = random_desc();
  switch (bits() % 12) {
    case 0: d.batch = r.batch; break;
    case 1: d.M = r.M; break;
    case 2: d.N = r.N; break;
    case 3: d.K = r.K; break;
    case 4: d.lda = r.lda; d.ldb = r.ldb; break;
    case 5: d.ldy = r.ldy; d.ldr = r.ldr; d.ldz = r.ldz; break;
    case 6: d.stride_a = r.stride_a; d.stride_b = r.stride_b; d.stride_y = r.stride_y; break;
    case 7: d.a_type = r.a_type; d.b_type = r.b_type; d.y_type = r.y_type; break;
    case 8: d.b_layout = r.b_layout; d.tile = r.tile; break;
    case 9: d.n_ops = r.n_ops; break;
    case 10: {
      const int i = static_cast<int>(bits() % GE_MAX_OPS);
      d.ops[i] = r.ops[i];
      break;
    }
    default: std::memcpy(d.ops, r.ops, sizeof d.ops); break;
  }
}

[[noreturn]] void fail(const char* what, int v, long it) {
  std::fprintf(stderr, "FAIL at iteration %ld: %s (%d)\n", it, what, v);
  std::abort();
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const long iters = argc > 2 ? std::strtol(argv[2], nullptr, 10) : 200000;
  rng.seed(seed);
  long hist[3] = {0, 0, 0};
  long created = 0, device_err = 0;
  for (long it = 0; it < iters; ++it) {
    ge_desc_t d;
    if (bits() % 2) {
      d = valid_desc(static_cast<int>(bits() % 6));
      const int muts = static_cast<int>(bits() % 3);
      for (int m = 0; m < muts; ++m) mutate(d);
    } else {
      d = random_desc();
    }
    const ge_status_t s = gemm_epilogue_validate(&d);
    if (s != GE_OK && s != GE_ERR_INVALID_ARG && s != GE_ERR_UNSUPPORTED) fail("validate status", s, it);
    if (gemm_epilogue_validate(&d) != s) fail("validate is not deterministic", s, it);
    ++hist[s];
    if (it % 64 == 0) {
      ge_handle_t h = reinterpret_cast<ge_handle_t>(0x1234);
      const ge_status_t c = gemm_epilogue_create(&d, &h);
      if (c != GE_OK && h != nullptr) fail("create left a handle on failure", c, it);
      if (s != GE_OK && c != s) fail("create disagrees with validate", c, it);
      if (c == GE_OK) {
        size_t ws = 0;
        if (gemm_epilogue_workspace_size(h, &ws) != GE_OK) fail("workspace_size", 0, it);
        char buf[64];
        if (gemm_epilogue_describe(h, buf, sizeof buf) != GE_OK || std::strlen(buf) >= sizeof buf) fail("describe", 0, it);
        gemm_epilogue_destroy(h);
        ++created;
      } else if (c == GE_ERR_DEVICE) {
        ++device_err;
      } else if (c != GE_ERR_INVALID_ARG && c != GE_ERR_UNSUPPORTED) {
        fail("create status", c, it);
      }
    }
    if (it % 97 == 0) {
      ge_tile_info_t info;
      const int32_t t = static_cast<int32_t>(bits() % 16) - 4;
      const ge_status_t ts = gemm_epilogue_tile_info(t, &info);
      if ((t >= 0 && t < GE_TILE_COUNT) != (ts == GE_OK)) fail("tile_info", t, it);
      if (ts == GE_OK && (info.bm <= 0 || info.bn <= 0 || info.lds_bytes > 160 * 1024)) fail("tile_info fields", t, it);
      if (!gemm_epilogue_status_string(static_cast<ge_status_t>(static_cast<int>(bits() % 32) - 8)))
        fail("status_string", 0, it);
    }
  }
  // NULL and degenerate arguments of every entry point
  if (gemm_epilogue_validate(nullptr) != GE_ERR_INVALID_ARG) fail("validate(NULL)", 0, -1);
  ge_desc_t d0 = valid_desc(0);
  if (gemm_epilogue_create(&d0, nullptr) != GE_ERR_INVALID_ARG) fail("create(desc, NULL)", 0, -1);
  ge_handle_t h = nullptr;
  if (gemm_epilogue_create(nullptr, &h) != GE_ERR_INVALID_ARG || h) fail("create(NULL, out)", 0, -1);
  size_t ws = 0;
  if (gemm_epilogue_workspace_size(nullptr, &ws) != GE_ERR_INVALID_ARG) fail("workspace_size(NULL)", 0, -1);
  if (gemm_epilogue_run(nullptr, nullptr, nullptr) != GE_ERR_INVALID_ARG) fail("run(NULL)", 0, -1);
  if (gemm_epilogue_run_noalloc(nullptr, nullptr, nullptr) != GE_ERR_INVALID_ARG) fail("run_noalloc(NULL)", 0, -1);
  char buf[8];
  if (gemm_epilogue_describe(nullptr, buf, sizeof buf) != GE_ERR_INVALID_ARG) fail("describe(NULL)", 0, -1);
  if (gemm_epilogue_tile_info(0, nullptr) != GE_ERR_INVALID_ARG) fail("tile_info(NULL)", 0, -1);
  gemm_epilogue_destroy(nullptr);
  std::printf("fuzz ok: seed %llu, %ld descriptors: GE_OK %ld, GE_ERR_INVALID_ARG %ld, GE_ERR_UNSUPPORTED %ld; "
              "create: %ld plans, %ld GE_ERR_DEVICE\n",
              (unsigned long long)seed, iters, hist[0], hist[1], hist[2], created, device_err);
  return 0;
}
