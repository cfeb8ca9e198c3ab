// libtpmlp: C ABI, argument validation, launch planning and the per-kernel
// timing hook.  The operations and their conventions are documented in
// include/tpmlp.h; the kernels live in gemm.hpp and reduce.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tpmlp.h"

#include "gemm.hpp"
#include "gemm_bf16.hpp"
#include "gemm_w4.hpp"
#include "reduce.hpp"
#include "attn.hpp"
#include "sp.hpp"
#include "swiglu.hpp"
#include "epilogue.hpp"

using namespace tpmlp;

namespace {

// ------------------------------------------------------------------ status --
thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TPMLP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TPMLP_TRY(expr)               \
  do {                                \
    int _st = (expr);                 \
    if (_st != TPMLP_OK) return _st;  \
  } while (0)

// -------------------------------------------------------------- profiling --
struct ProfRecord {
  std::string role, symbol;
  hipEvent_t start, stop;
  int clk_slot;  // slot of the clock buffer this launch wrote, or -1
};

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::string filter;
  std::vector<ProfRecord> records;
  std::vector<hipEvent_t> pool;
  // Clock samples of profiled GEMM launches: kClkSlots pairs of (shader
  // clock ticks, 100 MHz ticks), device memory allocated by
  // tpmlp_profile_enable on the device current then.
  static constexpr int kClkSlots = 4096;
  unsigned long long* clk = nullptr;
  int clk_device = -1;
  int clk_next = 0;
  int pending_slot = -1;  // slot handed to the launch being prepared

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Profiler& prof() {
  static Profiler p;
  return p;
}

// Launches `kernel` on `stream`; when profiling matches `role`, brackets the
// launch with two events on the same stream.
template <typename Kernel, typename... Args>
int launch(const char* role, const char* symbol, Kernel kernel, dim3 grid, dim3 block,
           hipStream_t stream, Args... args) {
  Profiler& P = prof();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int slot = -1;
  {
    std::lock_guard<std::mutex> lk(P.mu);
    slot = P.pending_slot;
    P.pending_slot = -1;
    if (P.enabled && std::strstr(role, P.filter.c_str()) != nullptr) {
      e0 = P.take();
      e1 = P.take();
    }
  }
  if (e0 && e1) {
    hipError_t e = hipEventRecord(e0, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(err, role);
  if (e0 && e1) {
    hipError_t e = hipEventRecord(e1, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    std::lock_guard<std::mutex> lk(P.mu);
    P.records.push_back({role, symbol, e0, e1, slot});
  }
  return TPMLP_OK;
}

// Clock-buffer slot for a GEMM launch of `role` when profiling covers it on
// the current device; null otherwise.
unsigned long long* prof_clock_slot(const char* role) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  P.pending_slot = -1;
  if (!P.enabled || P.clk == nullptr || std::strstr(role, P.filter.c_str()) == nullptr) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != P.clk_device) return nullptr;
  P.pending_slot = P.clk_next;
  P.clk_next = (P.clk_next + 1) % Profiler::kClkSlots;
  return P.clk + 2 * P.pending_slot;
}

// ------------------------------------------------------------ device info --
int device_cus(int* cus) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(TPMLP_E_HIP, "device index %d out of range", dev);
  if (cache[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    cache[dev] = n > 0 ? n : 256;
  }
  *cus = cache[dev];
  return TPMLP_OK;
}

// ------------------------------------------------------------- validation --
int elem_size(int dtype) { return dtype == TPMLP_BF16 ? 2 : 4; }
int chunk_elems(int dtype) { return 16 / elem_size(dtype); }

int check_dtype(int dtype) {
  if (dtype != TPMLP_BF16 && dtype != TPMLP_F32) return fail(TPMLP_E_DTYPE, "unknown dtype %d", dtype);
  return TPMLP_OK;
}

int check_act(int act) {
  if (act != TPMLP_ACT_NONE && act != TPMLP_ACT_GELU_TANH) return fail(TPMLP_E_ACT, "unknown activation %d", act);
  return TPMLP_OK;
}

int check_split(const char* what, int64_t n, int tp) {
  if (tp < 1) return fail(TPMLP_E_DIVISIBILITY, "tp_size %d < 1", tp);
  if (n >= 1 && n % tp != 0)
    return fail(TPMLP_E_DIVISIBILITY, "%s = %lld is not divisible by tp_size %d", what, (long long)n, tp);
  return TPMLP_OK;
}

constexpr int64_t kMaxDim = 0x7fffffff;

int check_rows(const char* what, int64_t t) {
  if (t < 0 || t > kMaxDim) return fail(TPMLP_E_SHAPE, "%s = %lld out of range [0, 2^31-1]", what, (long long)t);
  return TPMLP_OK;
}

int check_dim(const char* what, int64_t n) {
  if (n < 1 || n > kMaxDim) return fail(TPMLP_E_SHAPE, "%s = %lld out of range [1, 2^31-1]", what, (long long)n);
  return TPMLP_OK;
}

// A matrix operand: rows x width with leading dimension ld, element count
// multiple `vec` for width and ld, pointer 16-byte aligned.
int check_mat(const char* what, const void* p, int64_t rows, int64_t width, int64_t ld, int vec,
              bool required = true) {
  const bool empty = rows == 0 || width == 0;
  if (p == nullptr) {
    if (required && !empty) return fail(TPMLP_E_NULL, "%s is NULL", what);
    return TPMLP_OK;
  }
  if (ld < width) return fail(TPMLP_E_SHAPE, "%s: ld %lld < width %lld", what, (long long)ld, (long long)width);
  if (width % vec != 0 || ld % vec != 0)
    return fail(TPMLP_E_ALIGNMENT, "%s: width %lld and ld %lld must be multiples of %d elements", what,
                (long long)width, (long long)ld, vec);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(TPMLP_E_ALIGNMENT, "%s is not 16-byte aligned", what);
  return TPMLP_OK;
}

int check_vec(const char* what, const void* p, int64_t n, bool required) {
  if (p == nullptr) {
    if (required && n > 0) return fail(TPMLP_E_NULL, "%s is NULL", what);
    return TPMLP_OK;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(TPMLP_E_ALIGNMENT, "%s is not 16-byte aligned", what);
  return TPMLP_OK;
}

// --------------------------------------------------------------- planning --
struct TileCfg {
  int bm, bn, occ;   // tile, workgroups per CU
  float eff, eff_act; // measured relative throughput: plain fp32 epilogue / activation epilogues
  bool f32_epi_only;  // too many registers for the activation epilogues
};
// bf16: the four-wave kernel (gemm_w4.hpp) at 256x256 (128x128 per wave) is
// fastest when it fills the chip; at 128x128 (64x64 per wave, two workgroups
// per CU) it serves grids that 256x256 tiles would leave part idle: with
// whole rounds on both, 8192x4096x3072 ran 168 us at 256x256 and 224 us at
// 128x128 (0.75), and at 128x128 it beat the eight-wave kernel's 128x128
// tile on every MLP and attention product shape measured (by 5-20%; a
// 256x128 tile, one workgroup per CU, ran at 0.71 and never won by more than
// 2%).  The eight-wave kernel (gemm_bf16.hpp) keeps 256x320 (8 waves as
// 4 x 2, 64x160 per wave) for fp32 outputs whose width (5120) leaves 256x256
// a fraction of a round short: 4096x5120x3840 at 256 tiles of 256x320 ran
// 134 us in the attention block's step against 172 us at 256x256 (0.82 of
// the 256x256 rate per tile).  The four-wave kernel at 256x192 (128x96 per
// wave) serves widths of 1536, 3072 and 6144 that leave 256x256 a
// quarter or half round short: per tile it runs at 0.80 of 256x256's rate
// (2048x6144x12288 with bias+GeLU: 243 us in one round of 256x192 against
// 258 us in 3/4 of a round of 256x256; 8192x1536x4096: 79 against 92 us).
constexpr TileCfg kCfgBf16[] = {{256, 256, 1, 1.00f, 1.00f, false},
                                {128, 128, 2, 0.75f, 0.75f, false},
                                {256, 320, 1, 0.82f, 0.82f, true},
                                {256, 192, 1, 0.80f, 0.80f, false}};
constexpr TileCfg kCfgF32[] = {{128, 128, 1, 1.00f, 1.00f, false}, {64, 64, 1, 0.60f, 0.60f, false}};
constexpr int kMinBM = 64;  // smallest BM of any configuration (bounds per-tile column-sum rows)

int plan_cfg(int dtype, int M, int N, int epi, int cus) {
  const TileCfg* cfgs = dtype == TPMLP_BF16 ? kCfgBf16 : kCfgF32;
  const int n = dtype == TPMLP_BF16 ? (int)(sizeof(kCfgBf16) / sizeof(kCfgBf16[0]))
                                    : (int)(sizeof(kCfgF32) / sizeof(kCfgF32[0]));
  int best = 0;
  double best_score = -1.0;
  for (int i = 0; i < n; ++i) {
    if (cfgs[i].f32_epi_only && epi != kEpiF32) continue;
    const int64_t tiles = (int64_t)((M + cfgs[i].bm - 1) / cfgs[i].bm) * ((N + cfgs[i].bn - 1) / cfgs[i].bn);
    const int64_t slots = (int64_t)cus * cfgs[i].occ;
    const int64_t rounds = (tiles + slots - 1) / slots;
    // useful fraction of the workgroup slots over all rounds, times the
    // fraction of the padded tile area that is real output, times the
    // configuration's measured relative throughput
    const double fill = (double)tiles / (double)(rounds * slots);
    const double pad = ((double)M * N) / ((double)tiles * cfgs[i].bm * cfgs[i].bn);
    const double score = fill * pad * (epi == kEpiF32 ? cfgs[i].eff : cfgs[i].eff_act);
    if (score > best_score + 1e-9) {
      best_score = score;
      best = i;
    }
  }
  return best;
}

template <typename T, int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI>
int run_gemm_cfg(const char* role, GemmArgs a, hipStream_t s) {
  constexpr int BK = 8 * Elem<T>::kPerChunk;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  if (a.splits < 1) a.splits = 1;
  if (a.splits == 1) {
    a.k_per_split = ((a.K + BK - 1) / BK) * BK;
  } else {
    const int per = (a.K + a.splits - 1) / a.splits;
    a.k_per_split = ((per + BK - 1) / BK) * BK;
  }
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * a.splits;
  if (grid <= 0) return TPMLP_OK;
  if (grid > 0x7fffffff) return fail(TPMLP_E_SHAPE, "%s: grid too large", role);
  char sym[128];
  snprintf(sym, sizeof(sym), "gemm_kernel<%s,%d,%d,%d,%d,%d,%d,%d>", sizeof(T) == 2 ? "bf16" : "f32", BM, BN,
           WGM, WGN, (int)AK, (int)BKM, EPI);
  return launch(role, sym, gemm_kernel<T, BM, BN, WGM, WGN, AK, BKM, EPI>, dim3((unsigned)grid),
                dim3(WGM * WGN * 64), s, a);
}

template <int BM, int BN, bool AK, bool BKM, int EPI, int NS, int OCC, int BKT, int WGN = 2, int WGM = 2>
int run_gemm_bf16(const char* role, GemmArgs a, hipStream_t s, int group) {
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.group_m = group;
  if (a.splits < 1) a.splits = 1;
  const int per = (a.K + a.splits - 1) / a.splits;
  a.k_per_split = ((per + BKT - 1) / BKT) * BKT;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * a.splits;
  if (grid <= 0) return TPMLP_OK;
  if (grid > 0x7fffffff) return fail(TPMLP_E_SHAPE, "%s: grid too large", role);
  char sym[128];
  snprintf(sym, sizeof(sym), "gemm_bf16_kernel<%d,%d,%d,%d,%d,%d,%d,%d,%d,%d>", BM, BN, (int)AK, (int)BKM, EPI,
           NS, OCC, BKT, WGN, WGM);
  a.clk = prof_clock_slot(role);
  return launch(role, sym, gemm_bf16_kernel<BM, BN, AK, BKM, EPI, NS, OCC, BKT, WGN, WGM>, dim3((unsigned)grid),
                dim3(64 * WGM * WGN), s, a);
}

// The four-wave kernel (K steps of 64, two LDS stages) with BM x BN tiles.
template <int BM, int BN, bool AK, bool BKM, int EPI>
int run_gemm_w4(const char* role, GemmArgs a, hipStream_t s, int group) {
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.group_m = group;
  if (a.splits < 1) a.splits = 1;
  const int per = (a.K + a.splits - 1) / a.splits;
  a.k_per_split = ((per + 63) / 64) * 64;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * a.splits;
  if (grid <= 0) return TPMLP_OK;
  if (grid > 0x7fffffff) return fail(TPMLP_E_SHAPE, "%s: grid too large", role);
  char sym[96];
  snprintf(sym, sizeof(sym), "gemm_w4_kernel<%d,%d,%d,%d,%d>", BM, BN, (int)AK, (int)BKM, EPI);
  a.clk = prof_clock_slot(role);
  return launch(role, sym, gemm_w4_kernel<BM, BN, AK, BKM, EPI>, dim3((unsigned)grid), dim3(256), s, a);
}

// Two independent products in one launch of the four-wave kernel at BM x BN
// (gemm_w4_duo_kernel): a0's tiles first, a0's tile count a multiple of 8.
template <int BM, int BN, bool AK0, bool BK0, int E0, bool AK1, bool BK1, int E1>
int run_gemm_w4_duo(const char* role, GemmArgs a0, int g0, GemmArgs a1, int g1, hipStream_t s) {
  auto prep = [](GemmArgs& a, int group) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.group_m = group;
    a.splits = 1;
    a.k_per_split = ((a.K + 63) / 64) * 64;
    a.clk = nullptr;
    return (int64_t)a.tiles_m * a.tiles_n;
  };
  const int64_t n0 = prep(a0, g0), n1 = prep(a1, g1);
  if (n0 % 8 != 0) return fail(TPMLP_E_SHAPE, "%s: first product's tile count %lld is not a multiple of 8", role,
                               (long long)n0);
  char sym[96];
  snprintf(sym, sizeof(sym), "gemm_w4_duo_kernel<%d,%d,%d,%d,%d,%d,%d,%d>", BM, BN, (int)AK0, (int)BK0, E0, (int)AK1,
           (int)BK1, E1);
  a0.clk = prof_clock_slot(role);
  return launch(role, sym, gemm_w4_duo_kernel<BM, BN, AK0, BK0, E0, AK1, BK1, E1>, dim3((unsigned)(n0 + n1)),
                dim3(256), s, a0, a1, (int)n0);
}

// Buffer offsets inside a tile are 32-bit: a tile spans at most 320 rows of
// a K-contiguous operand (or 64 K-rows of an M/N-contiguous one).
constexpr int64_t kMaxLd = (int64_t)1 << 22;

// Entry points that launch several GEMMs check every operand's leading
// dimension before the first launch, so that no error can follow a launch.
int check_lds(std::initializer_list<int64_t> lds) {
  for (const int64_t ld : lds)
    if (ld >= kMaxLd) return fail(TPMLP_E_SHAPE, "leading dimension %lld above 2^22 elements", (long long)ld);
  return TPMLP_OK;
}

// Raster rows for tiles that share no operand with other XCDs (the weight
// gradients, whose operands are both activations): an XCD's `per_xcd` tiles
// form a block of g rows by ceil(per_xcd / g) columns with g + columns
// smallest, so they need as few 256-row operand blocks as possible.
int square_group(int per_xcd, int tiles_m) {
  int best = 1, cost = 1 << 30;
  for (int g = 1; g <= std::max(1, std::min(tiles_m, per_xcd)); ++g) {
    const int c = g + (per_xcd + g - 1) / g;
    if (c < cost) cost = c, best = g;
  }
  return best;
}

// Raster group of a product's own launch at tile configuration cfg: the tiles
// one XCD runs at once (CUs/8 x occupancy) span whole rows of tiles, so each
// round of an XCD shares its A rows; weight gradients (both operands
// activations, shared by no other XCD) and products of at most 8 tile rows
// (where whole rows would make every XCD stream all of B) take a square block
// of those tiles instead.
int raster_group(bool wgrad, int64_t M, int64_t N, int cfg, int cus) {
  const int bm = kCfgBf16[cfg].bm, bn = kCfgBf16[cfg].bn;
  const int tiles_m = (int)((M + bm - 1) / bm), tiles_n = (int)((N + bn - 1) / bn);
  if (wgrad || tiles_m <= 8) {
    const int64_t slots = (int64_t)cus * kCfgBf16[cfg].occ, tiles = (int64_t)tiles_m * tiles_n;
    return square_group((int)std::max<int64_t>(1, std::min(tiles, slots) / 8), tiles_m);
  }
  return std::max(1, std::min(tiles_m, (cus / 8) * kCfgBf16[cfg].occ / tiles_n));
}

// A weight gradient w (long K: the token count) and an independent product o
// of the same backward pass in one launch of 256x256 tiles, w's first, when
// w's tiles leave CUs idle (fewer than the CUs, a multiple of 8) and o's
// tiles, run on the idle CUs and then on the ones o's own tiles release,
// finish within one of w's tiles: the launch then takes about one w tile,
// against w's launch plus o's launch apart.
bool joins_under_wgrad(const GemmArgs& w, const GemmArgs& o, int cus) {
  if (w.M <= 0 || w.N <= 0 || o.M <= 0 || o.N <= 0) return false;
  const int64_t nw = ((w.M + 255) / 256) * ((w.N + 255) / 256), no = ((o.M + 255) / 256) * ((o.N + 255) / 256);
  if (nw % 8 != 0 || nw >= cus) return false;
  const int64_t kw = (w.K + 63) / 64, ko = (o.K + 63) / 64;
  const int64_t free_cus = cus - nw;
  return ((no + free_cus - 1) / free_cus) * ko <= kw;
}

// The two weight gradients of the MLP backward (A^T dZ and X^T dH) in one
// launch of the four-wave kernel when together they fill the chip once: at
// 256x256 (one workgroup per CU) when their tiles cover 3/4 to all of the
// CUs, else at 128x128 (up to two workgroups per CU) when theirs cover 3/4 of
// the CUs to all of the workgroup slots.  Past one round, at 256x256 when
// each would run as 256x256 tiles of its own (unsplit, the planner's choice)
// over the same K and their part-filled last rounds together save a round
// (GPT-3 shard: 1152 + 1152 tiles, 5 + 5 rounds apart, 9 together); each
// keeps the raster of its own launch, and the second's tiles start on the
// CUs the first's last round leaves free.  The first product's tile count
// must be a multiple of 8 (so each workgroup keeps its XCD within its
// product).  *done reports whether the pair ran; when it did not, nothing
// was launched.
int wgrad_splits(int dtype, int64_t M, int64_t N, int64_t K);

int run_wgrad_pair(const char* role, int dtype, GemmArgs a0, GemmArgs a1, hipStream_t s, bool* done) {
  *done = false;
  if (dtype != TPMLP_BF16 || a0.M <= 0 || a0.N <= 0 || a1.M <= 0 || a1.N <= 0) return TPMLP_OK;
  if (a0.lda >= kMaxLd || a0.ldb >= kMaxLd || a1.lda >= kMaxLd || a1.ldb >= kMaxLd) return TPMLP_OK;
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  constexpr int BKT = 64;
  auto prep = [&](GemmArgs& a, int bm, int bn) {
    a.tiles_m = (a.M + bm - 1) / bm;
    a.tiles_n = (a.N + bn - 1) / bn;
    // Each product holds about half of an XCD's workgroups; its tiles there
    // form a square block (16 tiles per XCD: 4 x 4, eight operand row
    // blocks of A and B, instead of 2 x 8, ten).
    a.group_m = square_group(std::max(1, (int)((int64_t)a.tiles_m * a.tiles_n / 8)), a.tiles_m);
    a.splits = 1;
    a.k_per_split = ((a.K + BKT - 1) / BKT) * BKT;
    a.clk = nullptr;
    return (int64_t)a.tiles_m * a.tiles_n;
  };
  auto fits = [&](int64_t n0, int64_t n1, int64_t slots) {
    return n0 % 8 == 0 && n0 + n1 <= slots && 4 * (n0 + n1) >= 3 * (int64_t)cus;
  };
  GemmArgs b0 = a0, b1 = a1;
  int64_t n0 = prep(b0, 256, 256), n1 = prep(b1, 256, 256);
  if (fits(n0, n1, cus)) {
    b0.clk = prof_clock_slot(role);   // the clock of the first product's workgroup 0
    *done = true;
    return launch(role, "gemm_w4_pair_kernel<256,256,0,0,0>", gemm_w4_pair_kernel<256, 256, false, false, kEpiF32>,
                  dim3((unsigned)(n0 + n1)), dim3(256), s, b0, b1, (int)n0);
  }
  b0 = a0, b1 = a1;
  n0 = prep(b0, 128, 128), n1 = prep(b1, 128, 128);
  if (fits(n0, n1, 2 * (int64_t)cus)) {
    b0.clk = prof_clock_slot(role);
    *done = true;
    return launch(role, "gemm_w4_pair_kernel<128,128,0,0,0>", gemm_w4_pair_kernel<128, 128, false, false, kEpiF32>,
                  dim3((unsigned)(n0 + n1)), dim3(256), s, b0, b1, (int)n0);
  }
  if (a0.K == a1.K && wgrad_splits(dtype, a0.M, a0.N, a0.K) == 1 && wgrad_splits(dtype, a1.M, a1.N, a1.K) == 1 &&
      plan_cfg(dtype, a0.M, a0.N, kEpiF32, cus) == 0 && plan_cfg(dtype, a1.M, a1.N, kEpiF32, cus) == 0) {
    b0 = a0, b1 = a1;
    n0 = prep(b0, 256, 256), n1 = prep(b1, 256, 256);
    b0.group_m = raster_group(true, b0.M, b0.N, 0, cus);
    b1.group_m = raster_group(true, b1.M, b1.N, 0, cus);
    auto rounds = [&](int64_t n) { return (n + cus - 1) / cus; };
    if (n0 % 8 == 0 && n0 + n1 <= 0x7fffffff && rounds(n0 + n1) < rounds(n0) + rounds(n1)) {
      b0.clk = prof_clock_slot(role);
      *done = true;
      return launch(role, "gemm_w4_pair_kernel<256,256,0,0,0>", gemm_w4_pair_kernel<256, 256, false, false, kEpiF32>,
                    dim3((unsigned)(n0 + n1)), dim3(256), s, b0, b1, (int)n0);
    }
  }
  return TPMLP_OK;
}

// The MLP backward's two weight gradients and its input gradient dX = dH W1^T
// (all three need only dH) in one launch:
//  * at 256x256 when the weight gradients fill one round of 256x256 tiles
//    (the 256x256 pair) and dX plans 256x256 tiles: dX's tiles follow the
//    pair's in the same grid (Llama-7B shard: 128 + 128 + 512 tiles);
//  * at 128x128 when the weight gradients would run as the 128x128 pair
//    (their 256x256 tiles too few) and all three together fit one round of
//    two workgroups per CU: the pair alone leaves half of the workgroup slots
//    empty, and dX then runs as a launch of its own (GPT-2-medium shard:
//    128 + 128 + 256 tiles).
// *done reports whether the launch ran; when it did not, nothing was launched.
int run_bwd_trio(const char* role, int dtype, GemmArgs a0, GemmArgs a1, GemmArgs a2, hipStream_t s, bool* done) {
  *done = false;
  if (dtype != TPMLP_BF16) return TPMLP_OK;
  for (const GemmArgs* a : {&a0, &a1, &a2}) {
    if (a->M <= 0 || a->N <= 0) return TPMLP_OK;
    if (a->lda >= kMaxLd || a->ldb >= kMaxLd) return TPMLP_OK;
  }
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  auto tiles = [](const GemmArgs& a, int b) { return (int64_t)((a.M + b - 1) / b) * ((a.N + b - 1) / b); };
  constexpr int BKT = 64;
  const int64_t w256 = tiles(a0, 256) + tiles(a1, 256);
  if (tiles(a0, 256) % 8 == 0 && w256 <= cus && 4 * w256 >= 3 * (int64_t)cus) {
    // The weight gradients fill one round of 256x256 tiles: dX joins them in
    // the same launch when its own plan is 256x256 too.  Its tiles come after
    // the pair's (the pair's workgroups are dispatched first and hold every
    // CU), so they start on each CU as soon as its weight-gradient tile ends,
    // with no launch boundary between the products.
    if (plan_cfg(dtype, a2.M, a2.N, kEpiF32, cus) != 0) return TPMLP_OK;
    auto prep256 = [&](GemmArgs& a, int group) {
      a.tiles_m = (a.M + 255) / 256;
      a.tiles_n = (a.N + 255) / 256;
      a.group_m = group;
      a.splits = 1;
      a.k_per_split = ((a.K + BKT - 1) / BKT) * BKT;
      a.clk = nullptr;
      return (int64_t)a.tiles_m * a.tiles_n;
    };
    const int64_t m0 = prep256(a0, square_group(std::max(1, (int)(tiles(a0, 256) / 8)), (int)((a0.M + 255) / 256)));
    const int64_t m1 = prep256(a1, square_group(std::max(1, (int)(tiles(a1, 256) / 8)), (int)((a1.M + 255) / 256)));
    const int64_t m2 = prep256(a2, raster_group(false, a2.M, a2.N, 0, cus));   // as dX's own launch
    a0.clk = prof_clock_slot(role);
    *done = true;
    return launch(role, "gemm_w4_trio_kernel<256,256>", gemm_w4_trio_kernel<256, 256>, dim3((unsigned)(m0 + m1 + m2)),
                  dim3(256), s, a0, a1, a2, (int)m0, (int)m1);
  }
  constexpr int B = 128;
  auto prep = [&](GemmArgs& a, bool square) {
    a.tiles_m = (a.M + B - 1) / B;
    a.tiles_n = (a.N + B - 1) / B;
    const int64_t t = (int64_t)a.tiles_m * a.tiles_n;
    a.group_m = square || a.tiles_m <= 8 ? square_group(std::max(1, (int)(t / 8)), a.tiles_m)
                                         : std::max(1, std::min(a.tiles_m, (cus / 8) * 2 / a.tiles_n));
    a.splits = 1;
    a.k_per_split = ((a.K + BKT - 1) / BKT) * BKT;
    a.clk = nullptr;
    return t;
  };
  const int64_t n0 = prep(a0, true), n1 = prep(a1, true), n2 = prep(a2, false);
  if (n0 % 8 != 0 || n1 % 8 != 0 || n0 + n1 > 2 * (int64_t)cus || 4 * (n0 + n1) < 3 * (int64_t)cus ||
      n0 + n1 + n2 > 2 * (int64_t)cus)
    return TPMLP_OK;
  a0.clk = prof_clock_slot(role);   // the clock of the first product's workgroup 0
  *done = true;
  return launch(role, "gemm_w4_trio_kernel<128,128>", gemm_w4_trio_kernel<B, B>, dim3((unsigned)(n0 + n1 + n2)),
                dim3(256), s, a0, a1, a2, (int)n0, (int)n1);
}

template <bool AK, bool BKM, int EPI>
int run_gemm(const char* role, int dtype, GemmArgs a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return TPMLP_OK;
  if (a.lda >= kMaxLd || a.ldb >= kMaxLd)
    return fail(TPMLP_E_SHAPE, "%s: leading dimension above 2^22 elements", role);
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  const int cfg = plan_cfg(dtype, a.M, a.N, EPI, cus);
  if (dtype == TPMLP_BF16) {
    const int group = raster_group(!AK && !BKM, a.M, a.N, cfg, cus);
    switch (cfg) {
      case 0: return run_gemm_w4<256, 256, AK, BKM, EPI>(role, a, s, group);
      case 3: return run_gemm_w4<256, 192, AK, BKM, EPI>(role, a, s, group);
      case 2:
        // 320 rows of 64-element K steps split evenly over 8 waves' loads.
        if constexpr (EPI == kEpiF32) return run_gemm_bf16<256, 320, AK, BKM, EPI, 2, 1, 64, 2, 4>(role, a, s, group);
        else return fail(TPMLP_E_SHAPE, "%s: no 256x320 tile for this epilogue", role);
      default: return run_gemm_w4<128, 128, AK, BKM, EPI>(role, a, s, group);
    }
  }
  if constexpr (EPI == kEpiSwiGLU || EPI == kEpiSwiGLUBwd) {
    return fail(TPMLP_E_DTYPE, "%s: the gated MLP epilogues are bf16 only", role);
  } else {
    switch (cfg) {
      case 0: return run_gemm_cfg<float, 128, 128, 2, 2, AK, BKM, EPI>(role, a, s);
      default: return run_gemm_cfg<float, 64, 64, 2, 2, AK, BKM, EPI>(role, a, s);
    }
  }
}

// A weight gradient whose 128x128 output tiles fill at most half of the
// chip's 512 workgroup slots (256 CUs x 2) is split along its long K = T
// into S slices of at least 1024 (fp32, in the workspace) that one launch
// computes side by side, then summed in slice order.  S depends on the
// shapes alone, so the workspace size does too.
constexpr int64_t kSplitSlots = 512;
int wgrad_splits(int dtype, int64_t M, int64_t N, int64_t K) {
  if (dtype != TPMLP_BF16) return 1;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (S < 8 && tiles * 2 * S <= kSplitSlots && K / (2 * S) >= 1024) S *= 2;
  return S;
}

int partial_sum(int tp, int64_t T, int64_t N, const float* P, int64_t stride, int64_t ldp, float* out,
                int64_t ldo, hipStream_t s, const char* role);

// A weight gradient (both operands M/N-contiguous, fp32 output) with its K
// split as wgrad_splits decides: the slices go to `slices` (M x N each, ld N)
// and are summed into a.C; unsplit, the planner's launch writes a.C directly.
int run_wgrad_split(const char* role, const char* sum_role, int dtype, GemmArgs a, float* slices,
                    hipStream_t s) {
  const int S = wgrad_splits(dtype, a.M, a.N, a.K);
  if (S == 1 || a.M <= 0 || a.N <= 0) return run_gemm<false, false, kEpiF32>(role, dtype, a, s);
  if (a.lda >= kMaxLd || a.ldb >= kMaxLd)
    return fail(TPMLP_E_SHAPE, "%s: leading dimension above 2^22 elements", role);
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  float* out = a.C;
  const int64_t ldo = a.ldc;
  a.C = slices;
  a.ldc = a.N;
  a.splits = S;
  a.split_stride = (int64_t)a.M * a.N;
  const int tiles_m = (a.M + 127) / 128, tiles_n = (a.N + 127) / 128;
  const int group = std::max(1, std::min(tiles_m, (cus / 8) * 2 / tiles_n));
  TPMLP_TRY((run_gemm_w4<128, 128, false, false, kEpiF32>(role, a, s, group)));
  return partial_sum(S, a.M, a.N, slices, a.split_stride, a.N, out, ldo, s, sum_role);
}

GemmArgs gemm_args(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t K) {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = A;
  a.lda = lda;
  a.B = B;
  a.ldb = ldb;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.splits = 1;
  a.act = kActNone;
  return a;
}

int fill_zero(float* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || p == nullptr) return TPMLP_OK;
  const int64_t total = rows * cols;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  return launch("fill_zero", "fill_zero_kernel", fill_zero_kernel, dim3(grid), dim3(256), s, p, (int)rows,
                (int)cols, ld);
}

int partial_sum(int tp, int64_t T, int64_t N, const float* P, int64_t stride, int64_t ldp, float* out,
                int64_t ldo, hipStream_t s, const char* role = "partial_sum") {
  if (T == 0) return TPMLP_OK;
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  const int nvec = (int)(N / 4);
  // Four 16-byte groups per thread for wide rows (measured 6.3 vs 6.1 TB/s at
  // N = 4096), two otherwise.
  if (nvec >= 1024) {
    const int64_t blocks = T * ((nvec + 1023) / 1024);
    const unsigned grid = (unsigned)std::min<int64_t>(blocks, (int64_t)cus * 16);
    return launch(role, "partial_sum_kernel<4>", partial_sum_kernel<4>, dim3(grid), dim3(256), s, P, stride, ldp,
                  out, ldo, tp, (int)T, nvec);
  }
  const int64_t blocks = T * ((nvec + 511) / 512);
  const unsigned grid = (unsigned)std::min<int64_t>(blocks, (int64_t)cus * 16);
  return launch(role, "partial_sum_kernel<2>", partial_sum_kernel<2>, dim3(grid), dim3(256), s, P, stride, ldp,
                out, ldo, tp, (int)T, nvec);
}

// Column-parallel forward body (arguments already validated).
int col_fwd(hipStream_t s, int dtype, int act, int64_t T, int64_t K, int64_t Ns, const void* X, int64_t ldx,
            const void* W, int64_t ldw, const void* bias, void* Y, int64_t ldy, void* H, int64_t ldh,
            const char* role) {
  if (T == 0) return TPMLP_OK;
  GemmArgs a = gemm_args(X, ldx, W, ldw, T, Ns, K);
  a.Y = Y;
  a.ldy = ldy;
  a.H = H;
  a.ldh = ldh;
  a.bias = bias;
  a.act = act;
  return run_gemm<true, false, kEpiBiasAct>(role, dtype, a, s);
}

int row_fwd(hipStream_t s, int dtype, int64_t T, int64_t Ks, int64_t N, const void* X, int64_t ldx,
            const void* W, int64_t ldw, float* Z, int64_t ldz, const char* role) {
  if (T == 0) return TPMLP_OK;
  GemmArgs a = gemm_args(X, ldx, W, ldw, T, N, Ks);
  a.C = Z;
  a.ldc = ldz;
  return run_gemm<true, false, kEpiF32>(role, dtype, a, s);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t dh_off, cs_off, split_off, total;
};

BwdLayout bwd_layout(int dtype, int64_t T, int64_t h, int64_t Fs) {
  BwdLayout L;
  L.dh_off = 0;
  const size_t dh = align256((size_t)T * Fs * elem_size(dtype));
  L.cs_off = dh;
  const size_t cs = align256((size_t)((T + kMinBM - 1) / kMinBM) * Fs * sizeof(float));
  L.split_off = dh + cs;
  // both weight gradients have h x Fs outputs
  const int S = std::max(wgrad_splits(dtype, Fs, h, T), wgrad_splits(dtype, h, Fs, T));
  const size_t split = S > 1 ? align256((size_t)S * h * Fs * sizeof(float)) : 0;
  L.total = L.split_off + split;
  return L;
}

// Operand checks of one shard's MLP backward (shared by the workspace and
// the allocation-free entry points).
int check_mlp_bwd_args(int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X, const void* W1_shard,
                       int64_t ldw1, const void* W2_shard, const void* H_save, const void* A_save, const void* dZ,
                       float* dX_partial, float* dW1_shard, float* db1_shard, float* dW2_shard) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X", X, T, h, h, v));
  TPMLP_TRY(check_mat("W1_shard", W1_shard, h, Fs, ldw1, v));
  TPMLP_TRY(check_mat("W2_shard", W2_shard, Fs, h, h, v));
  TPMLP_TRY(check_mat("H_save", H_save, T, Fs, Fs, v));
  TPMLP_TRY(check_mat("A_save", A_save, T, Fs, Fs, v));
  TPMLP_TRY(check_mat("dZ", dZ, T, h, h, v));
  TPMLP_TRY(check_mat("dX_partial", dX_partial, T, h, h, 4));
  TPMLP_TRY(check_mat("dW1_shard", dW1_shard, h, Fs, Fs, 4));
  TPMLP_TRY(check_vec("db1_shard", db1_shard, Fs, false));
  TPMLP_TRY(check_mat("dW2_shard", dW2_shard, Fs, h, h, 4));
  TPMLP_TRY(check_lds({h, ldw1, Fs}));
  return TPMLP_OK;
}

// One shard's MLP backward on a validated workspace of bwd_layout(...).total bytes.
int mlp_bwd_launch(hipStream_t s, int dtype, int64_t T, int64_t h, int64_t Fs, const void* X, const void* W1_shard,
                   int64_t ldw1, const void* W2_shard, const void* H_save, const void* A_save, const void* dZ,
                   float* dX_partial, float* dW1_shard, float* db1_shard, float* dW2_shard, void* workspace) {
  const BwdLayout L = bwd_layout(dtype, T, h, Fs);
  if (T == 0) {
    TPMLP_TRY(fill_zero(dW1_shard, h, Fs, Fs, s));
    TPMLP_TRY(fill_zero(dW2_shard, Fs, h, h, s));
    return fill_zero(db1_shard, 1, Fs, Fs, s);
  }
  char* ws = static_cast<char*>(workspace);
  void* dH = ws + L.dh_off;
  float* cs = reinterpret_cast<float*>(ws + L.cs_off);

  // dH = (dZ W2_i^T) * GeLU'(H_i), with per-tile column sums of dH.
  GemmArgs a = gemm_args(dZ, h, W2_shard, h, T, Fs, h);
  a.Y = dH;
  a.ldy = Fs;
  a.H = const_cast<void*>(H_save);
  a.ldh = Fs;
  a.colsum = db1_shard ? cs : nullptr;
  a.act = kActGeluTanh;
  // The tile rows used by the plan decide how many column-sum rows exist.
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  TPMLP_TRY((run_gemm<true, true, kEpiActBwd>("gemm.mlp_dgrad_act", dtype, a, s)));
  if (db1_shard) {
    const int cfg = plan_cfg(dtype, (int)T, (int)Fs, kEpiActBwd, cus);
    const int bm = dtype == TPMLP_BF16 ? kCfgBf16[cfg].bm : kCfgF32[cfg].bm;
    const int rows = (int)((T + bm - 1) / bm);
    TPMLP_TRY(launch("colsum", "colsum_reduce_kernel", colsum_reduce_kernel, dim3((unsigned)((Fs + 63) / 64)),
                     dim3(64), s, (const float*)cs, rows, (int)Fs, db1_shard));
  }
  // dW2_i = A_i^T dZ and dW1_i = X^T dH_i: one paired launch when together
  // they fill the chip once (joined by dX_i when all three fit one round of
  // 128x128 tiles), else one launch each.
  GemmArgs w2 = gemm_args(A_save, Fs, dZ, h, Fs, h, T);
  w2.C = dW2_shard;
  w2.ldc = h;
  GemmArgs w1 = gemm_args(X, h, dH, Fs, h, Fs, T);
  w1.C = dW1_shard;
  w1.ldc = Fs;
  // dX_i = dH_i W1_i^T
  a = gemm_args(dH, Fs, W1_shard, ldw1, T, h, Fs);
  a.C = dX_partial;
  a.ldc = h;
  bool joined = false;
  TPMLP_TRY(run_bwd_trio("gemm.mlp_wgrad2+gemm.mlp_wgrad1+gemm.mlp_dgrad1", dtype, w2, w1, a, s, &joined));
  if (joined) return TPMLP_OK;
  bool paired = false;
  TPMLP_TRY(run_wgrad_pair("gemm.mlp_wgrad2+gemm.mlp_wgrad1", dtype, w2, w1, s, &paired));
  if (!paired) {
    float* slices = reinterpret_cast<float*>(ws + L.split_off);
    TPMLP_TRY(run_wgrad_split("gemm.mlp_wgrad2", "wgrad_split_sum", dtype, w2, slices, s));
    TPMLP_TRY(run_wgrad_split("gemm.mlp_wgrad1", "wgrad_split_sum", dtype, w1, slices, s));
  }
  return run_gemm<true, true, kEpiF32>("gemm.mlp_dgrad1", dtype, a, s);
}


// -------------------------------------------------- allocation-free scratch --
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): tp_mlp_bwd_noalloc keeps
// its workspace in this file-scope device array instead of a caller buffer.
// Each device the library runs on holds its own copy until the process ends.
// In host code the array's name is only a host-side stand-in; its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed to kernels.  Calls on one device
// share the array, so calls that overlap on one device race; nothing in it
// needs to start at zero (every byte the backward reads it wrote first).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;   // 64 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of this device's scratch array (looked up on first use).
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(TPMLP_E_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TPMLP_OK;
}

}  // namespace

// ======================================================================= ABI
extern "C" {

const char* tpmlp_version(void) { return "libtpmlp 0.1 (gfx950)"; }

const char* tpmlp_status_string(int status) {
  switch (status) {
    case TPMLP_OK: return "TPMLP_OK";
    case TPMLP_E_NULL: return "TPMLP_E_NULL";
    case TPMLP_E_SHAPE: return "TPMLP_E_SHAPE";
    case TPMLP_E_DIVISIBILITY: return "TPMLP_E_DIVISIBILITY";
    case TPMLP_E_ALIGNMENT: return "TPMLP_E_ALIGNMENT";
    case TPMLP_E_DTYPE: return "TPMLP_E_DTYPE";
    case TPMLP_E_ACT: return "TPMLP_E_ACT";
    case TPMLP_E_WORKSPACE: return "TPMLP_E_WORKSPACE";
    case TPMLP_E_HIP: return "TPMLP_E_HIP";
    case TPMLP_E_VALUE: return "TPMLP_E_VALUE";
    default: return "TPMLP_E_UNKNOWN";
  }
}

const char* tpmlp_last_error(void) { return g_last_error.c_str(); }

int column_parallel_fwd(void* stream, int dtype, int act, int64_t T, int64_t K, int64_t N, int tp_size,
                        const void* X, int64_t ldx, const void* W_shard, int64_t ldw, const void* bias_shard,
                        void* Y_shard, int64_t ldy, void* H_save, int64_t ldh) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_act(act));
  TPMLP_TRY(check_split("N", N, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("K", K));
  TPMLP_TRY(check_dim("N", N));
  const int64_t Ns = N / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X", X, T, K, ldx, v));
  TPMLP_TRY(check_mat("W_shard", W_shard, K, Ns, ldw, v));
  TPMLP_TRY(check_vec("bias_shard", bias_shard, Ns, false));
  TPMLP_TRY(check_mat("Y_shard", Y_shard, T, Ns, ldy, v));
  TPMLP_TRY(check_mat("H_save", H_save, T, Ns, ldh, v, false));
  return col_fwd((hipStream_t)stream, dtype, act, T, K, Ns, X, ldx, W_shard, ldw, bias_shard, Y_shard, ldy, H_save,
                 ldh, "gemm.col_fwd");
}

int row_parallel_fwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size, const void* X_shard,
                     int64_t ldx, const void* W_shard, int64_t ldw, float* Z_partial, int64_t ldz) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("K", K, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("K", K));
  TPMLP_TRY(check_dim("N", N));
  const int64_t Ks = K / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X_shard", X_shard, T, Ks, ldx, v));
  TPMLP_TRY(check_mat("W_shard", W_shard, Ks, N, ldw, v));
  TPMLP_TRY(check_mat("Z_partial", Z_partial, T, N, ldz, 4));
  return row_fwd((hipStream_t)stream, dtype, T, Ks, N, X_shard, ldx, W_shard, ldw, Z_partial, ldz,
                 "gemm.row_fwd");
}

int shard_partial_sum(void* stream, int tp_size, int64_t T, int64_t N, const float* partials, int64_t shard_stride,
                      int64_t ldp, float* out, int64_t ldo) {
  if (tp_size < 1) return fail(TPMLP_E_DIVISIBILITY, "tp_size %d < 1", tp_size);
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("N", N));
  if (shard_stride < 0) return fail(TPMLP_E_SHAPE, "shard_stride %lld < 0", (long long)shard_stride);
  if (shard_stride % 4 != 0) return fail(TPMLP_E_ALIGNMENT, "shard_stride must be a multiple of 4 floats");
  TPMLP_TRY(check_mat("partials", partials, T, N, ldp, 4));
  TPMLP_TRY(check_mat("out", out, T, N, ldo, 4));
  if (out != partials && T > 0) {
    // out may alias partial 0 exactly; any other overlap with a partial is refused.
    const char* o0 = reinterpret_cast<const char*>(out);
    const char* o1 = o0 + ((T - 1) * ldo + N) * sizeof(float);
    for (int i = 0; i < tp_size; ++i) {
      const char* p0 = reinterpret_cast<const char*>(partials + (int64_t)i * shard_stride);
      const char* p1 = p0 + ((T - 1) * ldp + N) * sizeof(float);
      if (o0 < p1 && p0 < o1) return fail(TPMLP_E_SHAPE, "out overlaps partial %d", i);
    }
  } else if (out == partials && ldo != ldp) {
    return fail(TPMLP_E_SHAPE, "in-place sum into partial 0 needs ldo == ldp");
  }
  return partial_sum(tp_size, T, N, partials, shard_stride, ldp, out, ldo, (hipStream_t)stream);
}

int tp_mlp_fwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X,
               const void* W1_shard, int64_t ldw1, const void* b1_shard, const void* W2_shard, void* H_save,
               void* A_save, float* Z_partial) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X", X, T, h, h, v));
  TPMLP_TRY(check_mat("W1_shard", W1_shard, h, Fs, ldw1, v));
  TPMLP_TRY(check_vec("b1_shard", b1_shard, Fs, false));
  TPMLP_TRY(check_mat("W2_shard", W2_shard, Fs, h, h, v));
  TPMLP_TRY(check_mat("H_save", H_save, T, Fs, Fs, v, false));
  TPMLP_TRY(check_mat("A_save", A_save, T, Fs, Fs, v));
  TPMLP_TRY(check_mat("Z_partial", Z_partial, T, h, h, 4));
  TPMLP_TRY(check_lds({h, ldw1, Fs}));
  hipStream_t s = (hipStream_t)stream;
  TPMLP_TRY(col_fwd(s, dtype, TPMLP_ACT_GELU_TANH, T, h, Fs, X, h, W1_shard, ldw1, b1_shard, A_save, Fs, H_save, Fs,
                    "gemm.mlp_fwd1"));
  return row_fwd(s, dtype, T, Fs, h, A_save, Fs, W2_shard, h, Z_partial, h, "gemm.mlp_fwd2");
}

size_t tpmlp_bwd_workspace_bytes(int dtype, int64_t T, int64_t h, int64_t F, int tp_size) {
  if ((dtype != TPMLP_BF16 && dtype != TPMLP_F32) || tp_size < 1 || T < 0 || T > kMaxDim || h < 1 || F < 1 ||
      F % tp_size != 0)
    return 0;
  return bwd_layout(dtype, T, h, F / tp_size).total;
}

int tp_mlp_bwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X,
               const void* W1_shard, int64_t ldw1, const void* W2_shard, const void* H_save, const void* A_save,
               const void* dZ, float* dX_partial, float* dW1_shard, float* db1_shard, float* dW2_shard,
               void* workspace, size_t workspace_bytes) {
  TPMLP_TRY(check_mlp_bwd_args(dtype, T, h, F, tp_size, X, W1_shard, ldw1, W2_shard, H_save, A_save, dZ, dX_partial,
                               dW1_shard, db1_shard, dW2_shard));
  const int64_t Fs = F / tp_size;
  const BwdLayout L = bwd_layout(dtype, T, h, Fs);
  if (T > 0) {
    if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
    if (workspace_bytes < L.total)
      return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  }
  return mlp_bwd_launch((hipStream_t)stream, dtype, T, h, Fs, X, W1_shard, ldw1, W2_shard, H_save, A_save, dZ,
                        dX_partial, dW1_shard, db1_shard, dW2_shard, workspace);
}

int tp_mlp_bwd_noalloc(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X,
                       const void* W1_shard, int64_t ldw1, const void* W2_shard, const void* H_save,
                       const void* A_save, const void* dZ, float* dX_partial, float* dW1_shard, float* db1_shard,
                       float* dW2_shard) {
  TPMLP_TRY(check_mlp_bwd_args(dtype, T, h, F, tp_size, X, W1_shard, ldw1, W2_shard, H_save, A_save, dZ, dX_partial,
                               dW1_shard, db1_shard, dW2_shard));
  const int64_t Fs = F / tp_size;
  const BwdLayout L = bwd_layout(dtype, T, h, Fs);
  if (L.total > kNoAllocScratchBytes)
    return fail(TPMLP_E_WORKSPACE, "tp_mlp_bwd_noalloc: these sizes need %zu bytes of scratch, above the %zu-byte "
                "static scratch array (use tp_mlp_bwd with a caller workspace)", L.total, kNoAllocScratchBytes);
  void* ws = nullptr;
  TPMLP_TRY(noalloc_scratch(&ws));
  return mlp_bwd_launch((hipStream_t)stream, dtype, T, h, Fs, X, W1_shard, ldw1, W2_shard, H_save, A_save, dZ,
                        dX_partial, dW1_shard, db1_shard, dW2_shard, ws);
}

size_t tpmlp_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int column_parallel_bwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size, const void* X,
                        int64_t ldx, const void* W_shard, int64_t ldw, const void* dY, int64_t lddy,
                        float* dX_partial, int64_t lddx, float* dW_shard, int64_t lddw, float* db_shard) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("N", N, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("K", K));
  TPMLP_TRY(check_dim("N", N));
  const int64_t Ns = N / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X", X, T, K, ldx, v));
  TPMLP_TRY(check_mat("W_shard", W_shard, K, Ns, ldw, v));
  TPMLP_TRY(check_mat("dY", dY, T, Ns, lddy, v));
  TPMLP_TRY(check_mat("dX_partial", dX_partial, T, K, lddx, 4));
  TPMLP_TRY(check_mat("dW_shard", dW_shard, K, Ns, lddw, 4));
  TPMLP_TRY(check_vec("db_shard", db_shard, Ns, false));
  TPMLP_TRY(check_lds({ldx, ldw, lddy}));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    TPMLP_TRY(fill_zero(dW_shard, K, Ns, lddw, s));
    return fill_zero(db_shard, 1, Ns, Ns, s);
  }
  // dX_partial = dY W_i^T
  GemmArgs a = gemm_args(dY, lddy, W_shard, ldw, T, K, Ns);
  a.C = dX_partial;
  a.ldc = lddx;
  TPMLP_TRY((run_gemm<true, true, kEpiF32>("gemm.col_dgrad", dtype, a, s)));
  // dW_i = X^T dY
  a = gemm_args(X, ldx, dY, lddy, K, Ns, T);
  a.C = dW_shard;
  a.ldc = lddw;
  TPMLP_TRY((run_gemm<false, false, kEpiF32>("gemm.col_wgrad", dtype, a, s)));
  if (db_shard == nullptr) return TPMLP_OK;
  // db_i = column sums of dY
  const int cols = 8 * chunk_elems(dtype);
  const dim3 grid((unsigned)((Ns + cols - 1) / cols));
  if (dtype == TPMLP_BF16)
    return launch("colsum_rows", "colsum_rows_kernel<bf16>", colsum_rows_kernel<bf16_t>, grid, dim3(256), s,
                  static_cast<const bf16_t*>(dY), lddy, (int)T, (int)Ns, db_shard);
  return launch("colsum_rows", "colsum_rows_kernel<f32>", colsum_rows_kernel<float>, grid, dim3(256), s,
                static_cast<const float*>(dY), lddy, (int)T, (int)Ns, db_shard);
}

int row_parallel_bwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size, const void* X_shard,
                     int64_t ldx, const void* W_shard, int64_t ldw, const void* dY, int64_t lddy, float* dX_shard,
                     int64_t lddx, float* dW_shard, int64_t lddw) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("K", K, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("K", K));
  TPMLP_TRY(check_dim("N", N));
  const int64_t Ks = K / tp_size;
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("X_shard", X_shard, T, Ks, ldx, v));
  TPMLP_TRY(check_mat("W_shard", W_shard, Ks, N, ldw, v));
  TPMLP_TRY(check_mat("dY", dY, T, N, lddy, v));
  TPMLP_TRY(check_mat("dX_shard", dX_shard, T, Ks, lddx, 4));
  TPMLP_TRY(check_mat("dW_shard", dW_shard, Ks, N, lddw, 4));
  TPMLP_TRY(check_lds({ldx, ldw, lddy}));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) return fill_zero(dW_shard, Ks, N, lddw, s);
  // dX_i = dY W_i^T
  GemmArgs a = gemm_args(dY, lddy, W_shard, ldw, T, Ks, N);
  a.C = dX_shard;
  a.ldc = lddx;
  TPMLP_TRY((run_gemm<true, true, kEpiF32>("gemm.row_dgrad", dtype, a, s)));
  // dW_i = X_i^T dY
  a = gemm_args(X_shard, ldx, dY, lddy, Ks, N, T);
  a.C = dW_shard;
  a.ldc = lddw;
  return run_gemm<false, false, kEpiF32>("gemm.row_wgrad", dtype, a, s);
}

// ------------------------------------------- unfused GeLU epilogues --
namespace {
unsigned elementwise_grid(int64_t items) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 256 * 32));
}
}  // namespace

int bias_gelu_fwd(void* stream, int dtype, int64_t T, int64_t N, const float* Hin, int64_t ldin, const void* bias,
                  void* A_out, int64_t lda, void* H_out, int64_t ldh) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("N", N));
  const int v = chunk_elems(dtype);
  if (N % 8 != 0) return fail(TPMLP_E_ALIGNMENT, "N = %lld is not a multiple of 8", (long long)N);
  TPMLP_TRY(check_mat("Hin", Hin, T, N, ldin, 4));
  TPMLP_TRY(check_vec("bias", bias, N, false));
  TPMLP_TRY(check_mat("A_out", A_out, T, N, lda, v));
  TPMLP_TRY(check_mat("H_out", H_out, T, N, ldh, v, false));
  if (T == 0) return TPMLP_OK;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = elementwise_grid(T * (N / 8));
  if (dtype == TPMLP_BF16)
    return launch("bias_gelu_fwd", "bias_gelu_fwd_kernel<bf16>", bias_gelu_fwd_kernel<bf16_t>, dim3(grid), dim3(256),
                  s, Hin, ldin, static_cast<const bf16_t*>(bias), static_cast<bf16_t*>(A_out), lda,
                  static_cast<bf16_t*>(H_out), ldh, (int)T, (int)N);
  return launch("bias_gelu_fwd", "bias_gelu_fwd_kernel<f32>", bias_gelu_fwd_kernel<float>, dim3(grid), dim3(256), s,
                Hin, ldin, static_cast<const float*>(bias), static_cast<float*>(A_out), lda,
                static_cast<float*>(H_out), ldh, (int)T, (int)N);
}

int gelu_bwd(void* stream, int dtype, int64_t T, int64_t N, const float* dA, int64_t ldda, const void* H,
             int64_t ldh, void* dH_out, int64_t lddh) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("N", N));
  const int v = chunk_elems(dtype);
  if (N % 8 != 0) return fail(TPMLP_E_ALIGNMENT, "N = %lld is not a multiple of 8", (long long)N);
  TPMLP_TRY(check_mat("dA", dA, T, N, ldda, 4));
  TPMLP_TRY(check_mat("H", H, T, N, ldh, v));
  TPMLP_TRY(check_mat("dH_out", dH_out, T, N, lddh, v));
  if (T == 0) return TPMLP_OK;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = elementwise_grid(T * (N / 8));
  if (dtype == TPMLP_BF16)
    return launch("gelu_bwd", "gelu_bwd_kernel<bf16>", gelu_bwd_kernel<bf16_t>, dim3(grid), dim3(256), s, dA, ldda,
                  static_cast<const bf16_t*>(H), ldh, static_cast<bf16_t*>(dH_out), lddh, (int)T, (int)N);
  return launch("gelu_bwd", "gelu_bwd_kernel<f32>", gelu_bwd_kernel<float>, dim3(grid), dim3(256), s, dA, ldda,
                static_cast<const float*>(H), ldh, static_cast<float*>(dH_out), lddh, (int)T, (int)N);
}

// ------------------------------------------------- gated MLP (SwiGLU) --
int swiglu_pack_shard(void* stream, int dtype, int64_t h, int64_t F, int tp_size, int shard, const void* W_gate,
                      int64_t ldg, const void* W_up, int64_t ldu, void* W_gu_shard) {
  TPMLP_TRY(check_dtype(dtype));
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  if (Fs % 8 != 0) return fail(TPMLP_E_DIVISIBILITY, "F/tp_size = %lld is not a multiple of 8", (long long)Fs);
  if (shard < 0 || shard >= tp_size) return fail(TPMLP_E_SHAPE, "shard %d outside [0, %d)", shard, tp_size);
  const int v = chunk_elems(dtype);
  TPMLP_TRY(check_mat("W_gate", W_gate, h, F, ldg, v));
  TPMLP_TRY(check_mat("W_up", W_up, h, F, ldu, v));
  TPMLP_TRY(check_mat("W_gu_shard", W_gu_shard, h, 2 * Fs, 2 * Fs, v));
  if (h == 0) return TPMLP_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = h * (Fs / 4);
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  const int64_t c0 = (int64_t)shard * Fs;
  if (dtype == TPMLP_BF16)
    return launch("swiglu_pack", "swiglu_pack_kernel<bf16>", swiglu_pack_kernel<bf16_t>, dim3(grid), dim3(256), s,
                  static_cast<const bf16_t*>(W_gate), ldg, static_cast<const bf16_t*>(W_up), ldu, c0, (int)h,
                  (int)Fs, static_cast<bf16_t*>(W_gu_shard));
  return launch("swiglu_pack", "swiglu_pack_kernel<f32>", swiglu_pack_kernel<float>, dim3(grid), dim3(256), s,
                static_cast<const float*>(W_gate), ldg, static_cast<const float*>(W_up), ldu, c0, (int)h, (int)Fs,
                static_cast<float*>(W_gu_shard));
}

int swiglu_unpack_grad(void* stream, int64_t h, int64_t F, int tp_size, int shard, const float* dW_gu_shard,
                       float* dW_gate, int64_t ldg, float* dW_up, int64_t ldu) {
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  if (Fs % 8 != 0) return fail(TPMLP_E_DIVISIBILITY, "F/tp_size = %lld is not a multiple of 8", (long long)Fs);
  if (shard < 0 || shard >= tp_size) return fail(TPMLP_E_SHAPE, "shard %d outside [0, %d)", shard, tp_size);
  TPMLP_TRY(check_mat("dW_gu_shard", dW_gu_shard, h, 2 * Fs, 2 * Fs, 4));
  TPMLP_TRY(check_mat("dW_gate", dW_gate, h, F, ldg, 4));
  TPMLP_TRY(check_mat("dW_up", dW_up, h, F, ldu, 4));
  if (h == 0) return TPMLP_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = h * (Fs / 4);
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  return launch("swiglu_unpack", "swiglu_unpack_kernel", swiglu_unpack_kernel, dim3(grid), dim3(256), s,
                dW_gu_shard, (int)h, (int)Fs, (int64_t)shard * Fs, dW_gate, ldg, dW_up, ldu);
}

int tp_swiglu_fwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X,
                  const void* W_gu_shard, const void* W_down_shard, void* GU_save, void* A_save, float* Z_partial) {
  TPMLP_TRY(check_dtype(dtype));
  if (dtype != TPMLP_BF16) return fail(TPMLP_E_DTYPE, "the gated MLP is bf16 only");
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  if (Fs % 8 != 0) return fail(TPMLP_E_DIVISIBILITY, "F/tp_size = %lld is not a multiple of 8", (long long)Fs);
  TPMLP_TRY(check_mat("X", X, T, h, h, 8));
  TPMLP_TRY(check_mat("W_gu_shard", W_gu_shard, h, 2 * Fs, 2 * Fs, 8));
  TPMLP_TRY(check_mat("W_down_shard", W_down_shard, Fs, h, h, 8));
  TPMLP_TRY(check_mat("GU_save", GU_save, T, 2 * Fs, 2 * Fs, 8, false));
  TPMLP_TRY(check_mat("A_save", A_save, T, Fs, Fs, 8));
  TPMLP_TRY(check_mat("Z_partial", Z_partial, T, h, h, 4));
  if (T == 0) return TPMLP_OK;
  TPMLP_TRY(check_lds({h, 2 * Fs}));
  hipStream_t s = (hipStream_t)stream;
  // [gate | up] = X W_gu (packed), A = silu(gate) * up
  GemmArgs a = gemm_args(X, h, W_gu_shard, 2 * Fs, T, 2 * Fs, h);
  a.Y = A_save;
  a.ldy = Fs;
  a.H = GU_save;
  a.ldh = 2 * Fs;
  TPMLP_TRY((run_gemm<true, false, kEpiSwiGLU>("gemm.swiglu_fwd1", dtype, a, s)));
  // Z_i = A W_down_i
  a = gemm_args(A_save, Fs, W_down_shard, h, T, h, Fs);
  a.C = Z_partial;
  a.ldc = h;
  return run_gemm<true, false, kEpiF32>("gemm.swiglu_fwd2", dtype, a, s);
}

size_t tp_swiglu_bwd_workspace_bytes(int dtype, int64_t T, int64_t h, int64_t F, int tp_size) {
  if (dtype != TPMLP_BF16 || tp_size < 1 || T < 0 || T > kMaxDim || h < 1 || F < 1 || F % tp_size != 0 ||
      (F / tp_size) % 8 != 0)
    return 0;
  return align256((size_t)T * 2 * (F / tp_size) * sizeof(bf16_t));
}

int tp_swiglu_bwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size, const void* X,
                  const void* W_gu_shard, const void* W_down_shard, const void* GU_save, const void* A_save,
                  const void* dZ, float* dX_partial, float* dW_gu_shard, float* dW_down_shard, void* workspace,
                  size_t workspace_bytes) {
  TPMLP_TRY(check_dtype(dtype));
  if (dtype != TPMLP_BF16) return fail(TPMLP_E_DTYPE, "the gated MLP is bf16 only");
  TPMLP_TRY(check_split("F", F, tp_size));
  TPMLP_TRY(check_rows("T", T));
  TPMLP_TRY(check_dim("h", h));
  TPMLP_TRY(check_dim("F", F));
  const int64_t Fs = F / tp_size;
  if (Fs % 8 != 0) return fail(TPMLP_E_DIVISIBILITY, "F/tp_size = %lld is not a multiple of 8", (long long)Fs);
  TPMLP_TRY(check_mat("X", X, T, h, h, 8));
  TPMLP_TRY(check_mat("W_gu_shard", W_gu_shard, h, 2 * Fs, 2 * Fs, 8));
  TPMLP_TRY(check_mat("W_down_shard", W_down_shard, Fs, h, h, 8));
  TPMLP_TRY(check_mat("GU_save", GU_save, T, 2 * Fs, 2 * Fs, 8));
  TPMLP_TRY(check_mat("A_save", A_save, T, Fs, Fs, 8));
  TPMLP_TRY(check_mat("dZ", dZ, T, h, h, 8));
  TPMLP_TRY(check_mat("dX_partial", dX_partial, T, h, h, 4));
  TPMLP_TRY(check_mat("dW_gu_shard", dW_gu_shard, h, 2 * Fs, 2 * Fs, 4));
  TPMLP_TRY(check_mat("dW_down_shard", dW_down_shard, Fs, h, h, 4));
  const size_t need = align256((size_t)T * 2 * Fs * sizeof(bf16_t));
  if (T > 0) {
    if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
    if (workspace_bytes < need) return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  }
  TPMLP_TRY(check_lds({h, 2 * Fs}));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    TPMLP_TRY(fill_zero(dW_gu_shard, h, 2 * Fs, 2 * Fs, s));
    return fill_zero(dW_down_shard, Fs, h, h, s);
  }
  void* dGU = workspace;
  // dA = dZ W_down_i^T; packed [dgate | dup] from dA and the saved gate/up
  GemmArgs a = gemm_args(dZ, h, W_down_shard, h, T, Fs, h);
  a.Y = dGU;
  a.ldy = 2 * Fs;
  a.H = const_cast<void*>(GU_save);
  a.ldh = 2 * Fs;
  // dW_down_i = A^T dZ (needs dZ only, like dA)
  GemmArgs wd = gemm_args(A_save, Fs, dZ, h, Fs, h, T);
  wd.C = dW_down_shard;
  wd.ldc = h;
  int cus = 256;
  TPMLP_TRY(device_cus(&cus));
  if (joins_under_wgrad(wd, a, cus)) {
    TPMLP_TRY((run_gemm_w4_duo<256, 256, false, false, kEpiF32, true, true, kEpiSwiGLUBwd>(
        "gemm.swiglu_wgrad2+gemm.swiglu_dgrad_act", wd, raster_group(true, wd.M, wd.N, 0, cus), a,
        raster_group(false, a.M, a.N, 0, cus), s)));
  } else {
    TPMLP_TRY((run_gemm<true, true, kEpiSwiGLUBwd>("gemm.swiglu_dgrad_act", dtype, a, s)));
    TPMLP_TRY((run_gemm<false, false, kEpiF32>("gemm.swiglu_wgrad2", dtype, wd, s)));
  }
  // dW_gu = X^T dGU (packed)
  a = gemm_args(X, h, dGU, 2 * Fs, h, 2 * Fs, T);
  a.C = dW_gu_shard;
  a.ldc = 2 * Fs;
  TPMLP_TRY((run_gemm<false, false, kEpiF32>("gemm.swiglu_wgrad1", dtype, a, s)));
  // dX_i = dGU W_gu^T
  a = gemm_args(dGU, 2 * Fs, W_gu_shard, 2 * Fs, T, h, 2 * Fs);
  a.C = dX_partial;
  a.ldc = h;
  return run_gemm<true, true, kEpiF32>("gemm.swiglu_dgrad1", dtype, a, s);
}

// ------------------------------------------------ sequence-parallel region --
namespace {
constexpr int64_t kLnMaxWidth = 256 * 8 * kLnMaxChunks;  // one workgroup per row, held in registers

int check_sp_width(int64_t h) {
  TPMLP_TRY(check_dim("h", h));
  if (h % 8 != 0) return fail(TPMLP_E_ALIGNMENT, "h = %lld is not a multiple of 8", (long long)h);
  return TPMLP_OK;
}

int dropout_params(float p, uint32_t* thr, float* scale) {
  if (!(p >= 0.0f && p < 1.0f)) return fail(TPMLP_E_VALUE, "dropout probability %g outside [0, 1)", (double)p);
  *thr = (uint32_t)std::floor((double)p * 4294967296.0);
  *scale = (float)(1.0 / (1.0 - (double)p));
  return TPMLP_OK;
}

unsigned grid_for(int64_t items) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 16384)); }
}  // namespace

int layernorm_fwd(void* stream, int64_t rows, int64_t h, const void* X, int64_t ldx, const float* gamma,
                  const float* beta, float eps, void* Y, int64_t ldy, float* mean, float* rstd) {
  TPMLP_TRY(check_rows("rows", rows));
  TPMLP_TRY(check_sp_width(h));
  if (h > kLnMaxWidth) return fail(TPMLP_E_SHAPE, "h = %lld above %lld", (long long)h, (long long)kLnMaxWidth);
  if (!(eps > 0.0f)) return fail(TPMLP_E_VALUE, "eps = %g must be positive", (double)eps);
  TPMLP_TRY(check_mat("X", X, rows, h, ldx, 8));
  TPMLP_TRY(check_mat("Y", Y, rows, h, ldy, 8));
  TPMLP_TRY(check_vec("gamma", gamma, h, true));
  TPMLP_TRY(check_vec("beta", beta, h, true));
  TPMLP_TRY(check_vec("mean", mean, rows, true));
  TPMLP_TRY(check_vec("rstd", rstd, rows, true));
  if (rows == 0) return TPMLP_OK;
  return launch("layernorm_fwd", "layernorm_fwd_kernel", layernorm_fwd_kernel, dim3((unsigned)rows),
                dim3(256), (hipStream_t)stream, static_cast<const bf16_t*>(X), ldx, (int)rows, (int)h, gamma, beta,
                eps, static_cast<bf16_t*>(Y), ldy, mean, rstd);
}

int layernorm_bwd(void* stream, int64_t rows, int64_t h, const void* X, int64_t ldx, const float* gamma,
                  const float* mean, const float* rstd, const float* dY, int64_t lddy, const void* dRes,
                  int64_t ldr, float* dX, int64_t lddx, float* dgamma, float* dbeta) {
  TPMLP_TRY(check_rows("rows", rows));
  TPMLP_TRY(check_sp_width(h));
  if (h > kLnMaxWidth) return fail(TPMLP_E_SHAPE, "h = %lld above %lld", (long long)h, (long long)kLnMaxWidth);
  TPMLP_TRY(check_mat("X", X, rows, h, ldx, 8));
  TPMLP_TRY(check_mat("dY", dY, rows, h, lddy, 4));
  TPMLP_TRY(check_mat("dRes", dRes, rows, h, ldr, 8, false));
  TPMLP_TRY(check_mat("dX", dX, rows, h, lddx, 4));
  TPMLP_TRY(check_vec("gamma", gamma, h, true));
  TPMLP_TRY(check_vec("mean", mean, rows, true));
  TPMLP_TRY(check_vec("rstd", rstd, rows, true));
  TPMLP_TRY(check_vec("dgamma", dgamma, h, false));
  TPMLP_TRY(check_vec("dbeta", dbeta, h, false));
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0) {
    TPMLP_TRY(fill_zero(dgamma, 1, h, h, s));
    return fill_zero(dbeta, 1, h, h, s);
  }
  TPMLP_TRY(launch("layernorm_bwd", "layernorm_bwd_kernel", layernorm_bwd_kernel, dim3((unsigned)rows), dim3(256), s,
                   static_cast<const bf16_t*>(X), ldx, (int)rows, (int)h, gamma, mean, rstd, dY, lddy,
                   static_cast<const bf16_t*>(dRes), ldr, dX, lddx));
  if (dgamma == nullptr && dbeta == nullptr) return TPMLP_OK;
  return launch("layernorm_param_grad", "layernorm_param_grad_kernel", layernorm_param_grad_kernel,
                dim3((unsigned)((h + 15) / 16)), dim3(256), s, static_cast<const bf16_t*>(X), ldx, (int)rows, (int)h,
                mean, rstd, dY, lddy, dgamma, dbeta);
}

int sp_partial_sum_dropout_residual(void* stream, int tp_size, int64_t rows, int64_t h, const float* partials,
                                    int64_t shard_stride, int64_t ldp, const void* residual, int64_t ldr,
                                    float p, uint64_t seed, int64_t row0, void* out, int64_t ldo) {
  if (tp_size < 1) return fail(TPMLP_E_DIVISIBILITY, "tp_size %d < 1", tp_size);
  TPMLP_TRY(check_rows("rows", rows));
  TPMLP_TRY(check_sp_width(h));
  if (row0 < 0 || row0 > kMaxDim) return fail(TPMLP_E_SHAPE, "row0 = %lld out of range", (long long)row0);
  uint32_t thr;
  float scale;
  TPMLP_TRY(dropout_params(p, &thr, &scale));
  TPMLP_TRY(check_mat("partials", partials, rows, h, ldp, 4));
  if (tp_size > 1 && (shard_stride % 4 != 0 || shard_stride < 0))
    return fail(TPMLP_E_ALIGNMENT, "shard_stride %lld must be a non-negative multiple of 4", (long long)shard_stride);
  TPMLP_TRY(check_mat("residual", residual, rows, h, ldr, 8));
  TPMLP_TRY(check_mat("out", out, rows, h, ldo, 8));
  if (rows * (h / 8) > kMaxDim) return fail(TPMLP_E_SHAPE, "rows * h / 8 above 2^31 - 1");
  if (rows == 0) return TPMLP_OK;
  return launch("sp_partial_sum_dropout_residual", "sp_sum_dropout_residual_kernel", sp_sum_dropout_residual_kernel,
                dim3(grid_for(rows * (h / 8))), dim3(256), (hipStream_t)stream, partials, shard_stride, ldp,
                tp_size, (int)rows, (int)h, static_cast<const bf16_t*>(residual), ldr, thr, scale, seed, row0,
                static_cast<bf16_t*>(out), ldo);
}

int sp_dropout_bwd(void* stream, int64_t rows, int64_t h, const void* dOut, int64_t ldi, float p, uint64_t seed,
                   int64_t row0, void* dZ, int64_t ldz) {
  TPMLP_TRY(check_rows("rows", rows));
  TPMLP_TRY(check_sp_width(h));
  if (row0 < 0 || row0 > kMaxDim) return fail(TPMLP_E_SHAPE, "row0 = %lld out of range", (long long)row0);
  uint32_t thr;
  float scale;
  TPMLP_TRY(dropout_params(p, &thr, &scale));
  TPMLP_TRY(check_mat("dOut", dOut, rows, h, ldi, 8));
  TPMLP_TRY(check_mat("dZ", dZ, rows, h, ldz, 8));
  if (rows * (h / 8) > kMaxDim) return fail(TPMLP_E_SHAPE, "rows * h / 8 above 2^31 - 1");
  if (rows == 0) return TPMLP_OK;
  return launch("sp_dropout_bwd", "sp_dropout_bwd_kernel", sp_dropout_bwd_kernel, dim3(grid_for(rows * (h / 8))),
                dim3(256), (hipStream_t)stream, static_cast<const bf16_t*>(dOut), ldi, (int)rows, (int)h, thr, scale,
                seed, row0, static_cast<bf16_t*>(dZ), ldz);
}

// ------------------------------------------------------ attention core --
namespace {
// Causal key chunks (see attn_key_chunks): kc key blocks per chunk, min_kc or
// more (even) so that the longest query block has at most 8 chunks; the chunk
// count of that block; and the work items per (sequence, head).
struct AttnChunkPlan {
  int64_t kc, chunks, items;
};

AttnChunkPlan attn_chunk_plan(int64_t seq, int64_t min_kc = 16) {
  AttnChunkPlan pl{min_kc, 0, 0};
  if (seq <= 0) return pl;
  const int64_t nkb = (seq + 63) / 64, nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  const int64_t need = (nkb + 7) / 8;
  if (need > pl.kc) pl.kc = need + (need & 1);
  pl.chunks = (nkb + pl.kc - 1) / pl.kc;
  for (int64_t c = 0; c < pl.chunks && (pl.kc / 2) * c < nqb; ++c) pl.items += nqb - (pl.kc / 2) * c;
  return pl;
}

// Causal forward partials when some query block has several key chunks: fp32
// O [batch][heads][items][128][128], then fp32 base-2 lse [batch][heads][items][128].
struct AttnFwdWs {
  size_t lse_off, total;
};

// Key blocks per chunk (at least): 26 (1664 keys) measured best for 4096
// causal tokens and 10 heads on the current kernels, for the forward (62 + 9.5
// us merge, against 72 + 8 at 32, 68.6 + 9.8 at 30, 65.3 + 9.4 at 28 and
// 63 + 10 at 24) and for dQ (81 + 8.8 us sum, against 91 + 7.5 at 32 and
// 81 + 9.5 at 24): the longest work item shortens more than the merge grows.
constexpr int64_t kAttnFwdMinKc = 26;
constexpr int64_t kAttnDqMinKc = 26;

AttnFwdWs attn_fwd_ws(int64_t batch, int64_t seq, int64_t heads) {
  AttnFwdWs w{0, 0};
  const AttnChunkPlan pl = attn_chunk_plan(seq, kAttnFwdMinKc);
  if (pl.chunks <= 1) return w;
  const size_t slots = (size_t)batch * heads * pl.items;
  w.lse_off = align256(slots * kAttnBQ * kAttnD * sizeof(float));
  w.total = w.lse_off + align256(slots * kAttnBQ * sizeof(float));
  return w;
}

int check_attn(int64_t batch, int64_t seq, int heads, int head_dim, int causal, float scale) {
  if (head_dim != kAttnD) return fail(TPMLP_E_SHAPE, "head_dim %d: the attention kernels take head_dim 128 only", head_dim);
  if (heads < 1 || heads > 65535) return fail(TPMLP_E_SHAPE, "heads = %d out of range [1, 65535]", heads);
  if (batch < 0 || batch > 65535) return fail(TPMLP_E_SHAPE, "batch = %lld out of range", (long long)batch);
  TPMLP_TRY(check_rows("seq", seq));
  if (batch * seq > kMaxDim) return fail(TPMLP_E_SHAPE, "batch * seq above 2^31 - 1");
  // One-dimensional grids: key blocks (dK/dV) or work items (forward, dQ; at
  // most 4 per key block plus 8) times heads times batch.
  if (((seq + 63) / 64 * 4 + 8) * heads * batch > kMaxDim)
    return fail(TPMLP_E_SHAPE, "(4 * key blocks + 8) x heads x batch above 2^31 - 1");
  if (causal != 0 && causal != 1) return fail(TPMLP_E_VALUE, "causal = %d must be 0 or 1", causal);
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(TPMLP_E_VALUE, "scale must be finite and positive");
  return TPMLP_OK;
}
}  // namespace

size_t attn_fwd_workspace_bytes(int64_t batch, int64_t seq, int heads) {
  if (batch < 0 || seq < 0 || heads < 1 || batch * seq > kMaxDim) return 0;
  return attn_fwd_ws(batch, seq, heads).total;
}

int attn_fwd(void* stream, int64_t batch, int64_t seq, int heads, int head_dim, int causal, float scale,
             const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv, void* O,
             int64_t ldo, float* lse, void* workspace, size_t workspace_bytes) {
  TPMLP_TRY(check_attn(batch, seq, heads, head_dim, causal, scale));
  const int64_t T = batch * seq, w = (int64_t)heads * head_dim;
  TPMLP_TRY(check_mat("Q", Q, T, w, ldq, 8));
  TPMLP_TRY(check_mat("K", K, T, w, ldk, 8));
  TPMLP_TRY(check_mat("V", V, T, w, ldv, 8));
  TPMLP_TRY(check_mat("O", O, T, w, ldo, 8));
  TPMLP_TRY(check_vec("lse", lse, T * heads, false));
  if (T == 0) return TPMLP_OK;
  if (ldq >= kMaxLd || ldk >= kMaxLd || ldv >= kMaxLd)
    return fail(TPMLP_E_SHAPE, "leading dimension above 2^22 elements");
  // Only causal calls with more than one key chunk per block use the workspace.
  const AttnChunkPlan pl = attn_chunk_plan(seq, kAttnFwdMinKc);
  const AttnFwdWs W = causal ? attn_fwd_ws(batch, seq, heads) : AttnFwdWs{0, 0};
  if (W.total > 0) {
    if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
    if (workspace_bytes < W.total)
      return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, W.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  }
  AttnArgs a;
  a.Q = static_cast<const bf16_t*>(Q);
  a.K = static_cast<const bf16_t*>(K);
  a.V = static_cast<const bf16_t*>(V);
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.O = static_cast<bf16_t*>(O);
  a.ldo = ldo;
  a.lse = lse;
  a.batch = (int)batch;
  a.seq = (int)seq;
  a.heads = heads;
  a.causal = causal;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.chunks = (int)pl.chunks;
  a.kc = (int)pl.kc;
  a.items = (int)pl.items;
  a.o_part = W.total > 0 ? static_cast<float*>(workspace) : nullptr;
  a.lse_part = W.total > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + W.lse_off) : nullptr;
  // Causal: one workgroup per (query block, key chunk); blocks with several
  // chunks are merged by attn_fwd_combine_kernel.
  const int64_t nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)((causal ? pl.items : nqb) * heads * batch));
  TPMLP_TRY(launch("attn_fwd", "attn_fwd_kernel", attn_fwd_kernel, grid, dim3(256), s, a));
  if (W.total > 0 && nqb > pl.kc / 2)
    TPMLP_TRY(launch("attn_fwd_combine", "attn_fwd_combine_kernel", attn_fwd_combine_kernel,
                     dim3((unsigned)(8 * (nqb - pl.kc / 2)), (unsigned)heads, (unsigned)batch), dim3(256), s, a));
  return TPMLP_OK;
}

namespace {
struct AttnBwdWs {
  size_t d_bytes, l2_off, part_off, total;
};

// D [heads, T] fp32, the base-2 lse [heads, T] fp32, then (when some causal
// query block has several key chunks) the fp32 dQ partials
// [batch][heads][work items][128][128].
AttnBwdWs attn_bwd_ws(int64_t batch, int64_t seq, int64_t heads) {
  AttnBwdWs w;
  w.d_bytes = align256((size_t)batch * seq * heads * sizeof(float));
  w.l2_off = w.d_bytes;
  w.part_off = w.l2_off + w.d_bytes;
  const AttnChunkPlan pl = attn_chunk_plan(seq, kAttnDqMinKc);
  const size_t part = pl.chunks > 1 ? (size_t)batch * heads * pl.items * kAttnBQ * kAttnD * sizeof(float) : 0;
  w.total = w.part_off + align256(part);
  return w;
}
}  // namespace

size_t attn_bwd_workspace_bytes(int64_t batch, int64_t seq, int heads) {
  if (batch < 0 || seq < 0 || heads < 1 || batch * seq > kMaxDim) return 0;
  return attn_bwd_ws(batch, seq, heads).total;
}

int attn_bwd(void* stream, int64_t batch, int64_t seq, int heads, int head_dim, int causal, float scale,
             const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv, const void* O,
             int64_t ldo, const void* dO, int64_t lddo, const float* lse, void* dQ, int64_t lddq, void* dK,
             int64_t lddk, void* dV, int64_t lddv, void* workspace, size_t workspace_bytes) {
  TPMLP_TRY(check_attn(batch, seq, heads, head_dim, causal, scale));
  const int64_t T = batch * seq, w = (int64_t)heads * head_dim;
  TPMLP_TRY(check_mat("Q", Q, T, w, ldq, 8));
  TPMLP_TRY(check_mat("K", K, T, w, ldk, 8));
  TPMLP_TRY(check_mat("V", V, T, w, ldv, 8));
  TPMLP_TRY(check_mat("O", O, T, w, ldo, 8));
  TPMLP_TRY(check_mat("dO", dO, T, w, lddo, 8));
  TPMLP_TRY(check_mat("dQ", dQ, T, w, lddq, 8));
  TPMLP_TRY(check_mat("dK", dK, T, w, lddk, 8));
  TPMLP_TRY(check_mat("dV", dV, T, w, lddv, 8));
  TPMLP_TRY(check_vec("lse", lse, T * heads, true));
  if (T == 0) return TPMLP_OK;
  if (ldq >= kMaxLd || ldk >= kMaxLd || ldv >= kMaxLd || lddo >= kMaxLd)
    return fail(TPMLP_E_SHAPE, "leading dimension above 2^22 elements");
  const AttnBwdWs W = attn_bwd_ws(batch, seq, heads);
  const size_t need = W.total;
  if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
  if (workspace_bytes < need) return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  AttnBwdArgs a;
  a.Q = static_cast<const bf16_t*>(Q);
  a.K = static_cast<const bf16_t*>(K);
  a.V = static_cast<const bf16_t*>(V);
  a.O = static_cast<const bf16_t*>(O);
  a.dO = static_cast<const bf16_t*>(dO);
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.ldo = ldo;
  a.lddo = lddo;
  a.lse = lse;
  a.D = static_cast<float*>(workspace);
  a.L2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + W.l2_off);
  a.dQ = static_cast<bf16_t*>(dQ);
  a.dK = static_cast<bf16_t*>(dK);
  a.dV = static_cast<bf16_t*>(dV);
  a.lddq = lddq;
  a.lddk = lddk;
  a.lddv = lddv;
  a.batch = (int)batch;
  a.seq = (int)seq;
  a.heads = heads;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const AttnChunkPlan dqp = attn_chunk_plan(seq, kAttnDqMinKc);
  a.dq_chunks = (int)dqp.chunks;
  a.dq_kc = (int)dqp.kc;
  a.dq_items = (int)dqp.items;
  a.dq_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + W.part_off);
  hipStream_t s = (hipStream_t)stream;
  const int64_t items = T * heads;
  TPMLP_TRY(launch("attn_bwd_dot", "attn_bwd_dot_kernel", attn_bwd_dot_kernel, dim3((unsigned)((items + 15) / 16)),
                   dim3(256), s, a));
  // Causal dK/dV: each workgroup takes a long and a short block (pairs x, n-1-x).
  // Causal dQ: one workgroup per (query block, key chunk); blocks with several
  // chunks are summed by attn_bwd_dq_sum_kernel.
  const int64_t nkb = (seq + 63) / 64, nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  const int64_t dq_items = causal ? dqp.items : nqb;
  TPMLP_TRY(launch("attn_bwd_dkdv", "attn_bwd_dkdv_kernel", attn_bwd_dkdv_kernel,
                   dim3((unsigned)(nkb * heads * batch)), dim3(256), s, a));
  TPMLP_TRY(launch("attn_bwd_dq", "attn_bwd_dq_kernel", attn_bwd_dq_kernel,
                   dim3((unsigned)(dq_items * heads * batch)), dim3(256), s, a));
  if (causal && dqp.chunks > 1 && nqb > dqp.kc / 2)
    TPMLP_TRY(launch("attn_bwd_dq_sum", "attn_bwd_dq_sum_kernel", attn_bwd_dq_sum_kernel,
                     dim3((unsigned)(8 * (nqb - dqp.kc / 2)), (unsigned)heads, (unsigned)batch), dim3(256), s, a));
  return TPMLP_OK;
}

// ------------------------------------------- head-sharded attention block --
namespace {
struct AttnBlockDims {
  int64_t T, w, hs;
};

int check_attn_block(int64_t batch, int64_t seq, int64_t h, int heads, int head_dim, int tp_size, int causal,
                     float scale, AttnBlockDims* d) {
  TPMLP_TRY(check_attn(batch, seq, heads, head_dim, causal, scale));
  TPMLP_TRY(check_split("heads", heads, tp_size));
  TPMLP_TRY(check_dim("h", h));
  d->T = batch * seq;
  d->hs = heads / tp_size;
  d->w = d->hs * head_dim;
  return TPMLP_OK;
}

struct AttnBlockWs {
  size_t do_off, dqkv_off, d_off, total;
};

// dO and dQKV (bf16), then the attention backward's own workspace.
AttnBlockWs attn_block_ws(int64_t batch, int64_t seq, int64_t w, int64_t hs) {
  const int64_t T = batch * seq;
  AttnBlockWs L;
  L.do_off = 0;
  L.dqkv_off = align256((size_t)T * w * 2);
  L.d_off = L.dqkv_off + align256((size_t)T * 3 * w * 2);
  L.total = L.d_off + attn_bwd_ws(batch, seq, hs).total;
  return L;
}
}  // namespace

size_t tp_attn_fwd_workspace_bytes(int64_t batch, int64_t seq, int heads, int head_dim, int tp_size) {
  if (batch < 0 || seq < 0 || heads < 1 || head_dim != kAttnD || tp_size < 1 || heads % tp_size != 0 ||
      batch * seq > kMaxDim)
    return 0;
  return attn_fwd_ws(batch, seq, heads / tp_size).total;
}

int tp_attn_fwd(void* stream, int64_t batch, int64_t seq, int64_t h, int heads, int head_dim, int tp_size,
                int causal, float scale, const void* X, const void* Wqkv_shard, const void* Wo_shard,
                void* QKV_save, void* O_save, float* lse, float* Z_partial, void* workspace,
                size_t workspace_bytes) {
  AttnBlockDims d;
  TPMLP_TRY(check_attn_block(batch, seq, h, heads, head_dim, tp_size, causal, scale, &d));
  const int64_t T = d.T, w = d.w;
  TPMLP_TRY(check_mat("X", X, T, h, h, 8));
  TPMLP_TRY(check_mat("Wqkv_shard", Wqkv_shard, h, 3 * w, 3 * w, 8));
  TPMLP_TRY(check_mat("Wo_shard", Wo_shard, w, h, h, 8));
  TPMLP_TRY(check_mat("QKV_save", QKV_save, T, 3 * w, 3 * w, 8));
  TPMLP_TRY(check_mat("O_save", O_save, T, w, w, 8));
  TPMLP_TRY(check_vec("lse", lse, T * d.hs, true));
  TPMLP_TRY(check_mat("Z_partial", Z_partial, T, h, h, 4));
  if (T == 0) return TPMLP_OK;
  // The attention core's workspace is checked here, before the first launch.
  const size_t need = causal ? attn_fwd_ws(batch, seq, d.hs).total : 0;
  if (need > 0) {
    if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
    if (workspace_bytes < need)
      return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  }
  TPMLP_TRY(check_lds({h, 3 * w}));
  hipStream_t s = (hipStream_t)stream;
  TPMLP_TRY(col_fwd(s, TPMLP_BF16, kActNone, T, h, 3 * w, X, h, Wqkv_shard, 3 * w, nullptr, QKV_save, 3 * w,
                    nullptr, 0, "gemm.attn_qkv"));
  const bf16_t* qkv = static_cast<const bf16_t*>(QKV_save);
  TPMLP_TRY(attn_fwd(stream, batch, seq, (int)d.hs, head_dim, causal, scale, qkv, 3 * w, qkv + w, 3 * w,
                     qkv + 2 * w, 3 * w, O_save, w, lse, workspace, workspace_bytes));
  return row_fwd(s, TPMLP_BF16, T, w, h, O_save, w, Wo_shard, h, Z_partial, h, "gemm.attn_out");
}

size_t tp_attn_bwd_workspace_bytes(int64_t batch, int64_t seq, int heads, int head_dim, int tp_size) {
  if (batch < 0 || seq < 0 || heads < 1 || head_dim != kAttnD || tp_size < 1 || heads % tp_size != 0 ||
      batch * seq > kMaxDim)
    return 0;
  const int64_t hs = heads / tp_size;
  return attn_block_ws(batch, seq, hs * head_dim, hs).total;
}

int tp_attn_bwd(void* stream, int64_t batch, int64_t seq, int64_t h, int heads, int head_dim, int tp_size,
                int causal, float scale, const void* X, const void* Wqkv_shard, const void* Wo_shard,
                const void* QKV_save, const void* O_save, const float* lse, const void* dZ, float* dX_partial,
                float* dWqkv_shard, float* dWo_shard, void* workspace, size_t workspace_bytes) {
  AttnBlockDims d;
  TPMLP_TRY(check_attn_block(batch, seq, h, heads, head_dim, tp_size, causal, scale, &d));
  const int64_t T = d.T, w = d.w;
  TPMLP_TRY(check_mat("X", X, T, h, h, 8));
  TPMLP_TRY(check_mat("Wqkv_shard", Wqkv_shard, h, 3 * w, 3 * w, 8));
  TPMLP_TRY(check_mat("Wo_shard", Wo_shard, w, h, h, 8));
  TPMLP_TRY(check_mat("QKV_save", QKV_save, T, 3 * w, 3 * w, 8));
  TPMLP_TRY(check_mat("O_save", O_save, T, w, w, 8));
  TPMLP_TRY(check_vec("lse", lse, T * d.hs, true));
  TPMLP_TRY(check_mat("dZ", dZ, T, h, h, 8));
  TPMLP_TRY(check_mat("dX_partial", dX_partial, T, h, h, 4));
  TPMLP_TRY(check_mat("dWqkv_shard", dWqkv_shard, h, 3 * w, 3 * w, 4));
  TPMLP_TRY(check_mat("dWo_shard", dWo_shard, w, h, h, 4));
  const AttnBlockWs L = attn_block_ws(batch, seq, w, d.hs);
  TPMLP_TRY(check_lds({h, 3 * w}));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    TPMLP_TRY(fill_zero(dWqkv_shard, h, 3 * w, 3 * w, s));
    return fill_zero(dWo_shard, w, h, h, s);
  }
  if (workspace == nullptr) return fail(TPMLP_E_NULL, "workspace is NULL");
  if (workspace_bytes < L.total)
    return fail(TPMLP_E_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TPMLP_E_ALIGNMENT, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  bf16_t* dO = reinterpret_cast<bf16_t*>(ws + L.do_off);
  bf16_t* dqkv = reinterpret_cast<bf16_t*>(ws + L.dqkv_off);
  // dO = dZ Wo_i^T, straight to bf16 (no activation, so no pre-activation is read).
  GemmArgs a = gemm_args(dZ, h, Wo_shard, h, T, w, h);
  a.Y = dO;
  a.ldy = w;
  TPMLP_TRY((run_gemm<true, true, kEpiActBwd>("gemm.attn_out_dgrad", TPMLP_BF16, a, s)));
  // dWo_i = O^T dZ
  a = gemm_args(O_save, w, dZ, h, w, h, T);
  a.C = dWo_shard;
  a.ldc = h;
  TPMLP_TRY((run_gemm<false, false, kEpiF32>("gemm.attn_out_wgrad", TPMLP_BF16, a, s)));
  const bf16_t* qkv = static_cast<const bf16_t*>(QKV_save);
  TPMLP_TRY(attn_bwd(stream, batch, seq, (int)d.hs, head_dim, causal, scale, qkv, 3 * w, qkv + w, 3 * w,
                     qkv + 2 * w, 3 * w, O_save, w, dO, w, lse, dqkv, 3 * w, dqkv + w, 3 * w, dqkv + 2 * w, 3 * w,
                     ws + L.d_off, L.total - L.d_off));
  // dWqkv_i = X^T dQKV
  a = gemm_args(X, h, dqkv, 3 * w, h, 3 * w, T);
  a.C = dWqkv_shard;
  a.ldc = 3 * w;
  TPMLP_TRY((run_gemm<false, false, kEpiF32>("gemm.attn_qkv_wgrad", TPMLP_BF16, a, s)));
  // dX_i = dQKV Wqkv_i^T
  a = gemm_args(dqkv, 3 * w, Wqkv_shard, 3 * w, T, h, 3 * w);
  a.C = dX_partial;
  a.ldc = h;
  return run_gemm<true, true, kEpiF32>("gemm.attn_qkv_dgrad", TPMLP_BF16, a, s);
}

int tpmlp_profile_enable(const char* filter) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  P.enabled = filter != nullptr;
  P.filter = filter ? filter : "";
  if (P.enabled && P.clk == nullptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&P.clk), sizeof(unsigned long long) * 2 * Profiler::kClkSlots);
    if (e != hipSuccess) {
      P.clk = nullptr;
      return hip_fail(e, "profile clock buffer");
    }
    P.clk_device = dev;
  }
  return TPMLP_OK;
}

int tpmlp_profile_collect(char* buf, size_t len) {
  Profiler& P = prof();
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(P.mu);
    recs.swap(P.records);
  }
  int status = TPMLP_OK;
  std::vector<float> ms(recs.size(), 0.0f);
  for (size_t i = 0; i < recs.size(); ++i) {
    hipError_t e = hipEventSynchronize(recs[i].stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], recs[i].start, recs[i].stop);
    if (e != hipSuccess && status == TPMLP_OK) status = hip_fail(e, "profile event");
  }
  // All recorded launches have finished: their clock samples are final.
  std::vector<unsigned long long> clk;
  if (P.clk != nullptr && !recs.empty()) {
    clk.resize(2 * Profiler::kClkSlots);
    hipError_t e = hipMemcpy(clk.data(), P.clk, clk.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      clk.clear();
      if (status == TPMLP_OK) status = hip_fail(e, "profile clock copy");
    }
  }
  std::string out = "[";
  for (size_t i = 0; i < recs.size(); ++i) {
    // shader clock in GHz over workgroup 0's main loop, -1 when not sampled
    double ghz = -1.0;
    const int sl = recs[i].clk_slot;
    if (sl >= 0 && !clk.empty() && clk[2 * sl + 1] > 0) ghz = (double)clk[2 * sl] / ((double)clk[2 * sl + 1] * 10.0);
    char item[512];
    snprintf(item, sizeof(item), "%s[\"%s\", \"%s\", %.6f, %.4f]", i ? ", " : "", recs[i].role.c_str(),
             recs[i].symbol.c_str(), ms[i], ghz);
    out += item;
  }
  out += "]";
  {
    std::lock_guard<std::mutex> lk(P.mu);
    for (auto& r : recs) {
      P.pool.push_back(r.start);
      P.pool.push_back(r.stop);
    }
  }
  if (buf && len > 0) {
    std::strncpy(buf, out.c_str(), len - 1);
    buf[len - 1] = '\0';
  }
  if (status == TPMLP_OK && out.size() >= len) return fail(TPMLP_E_SHAPE, "profile buffer too small");
  return status;
}

}  // extern "C"
