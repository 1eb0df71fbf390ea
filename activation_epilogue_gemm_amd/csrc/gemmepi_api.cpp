// C ABI of libgemmepi: argument validation, the plan cache and the dispatch
// of the fused and unfused paths.  Host code only; the kernels live in the
// .hip files.
//
// The plan/execute split follows the pages' stateful Matmul object: a
// lazy, checks-only construction, a costly planning step that picks the
// algorithm and kernel configuration for the shape and is cached so its
// cost is amortised, then cheap executions ("Fusing bias addition with
// matrix multiplication using nvmath-python", paragraphs 3 and 5;
// "nvmath-python cuBLASLt bias fusion guide", section "Advanced techniques
// and engineering practice").  Here planning is a deterministic shape ->
// tile table lookup, done on the host without touching the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "gemmepi.h"
#include "gemm_tiles.h"
#include "kernels.h"

namespace gemmepi {

#define GEMMEPI_TILE_ENTRY(id, bm, bn, bk, wm, wn, ns, sched, mt) \
  {bm, bn, bk, wm, wn, ns, sched, mt,                              \
   #bm "x" #bn "x" #bk "_w" #wm "x" #wn "_s" #ns "_p" #sched "_m" #mt},
const TileCfg kTiles[kNumTiles] = {GEMMEPI_TILES(GEMMEPI_TILE_ENTRY)};
#undef GEMMEPI_TILE_ENTRY
// the single-pass norm's row counters (gemmepi_norm_stats_bytes) assume
// tiles of at least 64 rows
#define GEMMEPI_TILE_ROWS(id, bm, bn, bk, wm, wn, ns, sched, mt) \
  static_assert(bm >= 64, "norm row counters: tile rows");
GEMMEPI_TILES(GEMMEPI_TILE_ROWS)
#undef GEMMEPI_TILE_ROWS
// the deepest k slab and the most rows (of A, or of B stored [N,K]) that
// one workgroup addresses from a single buffer descriptor
#define GEMMEPI_TILE_BK(id, bm, bn, bk, wm, wn, ns, sched, mt) bk,
#define GEMMEPI_TILE_MN(id, bm, bn, bk, wm, wn, ns, sched, mt) (bm > bn ? bm : bn),
constexpr int kTileBk[] = {GEMMEPI_TILES(GEMMEPI_TILE_BK)};
constexpr int kTileMn[] = {GEMMEPI_TILES(GEMMEPI_TILE_MN)};
#undef GEMMEPI_TILE_BK
#undef GEMMEPI_TILE_MN
constexpr int max_of(const int* a, int n) {
  int m = 0;
  for (int i = 0; i < n; ++i) m = a[i] > m ? a[i] : m;
  return m;
}
constexpr int kMaxSlabK = max_of(kTileBk, kNumTiles);
constexpr int kMaxPanelRows = max_of(kTileMn, kNumTiles);

// Relative throughput of one CU on a full tile of each configuration, and
// how many of its workgroups fit on one CU (LDS and registers).  Used only
// to rank tiles for a shape: the grid runs in `rounds` of up to
// kNumCU * occ tiles; in one round a CU holds up to `occ` tiles that share
// its MFMA units, so
//   est = rounds * min(occ, ceil(tiles / kNumCU)) * BM * BN / eff.
static const double kTileEff[kNumTiles] = {1.0, 0.95, 0.85, 0.70, 0.66, 0.56, 1.07, 0.95, 1.08,
                                           0.60};
static const int kTileOcc[kNumTiles] = {1, 1, 1, 1, 2, 3, 1, 1, 1, 1};
// With B stored [N,K] both operands are K-contiguous; a 32-wide k slab then
// fetches 64-byte row segments of both, which measured 0.83x on the
// 65536 x 8192 x 16384 shape.  64-wide slabs fetch whole 128-byte lines and
// lose nothing; schedule 2 fetches both operands in 64-wide slabs.  With
// this factor at 1.0 the 2048 x 4096 x 11008 GEMM (B [N,K]) is split twice
// over schedule 2 (128 tiles of 256 x 256, 256 workgroups), measured
// 160.8 us against 170.9 us for tile 7 unsplit (interleaved, one box); no
// other shape of the suite changes plan.
double tile_eff(int t, bool bt) {
  if (!bt || kTiles[t].bk >= 64) return kTileEff[t];
  return kTileEff[t] * (kTiles[t].sched == 2 ? 1.0 : 0.83);
}
constexpr int kNumCU = 256;

hipError_t launch_gemm(int dtype, bool b_trans, int tile, const GemmArgs& a, hipStream_t s) {
  if (dtype == DT_F16)
    return b_trans ? launch_gemm_f16_bt(tile, a, s) : launch_gemm_f16_bn(tile, a, s);
  return b_trans ? launch_gemm_bf16_bt(tile, a, s) : launch_gemm_bf16_bn(tile, a, s);
}

// (cached: the kernels are built for one architecture)
hipError_t gemm_blocks_per_cu(int dtype, bool b_trans, int tile, int* n) {
  static std::atomic<int> cache[2][2][kNumTiles];
  if (tile < 0 || tile >= kNumTiles || (dtype != DT_F16 && dtype != DT_BF16))
    return hipErrorInvalidValue;
  std::atomic<int>& c = cache[dtype][b_trans ? 1 : 0][tile];
  int v = c.load(std::memory_order_relaxed);
  if (v > 0) {
    *n = v;
    return hipSuccess;
  }
  hipError_t e;
  if (dtype == DT_F16)
    e = b_trans ? blocks_per_cu_f16_bt(tile, &v) : blocks_per_cu_f16_bn(tile, &v);
  else
    e = b_trans ? blocks_per_cu_bf16_bt(tile, &v) : blocks_per_cu_bf16_bn(tile, &v);
  if (e != hipSuccess) return e;
  if (v > 0) c.store(v, std::memory_order_relaxed);
  *n = v;
  return hipSuccess;
}

}  // namespace gemmepi

using namespace gemmepi;

enum PlanPath { PATH_GEMM = 0, PATH_DECODE = 1 };

struct gemmepi_plan_s {
  int64_t M, N, K;
  int dtype, epi;
  uint32_t flags;
  int tile_req;
  int splits_req;  // -1 from the flags, 0 chosen, >= 1 requested
  int path;
  int tile;
  int tiles_m, tiles_n, group_m, xcd_remap;
  int sb_m, sb_n, xcd_m, xcd_n;
  int tuned;  // tile taken from a measured autotune result
  int stage_b;  // B stored [K,N] is first copied [N,K] into the workspace
  int splits, kt_split;  // split-K: K ranges per tile, k slabs per range
  int k_per_wave;
  int refs;
  std::string info;
};

namespace {

using Key = std::tuple<int64_t, int64_t, int64_t, int, int, uint32_t, int, int>;

std::mutex g_mu;
std::map<Key, gemmepi_plan_s*>& cache() {
  static std::map<Key, gemmepi_plan_s*> c;
  return c;
}
thread_local std::string g_err;

// Measured tile choices (gemmepi_autotune), keyed by shape, dtype, epilogue
// and flags.  With GEMMEPI_TUNE_CACHE=<path> they persist in a text file,
// one "gemmepi-tune-v1 M N K dtype epi flags tile" line per key, read once
// by the first plan() (host file I/O only) and rewritten by autotune.
using TuneKey = std::tuple<int64_t, int64_t, int64_t, int, int, uint32_t>;
std::map<TuneKey, int>& tuned() {
  static std::map<TuneKey, int> t;
  return t;
}
bool g_tune_loaded = false;

const char* tune_cache_path() {
  const char* s = getenv("GEMMEPI_TUNE_CACHE");
  return (s && s[0]) ? s : nullptr;
}

// Caller holds g_mu.
void load_tune_cache() {
  if (g_tune_loaded) return;
  g_tune_loaded = true;
  const char* path = tune_cache_path();
  if (!path) return;
  FILE* f = fopen(path, "r");
  if (!f) return;
  char line[256];
  while (fgets(line, sizeof line, f)) {
    long long M, N, K;
    int dtype, epi, tile;
    unsigned flags;
    char tag[32];
    if (sscanf(line, "%31s %lld %lld %lld %d %d %u %d", tag, &M, &N, &K, &dtype, &epi, &flags,
               &tile) != 8)
      continue;
    if (strcmp(tag, "gemmepi-tune-v1") != 0 || tile < 0 || tile >= kNumTiles || M < 1 || N < 1 ||
        K < 1)
      continue;
    tuned()[TuneKey{M, N, K, dtype, epi, flags}] = tile;
  }
  fclose(f);
}

// Caller holds g_mu.  Rewrites the whole file (write to <path>.tmp, rename).
bool save_tune_cache() {
  const char* path = tune_cache_path();
  if (!path) return true;
  std::string tmp = std::string(path) + ".tmp";
  FILE* f = fopen(tmp.c_str(), "w");
  if (!f) return false;
  for (auto& kv : tuned()) {
    const TuneKey& k = kv.first;
    fprintf(f, "gemmepi-tune-v1 %lld %lld %lld %d %d %u %d\n", (long long)std::get<0>(k),
            (long long)std::get<1>(k), (long long)std::get<2>(k), std::get<3>(k), std::get<4>(k),
            std::get<5>(k), kv.second);
  }
  const bool ok = fclose(f) == 0;
  return ok && rename(tmp.c_str(), path) == 0;
}

gemmepi_status_t fail(gemmepi_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr uint32_t kAllFlags = GEMMEPI_FLAG_B_TRANS | GEMMEPI_FLAG_BIAS_PER_COL |
                               GEMMEPI_FLAG_UNFUSED | GEMMEPI_FLAG_VALIDATE |
                               GEMMEPI_FLAG_NO_DECODE | GEMMEPI_FLAG_SPLIT_K |
                               GEMMEPI_FLAG_STAGE_B | GEMMEPI_FLAG_NORM_TWO_PASS;
constexpr int kMaxSplits = 64;
// Split-K cost model, fitted to a measured (tile, splits) sweep on one
// MI355X: a split unit pays for its partial-tile round trip about as much
// as kSplitCost k-steps of MFMA work on its tile, and a split plan must be
// estimated at least kSplitGain faster than the best unsplit plan.
constexpr double kSplitCost = 200.0;
constexpr double kSplitGain = 0.95;
constexpr int64_t kMaxDim = 0x7FFFFFFF;
// With GEMMEPI_FLAG_STAGE_B, B stored [K,N] is copied to [N,K] when the GEMM
// has at least this many rows: the copy (read and write of N K elements)
// then costs a few per cent of the GEMM, whose K-contiguous form ran ~10 %
// faster than the [K,N] form on the 65536 x 8192 x 16384 shape.
constexpr int64_t kStageMinM = 8192;

bool log_enabled() {
  static int v = [] {
    const char* e = getenv("GEMMEPI_LOG");
    return (e && *e && *e != '0') ? 1 : 0;
  }();
  return v != 0;
}

// Split-K ranges actually used for a request of `splits`: whole k slabs
// per range, no empty range.
void split_shape(int64_t K, int bk, int splits, int* eff_splits, int* kt_split) {
  const int64_t KT = (K + bk - 1) / bk;
  int64_t s = splits < 1 ? 1 : splits;
  if (s > KT) s = KT;
  const int64_t per = (KT + s - 1) / s;
  *kt_split = (int)per;
  *eff_splits = (int)((KT + per - 1) / per);
}

// Estimated time of tile t with `splits` K ranges: the units (tile, range)
// run in rounds of kNumCU * occ; a CU's share of a round costs its units'
// MFMA work (BM * BN * k) over the tile's efficiency, plus, when K is
// split, the partial-tile round trip (all splits' partials are read by the
// last one: kSplitCost * BM * BN * splits).
double tile_estimate(int t, int64_t M, int64_t N, int64_t K, bool bt, int splits) {
  const TileCfg& c = kTiles[t];
  int s = 1, per = 0;
  split_shape(K, c.bk, splits, &s, &per);
  const int64_t units = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * s;
  const int64_t slots = (int64_t)kNumCU * kTileOcc[t];
  const int64_t rounds = (units + slots - 1) / slots;
  const int64_t per_cu = (units + kNumCU - 1) / kNumCU;
  const int64_t share = per_cu < kTileOcc[t] ? per_cu : kTileOcc[t];
  double unit = (double)c.bm * c.bn * per * c.bk / tile_eff(t, bt);
  if (s > 1) unit += kSplitCost * c.bm * c.bn * s;
  return (double)rounds * share * unit;
}

int choose_tile(int64_t M, int64_t N, int64_t K, bool bt) {
  int best = 0;
  double best_est = 0.0;
  for (int t = 0; t < kNumTiles; ++t) {
    const double est = tile_estimate(t, M, N, K, bt, 1);
    if (t == 0 || est < best_est) {
      best = t;
      best_est = est;
    }
  }
  return best;
}

// Tile (when tile < 0) and split count for a split-K-enabled plan: the
// best unsplit estimate, unless some split count in {2, 3, 4, 6, 8, 16}
// is estimated kSplitGain faster.
void choose_split(int64_t M, int64_t N, int64_t K, bool bt, int* tile, int* splits) {
  const int t0 = *tile < 0 ? 0 : *tile, t1 = *tile < 0 ? kNumTiles : *tile + 1;
  static const int kCand[] = {2, 3, 4, 6, 8, 16};
  int b1 = t0, bst = t0, bss = 1;
  double best1 = 0.0, bests = 0.0;
  for (int t = t0; t < t1; ++t) {
    const double e1 = tile_estimate(t, M, N, K, bt, 1);
    if (t == t0 || e1 < best1) {
      best1 = e1;
      b1 = t;
    }
    for (int s : kCand) {
      const double es = tile_estimate(t, M, N, K, bt, s);
      if (bests == 0.0 || es < bests) {
        bests = es;
        bst = t;
        bss = s;
      }
    }
  }
  if (bests < kSplitGain * best1) {
    *tile = bst;
    *splits = bss;
  } else {
    *tile = b1;
    *splits = 1;
  }
}

void describe(gemmepi_plan_s* p) {
  char buf[384];
  static const char* epis[] = {"DEFAULT",     "BIAS",        "RELU_BIAS",
                               "RELU_AUX_BIAS", "GELU_BIAS", "DRELU_BGRAD",
                               "BIAS_RES_RMSNORM", "BIAS_RES_LAYERNORM",
                               "GELU_AUX_BIAS", "DGELU_BGRAD"};
  if (p->path == PATH_DECODE) {
    const DecodeKind kind = decode_kind((int)p->M, (int)p->N, (int)p->K);
    const int rows = decode_rows(kind);
    static const char* kinds[] = {"mfma", "rowstream", "rowwave"};
    snprintf(buf, sizeof(buf),
             "path=decode M=%lld N=%lld K=%lld dtype=%s epi=%s flags=0x%x kernel=%s rows=%d "
             "grid=%lld waves=%d%s",
             (long long)p->M, (long long)p->N, (long long)p->K, p->dtype ? "bf16" : "f16",
             epis[p->epi], p->flags, kinds[kind], rows, (long long)((p->N + rows - 1) / rows),
             decode_waves(kind), (p->flags & GEMMEPI_FLAG_UNFUSED) ? " unfused" : "");
  } else {
    const TileCfg& c = kTiles[p->tile];
    char split_buf[64] = "";
    if (p->splits > 1)
      snprintf(split_buf, sizeof(split_buf), " splits=%d kt_split=%d", p->splits, p->kt_split);
    snprintf(buf, sizeof(buf),
             "path=gemm M=%lld N=%lld K=%lld dtype=%s epi=%s flags=0x%x tile=%s tiles=%dx%d "
             "raster=%s%s%s%s%s",
             (long long)p->M, (long long)p->N, (long long)p->K, p->dtype ? "bf16" : "f16",
             epis[p->epi], p->flags, c.name, p->tiles_m, p->tiles_n,
             p->sb_m ? "chip16x16/xcd4x8" : (p->xcd_remap ? "xcd_remap,group8" : "group8"),
             split_buf, p->stage_b ? " stage_b" : "", p->tuned ? " tuned" : "",
             (p->flags & GEMMEPI_FLAG_UNFUSED) ? " unfused" : "");
  }
  p->info = buf;
}

// Lazily checked per device: the kernels are built for gfx950 only.
gemmepi_status_t check_device() {
  static int ok_dev[64] = {0};  // 0 unknown, 1 ok, -1 bad
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(GEMMEPI_ERR_DEVICE, "device index %d out of range", dev);
  if (ok_dev[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(GEMMEPI_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    ok_dev[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (ok_dev[dev] < 0)
      return fail(GEMMEPI_ERR_HIP, "device %d is %s; libgemmepi is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (ok_dev[dev] < 0) return fail(GEMMEPI_ERR_HIP, "device %d is not gfx950", dev);
  return GEMMEPI_OK;
}

// Poll bound of the single-pass norm's row wait: kNormWaitPolls, or
// GEMMEPI_NORM_WAIT_POLLS (read at every call) to force the give-up path in
// a test (0: a workgroup that is not the last of its band gives up at once).
uint32_t norm_wait_polls() {
  const char* e = getenv("GEMMEPI_NORM_WAIT_POLLS");
  if (!e || !*e) return kNormWaitPolls;
  char* end = nullptr;
  const unsigned long v = strtoul(e, &end, 10);
  if (!end || *end != '\0' || v > kNormWaitPolls) return kNormWaitPolls;
  return (uint32_t)v;
}

// Compute units of the current device (cached per device).
gemmepi_status_t device_cus(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(GEMMEPI_ERR_DEVICE, "device index %d out of range", dev);
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
      return fail(GEMMEPI_ERR_HIP, "compute unit count: %s", hipGetErrorString(e));
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return GEMMEPI_OK;
}

gemmepi_status_t check_device_ptr(const void* p, const char* name) {
  int dev = 0;
  hipGetDevice(&dev);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(GEMMEPI_ERR_DEVICE, "%s: not a HIP allocation (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice)
    return fail(GEMMEPI_ERR_DEVICE, "%s: not device memory (type %d)", name, (int)attr.type);
  if (attr.device != dev)
    return fail(GEMMEPI_ERR_DEVICE, "%s: on device %d, current device is %d", name, attr.device,
                dev);
  return GEMMEPI_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The shape, layout and raster fields of the tiled GEMM's arguments; the
// epilogue fields are zero.
GemmArgs gemm_args(const gemmepi_plan_s& p, const void* A, const void* B, void* out) {
  GemmArgs g{};
  const int N = (int)p.N, K = (int)p.K;
  g.A = A;
  g.B = B;
  g.out = out;
  g.M = (int)p.M;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldb = ((p.flags & GEMMEPI_FLAG_B_TRANS) || p.stage_b) ? K : N;
  g.ldo = N;
  g.aux_words = (N + 31) / 32;
  g.tiles_m = p.tiles_m;
  g.tiles_n = p.tiles_n;
  g.group_m = p.group_m;
  g.xcd_remap = p.xcd_remap;
  g.sb_m = p.sb_m;
  g.sb_n = p.sb_n;
  g.xcd_m = p.xcd_m;
  g.xcd_n = p.xcd_n;
  g.splits = p.splits;
  g.kt_split = p.kt_split;
  return g;
}

// Split-K layout of a tiled-GEMM plan (1 = none).
void set_split(gemmepi_plan_s* p, int splits) {
  split_shape(p->K, kTiles[p->tile].bk, splits, &p->splits, &p->kt_split);
  if (p->splits <= 1) {
    p->splits = 1;
    p->kt_split = 0;
  }
}

// Workspace of a split plan: the arrival counters (one per tile, padded to
// 256 bytes), then one fp32 partial tile per (tile, split).
size_t counter_bytes(const gemmepi_plan_s& p) {
  return ((size_t)p.tiles_m * p.tiles_n * 4 + 255) / 256 * 256;
}
// Staged plans keep the [N,K] copy of B at the start of the workspace.
size_t stage_bytes(const gemmepi_plan_s& p) {
  return p.stage_b ? ((size_t)p.N * (size_t)p.K * 2 + 255) / 256 * 256 : 0;
}
size_t workspace_bytes(const gemmepi_plan_s& p) {
  if (p.path != PATH_GEMM) return 0;
  size_t b = stage_bytes(p);
  if (p.splits > 1) {
    const TileCfg& c = kTiles[p.tile];
    b += counter_bytes(p) + (size_t)p.tiles_m * p.tiles_n * p.splits * c.bm * c.bn * 4;
  }
  return b;
}

// Tile, grid shape and raster of a tiled-GEMM plan.
void set_tile(gemmepi_plan_s* p, int tile) {
  const int64_t M = p->M, N = p->N;
  p->path = PATH_GEMM;
  p->tile = tile;
  const TileCfg& c = kTiles[tile];
  p->tiles_m = (int)((M + c.bm - 1) / c.bm);
  p->tiles_n = (int)((N + c.bn - 1) / c.bn);
  p->group_m = p->tiles_m < 8 ? p->tiles_m : 8;
  const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
  p->xcd_remap = (tiles % 8 == 0 && tiles >= 64) ? 1 : 0;
  // chip-block raster when one round of 16 x 16 tiles (one per CU) divides
  // the grid; XCDs take 4 x 8 sub-blocks (4 A panels, 8 B panels each)
  p->sb_m = p->sb_n = p->xcd_m = p->xcd_n = 0;
  const char* rast = getenv("GEMMEPI_RASTER");
  const bool chip_ok = kTileOcc[tile] == 1 && p->tiles_m % 16 == 0 && p->tiles_n % 16 == 0;
  if (chip_ok && !(rast && rast[0] == '0')) {
    p->sb_m = 16;
    p->sb_n = 16;
    p->xcd_m = 4;
    p->xcd_n = 2;
  }
}

gemmepi_status_t make_plan(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                           gemmepi_dtype_t dtype, gemmepi_epilogue_t epi, uint32_t flags,
                           int32_t tile_req, int32_t splits_req) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "plan: null output pointer");
  *plan = nullptr;
  if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "sizes must be in [1, 2^31-1]: M=%lld N=%lld K=%lld",
                (long long)M, (long long)N, (long long)K);
  if (dtype != GEMMEPI_F16 && dtype != GEMMEPI_BF16)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "unknown dtype %d", (int)dtype);
  if ((int)epi < GEMMEPI_EPI_DEFAULT || (int)epi > GEMMEPI_EPI_DGELU_BGRAD)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "unknown epilogue %d", (int)epi);
  if (flags & ~kAllFlags) return fail(GEMMEPI_ERR_INVALID_VALUE, "unknown flag bits 0x%x", flags);
  if (tile_req < -1 || tile_req >= kNumTiles)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "unknown tile id %d", tile_req);
  if (splits_req < -1 || splits_req > kMaxSplits)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "splits %d outside [0, %d]", splits_req, kMaxSplits);
  const bool norm_epi = epi == GEMMEPI_EPI_BIAS_RES_RMSNORM || epi == GEMMEPI_EPI_BIAS_RES_LAYERNORM;
  if (norm_epi && splits_req > 1)
    return fail(GEMMEPI_ERR_UNSUPPORTED, "the norm epilogues do not split K");
  // what plan() does about K splits: 1 never, 0 choose, > 1 as requested
  int split_mode = splits_req >= 0 ? splits_req : ((flags & GEMMEPI_FLAG_SPLIT_K) ? 0 : 1);
  if (norm_epi) split_mode = 1;
  const bool bt = flags & GEMMEPI_FLAG_B_TRANS;
  if (K % 8 != 0)
    return fail(GEMMEPI_ERR_MISALIGNED, "K=%lld must be a multiple of 8", (long long)K);
  if (!bt && N % 8 != 0)
    return fail(GEMMEPI_ERR_MISALIGNED,
                "N=%lld must be a multiple of 8 when B is stored [K,N] (no B_TRANS)",
                (long long)N);
  // 32-bit buffer offsets: the rows of A (or of B stored [N,K]) that one
  // workgroup addresses, and the k rows of one slab of B stored [K,N], must
  // stay below 2 GiB from the descriptor's base, whatever tile runs
  if (K * 2 * kMaxPanelRows >= 0x7FFFFFF0LL || (!bt && N * 2 * kMaxSlabK >= 0x7FFFFFF0LL))
    return fail(GEMMEPI_ERR_UNSUPPORTED, "leading dimension too large (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (M * N > (int64_t)1 << 40)
    return fail(GEMMEPI_ERR_UNSUPPORTED, "output too large");

  const Key key{M, N, K, (int)dtype, (int)epi, flags, tile_req, splits_req};
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = cache().find(key);
  if (it != cache().end()) {
    it->second->refs += 1;
    *plan = it->second;
    return GEMMEPI_OK;
  }
  gemmepi_plan_s* p = new (std::nothrow) gemmepi_plan_s();
  if (!p) return fail(GEMMEPI_ERR_NO_MEMORY, "plan allocation failed");
  p->M = M;
  p->N = N;
  p->K = K;
  p->dtype = (int)dtype;
  p->epi = (int)epi;
  p->flags = flags;
  p->tile_req = tile_req;
  p->splits_req = splits_req;
  p->splits = 1;
  p->refs = 1;
  const bool decode_epi = epi == GEMMEPI_EPI_DEFAULT || epi == GEMMEPI_EPI_BIAS ||
                          epi == GEMMEPI_EPI_RELU_BIAS || epi == GEMMEPI_EPI_GELU_BIAS;
  if (tile_req < 0 && split_mode <= 1 && !(flags & GEMMEPI_FLAG_NO_DECODE) && bt && M <= 16 &&
      decode_epi) {
    p->path = PATH_DECODE;
    p->tile = -1;
    const int64_t per = (K + 8 * 32 - 1) / (8 * 32) * 32;  // 8 waves, 32-wide steps
    p->k_per_wave = (int)per;
  } else {
    int tile = tile_req;
    int splits = split_mode;
    if (tile < 0) {
      load_tune_cache();
      auto t = tuned().find(TuneKey{M, N, K, (int)dtype, (int)epi, flags});
      if (t != tuned().end()) {
        tile = t->second;
        p->tuned = 1;
        if (splits == 0) splits = 1;
      }
    }
    // B as the kernel reads it: staged plans read the [N,K] copy
    bool stage = (flags & GEMMEPI_FLAG_STAGE_B) && !bt && !norm_epi && M >= kStageMinM;
    const int tile0 = tile, splits0 = splits;
    for (;;) {
      const bool bt_k = bt || stage;
      if (splits == 0)
        choose_split(M, N, K, bt_k, &tile, &splits);  // keeps an explicit tile
      else if (tile < 0)
        tile = choose_tile(M, N, K, bt_k);
      if (!stage || splits <= 1) break;
      // a shape that wants K split is too small to repay the copy
      stage = false;
      tile = tile0;
      splits = splits0;
    }
    p->stage_b = stage ? 1 : 0;
    set_tile(p, tile);
    set_split(p, splits);
    if ((int64_t)p->tiles_m * p->tiles_n * p->splits > 0x7FFFFFFFLL) {
      delete p;
      return fail(GEMMEPI_ERR_UNSUPPORTED, "grid too large");
    }
  }
  describe(p);
  if (log_enabled()) fprintf(stderr, "[gemmepi] plan %s\n", p->info.c_str());
  cache()[key] = p;
  *plan = p;
  return GEMMEPI_OK;
}

bool plan_live(gemmepi_plan_t plan) {
  for (auto& kv : cache())
    if (kv.second == plan) return true;
  return false;
}

// ws_static: the workspace is the library's static scratch (ws is its
// address on the current device): it is not checked as a caller allocation,
// and its counters are cleared here, since the previous call's contents
// remain in it.
gemmepi_status_t execute_impl(const gemmepi_plan_s& p, const void* A, const void* B, void* bias,
                              void* aux, void* out, void* ws, size_t ws_bytes, void* stream,
                              bool ws_static = false) {
  const int epi = p.epi;
  const bool bt = (p.flags & GEMMEPI_FLAG_B_TRANS) || p.stage_b;  // as the kernel reads B
  const bool per_col = p.flags & GEMMEPI_FLAG_BIAS_PER_COL;
  const bool unfused = p.flags & GEMMEPI_FLAG_UNFUSED;
  const bool bgrad_epi = epi == EPI_DRELU_BGRAD || epi == EPI_DGELU_BGRAD;
  const bool needs_bias = epi != EPI_DEFAULT;  // *_BGRAD: bgrad output
  const bool needs_aux = epi == EPI_RELU_AUX_BIAS || epi == EPI_DRELU_BGRAD ||
                         epi == EPI_GELU_AUX_BIAS || epi == EPI_DGELU_BGRAD;

  if (epi == EPI_BIAS_RES_RMSNORM || epi == EPI_BIAS_RES_LAYERNORM)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: norm epilogues run through execute_norm");
  if (!A || !B || !out) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: A, B and out are required");
  if (needs_bias && !bias)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: this epilogue needs the bias pointer%s",
                bgrad_epi ? " (fp32 bgrad output)" : "");
  if (needs_aux && !aux) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: this epilogue needs aux");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(out, 16))
    return fail(GEMMEPI_ERR_MISALIGNED, "execute: A, B and out must be 16-byte aligned");
  if (needs_bias && !aligned(bias, bgrad_epi ? 4 : 2))
    return fail(GEMMEPI_ERR_MISALIGNED, "execute: bias misaligned");
  if (needs_aux && !aligned(aux, 16))
    return fail(GEMMEPI_ERR_MISALIGNED, "execute: aux must be 16-byte aligned");
  const size_t ws_need = workspace_bytes(p);
  if (ws_need > 0) {
    if (!ws)
      return fail(GEMMEPI_ERR_INVALID_VALUE,
                  "execute: the plan %s and needs a workspace of %zu bytes "
                  "(gemmepi_execute_ws)", p.stage_b ? "stages B" : "splits K", ws_need);
    if (ws_bytes < ws_need)
      return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: workspace of %zu bytes, the plan needs %zu",
                  ws_bytes, ws_need);
    if (!aligned(ws, 256))
      return fail(GEMMEPI_ERR_MISALIGNED, "execute: workspace must be 256-byte aligned");
  }

  gemmepi_status_t st = check_device();
  if (st != GEMMEPI_OK) return st;
  if (p.flags & GEMMEPI_FLAG_VALIDATE) {
    if ((st = check_device_ptr(A, "A")) != GEMMEPI_OK) return st;
    if ((st = check_device_ptr(B, "B")) != GEMMEPI_OK) return st;
    if ((st = check_device_ptr(out, "out")) != GEMMEPI_OK) return st;
    if (needs_bias && (st = check_device_ptr(bias, "bias")) != GEMMEPI_OK) return st;
    if (needs_aux && (st = check_device_ptr(aux, "aux")) != GEMMEPI_OK) return st;
    if (ws_need > 0 && !ws_static && (st = check_device_ptr(ws, "workspace")) != GEMMEPI_OK)
      return st;
  }

  hipStream_t s = (hipStream_t)stream;
  const int M = (int)p.M, N = (int)p.N, K = (int)p.K;
  const int aux_ld = (int)gemmepi_aux_ld_words(N);
  const int core_epi = unfused ? EPI_DEFAULT : epi;
  hipError_t e = hipSuccess;
  (void)hipGetLastError();  // clear a stale error so it is not blamed on this call

  if (p.splits > 1 && ws_static) {
    // a fill kernel rather than hipMemsetAsync, so a captured stream
    // replays it correctly
    e = launch_fill_f32((float*)((uint8_t*)ws + stage_bytes(p)), (int64_t)(counter_bytes(p) / 4),
                        0.0f, s);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "scratch counter fill: %s", hipGetErrorString(e));
  }
  if (bgrad_epi) {
    e = launch_fill_f32((float*)bias, N, 0.0f, s);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "bgrad fill: %s", hipGetErrorString(e));
  }

  if (p.path == PATH_DECODE) {
    DecodeArgs d;
    d.x = A;
    d.W = B;
    d.bias = bias;
    d.out = out;
    d.M = M;
    d.N = N;
    d.K = K;
    d.ldx = K;
    d.ldw = K;
    d.ldo = N;
    d.k_per_wave = p.k_per_wave;
    d.epi = core_epi;
    d.bias_per_col = per_col ? 1 : 0;
    e = launch_decode(p.dtype, d, s);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "decode kernel: %s", hipGetErrorString(e));
  } else {
    GemmArgs g = gemm_args(p, A, B, out);
    g.bias = bias;
    g.aux = (uint32_t*)aux;
    g.bgrad = (float*)bias;
    g.aux_ld = aux_ld;
    g.epi = core_epi;
    g.bias_per_col = per_col ? 1 : 0;
    if (p.stage_b) {
      // B [K,N] -> its [N,K] copy at the start of the workspace
      e = launch_transpose16(B, ws, K, N, s);
      if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "B staging copy: %s", hipGetErrorString(e));
      g.B = ws;
    }
    if (p.splits > 1) {
      uint8_t* w = (uint8_t*)ws + stage_bytes(p);
      g.counters = (uint32_t*)w;
      g.ws = (float*)(w + counter_bytes(p));
    }
    e = launch_gemm(p.dtype, bt, p.tile, g, s);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "gemm kernel: %s", hipGetErrorString(e));
  }

  if (unfused) {
    switch (epi) {
      case EPI_DEFAULT:
        break;
      case EPI_DRELU_BGRAD:
        e = launch_mask_apply(p.dtype, out, (const uint32_t*)aux, M, N, N, aux_ld, s);
        if (e == hipSuccess) e = launch_colsum(p.dtype, out, (float*)bias, M, N, N, s);
        break;
      case EPI_DGELU_BGRAD:
        e = launch_dgelu_apply(p.dtype, out, aux, M, N, N, s);
        if (e == hipSuccess) e = launch_colsum(p.dtype, out, (float*)bias, M, N, N, s);
        break;
      default:
        e = launch_bias_add(p.dtype, out, bias, M, N, N, per_col ? 1 : 0, s);
        if (e == hipSuccess && epi != EPI_BIAS)
          e = launch_activation(p.dtype, epi, out, (uint32_t*)aux, M, N, N, aux_ld, s);
        break;
    }
    if (e != hipSuccess)
      return fail(GEMMEPI_ERR_HIP, "unfused elementwise kernel: %s", hipGetErrorString(e));
  }
  return GEMMEPI_OK;
}

}  // namespace

extern "C" {

gemmepi_status_t gemmepi_plan(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                              gemmepi_dtype_t dtype, gemmepi_epilogue_t epi, uint32_t flags) {
  return make_plan(plan, M, N, K, dtype, epi, flags, -1, -1);
}

gemmepi_status_t gemmepi_plan_tiled(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                                    gemmepi_dtype_t dtype, gemmepi_epilogue_t epi,
                                    uint32_t flags, int32_t tile_id) {
  return make_plan(plan, M, N, K, dtype, epi, flags, tile_id, -1);
}

gemmepi_status_t gemmepi_plan_split(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                                    gemmepi_dtype_t dtype, gemmepi_epilogue_t epi,
                                    uint32_t flags, int32_t tile_id, int32_t splits) {
  if (splits < 0)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "splits %d outside [0, %d]", splits, kMaxSplits);
  return make_plan(plan, M, N, K, dtype, epi, flags, tile_id, splits);
}

size_t gemmepi_workspace_bytes(gemmepi_plan_t plan) {
  if (!plan) return 0;
  return workspace_bytes(*plan);
}

gemmepi_status_t gemmepi_execute_ws(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                    void* aux, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: null plan");
  return execute_impl(*plan, A, B, bias, aux, out, workspace, workspace_bytes, stream);
}

gemmepi_status_t gemmepi_execute_noalloc(gemmepi_plan_t plan, const void* A, const void* B,
                                         void* bias, void* aux, void* out, void* stream) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute_noalloc: null plan");
  const size_t need = workspace_bytes(*plan);
  if (need == 0) return execute_impl(*plan, A, B, bias, aux, out, nullptr, 0, stream);
  if (need > kScratchBytes)
    return fail(GEMMEPI_ERR_UNSUPPORTED,
                "execute_noalloc: the plan's workspace is %zu bytes, more than the "
                "library's static scratch of %zu bytes (use gemmepi_execute_ws)",
                need, kScratchBytes);
  gemmepi_status_t st = check_device();
  if (st != GEMMEPI_OK) return st;
  void* ws = nullptr;
  const hipError_t e = scratch_pointer(&ws);
  if (e != hipSuccess)
    return fail(GEMMEPI_ERR_HIP, "execute_noalloc: static scratch address: %s", hipGetErrorString(e));
  return execute_impl(*plan, A, B, bias, aux, out, ws, kScratchBytes, stream, true);
}

size_t gemmepi_noalloc_scratch_bytes(void) { return kScratchBytes; }

gemmepi_status_t gemmepi_execute_norm(gemmepi_plan_t plan, const void* A, const void* B,
                                      const void* bias, const void* residual,
                                      const void* gamma, const void* beta, float eps,
                                      void* stats, void* out, void* stream) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute_norm: null plan");
  const gemmepi_plan_s& p = *plan;
  const int epi = p.epi;
  if (epi != EPI_BIAS_RES_RMSNORM && epi != EPI_BIAS_RES_LAYERNORM)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "execute_norm: the plan's epilogue is not a norm");
  const bool layernorm = epi == EPI_BIAS_RES_LAYERNORM;
  const bool unfused = p.flags & GEMMEPI_FLAG_UNFUSED;
  if (!layernorm) beta = nullptr;
  if (!A || !B || !out || !gamma || !stats)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "execute_norm: A, B, gamma, stats and out are required");
  if (!(eps > 0.0f) || !(eps < 3.0e38f))
    return fail(GEMMEPI_ERR_INVALID_VALUE, "execute_norm: eps must be positive and finite");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(out, 16) ||
      (residual && !aligned(residual, 16)))
    return fail(GEMMEPI_ERR_MISALIGNED, "execute_norm: A, B, residual and out must be 16-byte aligned");
  if ((bias && !aligned(bias, 2)) || !aligned(gamma, 2) || (beta && !aligned(beta, 2)) ||
      !aligned(stats, 8))
    return fail(GEMMEPI_ERR_MISALIGNED, "execute_norm: bias, gamma, beta or stats misaligned");

  gemmepi_status_t st = check_device();
  if (st != GEMMEPI_OK) return st;
  if (p.flags & GEMMEPI_FLAG_VALIDATE) {
    const void* ptrs[] = {A, B, out, gamma, stats, bias, residual, beta};
    const char* names[] = {"A", "B", "out", "gamma", "stats", "bias", "residual", "beta"};
    for (int i = 0; i < 8; ++i)
      if (ptrs[i] && (st = check_device_ptr(ptrs[i], names[i])) != GEMMEPI_OK) return st;
  }

  hipStream_t s = (hipStream_t)stream;
  const int M = (int)p.M, N = (int)p.N;
  const bool bt = (p.flags & GEMMEPI_FLAG_B_TRANS) != 0;
  hipError_t e = hipSuccess;
  (void)hipGetLastError();
  GemmArgs g = gemm_args(p, A, B, out);
  // Single pass when the whole grid is resident at once (every workgroup of
  // a tile row must reach the row wait); otherwise the GEMM writes y and a
  // second kernel normalises it.
  bool one_pass = false;
  if (!unfused && !(p.flags & GEMMEPI_FLAG_NORM_TWO_PASS)) {
    int per_cu = 0, cus = 0;
    if ((st = device_cus(&cus)) != GEMMEPI_OK) return st;
    e = gemm_blocks_per_cu(p.dtype, bt, p.tile, &per_cu);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
    one_pass = (int64_t)p.tiles_m * p.tiles_n <= (int64_t)per_cu * cus;
  }
  if (!unfused) {
    // the sums (and the row counters) start at zero; the whole buffer is
    // cleared, so row_sync[0] reads 0 after a two-pass execution
    e = launch_fill_f32((float*)stats, (int64_t)(gemmepi_norm_stats_bytes(M) / 4), 0.0f, s);
    if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "stats fill: %s", hipGetErrorString(e));
    g.bias = bias;
    g.residual = residual;
    g.stats = (double*)stats;
    g.bias_per_col = 1;
    if (one_pass) {
      g.epi = EPI_BIAS_RES_NORM;
      g.gamma = gamma;
      g.beta = beta;
      g.eps = eps;
      g.layernorm = layernorm ? 1 : 0;
      g.row_sums = (double*)stats + 2 * (size_t)M;
      g.row_sync = (uint32_t*)((double*)stats + 4 * (size_t)M);
      g.norm_wait_polls = norm_wait_polls();
    } else {
      g.epi = EPI_BIAS_RES_SUMS;
    }
  } else {
    g.epi = EPI_DEFAULT;
  }
  e = launch_gemm(p.dtype, bt, p.tile, g, s);
  if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "gemm kernel: %s", hipGetErrorString(e));
  if (one_pass) return GEMMEPI_OK;
  if (unfused) {
    if (bias) e = launch_bias_add(p.dtype, out, bias, M, N, N, 1, s);
    if (e == hipSuccess && residual) e = launch_residual_add(p.dtype, out, residual, M, N, N, s);
    if (e != hipSuccess)
      return fail(GEMMEPI_ERR_HIP, "unfused elementwise kernel: %s", hipGetErrorString(e));
  }
  e = launch_norm_rows(p.dtype, out, gamma, beta, (double*)stats, M, N, N, eps, layernorm ? 1 : 0,
                       unfused ? 0 : 1, s);
  if (e != hipSuccess) return fail(GEMMEPI_ERR_HIP, "norm kernel: %s", hipGetErrorString(e));
  return GEMMEPI_OK;
}

// (mean, rstd) [M][2] fp64, the row sums [M][2] fp64 of the single pass, then
// row_sync: a status word and one arrival count per tile row (every tile has
// at least 64 rows), rounded up to 16 bytes
size_t gemmepi_norm_stats_bytes(int64_t M) {
  if (M < 1) return 0;
  const size_t sync_words = 1 + (size_t)((M + 63) / 64);
  return ((size_t)M * 32 + sync_words * 4 + 15) & ~(size_t)15;
}

gemmepi_status_t gemmepi_plan_destroy(gemmepi_plan_t plan) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "plan_destroy: null plan");
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto it = cache().begin(); it != cache().end(); ++it) {
    if (it->second == plan) {
      if (--plan->refs == 0) {
        cache().erase(it);
        delete plan;
      }
      return GEMMEPI_OK;
    }
  }
  return fail(GEMMEPI_ERR_INVALID_VALUE, "plan_destroy: not a live plan");
}

gemmepi_status_t gemmepi_plan_info(gemmepi_plan_t plan, char* buf, size_t len) {
  if (!plan || !buf || len == 0) return fail(GEMMEPI_ERR_INVALID_VALUE, "plan_info: bad argument");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!plan_live(plan)) return fail(GEMMEPI_ERR_INVALID_VALUE, "plan_info: not a live plan");
  snprintf(buf, len, "%s", plan->info.c_str());
  return GEMMEPI_OK;
}

int32_t gemmepi_num_tiles(void) { return kNumTiles; }

const char* gemmepi_tile_name(int32_t tile_id) {
  if (tile_id < 0 || tile_id >= kNumTiles) return nullptr;
  return kTiles[tile_id].name;
}

int64_t gemmepi_aux_ld_words(int64_t N) {
  if (N < 1) return 0;
  return ((N + 31) / 32 + 3) / 4 * 4;
}

size_t gemmepi_aux_bytes(int64_t M, int64_t N) {
  if (M < 1 || N < 1) return 0;
  return (size_t)M * (size_t)gemmepi_aux_ld_words(N) * 4u;
}

const char* gemmepi_status_string(gemmepi_status_t s) {
  switch (s) {
    case GEMMEPI_OK: return "GEMMEPI_OK";
    case GEMMEPI_ERR_INVALID_VALUE: return "GEMMEPI_ERR_INVALID_VALUE";
    case GEMMEPI_ERR_MISALIGNED: return "GEMMEPI_ERR_MISALIGNED";
    case GEMMEPI_ERR_UNSUPPORTED: return "GEMMEPI_ERR_UNSUPPORTED";
    case GEMMEPI_ERR_DEVICE: return "GEMMEPI_ERR_DEVICE";
    case GEMMEPI_ERR_HIP: return "GEMMEPI_ERR_HIP";
    case GEMMEPI_ERR_NO_MEMORY: return "GEMMEPI_ERR_NO_MEMORY";
  }
  return "unknown status";
}

const char* gemmepi_last_error(void) { return g_err.c_str(); }

int32_t gemmepi_version(void) { return GEMMEPI_VERSION; }

gemmepi_status_t gemmepi_execute(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                 void* aux, void* out, void* stream) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "execute: null plan");
  // The plan is immutable after creation (autotune excepted); callers keep
  // it alive while they execute it, so no lock is taken on this path.
  return execute_impl(*plan, A, B, bias, aux, out, nullptr, 0, stream);
}

gemmepi_status_t gemmepi_autotune(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                  void* aux, void* out, int32_t reps, float* times_ms,
                                  void* stream) {
  if (!plan) return fail(GEMMEPI_ERR_INVALID_VALUE, "autotune: null plan");
  if (reps < 1 || reps > 10000) return fail(GEMMEPI_ERR_INVALID_VALUE, "autotune: reps %d", reps);
  gemmepi_plan_s& p = *plan;
  if (p.path != PATH_GEMM)
    return fail(GEMMEPI_ERR_UNSUPPORTED, "autotune: the decode kernel has no tile to tune");
  if (p.epi == EPI_BIAS_RES_RMSNORM || p.epi == EPI_BIAS_RES_LAYERNORM)
    return fail(GEMMEPI_ERR_UNSUPPORTED, "autotune: norm plans are not tuned");
  if (p.tile_req >= 0)
    return fail(GEMMEPI_ERR_INVALID_VALUE, "autotune: the plan has an explicit tile");
  if (p.splits > 1 || p.stage_b)
    return fail(GEMMEPI_ERR_UNSUPPORTED, "autotune: split-K and B-staging plans are not tuned");
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(GEMMEPI_ERR_HIP, "autotune: event creation failed");
  }
  int best = -1;
  float best_ms = 0.0f;
  gemmepi_status_t st = GEMMEPI_OK;
  for (int t = 0; t < kNumTiles && st == GEMMEPI_OK; ++t) {
    gemmepi_plan_s q = p;  // same operands, another tile
    set_tile(&q, t);
    st = execute_impl(q, A, B, bias, aux, out, nullptr, 0, stream);  // warm-up (validates the arguments)
    if (st != GEMMEPI_OK) break;
    hipError_t e = hipEventRecord(e0, s);
    for (int r = 0; r < reps && st == GEMMEPI_OK; ++r)
      st = execute_impl(q, A, B, bias, aux, out, nullptr, 0, stream);
    if (st != GEMMEPI_OK) break;
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) {
      st = fail(GEMMEPI_ERR_HIP, "autotune timing: %s", hipGetErrorString(e));
      break;
    }
    ms /= (float)reps;
    if (times_ms) times_ms[t] = ms;
    if (best < 0 || ms < best_ms) {
      best = t;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != GEMMEPI_OK) return st;
  std::lock_guard<std::mutex> lock(g_mu);
  load_tune_cache();
  tuned()[TuneKey{p.M, p.N, p.K, p.dtype, p.epi, p.flags}] = best;
  set_tile(&p, best);
  p.tuned = 1;
  describe(&p);
  if (!save_tune_cache())
    return fail(GEMMEPI_ERR_HIP, "autotune: could not write %s", tune_cache_path());
  return GEMMEPI_OK;
}

}  // extern "C"
