// C-ABI front end: argument validation (before any HIP call), blob layout, work
// planning and kernel dispatch. See include/qgemm.h for the contract.
#include "qgemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qgemm_internal.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_force_nb{0};
std::atomic<int> g_force_wpt{0};
std::atomic<int> g_force_splits{0};
std::atomic<int> g_force_kernel{0};

constexpr int64_t kMaxM = 65535;
constexpr int64_t kMaxKN = int64_t(1) << 20;
constexpr int64_t kMaxKW4A8 = 16384;
constexpr int64_t kMaxWeights = int64_t(1) << 32;   // K*N: at most 2 GiB of 4-bit codes
constexpr int64_t kMaxKBitplane = 65536;            // K*127*255 < 2^31: exact int32

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return QGEMM_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

bool valid_fmt(int fmt) {
  return fmt == QGEMM_FMT_W4A16 || fmt == QGEMM_FMT_W4A8 || fmt == QGEMM_FMT_W2W4 || fmt == QGEMM_FMT_W4A16_SP24;
}

int check_kn(int fmt, int64_t K, int64_t N) {
  if (K <= 0 || K % qg::kGroup != 0 || K > kMaxKN) return QGEMM_ERR_SHAPE;
  if (N <= 0 || N % 64 != 0 || N > kMaxKN) return QGEMM_ERR_SHAPE;
  if (fmt == QGEMM_FMT_W4A8 && K > kMaxKW4A8) return QGEMM_ERR_SHAPE;
  if (fmt == QGEMM_FMT_BITPLANE && K > kMaxKBitplane) return QGEMM_ERR_SHAPE;
  if (K * N > kMaxWeights) return QGEMM_ERR_SHAPE;   // 32-bit buffer offsets into the blob
  return QGEMM_OK;
}

// General grid: 64, or a multiple of 128 dividing K (K itself: one group per column).
bool valid_group_size(int64_t K, int64_t gs) {
  return gs == 64 || (gs > 0 && gs % qg::kGroup == 0 && K % gs == 0);
}

// The current device must be a gfx950 GPU; cached per device ordinal.
int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::map<int, int> cache;
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) {
      if (it->second != QGEMM_OK) g_last_error = "current device is not gfx950";
      return it->second;
    }
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const int st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? QGEMM_OK : QGEMM_ERR_DEVICE;
  if (st != QGEMM_OK) g_last_error = std::string("device arch ") + prop.gcnArchName + " is not gfx950";
  std::lock_guard<std::mutex> lk(mu);
  cache[dev] = st;
  return st;
}

int no_plan() {
  g_last_error = "no launch shape of this call fits the 160 KB of LDS of a workgroup";
  return QGEMM_ERR_SHAPE;
}

int64_t count_bits(const uint32_t* bitmap, int64_t G, int64_t N, bool* stray) {
  const int64_t W = (N + 31) / 32;
  int64_t n = 0;
  *stray = false;
  for (int64_t g = 0; g < G; ++g)
    for (int64_t w = 0; w < W; ++w) {
      uint32_t v = bitmap[g * W + w];
      const int64_t valid = std::min<int64_t>(32, N - 32 * w);
      if (valid < 32 && (v >> valid) != 0) *stray = true;
      n += __builtin_popcount(v);
    }
  return n;
}

}  // namespace

namespace qg {

BlobLayout blob_layout(int fmt, int64_t K, int64_t N, int64_t n4) {
  BlobLayout L;
  L.K = K;
  L.N = N;
  L.G = K / kGroup;
  L.NB = N / 16;
  L.G8 = (L.G + 7) / 8;
  const size_t chunks = (size_t)(L.NB * L.G);
  if (fmt == QGEMM_FMT_W4A16) {
    L.codes = 0;
    L.scales = align256(chunks * 1024);
    L.total = L.scales + align256((size_t)L.NB * L.G8 * 256);
  } else if (fmt == QGEMM_FMT_W4A8) {
    L.codes = 0;
    L.scales = align256(chunks * 1024);
    L.aux = L.scales + align256((size_t)L.NB * L.G8 * 128);
    L.total = L.aux + align256((size_t)N * 2);
  } else if (fmt == QGEMM_FMT_W4A16_SP24) {
    L.codes = 0;
    L.scales = align256(chunks * 768);
    L.high = L.scales + align256((size_t)L.NB * L.G8 * 256);
    L.total = L.high + 256;
  } else {
    L.codes = 0;
    L.aux = align256(chunks * 512);
    L.scales = L.aux + align256(chunks * 8);
    L.high = L.scales + align256((size_t)L.NB * L.G8 * 256);
    L.total = L.high + align256((size_t)n4 * 32);
  }
  return L;
}

BlobLayout blob_layout_w4g(int64_t K, int64_t N, int gs, bool zeros) {
  BlobLayout L;
  L.K = K;
  L.N = N;
  L.G = K / kGroup;
  L.NB = N / 16;
  L.G8 = (L.G + 7) / 8;
  L.codes = 0;
  L.scales = align256((size_t)(L.NB * L.G) * 1024);
  L.total = L.scales + align256((size_t)(K / gs) * (size_t)N * (zeros ? 4 : 2));
  return L;
}

BlobLayout blob_layout_bitplane(int64_t K, int64_t N, int bits) {
  BlobLayout L;
  L.K = K;
  L.N = N;
  L.G = K / kGroup;
  L.NB = N / 16;
  L.G8 = (L.G + 7) / 8;
  L.codes = 0;
  L.aux = align256((size_t)(L.NB * L.G) * 256 * bits);
  L.total = L.aux + align256((size_t)N * 2);
  return L;
}

// Large-M W4A16 plan: 8-wave workgroups own 16*mb x 256 tiles. K is split across
// workgroups until about one workgroup per CU is busy: measured on MI355X, a
// second resident workgroup per CU does not pay for the extra partial-sum
// traffic of the splits it needs.
// nb = 4: 256-column tiles of 8-wave K-parts; nb = 2: 128-column tiles of two
// 4-wave K-parts (the same 64 x 32 wave tile)
Plan make_wide_plan_nb(int64_t M, int64_t K, int64_t N, int nb) {
  Plan pl;
  const int G = (int)(K / kGroup);
  pl.kernel = 2;
  // 64-row tiles at every M: larger M takes more row tiles, which re-read the
  // same weights from L2 (row tiles of one column tile sit on one XCD), rather
  // than taller tiles that would need more k-splits (measured on MI355X:
  // 128 x 8192 x 28672 in 78 us as 2 x 64 rows vs 93 us as one 128-row tile)
  pl.mb = 4;
  pl.nb = nb;
  // 8 waves (two per SIMD), or 16 as two K-parts of 8: on layers of at least
  // 2^27 weights at M > 64 (two row tiles) the extra waves hide more of the
  // weight stream (measured on MI355X, 70B layers: 48.3 vs 52.1 us at M = 96,
  // 48.8 vs 52.2 us at M = 128; at M = 48-64, and on 7B-class layers at every
  // M, 8 waves were faster: 21.7 vs 23.3 us at 128 x 4096 x 11008)
  const int fw = g_force_wpt.load();
  pl.wpt = fw == 16 ? 16 : fw != 0 ? 8 : (M > 64 && K * N >= (int64_t(1) << 27) ? 16 : 8);
  if (nb == 2) pl.wpt = 8;
  pl.mt = (int)((M + 16 * pl.mb - 1) / (16 * pl.mb));
  pl.nt = (int)(N / (64 * nb));
  const int64_t tiles = (int64_t)pl.mt * pl.nt;
  const int force_splits = g_force_splits.load();
  const int best = (int)std::max<int64_t>(1, std::min<int64_t>(std::max(1, G / 2), device_cu_count() / tiles));
  const int splits = force_splits ? std::min(force_splits, G) : best;
  pl.gps = (G + splits - 1) / splits;
  pl.splits = (G + pl.gps - 1) / pl.gps;
  pl.workgroups = launch_workgroups(pl.nt, pl.mt, pl.splits);
  pl.waves = pl.workgroups * pl.wpt;
  pl.lds_bytes = wide_lds_bytes(pl);
  if (pl.splits > 1) {
    // partial tiles are kept whole (rows padded to the tile) in fragment order
    pl.counter_bytes = counter_region_bytes(tiles);
    pl.ws_bytes = pl.counter_bytes + align256((size_t)pl.splits * pl.mt * 16 * pl.mb * N * 4);
  }
  return pl;
}

// The 256-column plan, or the 128-column one where it needs fewer k-splits for
// at most one workgroup per CU while the 256-column plan runs 8 waves: the
// same workgroups with fewer partial sums (measured on MI355X in one process:
// 128 x 4096 x 11008 22.5 against 25.6 us, 28672 x 8192 at M = 48 / 64 48.1 /
// 45.9 against 50.0 / 47.0 us, 8192 x 28672 at M = 48 / 64 50.8 / 52.0 against
// 52.1 / 52.3 us; where the 256-column plan runs 16 waves, at M > 64 on the
// 70B layers, the 128-column tiles were 5-21 % slower).
Plan make_wide_plan(int64_t M, int64_t K, int64_t N) {
  const int fnb = g_force_nb.load();
  if (fnb == 2 || fnb == 4) return make_wide_plan_nb(M, K, N, fnb);
  const Plan p256 = make_wide_plan_nb(M, K, N, 4);
  if (p256.wpt != 8 || p256.splits == 1) return p256;
  const Plan p128 = make_wide_plan_nb(M, K, N, 2);
  if ((int64_t)p128.mt * p128.nt <= device_cu_count() && p128.splits < p256.splits) return p128;
  return p256;
}

// Waves per SIMD that the register use of each streaming kernel allows, as
// the gfx950 compiler reports it (-Rpass-analysis=kernel-resource-usage), and
// whether the kernel spills to scratch. Rows: format; characters: tile shape
// (mb, nb) = (1,1) (1,2) (2,1) (2,2), each for kp = 1, 2, 4 waves per column
// block; 'a'..'h' = 1..8 waves and spilled, '1'..'8' = not spilled. The
// general-grid rows are per activation type, each the minimum over the
// variants with and without zero points; the bit-plane rows are b = 1..8.
// For the general grid the planner takes the spill flag of the call's type
// and the waves per SIMD of the lower type: residency counted with the fp16
// rows alone moved plans that then measured 6-12 % slower on MI355X
// (11008 x 4096 at M = 80, 8192 x 28672 at M = 1-4), while excluding only the
// type's own spilling instances admits the 16-wave two-block fp16 tiles
// (8192 x 28672 at M = 24-32: 32.8-33.3 against 36.0-36.9 us).
namespace {
const char* const kOccW4A16 = "888555777555";   // 32-row two-block tiles: the M32 policy
const char* const kOccW4A8 = "888555677444";
const char* const kOccW2W4 = "666444655444";
const char* const kOccW4GH = "677455455344";   // fp16, grid entries staged in LDS
const char* const kOccW4GLH = "677445455344";  // fp16, grid entries loaded per lane
const char* const kOccW4GB = "55544434423d";   // bf16, staged
const char* const kOccW4GLB = "55544434423d";  // bf16, per lane
const char* const kOccSP24 = "666555555444";
const char* const kOccBP[8] = {"888888888777", "888888788555", "888777566444", "788566455344", "67755544443d", "56645534433d", "55544434433d", "55544423d13d"};
}  // namespace

KernelOccupancy skinny_occupancy(int fmt, int mb, int nb, int kp, int bits, int kernel, bool act_bf16) {
  const int idx = ((mb - 1) * 2 + (nb - 1)) * 3 + (kp == 1 ? 0 : kp == 2 ? 1 : 2);
  auto waves = [](char ch) { return ch >= 'a' ? ch - 'a' + 1 : ch - '0'; };
  KernelOccupancy o;
  if (fmt == QGEMM_FMT_W4G) {
    const char* own = kernel == 3 ? (act_bf16 ? kOccW4GLB : kOccW4GLH) : (act_bf16 ? kOccW4GB : kOccW4GH);
    const char* other = kernel == 3 ? (act_bf16 ? kOccW4GLH : kOccW4GLB) : (act_bf16 ? kOccW4GH : kOccW4GB);
    o.spills = own[idx] >= 'a';
    o.waves_per_simd = std::min(waves(own[idx]), waves(other[idx]));
    return o;
  }
  const char* row = fmt == QGEMM_FMT_W4A16 ? kOccW4A16
                    : fmt == QGEMM_FMT_W4A8 ? kOccW4A8
                    : fmt == QGEMM_FMT_W2W4 ? kOccW2W4
                    : fmt == QGEMM_FMT_W4A16_SP24 ? kOccSP24
                    : kOccBP[std::min(std::max(bits, 1), 8) - 1];
  const char ch = row[idx];
  o.spills = ch >= 'a';
  o.waves_per_simd = waves(ch);
  return o;
}

namespace {
// dynamic LDS of a streaming-kernel launch of plan c
size_t plan_lds(int fmt, const Plan& c, int G, int bits, int gs, bool zeros) {
  (void)bits;
  return fmt == QGEMM_FMT_W4A16         ? lds_bytes_w4a16(c, G)
         : fmt == QGEMM_FMT_W4A8        ? lds_bytes_w4a8(c, G)
         : fmt == QGEMM_FMT_W4G         ? lds_bytes_w4g(c, G, gs, zeros)
         : fmt == QGEMM_FMT_W4A16_SP24  ? lds_bytes_sp24(c, G)
         : fmt == QGEMM_FMT_BITPLANE    ? lds_bytes_bitplane(c, G)
                                        : lds_bytes_w2w4(c, G);
}
}  // namespace

int device_cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  static bool no_device = false;
  std::lock_guard<std::mutex> lk(mu);
  if (no_device) return kDefaultCUs;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    no_device = true;
    return kDefaultCUs;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = kDefaultCUs;
  cache[dev] = cus;
  return cus;
}

namespace {
// Two 32-row tiles (M = 33..64) of W4A16, W4A8, the 2:4 sparse format and the
// general grid on a layer of 128-column tiles whose 2 x N/128 workgroups cover
// between half and all of the CUs, with each busy CU streaming under 96 KB more
// than on a launch over every CU: one workgroup per tile and no k-split (see
// make_plan).
bool two_row_tiles_unsplit(int fmt, int64_t M, int64_t K, int64_t N, double chunk, int cus) {
  if (fmt != QGEMM_FMT_W4A16 && fmt != QGEMM_FMT_W4A8 && fmt != QGEMM_FMT_W4A16_SP24 && fmt != QGEMM_FMT_W4G)
    return false;
  if (M <= 32 || M > 64 || N % 128 != 0 || K / kGroup < 4) return false;
  const int64_t T = 2 * (N / 128);
  const double blob = (double)(K / kGroup) * (double)(N / 16) * chunk;
  const double extra = 2.0 * blob * (1.0 / (double)T - 1.0 / (double)cus);
  return 2 * T >= cus && T <= cus && extra < 96.0 * 1024.0;
}
}  // namespace

Plan make_plan(int fmt, int64_t M, int64_t K, int64_t N, int bits, int gs, bool zeros, bool act_bf16) {
  const int force_kernel = g_force_kernel.load();
  const int cus = device_cu_count();
  // the wide kernel: W4A16, and the general grid with fp16 activations
  const bool wide_ok = (fmt == QGEMM_FMT_W4A16 || (fmt == QGEMM_FMT_W4G && !act_bf16)) && N % kWideCols == 0;
  if (wide_ok && (force_kernel == 2 || (force_kernel == 0 && M >= kWideMinM))) {
    // The wide tile (256 columns, all rows of the batch) needs many k-splits on
    // narrow layers, and their partial sums then cost more than re-streaming
    // the weights once per 32-row tile of the streaming kernel (measured on
    // MI355X: 7B-class layers at M = 64..128 and N = 8192 at M = 128).
    // (decided on the 256-column plan's k-splits). On layers below 2^27
    // weights at M <= 64 whose two 32-row tiles take the unsplit streaming
    // plan, that plan measured faster (4096 x 14336 at M = 48-64: 16.3-16.4
    // against 22.7-23.2 us; 5120 x 13824: 19.8-19.9 against 24.1-25.2 us).
    const Plan wide = make_wide_plan_nb(M, K, N, 4);
    const bool big = K * N >= (int64_t(1) << 27);
    const bool unsplit32 = fmt == QGEMM_FMT_W4A16 && !big && two_row_tiles_unsplit(fmt, M, K, N, 1024.0, cus);
    if (force_kernel == 2 || (!unsplit32 && (wide.splits <= 4 || (big && M <= 64))))
      return make_wide_plan(M, K, N);
  }
  // Streaming kernel: 4*KP-wave workgroups own 16*mb x 64*nb tiles; the 4
  // column waves of each of the KP K-parts share activations through LDS.
  //
  // With group-major weight chunks, every K position that is streamed at the
  // same time (one per K-part and k-split) is a contiguous front sweeping
  // through the blob. Measured on MI355X, the fewer such fronts the better,
  // provided that (a) at least ~3/4 of the CUs get a workgroup, (b) enough
  // weight loads are in flight (each wave keeps two groups of nb chunks in
  // flight; about 7-8 MB in total covers HBM latency at full bandwidth, half the
  // blob on smaller layers), and (c) every workgroup is resident at once, by LDS and by the
  // register-limited occupancy of its kernel. Among plans meeting these, the
  // search prefers nb = 2 when M > 4 (W4A16 on blobs of 64 MB: any M) and the
  // blob is at least 32 MB (half the activation traffic per weight; on smaller
  // blobs one-block tiles give twice the workgroups at fewer k-splits, which
  // measured faster) and nb = 1
  // otherwise, then the lowest fronts + k-splits (a k-split also costs
  // partial-sum traffic and a second reduction), then fewer k-splits. Over
  // 1k x 1k to 8k x 28k layers of every format at M = 1..128 this lands
  // within 13% of the best measured plan (geometric mean).
  Plan pl;
  const int G = (int)(K / kGroup);
  pl.kernel = 1;
  pl.mb = M <= 16 ? 1 : 2;
  pl.mt = (int)std::max<int64_t>(1, (M + 16 * pl.mb - 1) / (16 * pl.mb));
  const int force_nb = g_force_nb.load();
  const int force_wpt = g_force_wpt.load();
  const int force_splits = g_force_splits.load();
  const double chunk = fmt == QGEMM_FMT_W2W4 ? 560.0 : fmt == QGEMM_FMT_W4A16_SP24 ? 768.0
                       : fmt == QGEMM_FMT_BITPLANE ? 256.0 * bits : 1024.0;   // streamed bytes per 16 x 128 chunk
  const double blob = (double)G * (double)(N / 16) * chunk;
  const double big_blob = 32.0 * 1048576.0;
  // W4A16: 7 MB (the 70B up projection's 8-wave two-block tiles keep 7.3 MB in
  // flight; measured on MI355X they beat 16-wave tiles by 5-8 % at M <= 32, and
  // 8192 x 10240 by 17-24 %); mixed 2/4-bit also 7 MB with one row tile (its
  // 16-wave two-block tiles without k-splits keep 7.7 MB in flight on the 70B
  // up projection and measured 18-25 % faster at M = 1-32 than the three-split
  // plans an 8 MB target chose; with several row tiles 8 MB stayed 2-4 %
  // faster); W4A8 16-row tiles on blobs of 64 MB also 7 MB (8-wave two-block
  // tiles on the 70B up projection: 20.8 against 21.9-22.6 us at M = 1-16); the
  // other formats keep the 8 MB of their sweep
  const bool mixed = fmt == QGEMM_FMT_W2W4;
  const bool big64 = blob >= 64.0 * 1048576.0;
  const bool target7 = fmt == QGEMM_FMT_W4A16 || (mixed && pl.mt == 1) ||
                       (fmt == QGEMM_FMT_W4A8 && pl.mb == 1 && big64);
  const double inflight_target = std::min((target7 ? 7.0 : 8.0) * 1048576.0, blob / 2);
  // the bit-plane kernel is bound by its plane unpacking: one-block tiles (twice
  // the waves) measured faster on every layer and batch
  // (W4A16 also at M <= 4 once the blob reaches 64 MB: 21.7 vs 22.5 us on the 70B
  // up projection at M = 1-4)
  // (mixed 2/4-bit on blobs of 64 MB: 24.1 against 34.4 us for one-block tiles
  // on the 70B up projection at M = 1; W4A8 20.8 against 22.6 us)
  const bool w4a16_big = (fmt == QGEMM_FMT_W4A16 || mixed || fmt == QGEMM_FMT_W4A8) && big64;
  const int pref_nb = (fmt != QGEMM_FMT_BITPLANE && (M > 4 || w4a16_big) && blob >= big_blob) ? 2 : 1;
  struct Score {
    int violations, kp_pen, nb_pen, cost, splits;
    int64_t neg_waves;
    bool operator<(const Score& o) const {
      if (violations != o.violations) return violations < o.violations;
      if (kp_pen != o.kp_pen) return kp_pen < o.kp_pen;
      if (nb_pen != o.nb_pen) return nb_pen < o.nb_pen;
      if (cost != o.cost) return cost < o.cost;
      if (splits != o.splits) return splits < o.splits;
      return neg_waves < o.neg_waves;
    }
  };
  // General-grid kernel: 1 stages the grid entries in LDS, 3 (only on request)
  // loads them per lane. Measured on MI355X over 1k x 4k to 57k x 8k layers at
  // M = 1..128, staging is faster in all but a few cases at M >= 32 with group
  // length 64 and zero points (8-byte entries per column and chunk), and 10%
  // faster in total; a plan whose staged entries alone cut a launch of more
  // workgroups than CUs down to one workgroup per CU counts a violation.
  const bool w4g = fmt == QGEMM_FMT_W4G;
  const int var = w4g && force_kernel == 3 ? 3 : 1;
  bool have = false;
  Score best{};
  int best_nb = 1, best_kp = 1, best_s = 1;
  {
    for (int nb = 1; nb <= 2; ++nb) {
      if (force_nb && nb != std::min(force_nb, 2)) continue;
      if (N % (64 * nb) != 0) continue;
      const int64_t tiles = (int64_t)pl.mt * (N / (64 * nb));
      for (int kp = 1; kp <= 4; kp *= 2) {
        if (force_wpt && kp != std::max(1, force_wpt / 4)) continue;
        if (kp > G) continue;
        const KernelOccupancy occ = skinny_occupancy(fmt, pl.mb, nb, kp, bits, var, act_bf16);
        if (occ.spills && !force_wpt) continue;
        const int smax = std::min(G, 64);
        for (int s0 = 1; s0 <= smax; ++s0) {
          if (force_splits && s0 != std::min(force_splits, G)) continue;
          const int gps = (G + s0 - 1) / s0;
          const int s = (G + gps - 1) / gps;
          if (s != s0) continue;                       // the same plan as a smaller s0
          if (kp > gps) continue;                      // every K-part gets a group
          Plan c = pl;
          c.kernel = var;
          c.nb = nb;
          c.wpt = 4 * kp;
          c.gps = gps;
          const size_t lds = plan_lds(fmt, c, G, bits, gs, zeros);
          if (lds > kSkinnyLdsBudget) continue;
          const int64_t wgs = tiles * s;
          const int64_t waves = wgs * 4 * kp;
          // resident workgroups per CU: LDS, and registers (a workgroup puts kp
          // waves on each of the 4 SIMDs)
          const int64_t lds_cap = std::max<int64_t>(1, kLdsPerWorkgroup / std::max<size_t>(lds, 1));
          const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(lds_cap, occ.waves_per_simd / kp));
          Score sc;
          // too few loads in flight costs more than workgroups in a second round
          bool staged_pen = false;
          if (w4g && var == 1 && wgs > cus && kLdsPerWorkgroup / (lds + 16) < 2) {
            Plan c3 = c;
            c3.kernel = 3;
            staged_pen = kLdsPerWorkgroup / (lds_bytes_w4g(c3, G, gs, zeros) + 16) >= 2;
          }
          sc.violations = (wgs * 4 < 3 * cus) + 2 * (waves * nb * 2.0 * chunk < inflight_target) +
                          (wgs > cap * cus) + staged_pen;
          sc.cost = s * kp + s;   // fronts + k-splits
          sc.splits = s;
          sc.nb_pen = nb == pref_nb ? 0 : 1;
          // general grid at 32-row tiles: one K-part per workgroup measured 10-30 %
          // slower than two or four on every layer of a forced-plan sweep on MI355X
          // (4096 x 11008 to 57344 x 8192, M = 32..128)
          sc.kp_pen = (w4g && pl.mb == 2 && kp == 1) ? 1 : 0;
          sc.neg_waves = -waves;
          if (!have || sc < best) {
            have = true;
            best = sc;
            best_nb = nb;
            best_kp = kp;
            best_s = s;
          }
        }
      }
    }
  }
  // Small batches (16-row tiles) of W4A16 and W4A8 on layers with between half
  // as many and as many 64-column tiles as CUs: one workgroup of four K-parts
  // per tile and no k-split, when the extra bytes each busy CU streams over a
  // launch on all CUs stay under 96 KB. Measured on MI355X: 4096 x 11008 at
  // M = 1-16 in 7.9-8.6 us against 10.6-11.2 us with three k-splits (W4A8 at
  // M = 16: 7.9 against 11.2 us); the cross-workgroup reduction costs more
  // than the unused CUs there. Layers whose CUs would each stream much more
  // (28672 x 8192) keep their k-splits. W4A16 and the general 4-bit grid take
  // the same rule at 32-row tiles (one row tile): 4096 x 11008 at M = 32 in
  // 10.7 against 14.4 us with three k-splits (W4A16, one process), and the
  // general grid's forced-plan sweep on the same layers ranked the unsplit
  // four-K-part shape first there. The 2:4 format takes it at 16-row tiles
  // (4096 x 11008 at M = 16: 7.7 against 9.4 us with four k-splits).
  if (have && !force_nb && !force_wpt && !force_splits && pl.mt == 1 &&
      ((fmt == QGEMM_FMT_W4A16 && pl.mb <= 2) ||
       ((fmt == QGEMM_FMT_W4A8 || fmt == QGEMM_FMT_W4A16_SP24) && pl.mb == 1) || w4g) && G >= 4) {
    const int64_t T = N / 64;
    const double extra = blob * (1.0 / (double)T - 1.0 / (double)cus);
    if (2 * T >= cus && T <= cus && extra < 96.0 * 1024.0 && !skinny_occupancy(fmt, pl.mb, 1, 4, bits, var, act_bf16).spills) {
      Plan c = pl;
      c.kernel = var;
      c.nb = 1;
      c.wpt = 16;
      c.gps = G;
      if (plan_lds(fmt, c, G, bits, gs, zeros) <= kSkinnyLdsBudget) {
        best_nb = 1;
        best_kp = 4;
        best_s = 1;
      }
    }
  }
  // Two 32-row tiles on such layers (M = 33..64): the same unsplit shape with
  // two-block tiles, 8 waves for W4A16 (its 32 x 32 wave tiles) and 16 for
  // the other formats. Measured on MI355X in one process against the
  // scored plans: 4096 x 11008 at M = 33-64 15.8-16.1 against 17.2-17.5 us
  // (W4A16), 14.2-14.6 against 16.3-17.1 (W4A8), 13.6-14.0 against 17.4-17.8
  // (2:4); 4096 x 14336 W4A8 14.6-15.0 against 21.7-22.4 us; the general grid
  // (group 128, zero points, fp16) 18.1-18.4 against 21.3-21.5 us. Its bf16
  // 16-wave two-block instance spills and keeps the scored plan.
  if (have && !force_nb && !force_wpt && !force_splits && pl.mb == 2 && pl.mt == 2 &&
      two_row_tiles_unsplit(fmt, M, K, N, chunk, cus)) {
    const int kp2 = fmt == QGEMM_FMT_W4A16 ? 2 : 4;
    Plan c = pl;
    c.kernel = var;
    c.nb = 2;
    c.wpt = 4 * kp2;
    c.gps = G;
    if (plan_lds(fmt, c, G, bits, gs, zeros) <= kSkinnyLdsBudget && !skinny_occupancy(fmt, 2, 2, kp2, bits, var, act_bf16).spills) {
      best_nb = 2;
      best_kp = kp2;
      best_s = 1;
    }
  }
  if (!have) {   // a forced shape outside the search space: fall back to its literal values
    best_nb = (force_nb && N % (64 * std::min(force_nb, 2)) == 0) ? std::min(force_nb, 2) : 1;
    best_s = std::max(1, std::min(force_splits ? force_splits : 1, G));
    best_kp = force_wpt ? std::max(1, std::min(4, force_wpt / 4)) : 1;
    if (best_kp == 3) best_kp = 2;
  }
  const int64_t tiles = (int64_t)pl.mt * (N / (64 * best_nb));
  int splits = best_s;
  const int gps = (G + splits - 1) / splits;
  splits = (G + gps - 1) / gps;
  int kp = best_kp;
  while (kp > 1 && kp > gps) kp /= 2;       // every K-part gets at least one group
  pl.kernel = var;
  pl.nb = best_nb;
  pl.nt = (int)(N / (64 * best_nb));
  pl.wpt = 4 * kp;
  pl.splits = splits;
  pl.gps = gps;
  pl.workgroups = launch_workgroups(pl.nt, pl.mt, splits);
  pl.waves = pl.workgroups * pl.wpt;
  pl.lds_bytes = plan_lds(fmt, pl, G, bits, gs, zeros);
  // no shape of the search fits (or a forced shape does not): refuse the call
  // rather than launch more LDS than a workgroup can hold
  if ((!have && !(force_nb || force_wpt || force_splits)) || pl.lds_bytes > kSkinnyLdsBudget) pl.kernel = 0;
  if (pl.splits > 1) {
    // partial tiles are kept whole (rows padded to the tile) in fragment order
    pl.counter_bytes = counter_region_bytes(tiles);
    pl.ws_bytes = pl.counter_bytes + align256((size_t)pl.splits * pl.mt * 16 * pl.mb * N * 4);
  }
  return pl;
}

}  // namespace qg

extern "C" {

const char* qgemm_status_str(int status) {
  switch (status) {
    case QGEMM_OK: return "QGEMM_OK";
    case QGEMM_ERR_NULL: return "QGEMM_ERR_NULL";
    case QGEMM_ERR_SHAPE: return "QGEMM_ERR_SHAPE";
    case QGEMM_ERR_ALIGN: return "QGEMM_ERR_ALIGN";
    case QGEMM_ERR_WORKSPACE: return "QGEMM_ERR_WORKSPACE";
    case QGEMM_ERR_FORMAT: return "QGEMM_ERR_FORMAT";
    case QGEMM_ERR_RANGE: return "QGEMM_ERR_RANGE";
    case QGEMM_ERR_ALIAS: return "QGEMM_ERR_ALIAS";
    case QGEMM_ERR_HIP: return "QGEMM_ERR_HIP";
    case QGEMM_ERR_DEVICE: return "QGEMM_ERR_DEVICE";
    case QGEMM_ERR_SIZE: return "QGEMM_ERR_SIZE";
    default: return "QGEMM_ERR_UNKNOWN";
  }
}

const char* qgemm_last_error(void) { return g_last_error.c_str(); }

int qgemm_version(void) { return 100; }

int qgemm_packed_bytes(int fmt, int64_t K, int64_t N, const uint32_t* bitmap_host, size_t* bytes) {
  if (!valid_fmt(fmt)) return QGEMM_ERR_FORMAT;
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(fmt, K, N);
  if (st) return st;
  int64_t n4 = 0;
  if (fmt == QGEMM_FMT_W2W4) {
    if (!bitmap_host) return QGEMM_ERR_NULL;
    bool stray = false;
    n4 = count_bits(bitmap_host, K / qg::kGroup, N, &stray);
    if (stray) return QGEMM_ERR_RANGE;
  }
  *bytes = qg::blob_layout(fmt, K, N, n4).total;
  return QGEMM_OK;
}

int qgemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N, size_t* bytes) {
  if (!valid_fmt(fmt)) return QGEMM_ERR_FORMAT;
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(fmt, K, N);
  if (st) return st;
  if (M < 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  if (M == 0) {
    *bytes = 0;
    return QGEMM_OK;
  }
  const qg::Plan pl = qg::make_plan(fmt, M, K, N);
  if (pl.kernel == 0) return no_plan();
  *bytes = pl.ws_bytes;
  return QGEMM_OK;
}

int qgemm_plan(int fmt, int64_t M, int64_t K, int64_t N, int64_t* out10) {
  if (!valid_fmt(fmt) && fmt != QGEMM_FMT_W4G) return QGEMM_ERR_FORMAT;
  if (!out10) return QGEMM_ERR_NULL;
  int st = check_kn(fmt, K, N);
  if (st) return st;
  if (M <= 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  const qg::Plan pl = qg::make_plan(fmt, M, K, N);
  if (pl.kernel == 0) return no_plan();
  const int64_t v[10] = {pl.kernel, pl.mb, pl.nb, pl.wpt, pl.splits, pl.gps,
                         pl.mt, pl.nt, pl.workgroups, pl.waves};
  std::memcpy(out10, v, sizeof(v));
  return QGEMM_OK;
}

int qgemm_bitplane_plan(int64_t M, int64_t K, int64_t N, int32_t bits, int64_t* out10) {
  if (!out10) return QGEMM_ERR_NULL;
  if (bits < 1 || bits > 8) return QGEMM_ERR_RANGE;
  int st = check_kn(QGEMM_FMT_BITPLANE, K, N);
  if (st) return st;
  if (M <= 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  const qg::Plan pl = qg::make_plan(QGEMM_FMT_BITPLANE, M, K, N, bits);
  if (pl.kernel == 0) return no_plan();
  const int64_t v[10] = {pl.kernel, pl.mb, pl.nb, pl.wpt, pl.splits, pl.gps,
                         pl.mt, pl.nt, pl.workgroups, pl.waves};
  std::memcpy(out10, v, sizeof(v));
  return QGEMM_OK;
}

int qgemm_plan_info(int fmt, int64_t M, int64_t K, int64_t N, int32_t bits, int32_t group_size,
                    int32_t has_zeros, int32_t act_dtype, int64_t* out12) {
  if (!valid_fmt(fmt) && fmt != QGEMM_FMT_W4G && fmt != QGEMM_FMT_BITPLANE) return QGEMM_ERR_FORMAT;
  if (!out12) return QGEMM_ERR_NULL;
  int st = check_kn(fmt, K, N);
  if (st) return st;
  if (M <= 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  if (fmt == QGEMM_FMT_BITPLANE && (bits < 1 || bits > 8)) return QGEMM_ERR_RANGE;
  if (fmt == QGEMM_FMT_W4G && (!valid_group_size(K, group_size) || (has_zeros != 0 && has_zeros != 1) ||
                               (act_dtype != QGEMM_DT_F16 && act_dtype != QGEMM_DT_BF16)))
    return QGEMM_ERR_RANGE;
  const qg::Plan pl = qg::make_plan(fmt, M, K, N, fmt == QGEMM_FMT_BITPLANE ? bits : 4,
                                    fmt == QGEMM_FMT_W4G ? group_size : qg::kGroup, has_zeros != 0,
                                    fmt == QGEMM_FMT_W4G && act_dtype == QGEMM_DT_BF16);
  if (pl.kernel == 0) return no_plan();
  const int64_t v[12] = {pl.kernel, pl.mb, pl.nb, pl.wpt, pl.splits, pl.gps, pl.mt, pl.nt,
                         pl.workgroups, pl.waves, (int64_t)pl.ws_bytes, (int64_t)pl.lds_bytes};
  std::memcpy(out12, v, sizeof(v));
  return QGEMM_OK;
}

int qgemm_set_plan_override(int kernel, int nb_per_tile, int waves_per_tile, int k_splits) {
  if (kernel < 0 || kernel > 3) return QGEMM_ERR_RANGE;
  if (!(nb_per_tile == 0 || nb_per_tile == 1 || nb_per_tile == 2 || nb_per_tile == 4))
    return QGEMM_ERR_RANGE;
  if (!(waves_per_tile == 0 || waves_per_tile == 4 || waves_per_tile == 8 || waves_per_tile == 16))
    return QGEMM_ERR_RANGE;
  if (k_splits < 0 || k_splits > 4096) return QGEMM_ERR_RANGE;
  g_force_kernel.store(kernel);
  g_force_nb.store(nb_per_tile);
  g_force_wpt.store(waves_per_tile);
  g_force_splits.store(k_splits);
  return QGEMM_OK;
}

int qgemm_repack(int fmt, int64_t K, int64_t N, const void* codes, const void* group_scales,
                 const void* chan_scales, const uint32_t* bitmap_host, void* packed,
                 size_t packed_bytes, void* stream) {
  if (!valid_fmt(fmt)) return QGEMM_ERR_FORMAT;
  if (!codes || !group_scales || !packed) return QGEMM_ERR_NULL;
  if (fmt == QGEMM_FMT_W4A8 && !chan_scales) return QGEMM_ERR_NULL;
  if (fmt == QGEMM_FMT_W2W4 && !bitmap_host) return QGEMM_ERR_NULL;
  int st = check_kn(fmt, K, N);
  if (st) return st;
  const int64_t G = K / qg::kGroup;
  int64_t n4 = 0;
  if (fmt == QGEMM_FMT_W2W4) {
    bool stray = false;
    n4 = count_bits(bitmap_host, G, N, &stray);
    if (stray) return QGEMM_ERR_RANGE;
  }
  const qg::BlobLayout L = qg::blob_layout(fmt, K, N, n4);
  if (packed_bytes != L.total) return QGEMM_ERR_SIZE;
  if (!aligned(packed, 16) || !aligned(codes, fmt == QGEMM_FMT_W2W4 ? 1 : 4) ||
      !aligned(group_scales, fmt == QGEMM_FMT_W4A8 ? 1 : 2) || (chan_scales && !aligned(chan_scales, 2)))
    return QGEMM_ERR_ALIGN;
  const size_t code_bytes = fmt == QGEMM_FMT_W2W4 ? (size_t)(K * N) : (size_t)(K / 2 * N);
  const size_t gs_bytes = (size_t)(G * N) * (fmt == QGEMM_FMT_W4A8 ? 1 : 2);
  if (overlap(packed, L.total, codes, code_bytes) || overlap(packed, L.total, group_scales, gs_bytes) ||
      (fmt == QGEMM_FMT_W4A8 && overlap(packed, L.total, chan_scales, (size_t)N * 2)))
    return QGEMM_ERR_ALIAS;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // padding and alignment gaps are defined as zero bytes
  hipError_t e = qg::launch_zero_fill(packed, L.total, s);
  if (e != hipSuccess) return hip_fail(e, "zero fill");
  if (fmt == QGEMM_FMT_W4A16) {
    e = qg::launch_repack_w4a16(L, codes, group_scales, packed, s);
  } else if (fmt == QGEMM_FMT_W4A16_SP24) {
    e = qg::launch_repack_sp24(L, codes, group_scales, packed, s);
    if (e != hipSuccess) return hip_fail(e, "repack launch");
    // the structure check: the kernel counted quads with more than two nonzero codes
    uint32_t bad = 0;
    e = hipMemcpyAsync(&bad, static_cast<char*>(packed) + L.high, 4, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (bad != 0) {
      g_last_error = std::to_string(bad) + " runs of 4 consecutive k hold more than two nonzero codes";
      return QGEMM_ERR_RANGE;
    }
  } else if (fmt == QGEMM_FMT_W4A8) {
    e = qg::launch_repack_w4a8(L, codes, group_scales, chan_scales, packed, s);
  } else {
    // per-chunk descriptors: (high-plane slot offset, 16-bit column mask)
    std::vector<uint32_t> desc((size_t)L.NB * L.G * 2);
    const int64_t W = (N + 31) / 32;
    uint32_t off = 0;
    for (int64_t g = 0; g < G; ++g)          // chunk order g*NB + b, as the base plane
      for (int64_t b = 0; b < L.NB; ++b) {
        const uint32_t word = bitmap_host[g * W + (16 * b) / 32];
        const uint32_t m16 = (word >> ((16 * b) % 32)) & 0xFFFFu;
        desc[(size_t)(g * L.NB + b) * 2] = off;
        desc[(size_t)(g * L.NB + b) * 2 + 1] = m16;
        off += (uint32_t)__builtin_popcount(m16);
      }
    e = hipMemcpyAsync(static_cast<char*>(packed) + L.aux, desc.data(), desc.size() * 4,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = qg::launch_repack_w2w4(L, codes, group_scales, packed, s);
    if (e != hipSuccess) return hip_fail(e, "repack launch");
    e = hipStreamSynchronize(s);   // keeps the host descriptor table alive until consumed
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  }
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  return QGEMM_OK;
}

}  // extern "C"

namespace {

struct GemmCall {
  int fmt;
  const void* A;
  int64_t lda;
  const void* a_scale;
  const void* packed;
  void* C;
  int64_t ldc;
  int32_t* acc_out;
  int64_t M, K, N;
  void* ws;
  size_t ws_bytes;
  void* stream;
  int gs = qg::kGroup;    // general grid only
  bool zeros = false;
  bool bf16 = false;
  int bits = 4;           // bit-plane format only
  bool dry = false;       // validate only: no workspace checks, no launch
};

int run_gemm(const GemmCall& g) {
  if (!valid_fmt(g.fmt) && g.fmt != QGEMM_FMT_W4G && g.fmt != QGEMM_FMT_BITPLANE) return QGEMM_ERR_FORMAT;
  const bool int8_act = g.fmt == QGEMM_FMT_W4A8 || g.fmt == QGEMM_FMT_BITPLANE;
  int st = check_kn(g.fmt, g.K, g.N);
  if (st) return st;
  if (g.M < 0 || g.M > kMaxM) return QGEMM_ERR_SHAPE;
  if (g.M == 0) return QGEMM_OK;
  if (!g.A || !g.packed || !g.C) return QGEMM_ERR_NULL;
  if (int8_act && !g.a_scale) return QGEMM_ERR_NULL;
  const int64_t aelt = int8_act ? 1 : 2;
  if (!aligned(g.A, 16) || !aligned(g.packed, 16) || !aligned(g.C, 16)) return QGEMM_ERR_ALIGN;
  if (g.lda < g.K || (g.lda * aelt) % 16 != 0) return QGEMM_ERR_ALIGN;
  if (g.ldc < g.N || g.ldc % 8 != 0) return QGEMM_ERR_ALIGN;
  if (g.a_scale && !aligned(g.a_scale, 2)) return QGEMM_ERR_ALIGN;
  if (g.acc_out && !aligned(g.acc_out, 4)) return QGEMM_ERR_ALIGN;
  const qg::Plan pl = qg::make_plan(g.fmt, g.M, g.K, g.N, g.bits, g.gs, g.zeros, g.bf16);
  if (pl.kernel == 0) return no_plan();
  if (pl.ws_bytes > 0 && !g.dry) {
    if (!g.ws) return QGEMM_ERR_NULL;
    if (g.ws_bytes < pl.ws_bytes) return QGEMM_ERR_WORKSPACE;
    if (!aligned(g.ws, 16)) return QGEMM_ERR_ALIGN;
  }
  // the fixed-size part of the blob (everything before a mixed blob's high plane)
  const qg::BlobLayout L = g.fmt == QGEMM_FMT_W4G       ? qg::blob_layout_w4g(g.K, g.N, g.gs, g.zeros)
                           : g.fmt == QGEMM_FMT_BITPLANE ? qg::blob_layout_bitplane(g.K, g.N, g.bits)
                                                         : qg::blob_layout(g.fmt, g.K, g.N, 0);
  const size_t blob_fixed = g.fmt == QGEMM_FMT_W2W4 ? L.high : L.total;
  const size_t c_bytes = (size_t)((g.M - 1) * g.ldc + g.N) * 2;
  const size_t a_bytes = (size_t)((g.M - 1) * g.lda + g.K) * aelt;
  const size_t acc_bytes = g.acc_out ? (size_t)(g.M * g.N) * 4 : 0;
  if (overlap(g.C, c_bytes, g.A, a_bytes) || overlap(g.C, c_bytes, g.packed, blob_fixed) ||
      (pl.ws_bytes && overlap(g.C, c_bytes, g.ws, pl.ws_bytes)) ||
      (g.a_scale && overlap(g.C, c_bytes, g.a_scale, (size_t)g.M * 2)) ||
      (g.acc_out && (overlap(g.acc_out, acc_bytes, g.C, c_bytes) ||
                     overlap(g.acc_out, acc_bytes, g.A, a_bytes) ||
                     overlap(g.acc_out, acc_bytes, g.packed, blob_fixed) ||
                     (pl.ws_bytes && overlap(g.acc_out, acc_bytes, g.ws, pl.ws_bytes)))))
    return QGEMM_ERR_ALIAS;
  st = check_device();
  if (st) return st;
  if (g.dry) return QGEMM_OK;

  qg::GemmArgs a{};
  const char* blob = static_cast<const char*>(g.packed);
  a.A = g.A;
  a.codes = blob + L.codes;
  a.scales = blob + L.scales;
  a.aux = blob + L.aux;
  a.high = blob + L.high;
  a.a_scale = g.a_scale;
  a.C = g.C;
  a.acc_out = g.acc_out;
  a.lda = g.lda;
  a.ldc = g.ldc;
  a.M = (int)g.M;
  a.K = (int)g.K;
  a.N = (int)g.N;
  a.G = (int)L.G;
  a.G8 = (int)L.G8;
  a.splits = pl.splits;
  a.gps = pl.gps;
  a.mt = pl.mt;
  a.nt = pl.nt;
  a.gs = g.gs;
  a.bits = g.bits;
  if (pl.ws_bytes) {
    a.counters = static_cast<uint32_t*>(g.ws);
    a.partial = static_cast<char*>(g.ws) + pl.counter_bytes;
  }
  hipStream_t s = static_cast<hipStream_t>(g.stream);
  hipError_t e;
  if (pl.ws_bytes && pl.counter_bytes > qg::kCounterBytes) {
    // a counter region beyond the fixed one may hold other plans' partial sums
    e = qg::launch_zero_fill(g.ws, pl.counter_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "counter clear");
  }
  if (g.fmt == QGEMM_FMT_W4A16) e = pl.kernel == 2 ? qg::launch_w4a16_wide(pl, a, s) : qg::launch_w4a16(pl, a, s);
  else if (g.fmt == QGEMM_FMT_W4A8) e = qg::launch_w4a8(pl, a, s);
  else if (g.fmt == QGEMM_FMT_W4G)
    e = pl.kernel == 2 ? qg::launch_w4g_wide(pl, a, g.zeros, s) : qg::launch_w4g(pl, a, g.bf16, g.zeros, s);
  else if (g.fmt == QGEMM_FMT_W4A16_SP24) e = qg::launch_sp24(pl, a, s);
  else if (g.fmt == QGEMM_FMT_BITPLANE)
    e = g.bits <= 4 ? qg::launch_bitplane_lo(pl, a, g.bits, s) : qg::launch_bitplane_hi(pl, a, g.bits, s);
  else e = qg::launch_w2w4(pl, a, s);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return QGEMM_OK;
}

}  // namespace

namespace qg {

int fail_hip(hipError_t e, const char* what) { return hip_fail(e, what); }

void set_last_error(const std::string& text) { g_last_error = text; }

int validate_w4a16(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M, int64_t K,
                   int64_t N) {
  GemmCall g{QGEMM_FMT_W4A16, A, lda, nullptr, packed, C, ldc, nullptr, M, K, N, nullptr, 0, nullptr};
  g.dry = true;
  return run_gemm(g);
}

}  // namespace qg

extern "C" {

int qgemm_w4a16(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
                int64_t K, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gemm({QGEMM_FMT_W4A16, A, lda, nullptr, packed, C, ldc, nullptr, M, K, N, workspace,
                   workspace_bytes, stream});
}

int qgemm_w4a8(const void* A, int64_t lda, const void* a_scale, const void* packed, void* C,
               int64_t ldc, int32_t* acc_out, int64_t M, int64_t K, int64_t N, void* workspace,
               size_t workspace_bytes, void* stream) {
  return run_gemm({QGEMM_FMT_W4A8, A, lda, a_scale, packed, C, ldc, acc_out, M, K, N, workspace,
                   workspace_bytes, stream});
}

int qgemm_w4a16_sp24(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
                     int64_t K, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gemm({QGEMM_FMT_W4A16_SP24, A, lda, nullptr, packed, C, ldc, nullptr, M, K, N, workspace,
                   workspace_bytes, stream});
}

int qgemm_w2w4_mixed(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc,
                     int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return run_gemm({QGEMM_FMT_W2W4, A, lda, nullptr, packed, C, ldc, nullptr, M, K, N, workspace,
                   workspace_bytes, stream});
}

int qgemm_w4g_packed_bytes(int64_t K, int64_t N, int32_t group_size, int32_t has_zeros,
                           size_t* bytes) {
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_W4G, K, N);
  if (st) return st;
  if (!valid_group_size(K, group_size) || (has_zeros != 0 && has_zeros != 1)) return QGEMM_ERR_RANGE;
  *bytes = qg::blob_layout_w4g(K, N, group_size, has_zeros != 0).total;
  return QGEMM_OK;
}

int qgemm_w4g_workspace_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes) {
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_W4G, K, N);
  if (st) return st;
  if (M < 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  // the plan depends on the grid and the activation type; size for every
  // grid and type (a grid with no plan that fits is refused by the GEMM call)
  size_t ws = 0;
  for (int gs : {64, 128})
    for (bool z : {false, true})
      for (bool bf : {false, true})
        ws = std::max(ws, M == 0 ? 0 : qg::make_plan(QGEMM_FMT_W4G, M, K, N, 4, gs, z, bf).ws_bytes);
  *bytes = ws;
  return QGEMM_OK;
}

int qgemm_w4g_plan(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t has_zeros, int32_t act_dtype,
                   int64_t* out10) {
  if (!out10) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_W4G, K, N);
  if (st) return st;
  if (!valid_group_size(K, group_size) || (has_zeros != 0 && has_zeros != 1) ||
      (act_dtype != QGEMM_DT_F16 && act_dtype != QGEMM_DT_BF16))
    return QGEMM_ERR_RANGE;
  if (M <= 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  const qg::Plan pl =
      qg::make_plan(QGEMM_FMT_W4G, M, K, N, 4, group_size, has_zeros != 0, act_dtype == QGEMM_DT_BF16);
  if (pl.kernel == 0) return no_plan();
  const int64_t v[10] = {pl.kernel, pl.mb, pl.nb, pl.wpt, pl.splits, pl.gps,
                         pl.mt, pl.nt, pl.workgroups, pl.waves};
  std::memcpy(out10, v, sizeof(v));
  return QGEMM_OK;
}

int qgemm_w4g_repack(int64_t K, int64_t N, int32_t group_size, const void* codes, const void* scales,
                     const void* zeros, void* packed, size_t packed_bytes, void* stream) {
  if (!codes || !scales || !packed) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_W4G, K, N);
  if (st) return st;
  if (!valid_group_size(K, group_size)) return QGEMM_ERR_RANGE;
  const qg::BlobLayout L = qg::blob_layout_w4g(K, N, group_size, zeros != nullptr);
  if (packed_bytes != L.total) return QGEMM_ERR_SIZE;
  if (!aligned(packed, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return QGEMM_ERR_ALIGN;
  const size_t ng = (size_t)(K / group_size) * (size_t)N;
  if (overlap(packed, L.total, codes, (size_t)(K / 2 * N)) || overlap(packed, L.total, scales, ng * 2) ||
      overlap(packed, L.total, zeros, zeros ? ng : 0))
    return QGEMM_ERR_ALIAS;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = qg::launch_zero_fill(packed, L.total, s);
  if (e != hipSuccess) return hip_fail(e, "zero fill");
  e = qg::launch_repack_w4g(L, group_size, codes, scales, zeros, packed, s);
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  return QGEMM_OK;
}

int qgemm_w4g(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
              int64_t K, int64_t N, int32_t group_size, int32_t has_zeros, int32_t act_dtype,
              void* workspace, size_t workspace_bytes, void* stream) {
  if (check_kn(QGEMM_FMT_W4G, K, N) == QGEMM_OK &&
      (!valid_group_size(K, group_size) || (has_zeros != 0 && has_zeros != 1) ||
       (act_dtype != QGEMM_DT_F16 && act_dtype != QGEMM_DT_BF16)))
    return QGEMM_ERR_RANGE;
  GemmCall g{QGEMM_FMT_W4G, A, lda, nullptr, packed, C, ldc, nullptr, M, K, N, workspace,
             workspace_bytes, stream};
  g.gs = group_size;
  g.zeros = has_zeros != 0;
  g.bf16 = act_dtype == QGEMM_DT_BF16;
  return run_gemm(g);
}

int qgemm_bitplane_packed_bytes(int64_t K, int64_t N, int32_t bits, size_t* bytes) {
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_BITPLANE, K, N);
  if (st) return st;
  if (bits < 1 || bits > 8) return QGEMM_ERR_RANGE;
  *bytes = qg::blob_layout_bitplane(K, N, bits).total;
  return QGEMM_OK;
}

int qgemm_bitplane_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t bits, size_t* bytes) {
  if (!bytes) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_BITPLANE, K, N);
  if (st) return st;
  if (bits < 1 || bits > 8) return QGEMM_ERR_RANGE;
  if (M < 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  if (M == 0) {
    *bytes = 0;
    return QGEMM_OK;
  }
  const qg::Plan pl = qg::make_plan(QGEMM_FMT_BITPLANE, M, K, N, bits);
  if (pl.kernel == 0) return no_plan();
  *bytes = pl.ws_bytes;
  return QGEMM_OK;
}

int qgemm_bitplane_repack(int64_t K, int64_t N, int32_t bits, const void* codes, const void* chan_scales,
                          void* packed, size_t packed_bytes, void* stream) {
  if (!codes || !chan_scales || !packed) return QGEMM_ERR_NULL;
  int st = check_kn(QGEMM_FMT_BITPLANE, K, N);
  if (st) return st;
  if (bits < 1 || bits > 8) return QGEMM_ERR_RANGE;
  const qg::BlobLayout L = qg::blob_layout_bitplane(K, N, bits);
  if (packed_bytes != L.total) return QGEMM_ERR_SIZE;
  if (!aligned(packed, 16) || !aligned(chan_scales, 2)) return QGEMM_ERR_ALIGN;
  if (overlap(packed, L.total, codes, (size_t)(K * N)) || overlap(packed, L.total, chan_scales, (size_t)N * 2))
    return QGEMM_ERR_ALIAS;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = qg::launch_zero_fill(packed, L.total, s);
  if (e != hipSuccess) return hip_fail(e, "zero fill");
  e = qg::launch_repack_bitplane(L, bits, codes, chan_scales, packed, s);
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  return QGEMM_OK;
}

int qgemm_bitplane_a8(const void* A, int64_t lda, const void* a_scale, const void* packed, void* C, int64_t ldc,
                      int32_t* acc_out, int64_t M, int64_t K, int64_t N, int32_t bits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (check_kn(QGEMM_FMT_BITPLANE, K, N) == QGEMM_OK && (bits < 1 || bits > 8)) return QGEMM_ERR_RANGE;
  GemmCall g{QGEMM_FMT_BITPLANE, A, lda, a_scale, packed, C, ldc, acc_out, M, K, N, workspace,
             workspace_bytes, stream};
  g.bits = bits;
  return run_gemm(g);
}

int qgemm_quantize_a8(const void* A, int64_t lda, int64_t M, int64_t K, void* A_q, int64_t ldq,
                      void* a_scale, void* stream) {
  if (K <= 0 || K % 8 != 0 || K > kMaxKN) return QGEMM_ERR_SHAPE;
  if (M < 0 || M > kMaxM) return QGEMM_ERR_SHAPE;
  if (M == 0) return QGEMM_OK;
  if (!A || !A_q || !a_scale) return QGEMM_ERR_NULL;
  if (!aligned(A, 16) || !aligned(A_q, 16) || !aligned(a_scale, 2)) return QGEMM_ERR_ALIGN;
  if (lda < K || lda % 8 != 0 || ldq < K || ldq % 16 != 0) return QGEMM_ERR_ALIGN;
  const size_t a_bytes = (size_t)((M - 1) * lda + K) * 2;
  const size_t q_bytes = (size_t)((M - 1) * ldq + K);
  if (overlap(A_q, q_bytes, A, a_bytes) || overlap(a_scale, (size_t)M * 2, A, a_bytes) ||
      overlap(a_scale, (size_t)M * 2, A_q, q_bytes))
    return QGEMM_ERR_ALIAS;
  const int st = check_device();
  if (st) return st;
  const hipError_t e = qg::launch_quantize_a8(A, lda, M, K, A_q, ldq, a_scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return QGEMM_OK;
}

}  // extern "C"
