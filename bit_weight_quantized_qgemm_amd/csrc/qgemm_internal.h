// Host-side internals shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace qg {

constexpr int kGroup = 128;          // k per quantization group
constexpr int kWave = 64;            // lanes per wavefront (CDNA)
constexpr int kWavesPerBlock = 4;    // one wave per SIMD of a CU
constexpr int kDefaultCUs = 256;     // MI355X compute units (8 XCDs x 32)
// Compute units of the current device, queried once per device and cached;
// kDefaultCUs when no device is visible (host-only queries).
int device_cu_count();
constexpr int kMaxWavesPerTile = 16;
// LDS of one workgroup on gfx950, and the dynamic part the streaming kernels
// may request: their static LDS (the arrival flag, 16 bytes) comes on top,
// and a launch whose total exceeds the limit aborts the queue.
constexpr size_t kLdsPerWorkgroup = 160 * 1024;
constexpr size_t kSkinnyLdsBudget = kLdsPerWorkgroup - 256;
constexpr int kWideCols = 256;        // columns per tile of the wide kernel (also 128: plan nb = 2)
constexpr int kWideSlots = 4;         // activation LDS slots per K-part of the wide kernel
constexpr int kWideMinM = 33;         // batches from which the wide kernel is used
// Split-K arrival counters live in a fixed region at the start of every
// workspace, so that calls with different plans sharing one workspace never see
// another plan's partial sums in place of zero counters. A plan with more tiles
// than that region holds gets a larger counter region, which its call clears
// first (the fixed region's calls may have left partial sums beyond it).
constexpr size_t kCounterBytes = 65536;
constexpr int64_t kMaxCounters = kCounterBytes / 4;
inline size_t counter_region_bytes(int64_t tiles) {
  return tiles > kMaxCounters ? (size_t)((tiles * 4 + 255) / 256 * 256) : kCounterBytes;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Blob region offsets (bytes) for one weight shape; see the layout notes in
// repack.hip. All regions start on 256-byte boundaries.
struct BlobLayout {
  int64_t K = 0, N = 0, G = 0, NB = 0, G8 = 0;
  size_t codes = 0;    // W4A16/W4A8 1 KB chunks; W2W4 512 B base chunks
  size_t scales = 0;   // fp16 (W4A16, W2W4) or int8 (W4A8) group scales
  size_t aux = 0;      // W4A8: fp16 channel scales; W2W4: per-chunk descriptors
  size_t high = 0;     // W2W4: 4-bit high plane; SP24: status word
  size_t total = 0;
};

BlobLayout blob_layout(int fmt, int64_t K, int64_t N, int64_t n4);

// Work decomposition of one GEMM call. Kernel 1: workgroups of wpt = 4*KP
// waves own tiles of 16*mb rows x 64*nb columns, KP K-parts of 4 column waves;
// kernel 2: wpt-wave workgroups own 16*mb x 64*nb tiles as K-parts of 2*nb
// column waves of 32 columns. `splits` > 1 additionally
// splits K across workgroups.
struct Plan {
  // 1 = streaming skinny kernel, 2 = wide (large-M) W4A16 kernel, 3 = streaming
  // general-grid kernel with per-lane grid entries; 0 = no launch shape fits
  // the workgroup's LDS (the call is refused with QGEMM_ERR_SHAPE)
  int kernel = 1;
  int mb = 1;            // 16-row blocks per tile (per wave for kernel 2)
  int nb = 1;            // 16-column blocks per wave
  int wpt = 1;           // waves per tile (workgroup size / 64)
  int splits = 1;        // k-splits across workgroups
  int gps = 0;           // groups per k-split
  int mt = 1;            // m-tiles
  int nt = 1;            // n-tiles
  int64_t workgroups = 0;
  int64_t waves = 0;
  size_t counter_bytes = 0;
  size_t ws_bytes = 0;   // total workspace (0 when splits == 1)
  size_t lds_bytes = 0;  // dynamic LDS the launch requests
};

// Workgroups of a launch of nt x mt tiles and `splits` k-splits: one per tile
// and k-split (the kernels' tile_of_block orders them).
inline int64_t launch_workgroups(int64_t nt, int64_t mt, int64_t splits) { return nt * mt * splits; }

// dynamic LDS of a wide-kernel launch: per K-part of 8 waves, kWideSlots slots
// of 16*mb rows x 128 k fp16
// K-parts of 2*nb waves (nb = 4: 256-column tiles, 2: 128-column tiles)
inline size_t wide_lds_bytes(const Plan& pl) {
  return (size_t)(pl.wpt / (2 * pl.nb)) * kWideSlots * pl.mb * 4 * 1024;
}

// bits: planes per weight of the bit-plane format (ignored by the others)
// gs / zeros: the general-grid format's group length and zero points (its
// staged grid entries size the LDS); act_bf16: its activation type (fp16 calls
// may take the wide kernel); ignored by the other formats
Plan make_plan(int fmt, int64_t M, int64_t K, int64_t N, int bits = 4, int gs = 128, bool zeros = true,
               bool act_bf16 = false);
struct KernelOccupancy {
  int waves_per_simd;
  bool spills;
};
// register-limited occupancy of a streaming-kernel instance (tile 16*mb x 64*nb,
// kp waves per SIMD per workgroup; act_bf16 selects the general grid's bf16 rows)
KernelOccupancy skinny_occupancy(int fmt, int mb, int nb, int kp, int bits, int kernel, bool act_bf16);

// Arguments of every GEMM kernel (passed by value).
struct GemmArgs {
  const void* A;
  const void* codes;      // chunk region
  const void* scales;     // group-scale region
  const void* aux;        // W4A8: fp16 channel scales; W2W4: descriptors
  const void* high;       // W2W4: high plane
  const void* a_scale;    // W4A8: fp16 per-row scales
  void* C;
  int32_t* acc_out;       // W4A8, nullable
  void* partial;          // split-K partials [splits][M][N] (fp32 or int32)
  uint32_t* counters;     // per (m-tile, n-tile) arrival counters
  int64_t lda, ldc;
  int M, K, N, G, G8;
  int splits, gps, mt, nt;
  int gs;                 // general-grid format: k per quantization group
  int bits;               // bit-plane format: planes per weight
};

size_t lds_bytes_w4a16(const Plan& pl, int G);
size_t lds_bytes_w4a8(const Plan& pl, int G);
size_t lds_bytes_w2w4(const Plan& pl, int G);
size_t lds_bytes_w4g(const Plan& pl, int G, int gs, bool zeros);
size_t lds_bytes_sp24(const Plan& pl, int G);
size_t lds_bytes_bitplane(const Plan& pl, int G);
hipError_t launch_w4a16(const Plan& pl, const GemmArgs& a, hipStream_t s);
hipError_t launch_w4a16_wide(const Plan& pl, const GemmArgs& a, hipStream_t s);
// general grid, fp16 activations, on the wide kernel (kernel 2)
hipError_t launch_w4g_wide(const Plan& pl, const GemmArgs& a, bool zeros, hipStream_t s);
hipError_t launch_w4a8(const Plan& pl, const GemmArgs& a, hipStream_t s);
hipError_t launch_w2w4(const Plan& pl, const GemmArgs& a, hipStream_t s);
hipError_t launch_w4g(const Plan& pl, const GemmArgs& a, bool bf16, bool zeros, hipStream_t s);
hipError_t launch_sp24(const Plan& pl, const GemmArgs& a, hipStream_t s);
hipError_t launch_bitplane_lo(const Plan& pl, const GemmArgs& a, int bits, hipStream_t s);   // bits 1..4
hipError_t launch_bitplane_hi(const Plan& pl, const GemmArgs& a, int bits, hipStream_t s);   // bits 5..8

hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t s);

// Error plumbing and argument checks shared by the C-ABI entry points: record
// a HIP failure (returns QGEMM_ERR_HIP), record an error text, and run every
// check of qgemm_w4a16 except the workspace's without launching anything.
int fail_hip(hipError_t e, const char* what);
void set_last_error(const std::string& text);
int validate_w4a16(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M, int64_t K,
                   int64_t N);
hipError_t launch_quantize_a8(const void* A, int64_t lda, int64_t M, int64_t K, void* Q, int64_t ldq,
                              void* S, hipStream_t s);
hipError_t launch_repack_w4a16(const BlobLayout& L, const void* codes, const void* scales,
                               void* packed, hipStream_t s);
hipError_t launch_repack_w4a8(const BlobLayout& L, const void* codes, const void* gscales,
                              const void* cscales, void* packed, hipStream_t s);
// General-grid blob: W4A16 codes, then one entry per (group, column) in the
// scales region (see repack.hip); Gs = K / gs groups, P = 2 entries per 128-k
// chunk when gs = 64, else 1.
BlobLayout blob_layout_w4g(int64_t K, int64_t N, int gs, bool zeros);
// Bit-plane W_b A8: chunks of 256*bits bytes (codes), then fp16 channel scales (aux).
BlobLayout blob_layout_bitplane(int64_t K, int64_t N, int bits);
hipError_t launch_repack_bitplane(const BlobLayout& L, int bits, const void* codes, const void* cscales,
                                  void* packed, hipStream_t s);
// 2:4 sparse W4A16: 768-byte chunks of kept codes and positions, scales, status word (high).
hipError_t launch_repack_sp24(const BlobLayout& L, const void* codes, const void* scales, void* packed,
                              hipStream_t s);
hipError_t launch_repack_w4g(const BlobLayout& L, int gs, const void* codes, const void* scales,
                             const void* zeros, void* packed, hipStream_t s);
// desc (already uploaded into the blob's descriptor region) gives the high-plane slots.
hipError_t launch_repack_w2w4(const BlobLayout& L, const void* codes, const void* scales,
                              void* packed, hipStream_t s);

}  // namespace qg
