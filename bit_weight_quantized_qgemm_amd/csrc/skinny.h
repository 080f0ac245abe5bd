// Shared driver of the streaming quantized-weight GEMM kernels (gfx950), used for
// small and medium batches (the memory-bound regime of the MARLIN abstract).
//
// Work decomposition (the MARLIN abstract's scheduling of the work across the
// GPU, re-derived for CDNA4):
//   * a workgroup owns one output tile of 16*MB rows x 64*NBW columns over the K
//     range of its k-split (usually all of K);
//   * its 4*KP waves form KP K-parts of 4 column waves: column wave n streams
//     16*NBW columns, K-part k the k-th contiguous share of the tile's groups;
//   * the 4 column waves of a K-part share the activations through LDS: each
//     group's A rows (1 KB loads of 4 fp16 or 8 int8 whole rows, chunk-swizzled,
//     see ARows16 / ARows8) arrive by direct buffer-to-LDS loads two groups
//     ahead into a 3-slot ring, each column wave fetching a quarter, published
//     by one barrier per group;
//   * weights stream per wave into a 3-stage register ring, also two groups
//     ahead, so every wave keeps two groups of loads in flight;
//   * at the end the KP partial tiles are summed in LDS in K-part order
//     (deterministic) and written as fp16;
//   * only when a layer has too few tiles does the plan also split K across
//     workgroups; those partials go through a global workspace in fragment order
//     with device-coherent 16-byte stores and loads and one arrival counter per
//     tile; the last workgroup to arrive adds them in split order.
//
// A format policy F supplies the per-group weight stage (load and math), the
// activation slot layout and the output conversion. Group scales of the tile are
// staged in LDS once per workgroup, after the first loads are already in flight.
#pragma once

#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// vmcnt(n) with the other counters left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence: __syncthreads() is a release fence,
// which would also wait for every direct-to-LDS prefetch in flight. Callers make
// their own completions explicit with wait_vmcnt; the compiler fences keep LDS
// accesses on their side of the barrier.
__device__ __forceinline__ void raw_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct TileInfo {
  int b0;      // first 16-column block of the tile
  int row0;    // first row of the tile
  int rows;    // valid rows in the tile (>= 1)
  int G0, G1;  // group range of the workgroup
  int c8;      // first 8-group scale chunk (G0 / 8)
  int n8;      // scale chunks staged per column block
};

// The tile (column tile, row tile, k-split) of this workgroup. With several row
// tiles (mt > 1) the row tiles of one column tile and k-split get block indices
// 8 apart: the hardware hands workgroups to the 8 XCDs in turn, so they run on
// one XCD, and its L2 serves the repeated reads of the same weights (only speed
// depends on that order, not results). The (column tile, k-split) pairs past
// the last whole group of 8 keep the plain order, so the grid is exactly
// nt x mt x splits and no XCD gets more workgroups than in plain order.
struct TileIndex {
  int nt, mt, split;
};
__device__ __forceinline__ TileIndex tile_of_block(const GemmArgs& p) {
  const int b = blockIdx.x;
  const int pairs = p.nt * p.splits;
  const int whole = pairs & ~7;
  int g, r;
  if (b < whole * p.mt) {
    const int q = b >> 3;
    g = (q / p.mt) * 8 + (b & 7);
    r = q % p.mt;
  } else {
    const int j = b - whole * p.mt, rest = pairs - whole;
    g = whole + j % rest;
    r = j / rest;
  }
  return TileIndex{g % p.nt, r, g / p.nt};
}

// Returns true in every thread of the workgroup that arrived last.
__device__ __forceinline__ bool workgroup_arrive_last(uint32_t* counter, uint32_t total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = prev == total - 1;
    if (prev == total - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
}

// Direct buffer-to-LDS copy of `pieces` 16-byte pieces to dst .. dst + 16*pieces
// (dst 16-byte aligned): piece p comes from byte offset src_of(p) of resource
// r. The workgroup's waves take 1 KB rows of the destination in turn; lanes
// past the last piece are masked off, so nothing beyond the destination is
// written. The copies count on the vector memory counter like any load, and
// become visible to other waves after their issuing wave has waited for them
// and passed a barrier.
template <class SrcOf>
__device__ __forceinline__ void dma16(rsrc_t r, char* dst, int pieces, const SrcOf& src_of, int wave, int nwaves,
                                      int lane) {
  const int rows = (pieces + 63) >> 6;
  for (int t = wave; t < rows; t += nwaves) {
    const int p = (t << 6) + lane;
    if (p < pieces) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + (t << 10)), 16, src_of(p), 0, 0, 0);
  }
}

// The tile's group-scale chunks into LDS by direct loads: for each of the NB
// column blocks, n8 chunks of `chunk` bytes starting at chunk c8 ([NB][n8][chunk]).
__device__ __forceinline__ void stage_scales(const void* scales, char* lds, int NB, int G8, int b0,
                                             int c8, int n8, int chunk, int wave, int nwaves, int lane) {
  const int per_blk = n8 * chunk / 16;      // 16-byte pieces per block
  const rsrc_t r = make_rsrc(static_cast<const char*>(scales) + (size_t)b0 * G8 * chunk, (uint32_t)(NB * G8 * chunk));
  dma16(r, lds, NB * per_blk, [&](int p) {
    const int j = p / per_blk, o = p - j * per_blk;
    return (uint32_t)((j * G8 + c8) * chunk + o * 16);
  }, wave, nwaves, lane);
}

// Geometry shared by the policies built on 16 x 16 MFMA tiles: the position
// (row_of, col_of) of accumulator element i of lane ln in fragment (mb, j) of
// a wave's tile.
struct Tile16 {
  __device__ static int row_of(int mb, int, int i, int ln) { return mb * 16 + 4 * (ln >> 4) + i; }
  __device__ static int col_of(int, int j, int, int ln) { return j * 16 + (ln & 15); }
};

// fp16 / bf16 activation slots in LDS: [rows][128 k], 256 B per row, with the
// 16-byte chunk c (k = 8c .. 8c + 7) of row r at chunk position c ^ (r & 15).
// Each direct-to-LDS load moves four whole rows (lane j: row 4*fr + j/16,
// position j % 16), i.e. 1 KB in 8 full cache lines, where MFMA operand order
// would touch 16 or 32 rows per load; the operand reads, whose lanes take 16
// or 32 consecutive rows at one chunk, see 16 distinct positions per 16 rows,
// so they stay free of bank conflicts.
struct ARows16 {
  // byte offset in A (row stride arow bytes) of this lane's 16 bytes of load fr
  __device__ static uint32_t dma_voff(int fr, int lane, int rows, size_t arow) {
    const int r = 4 * fr + (lane >> 4);
    return (uint32_t)((size_t)min(r, rows - 1) * arow + (uint32_t)(((lane & 15) ^ (r & 15)) << 4));
  }
  // the 8 activations of row r, chunk c of a slot
  __device__ static const char* at(const char* slot, int r, int c) { return slot + r * 256 + ((c ^ (r & 15)) << 4); }
};

// int8 activation slots: [rows][128 k], 128 B per row, chunk c at position
// c ^ ((r >> 1) & 7); a 1 KB load moves eight whole rows (lane j: row
// 8*fr + j/8, position j % 8), and the 16x16x64 operand reads (16 rows at one
// chunk) cover all 64 banks once.
struct ARows8 {
  __device__ static uint32_t dma_voff(int fr, int lane, int rows, size_t arow) {
    const int r = 8 * fr + (lane >> 3);
    return (uint32_t)((size_t)min(r, rows - 1) * arow + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4));
  }
  __device__ static const char* at(const char* slot, int r, int c) {
    return slot + r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  }
};

// LDS layout of a launch: [scales | extra | A rings (KP x 3 slots)]; the
// reduction buffer reuses the start of LDS after the main loop.
struct SkinnyLds {
  int scale_bytes, extra_off, ring_off, slot_bytes, total;
};

template <class F>
__host__ __device__ inline SkinnyLds skinny_lds(int MB, int NBW, int KP, int n8_max, int ng_max, int gs) {
  constexpr int WD = F::kWeightDepth;
  SkinnyLds L;
  const int NB = 4 * NBW;
  L.scale_bytes = F::kStageScales ? NB * n8_max * F::kScaleChunk : 0;
  L.extra_off = L.scale_bytes;
  const int extra = F::extra_lds(NB, ng_max, gs);
  L.ring_off = (L.extra_off + extra + 255) / 256 * 256;
  L.slot_bytes = MB * F::kFrag * 1024;
  const int rings = L.ring_off + KP * (WD + 1) * L.slot_bytes;
  const int red = KP * 4 * MB * NBW * 1024;   // one 1 KB fragment of floats per (wave, block)
  L.total = rings > red ? rings : red;
  return L;
}

template <class F, int MB, int NBW, int KP>
__device__ __forceinline__ void skinny_body(const GemmArgs& p, char* lds, int* flag) {
  constexpr int WD = F::kWeightDepth;
  using Acc = typename F::Acc;
  using Stage = typename F::template Stage<NBW>;
  using View = typename F::template View<NBW>;
  constexpr int NB = 4 * NBW;
  constexpr int kFrags = MB * F::kFrag;          // 1 KB activation loads per group per K-part

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kp = wave >> 2, nw = wave & 3;
  const int c = lane & 15, h = lane >> 4;
  const TileIndex tix = tile_of_block(p);
  const int nt = tix.nt, mt = tix.mt, split = tix.split;

  TileInfo ti;
  ti.b0 = nt * NB;
  ti.row0 = mt * MB * 16;
  ti.rows = min(MB * 16, p.M - ti.row0);
  ti.G0 = split * p.gps;
  ti.G1 = min(p.G, ti.G0 + p.gps);
  ti.c8 = ti.G0 >> 3;
  ti.n8 = ((ti.G1 - 1) >> 3) - ti.c8 + 1;
  const int ngw = ti.G1 - ti.G0;
  const SkinnyLds L = skinny_lds<F>(MB, NBW, KP, (min(p.G, p.gps) + 7) / 8 + 1, min(p.G, p.gps), p.gs);

  // this K-part's groups [gk0, gk0 + ngk); every K-part runs `iters` iterations
  const int iters = (ngw + KP - 1) / KP;
  const int gk0 = ti.G0 + kp * iters;
  const int ngk = max(0, min(ti.G1 - gk0, iters));
  const int nload = max(ngk, 1);                  // clamp target for reloads
  const int gk0c = ngk > 0 ? gk0 : ti.G0;         // empty K-parts re-read the first group

  // ---- activations: this K-part's 1 KB row loads, a quarter per column wave
  const size_t arow = (size_t)p.lda * F::kAElem;
  const rsrc_t ra = make_rsrc(static_cast<const char*>(p.A) + (size_t)ti.row0 * arow + (size_t)gk0c * 128 * F::kAElem,
                              (uint32_t)((size_t)(ti.rows - 1) * arow + (size_t)nload * 128 * F::kAElem));
  constexpr int kAPerWave = (kFrags + 3) / 4;     // activation loads per column wave per group
  uint32_t avoff[kAPerWave];
  int afrag[kAPerWave];
#pragma unroll
  for (int q = 0; q < kAPerWave; ++q) {
    const int fr = min(nw + 4 * q, kFrags - 1);   // waves past the last load duplicate it
    afrag[q] = fr;
    avoff[q] = F::a_voff(fr, lane, ti.rows, arow);
  }
  char* ring = lds + L.ring_off + kp * (WD + 1) * L.slot_bytes;
  auto issue_a = [&](int rel, int slot, uint32_t oob) {
#pragma unroll
    for (int q = 0; q < kAPerWave; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(ring + slot * L.slot_bytes + afrag[q] * 1024), 16,
                                               avoff[q] + oob, rel * (128u * F::kAElem), 0, 0);
  };

  const View v(p, lds, L, ti, ti.b0 + nw * NBW, gk0c, nload, lane);
  Acc acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[mb][j] = Acc{0, 0, 0, 0};

  // ---- prologue. Weights and activations both run kWD = F::kWeightDepth
  // groups ahead, in a register ring of kWD + 1 stages and an LDS ring of
  // kWD + 1 slots. (A deeper ring measured slower on MI355X: three and four
  // groups ahead by 0-29 %, and eight groups - every group of a short K-part in
  // flight at once - by 5-50 % on 4096 x 4096 to 28672 x 8192 layers at
  // M <= 16, also with its loads past the K-part's end reading nothing.)
  // The tile's staged data (group scales, grid entries, descriptors) goes to
  // LDS first, by direct loads, then the first groups' loads; a counted wait
  // then retires only the staging copies, so the first groups stay in flight
  // while the barrier publishes the staged data (a full __syncthreads here
  // would drain every load in flight).
  constexpr int kWD = WD, kWS = kWD + 1, kAS = kWD + 1;
  static_assert(kWD >= 2, "at least two groups in flight");
  constexpr bool kStaged = F::kStageScales || F::kStageExtra;
  // Group g of the K-part (relative to its first): loads past the K-part's last
  // group keep the fixed count but read nothing: their per-lane offsets move
  // past the buffer's size (2^31 and up), so the hardware returns zeros
  // without a memory access (and direct-to-LDS loads write zeros to their
  // slot, which no later group uses).
  auto wl = [&](int g) { return min(g, nload - 1); };
  auto oob = [&](int g) { return g >= nload ? 0x80000000u : 0u; };
  if constexpr (kStaged) {
    if constexpr (F::kStageScales)
      stage_scales(p.scales, lds, NB, p.G8, ti.b0, ti.c8, ti.n8, F::kScaleChunk, wave, 4 * KP, lane);
    F::stage_extra(p, lds + L.extra_off, ti, NB, wave, 4 * KP, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  Stage st[kWS];
#pragma unroll
  for (int d = 0; d < kWD; ++d) {
    issue_a(wl(d), d, oob(d));
    __builtin_amdgcn_sched_barrier(0);
    v.load_vmem(st[d], wl(d), oob(d));
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kStaged) {
    // loads issued after the staging copies: kWD groups of activations and weights
    wait_vmcnt<kWD * (kAPerWave + Stage::kVmemFirst)>();
    raw_barrier();
  }
#pragma unroll
  for (int d = 0; d < kWD; ++d) v.load_lds(st[d], wl(d), oob(d));

  const typename F::Consts k;
  // Per iteration each wave first issues the weights of group i + kWD (their
  // register stage held group i - 1, already consumed), waits, passes the
  // barrier, then issues its A loads of group i + kWD (their slot held group
  // i - 1, which the barrier shows every wave has finished reading). At the
  // wait of iteration i >= kWD exactly the batches of iterations i - kWD + 1 ..
  // i - 1 and the weights of iteration i were issued after the wave's last
  // A(i) load (earlier iterations have more loads after it, so they wait for
  // more), and the counter retires loads in order. Issuing the weights before
  // the wait keeps them in flight while the wave waits at the barrier
  // (measured on MI355X: 3-6 % at M = 4-32 on the down projection).
  //
  // Loads keep this fixed count to the end: the last kWD iterations issue
  // out-of-range loads (see oob) instead of skipping their loads. A variant
  // that skipped them, with exact smaller waits in those iterations, measured
  // 5-45 % slower on MI355X (the compiler's own waits around the conditional
  // loads serialized the ring).
  constexpr int kAfter = Stage::kVmem + (kWD - 1) * (kAPerWave + Stage::kVmem);
  for (int base = 0; base < iters; base += kWS) {
#pragma unroll
    for (int r = 0; r < kWS; ++r) {
      const int i = base + r;
      if (i < iters) {   // uniform over the workgroup
        v.load_vmem(st[(r + kWD) % kWS], wl(i + kWD), oob(i + kWD));
        // the count relies on this order: keep the compiler from moving loads
        // across the wait or between the weights and the activations
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kAfter>();
        raw_barrier();
        issue_a(wl(i + kWD), (r + kWD) % kAS, oob(i + kWD));
        __builtin_amdgcn_sched_barrier(0);
        v.load_lds(st[(r + kWD) % kWS], wl(i + kWD), oob(i + kWD));
        F::template compute<MB, NBW>(st[r], ring + (r % kAS) * L.slot_bytes, acc, i < ngk, k, lane);
      }
    }
  }
  // The last iterations left loads in flight, the last of them activation DMA
  // into the ring: retire everything before LDS is reused.
  wait_vmcnt<0>();
  __syncthreads();   // all LDS reads done: reuse LDS for the reduction

  // ---- reduce the KP K-parts in K-part order; fragment (wave, mb, j) = 1 KB
  using E = typename F::Elem;
  E* red = reinterpret_cast<E*>(lds);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(((wave * MB + mb) * NBW + j) * 64 + lane) * 4 + i] = acc[mb][j][i];
  __syncthreads();
  constexpr int kTileElems = 4 * MB * NBW * 256;   // 4 column waves x fragments x 256
  const int tid = threadIdx.x;
  if (p.splits == 1) {
    for (int e = tid; e < kTileElems; e += KP * 256) {
      E s = red[e];
      for (int q = 1; q < KP; ++q) s += red[q * kTileElems + e];
      const int i = e & 3, ln = (e >> 2) & 63, fj = e >> 8;      // fj = (nw*MB + mb)*NBW + j
      const int j = fj % NBW, mb = (fj / NBW) % MB, w = fj / (NBW * MB);
      const int row = ti.row0 + F::row_of(mb, j, i, ln);
      const int col = (ti.b0 + w * NBW) * 16 + F::col_of(mb, j, i, ln);
      if (row < ti.row0 + ti.rows) F::store(p, row, col, s);
    }
    return;
  }
  // cross-workgroup split: publish the reduced tile in fragment order
  const size_t tile_id = (size_t)mt * p.nt + nt;
  const size_t ntiles = (size_t)p.mt * p.nt;
  constexpr uint32_t kRegion = kTileElems * 4;
  auto region = [&](int q) {
    return make_rsrc(static_cast<char*>(p.partial) + ((size_t)q * ntiles + tile_id) * kRegion, kRegion);
  };
  {
    const rsrc_t mine = region(split);
    for (int e4 = tid; e4 < kTileElems / 4; e4 += KP * 256) {
      f32x4 s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        E x = red[e4 * 4 + i];
        for (int q = 1; q < KP; ++q) x += red[q * kTileElems + e4 * 4 + i];
        s[i] = __builtin_bit_cast(float, x);
      }
      store16_coherent(s, mine, e4 * 16u);
    }
  }
  if (!workgroup_arrive_last(p.counters + tile_id, (uint32_t)p.splits, flag)) return;
  constexpr int kBatch = 8;   // splits whose loads are in flight together
  for (int e4 = tid; e4 < kTileElems / 4; e4 += KP * 256) {
    E s[4] = {0, 0, 0, 0};
    for (int q0 = 0; q0 < p.splits; q0 += kBatch) {
      f32x4 x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x[u] = load16_coherent(region(min(q0 + u, p.splits - 1)), e4 * 16u);
      // in split order; splits past the last were re-reads and add nothing
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (q0 + u < p.splits) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // copy the lane out first: this compiler's bit_cast of a vector-element
            // lvalue reads element 0 whatever the index
            const float xi = x[u][i];
            s[i] += __builtin_bit_cast(E, xi);
          }
        }
      }
    }
    const int ln = e4 & 63, fj = e4 >> 6;
    const int j = fj % NBW, mb = (fj / NBW) % MB, w = fj / (NBW * MB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = (ti.b0 + w * NBW) * 16 + F::col_of(mb, j, i, ln);
      const int row = ti.row0 + F::row_of(mb, j, i, ln);
      if (row < ti.row0 + ti.rows) F::store(p, row, col, s[i]);
    }
  }
}

// One kernel per workgroup size, so each gets its own register budget (a
// template-dependent launch bound would not do here).
#define QG_SKINNY_KERNEL(KPV, THREADS)                                          \
  template <class F, int MB, int NBW>                                           \
  __global__ void __launch_bounds__(THREADS) skinny_gemm_kp##KPV(GemmArgs p) { \
    extern __shared__ __attribute__((aligned(16))) char lds[];                 \
    __shared__ int flag;                                                        \
    skinny_body<F, MB, NBW, KPV>(p, lds, &flag);                               \
  }
QG_SKINNY_KERNEL(1, 256)
QG_SKINNY_KERNEL(2, 512)
QG_SKINNY_KERNEL(4, 1024)
#undef QG_SKINNY_KERNEL

// LDS bytes of a launch (the largest split range bounds the staged chunks)
template <class F>
inline size_t skinny_lds_bytes(const Plan& pl, int G, int gs = 0) {
  const int ng_max = std::min(G, pl.gps);
  return (size_t)skinny_lds<F>(pl.mb, pl.nb, pl.wpt / 4, (ng_max + 7) / 8 + 1, ng_max, gs).total;
}

template <class F, int MB, int NBW>
hipError_t dispatch_kp(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  const size_t lds = skinny_lds_bytes<F>(pl, a.G, a.gs);
  if (lds > kSkinnyLdsBudget) return hipErrorInvalidValue;   // the planner keeps plans within it
  const dim3 grid((unsigned)pl.workgroups);
  switch (pl.wpt / 4) {
    case 1: hipLaunchKernelGGL((skinny_gemm_kp1<F, MB, NBW>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((skinny_gemm_kp2<F, MB, NBW>), grid, dim3(512), lds, s, a); break;
    case 4: hipLaunchKernelGGL((skinny_gemm_kp4<F, MB, NBW>), grid, dim3(1024), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class F>
hipError_t dispatch_skinny(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  switch (pl.mb * 10 + pl.nb) {
    case 11: return dispatch_kp<F, 1, 1>(pl, a, s);
    case 12: return dispatch_kp<F, 1, 2>(pl, a, s);
    case 21: return dispatch_kp<F, 2, 1>(pl, a, s);
    case 22: return dispatch_kp<F, 2, 2>(pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
