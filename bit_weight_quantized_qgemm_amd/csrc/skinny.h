// Shared driver of the streaming quantized-weight GEMM kernels (gfx950).
//
// Work decomposition (the "task scheduling" of the MARLIN abstract, re-derived
// for CDNA4):
//   * one workgroup = one output tile of 16*MB rows x 16*NB columns, over the
//     K range of its k-split (almost always the whole K);
//   * its W waves (1..8) split that K range into W contiguous group ranges and
//     stream them concurrently: small-M layers have few tiles, so parallelism
//     comes from K (split-K inside the workgroup);
//   * each wave keeps D groups of weights and activations in flight in a
//     register ring (the "asynchronous memory access and pipelining");
//   * the W partial tiles are summed in LDS in wave order (deterministic), and
//     the workgroup writes fp16 C. No global workspace, no atomics.
//   * Only when a layer has too few tiles even for 8 waves each does the plan
//     also split K across workgroups; those partial tiles go through a global
//     workspace with device-coherent stores and one arrival counter per tile;
//     the last workgroup to arrive adds them in split order.
//
// A format policy F supplies the per-group stage (what one wave loads for one
// group), its load and its math. Group scales of the tile are staged in LDS once
// per workgroup, so a wave's K range may start at any group.
#pragma once

#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {

// LDS layout: [scale region | (after the main loop) reduction region]
struct TileInfo {
  int b0;      // first 16-column block of the tile
  int row0;    // first row of the tile
  int rows;    // valid rows in the tile (>= 1)
  int G0, G1;  // group range of the workgroup
  int c8;      // first 8-group scale chunk (G0 / 8)
  int n8;      // scale chunks staged per column block
};

// Reduce W waves' accumulators through LDS and hand each output element to
// `emit(row, col, value)` exactly once. Accumulators are 4-vectors of float or
// int32; lane (c, h) of a wave holds rows 4h..4h+3 of column c of each 16x16 block.
template <int MB, int NB, typename V, typename Emit>
__device__ __forceinline__ void reduce_tile(const V (&acc)[MB][NB], char* lds, int W, int lane,
                                            int wave, const TileInfo& ti, Emit emit) {
  using E = decltype(acc[0][0][0] + acc[0][0][0]);
  E* red = reinterpret_cast<E*>(lds);
  constexpr int kPer = MB * NB * 4;   // elements per lane per wave
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[((wave * kPer) + (mb * NB + j) * 4 + i) * 64 + lane] = acc[mb][j][i];
  __syncthreads();
  const int nthreads = W * 64;
  for (int e = threadIdx.x; e < kPer * 64; e += nthreads) {
    E v = red[e];
    for (int w = 1; w < W; ++w) v += red[w * kPer * 64 + e];
    const int ln = e & 63, idx = e >> 6;
    const int i = idx & 3, blk = idx >> 2;
    const int j = blk % NB, mb = blk / NB;
    const int row = ti.row0 + mb * 16 + 4 * (ln >> 4) + i;
    const int col = (ti.b0 + j) * 16 + (ln & 15);
    if (row < ti.row0 + ti.rows) emit(row, col, v);
  }
}

// Cross-workgroup k-split: publish this workgroup's reduced tile, count arrivals,
// and let the last arriver finish the tile. Partial stores and loads are
// device-scope atomics (cache-coherent across XCDs without whole-cache
// maintenance); every thread waits for its own stores before the barrier that
// precedes the counter increment.
template <typename E>
struct CrossSplit {
  E* part;              // [splits][M][N]
  uint32_t* counter;    // this tile's counter
  int split, splits, M, N;

  __device__ __forceinline__ void publish(int row, int col, E v) const {
    __hip_atomic_store(part + ((size_t)split * M + row) * N + col, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ E gather(int row, int col) const {
    E s = 0;
    for (int q = 0; q < splits; ++q)
      s += __hip_atomic_load(part + ((size_t)q * M + row) * N + col, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return s;
  }
};

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

// Cooperative copy of the tile's group-scale chunks into LDS: for each of the NB
// column blocks, n8 chunks of `chunk` bytes starting at chunk c8.
__device__ __forceinline__ void stage_scales(const void* scales, char* lds, int NB, int G8, int b0,
                                             int c8, int n8, int chunk) {
  const int per_blk = n8 * chunk / 16;      // 16-byte pieces per block
  const int total = NB * per_blk;
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    const int j = t / per_blk, o = t % per_blk;
    const u32x4* src = static_cast<const u32x4*>(scales) +
                       ((size_t)(b0 + j) * G8 + c8) * (chunk / 16) + o;
    reinterpret_cast<u32x4*>(lds)[t] = *src;
  }
}

template <class F, int MB, int NB, int D>
__global__ void __launch_bounds__(512) skinny_gemm(GemmArgs p) {
  using Acc = typename F::Acc;
  using Stage = typename F::template Stage<MB, NB>;
  using View = typename F::template View<MB, NB>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_flag;

  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = blockIdx.x % p.nt;
  const int rest = blockIdx.x / p.nt;
  const int mt = rest % p.mt;
  const int split = rest / p.mt;

  TileInfo ti;
  ti.b0 = nt * NB;
  ti.row0 = mt * MB * 16;
  ti.rows = min(MB * 16, p.M - ti.row0);
  ti.G0 = split * p.gps;
  ti.G1 = min(p.G, ti.G0 + p.gps);
  ti.c8 = ti.G0 >> 3;
  ti.n8 = ((ti.G1 - 1) >> 3) - ti.c8 + 1;

  stage_scales(p.scales, lds, NB, p.G8, ti.b0, ti.c8, ti.n8, F::kScaleChunk);
  F::stage_extra(p, lds, ti, NB);
  __syncthreads();

  // this wave's groups [gw0, gw0 + ng)
  const int ngw = ti.G1 - ti.G0;
  const int gpw = (ngw + W - 1) / W;
  const int gw0 = ti.G0 + wave * gpw;
  const int ng = min(ti.G1, gw0 + gpw) - gw0;

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = Acc{0, 0, 0, 0};

  if (ng > 0) {
    const View v(p, lds, ti, gw0, ng, lane);
    typename F::Consts k;
    // Register ring of 4 stages with static slots: loads for group g + D are
    // issued before the math of group g. Groups past the end (ragged tail of the
    // 4-group body) reload the last group and are scaled by zero, so the body
    // stays one basic block.
    Stage st[4];
#pragma unroll
    for (int d = 0; d < D; ++d) v.load(st[d], min(d, ng - 1));
    for (int base = 0; base < ng; base += 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v.load(st[(r + D) & 3], min(base + r + D, ng - 1));
        __builtin_amdgcn_sched_barrier(0);
        F::template compute<MB, NB>(st[r], acc, base + r < ng, k, lane);
      }
    }
  }
  __syncthreads();   // scale/extra LDS regions are dead: reuse LDS for the reduction

  if (p.splits == 1) {
    auto emit = [&](int row, int col, typename F::Elem v) { F::store(p, row, col, v); };
    reduce_tile<MB, NB>(acc, lds, W, lane, wave, ti, emit);
    return;
  }
  CrossSplit<typename F::Elem> cs{static_cast<typename F::Elem*>(p.partial),
                                  p.counters + (size_t)mt * p.nt + nt, split, p.splits, p.M, p.N};
  reduce_tile<MB, NB>(acc, lds, W, lane, wave, ti,
                      [&](int row, int col, typename F::Elem v) { cs.publish(row, col, v); });
  if (!workgroup_arrive_last(cs.counter, (uint32_t)p.splits, &s_flag)) return;
  constexpr int kElems = MB * NB * 256;
  for (int e = threadIdx.x; e < kElems; e += blockDim.x) {
    const int ln = e & 63, idx = e >> 6;
    const int i = idx & 3, blk = idx >> 2;
    const int j = blk % NB, mb = blk / NB;
    const int row = ti.row0 + mb * 16 + 4 * (ln >> 4) + i;
    const int col = (ti.b0 + j) * 16 + (ln & 15);
    if (row < ti.row0 + ti.rows) F::store(p, row, col, cs.gather(row, col));
  }
}

// LDS bytes a launch needs: max(staged scales + extras, reduction buffer).
template <class F>
inline size_t skinny_lds_bytes(const Plan& pl, int G) {
  const int n8 = (std::min(G, pl.gps) + 7) / 8 + 1;   // chunks touched by one split, worst case
  const size_t stage = (size_t)pl.nb * n8 * F::kScaleChunk + F::extra_lds(pl);
  const size_t red = (size_t)pl.wpt * pl.mb * pl.nb * 4 * 64 * 4;
  return std::max(stage, red);
}

template <class F, int MB, int NB>
hipError_t launch_skinny(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  constexpr int D = F::kDepth;
  const size_t lds = skinny_lds_bytes<F>(pl, a.G);
  hipLaunchKernelGGL((skinny_gemm<F, MB, NB, D>), dim3((unsigned)pl.workgroups),
                     dim3(kWave * pl.wpt), lds, s, a);
  return hipGetLastError();
}

template <class F>
hipError_t dispatch_skinny(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  switch (pl.mb * 10 + pl.nb) {
    case 11: return launch_skinny<F, 1, 1>(pl, a, s);
    case 12: return launch_skinny<F, 1, 2>(pl, a, s);
    case 14: return launch_skinny<F, 1, 4>(pl, a, s);
    case 21: return launch_skinny<F, 2, 1>(pl, a, s);
    case 22: return launch_skinny<F, 2, 2>(pl, a, s);
    case 24: return launch_skinny<F, 2, 4>(pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
