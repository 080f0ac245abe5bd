// W4A16 GEMM for larger batches (M > 32) on gfx950: the compute-bound end of the
// batch range of the MARLIN abstract, where its speedup shrinks with batch size
// but persists up to 64-128. The same kernel runs the general 4-bit grid with
// fp16 activations (per group and column a scale and optionally a zero point;
// the abstract of the "Enabling Fast 2-bit LLM on GPUs" page quantizes weights
// by groups without fixing their length).
//
// Each workgroup owns a tile of 16*MBW = 64 rows x TC = 256 columns; its eight
// waves (two per SIMD, so one wave's dequantization and LDS reads overlap the
// other's matrix operations) form a grid of NWC column waves x 8/NWC row waves,
// each owning 256/NWC columns and 16*MBW*NWC/8 rows. Layers whose 256-column
// tiles would need more k-splits take 64 x 128 tiles, whose eight waves are
// two K-parts of four (WPK) 32-column waves. Each weight is dequantized
// by the WPK/NWC row waves of its columns and reused by all of their rows. The products
// run on v_mfma_f32_32x32x16_f16, which does twice the work of the 16x16x32 form
// for the same operand bytes and sustains a higher rate on gfx950:
//   * operands of one 32x32x16 step: lane l holds row (A) or column (B) l % 32
//     and k = 8*(l/32) .. +7 of the 16-k step; the result's element i of lane l
//     is row 8*(i/4) + 4*(l/32) + i%4, column l % 32;
//   * the blob keeps its 16-column chunk order (shared with the streaming
//     kernel): the B operand of 32-column block jb for k-step u is word u/2 of
//     blob lane 16*(2*(u%2) + l/32) + l%16 of 16-column block 2*jb + (l%32)/16,
//     so every lane fetches two 16-byte pieces per 32-column block and group
//     (its "even" and "odd" k-steps) at lane-dependent offsets - each byte of
//     the chunk pair is still loaded exactly once per wave;
//   * per group of 128 k the tile's activations arrive as whole rows (the
//     swizzled row-major slot of ARows16, four rows per 1 KB load) by direct
//     buffer-to-LDS loads, issued kDepth groups ahead into an LDS ring, each
//     wave fetching an eighth; one
//     barrier per group publishes a slot after the wave's own loads of it are
//     counted complete (s_waitcnt on the in-order vector memory counter), and the
//     slot written next is the one all waves finished reading before that
//     barrier.
// Weights stream per wave into a register ring (kDepth groups ahead) together
// with the lane's fp16 group scales (or grid entries); dequantization is exact
// to fp16 (q - 8, or q - z),
// then one packed multiply by the scale rounds once (the scale cannot be applied
// after the MFMA here without doubling the accumulators). Accumulation is fp32.
// When a layer has too few tiles for the chip, K is also split across workgroups
// and finished with the coherent-store / arrival-counter fix-up.
#include "skinny.h"

#include <mutex>
#include <set>
#include <utility>

namespace qg {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWideWaves = 8;
constexpr int kDepth = 3;                              // groups of loads in flight ahead
constexpr int kASlots = kDepth + 1;                    // LDS slots and register stages

// Weight formats of the wide kernel: the W4A16 blob, or the general-grid blob
// (the same code chunks, then one 16-bit scale or 32-bit scale | zero-point
// entry per (group, column)) with fp16 activations, as one kernel per entry
// layout: group length a multiple of 128 (one entry per chunk-column) or 64
// (two, adjacent), without or with zero points. A compile-time layout keeps
// the stage loads free of branches and of register copies, either of which
// makes the compiler wait for the load at issue (a full drain of the ring).
enum WideFmt { kWideW4A16 = 0, kWideGrid = 1, kWideGridZ = 2, kWideGrid64 = 3, kWideGrid64Z = 4 };

template <int JB>
struct WideStage {
  u32x4 even[JB];   // words t = k-steps 2t of each 32-column block
  u32x4 odd[JB];    // words t = k-steps 2t + 1
  u32x2 s[JB];      // W4A16 and grid groups of 128+ k: the lane's fp16 scale or
                    // entry in [0]; group length 64: both entries of the chunk
                    // (in [0] as two 16-bit scales, or in [0] and [1])
};

}  // namespace

template <int MBW, int NWC, int KPW, int WF = kWideW4A16, int WPK = kWideWaves, int TC = kWideCols>
__device__ __forceinline__ void wide_body(const GemmArgs& p, char* lds, int* flag) {
  constexpr int NWR = WPK / NWC;                    // row waves
  constexpr int kWideJB = TC / 32 / NWC;            // 32-column blocks per wave
  constexpr int R32T = MBW / 2;                     // 32-row blocks of the tile
  constexpr int R32 = R32T / NWR;                   // 32-row blocks per wave
  static_assert(R32 >= 1 && kWideJB >= 1, "wave grid");
  constexpr int kSlotBytes = R32T * 8 * 1024;       // 32-row blocks x 8 k-steps x 1 KB
  constexpr int kAPerWave = R32T * 8 / WPK;         // 1 KB activation loads per wave per group
  using Stage = WideStage<kWideJB>;

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kpi = wave_all / WPK;                    // K-part of this wave
  const int wave = wave_all % WPK;                   // wave within its K-part
  const int wc = wave % NWC, wr = wave / NWC;
  const int c32 = lane & 31, hh = lane >> 5;
  const TileIndex tix = tile_of_block(p);
  const int nt = tix.nt, mt = tix.mt, split = tix.split;
  const int G0s = split * p.gps;
  const int ngw = min(p.G, G0s + p.gps) - G0s;
  // this K-part's groups [G0, G0 + ng); every K-part runs `iters` iterations
  const int iters = (ngw + KPW - 1) / KPW;
  const int gk0 = G0s + kpi * iters;
  const int ng = max(0, min(G0s + ngw - gk0, iters));
  const int nload = max(ng, 1);                      // clamp target for reloads
  const int G0 = ng > 0 ? gk0 : G0s;                 // an empty K-part re-reads the first group
  const int row0 = mt * MBW * 16;
  const int rows = min(MBW * 16, p.M - row0);
  const int bw = nt * (TC / 16) + wc * 2 * kWideJB;     // first 16-column block of the wave
  const int rw0 = wr * R32 * 32;                                // first tile row of the wave

  // activations: rows of the tile from k = 128*G0; rows beyond M re-read a valid row
  const rsrc_t ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)row0 * p.lda + (size_t)G0 * kGroup,
                              (uint32_t)(((size_t)(rows - 1) * p.lda + (size_t)nload * kGroup) * 2));
  // load f moves rows 4f .. 4f + 3 of the group (1 KB); this wave issues f = wave*kAPerWave ..
  uint32_t avoff[kAPerWave];
  int afrag[kAPerWave];
#pragma unroll
  for (int q = 0; q < kAPerWave; ++q) {
    const int f = wave * kAPerWave + q;
    afrag[q] = f;
    avoff[q] = ARows16::dma_voff(f, lane, rows, (size_t)p.lda * 2);
  }
  char* ring = lds + kpi * kASlots * kSlotBytes;     // this K-part's activation ring
  auto issue_a = [&](int rel, int slot) {
#pragma unroll
    for (int q = 0; q < kAPerWave; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(ring + slot * kSlotBytes + afrag[q] * 1024), 16,
                                               avoff[q], rel * 256u, 0, 0);
  };

  // weights and scales of this wave's 32-column blocks (group-major chunks)
  const uint32_t gstep = (uint32_t)(p.N / 16) * 1024u;
  const rsrc_t rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)G0 * (p.N / 16) + bw) * 1024,
                              (uint32_t)(nload - 1) * gstep + 2 * kWideJB * 1024u);
  uint32_t cvoff[kWideJB];
#pragma unroll
  for (int jb = 0; jb < kWideJB; ++jb)
    cvoff[jb] = (uint32_t)((2 * jb + (c32 >> 4)) * 1024 + (16 * hh + (c32 & 15)) * 16);
  // W4A16 scales [NB][G8][16][8] fp16; grid entries [row][N][per] of kEntry
  // bytes, row = the group (per = 2: the chunk's two 64-k groups, group length
  // 64) or the group that holds the chunk (per = 1)
  constexpr bool kGrid = WF != kWideW4A16;
  constexpr bool kG64 = WF == kWideGrid64 || WF == kWideGrid64Z;
  constexpr bool kZero = WF == kWideGridZ || WF == kWideGrid64Z;
  constexpr uint32_t kEntry = kZero ? 4u : 2u;
  constexpr uint32_t per = kG64 ? 2u : 1u;
  // chunks per group (groups of 128+ k); the group of chunk g is
  // (g * cmag) >> 31 with cmag = ceil(2^31 / cpg), exact while g * cpg < 2^31
  // (g < 2^13 chunks)
  const uint32_t cpg = (kGrid && !kG64) ? (uint32_t)p.gs / 128u : 1u;
  const uint32_t cmag = 0x7FFFFFFFu / cpg + 1u;
  const uint32_t sblk = (uint32_t)p.G8 * 256u;
  const uint32_t erow = (uint32_t)p.N * per * kEntry;   // bytes per entry row
  const rsrc_t rs = kGrid ? make_rsrc(p.scales, (kG64 ? (uint32_t)p.G : (uint32_t)p.G / cpg) * erow)
                          : make_rsrc(static_cast<const char*>(p.scales) + (size_t)bw * p.G8 * 256,
                                      2 * kWideJB * sblk);
  uint32_t svoff[kWideJB];
#pragma unroll
  for (int jb = 0; jb < kWideJB; ++jb)
    svoff[jb] = kGrid ? (uint32_t)((bw + 2 * jb) * 16 + c32) * per * kEntry
                      : (uint32_t)((2 * jb + (c32 >> 4)) * sblk + (c32 & 15) * 16);
  auto issue_b = [&](Stage& st, int rel) {
#pragma unroll
    for (int jb = 0; jb < kWideJB; ++jb) {
      st.even[jb] = load16(rc, cvoff[jb], rel * gstep);
      st.odd[jb] = load16(rc, cvoff[jb] + 512u, rel * gstep);
    }
    const int g = G0 + rel;
    if constexpr (!kGrid) {
      const uint32_t soff = (uint32_t)(g >> 3) * 256u + (uint32_t)(g & 7) * 2u;
#pragma unroll
      for (int jb = 0; jb < kWideJB; ++jb)
        st.s[jb] = u32x2{__builtin_amdgcn_raw_buffer_load_b16(rs, svoff[jb], soff, 0), 0u};
    } else {
      // one load per block in every layout, so the counted waits see the
      // same number of loads; loaded words are used as they are (unpacked at
      // the dequantization)
      const uint32_t row = kG64 ? (uint32_t)g : (uint32_t)(((uint64_t)(uint32_t)g * cmag) >> 31);
      const uint32_t soff = row * erow;
#pragma unroll
      for (int jb = 0; jb < kWideJB; ++jb) {
        if constexpr (WF == kWideGrid64Z)
          st.s[jb] = load8(rs, svoff[jb], soff);
        else if constexpr (WF == kWideGrid)
          st.s[jb] = u32x2{__builtin_amdgcn_raw_buffer_load_b16(rs, svoff[jb], soff, 0), 0u};
        else
          st.s[jb] = u32x2{__builtin_amdgcn_raw_buffer_load_b32(rs, svoff[jb], soff, 0), 0u};
      }
    }
  };
  constexpr int kBPerGroup = 3 * kWideJB;           // vector memory operations of issue_b

  f32x16 acc[R32][kWideJB];
#pragma unroll
  for (int rb = 0; rb < R32; ++rb)
#pragma unroll
    for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][jb][i] = 0.f;

  const f16x2 lo_off = splat_h2(-1032.0f), hi_off = splat_h2(-72.0f);
  const uint32_t magic = 0x64006400u;

  // Prologue: activations and weights of groups 0 .. kDepth-1. Each later
  // iteration issues the weights and scales of group i + kDepth, waits, passes
  // the barrier and issues the activations of group i + kDepth, so at the wait
  // of iteration i >= kDepth exactly kAfter loads (the batches of groups
  // i+1 .. i+kDepth-1 and the weights of group i + kDepth) were issued after
  // the last activation load of group i, and earlier iterations wait for more;
  // the vector memory counter retires loads in order. Slots and stages are
  // static inside the unrolled body, and the iterations past the end only
  // re-issue in-bounds loads and skip the math.
  Stage st[kASlots];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    issue_a(min(d, nload - 1), d);
    __builtin_amdgcn_sched_barrier(0);
    issue_b(st[d], min(d, nload - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int kAfter = kBPerGroup + (kDepth - 1) * (kAPerWave + kBPerGroup);
  static_assert(kAfter < 64, "vmcnt range");

  // B operand of k-step u for both 32-column blocks, scaled. The grid formats
  // take the zero point and scale of the k-step's 64-k half (k-steps 0-3 and
  // 4-7) from the lane's entry: -(1024 + z) and -(64 + z) are exact fp16
  // patterns (the ulp is 1 at 1024 and 1/16 at 64).
  auto dequant_step = [&](const Stage& cur, int u, f16x8 (&bf)[kWideJB]) {
#pragma unroll
    for (int jb = 0; jb < kWideJB; ++jb) {
      const uint32_t w = (u & 1) ? cur.odd[jb][u >> 1] : cur.even[jb][u >> 1];
      // the k-step's entry: steps 0-3 and 4-7 are the chunk's two 64-k halves
      const uint32_t e = WF == kWideGrid64 ? ((u >> 2) ? cur.s[jb][0] >> 16 : cur.s[jb][0])
                                           : cur.s[jb][WF == kWideGrid64Z ? (u >> 2) : 0];
      const f16 sh = as_h2(e & 0xFFFFu)[0];
      const f16x8 sc8 = {sh, sh, sh, sh, sh, sh, sh, sh};
      if constexpr (kZero) {
        const uint32_t z = (e >> 16) & 0xFu;
        const uint32_t zz = z | (z << 16);
        bf[jb] = dequant_u4x8(w, as_h2(zz | 0xE400E400u), as_h2((zz << 4) | 0xD400D400u), magic) * sc8;
      } else {
        bf[jb] = dequant_u4x8(w, lo_off, hi_off, magic) * sc8;
      }
    }
  };
  auto read_a = [&](const char* slot, int u, f16x8 (&a)[R32]) {
#pragma unroll
    for (int rb = 0; rb < R32; ++rb)
      a[rb] = *reinterpret_cast<const f16x8*>(ARows16::at(slot, (wr * R32 + rb) * 32 + c32, 2 * u + hh));
  };

  for (int base = 0; base < iters; base += kASlots) {
#pragma unroll
    for (int r = 0; r < kASlots; ++r) {
      const int i = base + r;
      // weights first (their stage held group i - 1, already consumed), so
      // they are in flight during the wait; raw_barrier() publishes only the
      // counted completion (see skinny.h)
      issue_b(st[(r + kDepth) % kASlots], min(i + kDepth, nload - 1));
      // the count relies on this order: no load moves across the wait
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kAfter>();
      raw_barrier();
      issue_a(min(i + kDepth, nload - 1), (r + kDepth) % kASlots);
      __builtin_amdgcn_sched_barrier(0);
      if (i < ng) {
        const Stage& cur = st[r];
        const char* slot = ring + r * kSlotBytes;
        // software pipeline over the 8 k-steps: the A operands and dequantized
        // weights of step u+1 are fetched while the MFMAs of step u run
        f16x8 a[2][R32], bf[2][kWideJB];
        read_a(slot, 0, a[0]);
        dequant_step(cur, 0, bf[0]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (u < 7) {
            read_a(slot, u + 1, a[(u + 1) & 1]);
            dequant_step(cur, u + 1, bf[(u + 1) & 1]);
          }
#pragma unroll
          for (int rb = 0; rb < R32; ++rb)
#pragma unroll
            for (int jb = 0; jb < kWideJB; ++jb)
              acc[rb][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[u & 1][rb], bf[u & 1][jb], acc[rb][jb], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (KPW > 1) {
    // The last iterations left loads in flight, the last of them activation
    // DMA into the ring: retire everything before LDS is reused. K-parts 1..
    // then publish their accumulators and K-part 0 adds them in K-part order.
    wait_vmcnt<0>();
    __syncthreads();
    constexpr int kAcc4 = R32 * kWideJB * 4;         // f32x4 per lane
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    auto at = [&](int q, int e4) -> f32x4& { return red[(((q - 1) * WPK + wave) * kAcc4 + e4) * 64 + lane]; };
    if (kpi > 0) {
#pragma unroll
      for (int rb = 0; rb < R32; ++rb)
#pragma unroll
        for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            at(kpi, (rb * kWideJB + jb) * 4 + q4) = f32x4{acc[rb][jb][4 * q4], acc[rb][jb][4 * q4 + 1],
                                                          acc[rb][jb][4 * q4 + 2], acc[rb][jb][4 * q4 + 3]};
    }
    __syncthreads();
    if (kpi == 0) {
#pragma unroll
      for (int q = 1; q < KPW; ++q)
#pragma unroll
        for (int rb = 0; rb < R32; ++rb)
#pragma unroll
          for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 v = at(q, (rb * kWideJB + jb) * 4 + q4);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[rb][jb][4 * q4 + e] += v[e];
            }
    }
  }

  // ---- epilogue (K-part 0): element i of lane l is row 8*(i/4) + 4*hh + i%4 of the 32-row
  // block, column c32 of the 32-column block
  auto store_tile = [&]() {
    f16* C = static_cast<f16*>(p.C);
#pragma unroll
    for (int rb = 0; rb < R32; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rw0 + rb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (r < rows) {
#pragma unroll
          for (int jb = 0; jb < kWideJB; ++jb)
            C[(size_t)(row0 + r) * p.ldc + (bw + 2 * jb) * 16 + c32] = (f16)acc[rb][jb][i];
        }
      }
  };
  if (p.splits == 1) {
    if (kpi == 0) store_tile();
    return;
  }
  // Cross-workgroup split: partials in accumulator order, four 1 KB pieces per
  // (wave, 32-row block, 32-column block), so every access is a coalesced
  // 16-byte device-coherent buffer operation. Region of (split, tile):
  // kWideWaves * R32 * kWideJB * 4 KB.
  constexpr int kFrag = R32 * kWideJB * 4;
  constexpr uint32_t kRegion = WPK * kFrag * 1024;
  const size_t tile_id = (size_t)mt * p.nt + nt;
  const size_t ntiles = (size_t)p.mt * p.nt;
  auto region = [&](int q) {
    return make_rsrc(static_cast<char*>(p.partial) + ((size_t)q * ntiles + tile_id) * kRegion, kRegion);
  };
  auto voff = [&](int rb, int jb, int q4) {
    return (uint32_t)((((wave * R32 + rb) * kWideJB + jb) * 4 + q4) * 1024 + lane * 16);
  };
  if (kpi == 0) {
    const rsrc_t mine = region(split);
#pragma unroll
    for (int rb = 0; rb < R32; ++rb)
#pragma unroll
      for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {acc[rb][jb][4 * q4], acc[rb][jb][4 * q4 + 1], acc[rb][jb][4 * q4 + 2],
                           acc[rb][jb][4 * q4 + 3]};
          store16_coherent(v, mine, voff(rb, jb, q4));
        }
  }
  // every wave takes part in the arrival barriers; only K-part 0 continues
  if (!workgroup_arrive_last(p.counters + tile_id, (uint32_t)p.splits, flag) || kpi > 0) return;
  // last arriver: sum the splits in split order (deterministic), then store fp16
  // (measured faster than prefetching the next split or reusing the own partial
  // from registers, which raise register pressure)
#pragma unroll
  for (int rb = 0; rb < R32; ++rb)
#pragma unroll
    for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][jb][i] = 0.f;
  // kEpi splits' loads in flight at a time (a split past the last re-reads the
  // last and adds nothing); the sum stays in split order. The 16-wave build
  // keeps one at a time to stay within 128 registers.
  constexpr int kEpi = KPW == 1 ? 2 : 1;
  for (int q = 0; q < p.splits; q += kEpi) {
    f32x4 v[kEpi][R32][kWideJB][4];
#pragma unroll
    for (int u = 0; u < kEpi; ++u) {
      const rsrc_t r = region(min(q + u, p.splits - 1));
#pragma unroll
      for (int rb = 0; rb < R32; ++rb)
#pragma unroll
        for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) v[u][rb][jb][q4] = load16_coherent(r, voff(rb, jb, q4));
    }
#pragma unroll
    for (int u = 0; u < kEpi; ++u) {
      const bool has = q + u < p.splits;
#pragma unroll
      for (int rb = 0; rb < R32; ++rb)
#pragma unroll
        for (int jb = 0; jb < kWideJB; ++jb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (has) acc[rb][jb][4 * q4 + e] += v[u][rb][jb][q4][e];
    }
  }
  store_tile();
}

__global__ void __launch_bounds__(512) w4a16_wide_m64(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 8, 1>(p, lds, &flag);   // eight column waves of 32 columns
}

// the same tile with two K-parts of eight waves (four waves per SIMD)
__global__ void __launch_bounds__(1024) w4a16_wide_m64_kp2(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 8, 2>(p, lds, &flag);
}

// 64 x 128 tiles: two K-parts of four 32-column waves (two waves per SIMD),
// for layers where 256-column tiles would need more k-splits
__global__ void __launch_bounds__(512) w4a16_wide_m64_n128(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 4, 2, kWideW4A16, 4, 128>(p, lds, &flag);
}

// the general grid with fp16 activations (WF: the entry layout)
template <int WF>
__global__ void __launch_bounds__(512) w4g_wide_m64(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 8, 1, WF>(p, lds, &flag);
}
template <int WF>
__global__ void __launch_bounds__(1024) w4g_wide_m64_kp2(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 8, 2, WF>(p, lds, &flag);
}
template <int WF>
__global__ void __launch_bounds__(512) w4g_wide_m64_n128(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4, 4, 2, WF, 4, 128>(p, lds, &flag);
}



namespace {

// KPW K-parts of eight waves; the LDS size is fixed per kernel: opt in to it
// (above 64 KiB) once per kernel and device
template <int KPW, int WPK = kWideWaves>
hipError_t launch_wide_k(void (*kernel)(GemmArgs), int mbw, const Plan& pl, const GemmArgs& a, hipStream_t s) {
  static_assert(kASlots == kWideSlots, "the planner sizes the LDS ring");
  const size_t lds = wide_lds_bytes(pl);
  if (lds != (size_t)KPW * kASlots * mbw * 4 * 1024) return hipErrorInvalidValue;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;   // (kernel, device) pairs opted in
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    const void* key = reinterpret_cast<const void*>(kernel);
    std::lock_guard<std::mutex> lk(mu);
    if (!done.count({key, dev})) {
      e = hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      done.insert({key, dev});
    }
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)pl.workgroups), dim3(kWave * WPK * KPW), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16_wide(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  if (pl.mb != 4) return hipErrorInvalidValue;
  if (pl.nb == 2) return pl.wpt == 8 ? launch_wide_k<2, 4>(w4a16_wide_m64_n128, 4, pl, a, s) : hipErrorInvalidValue;
  if (pl.nb != 4) return hipErrorInvalidValue;
  switch (pl.wpt) {
    case 8: return launch_wide_k<1>(w4a16_wide_m64, 4, pl, a, s);
    case 16: return launch_wide_k<2>(w4a16_wide_m64_kp2, 4, pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

namespace {
template <int WF>
hipError_t launch_w4g_wide_f(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  if (pl.nb == 2) return pl.wpt == 8 ? launch_wide_k<2, 4>(w4g_wide_m64_n128<WF>, 4, pl, a, s) : hipErrorInvalidValue;
  if (pl.nb != 4) return hipErrorInvalidValue;
  if (pl.wpt == 8) return launch_wide_k<1>(w4g_wide_m64<WF>, 4, pl, a, s);
  if (pl.wpt == 16) return launch_wide_k<2>(w4g_wide_m64_kp2<WF>, 4, pl, a, s);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_w4g_wide(const Plan& pl, const GemmArgs& a, bool zeros, hipStream_t s) {
  if (pl.mb != 4 || (a.gs != 64 && a.gs % 128 != 0)) return hipErrorInvalidValue;
  if (a.gs == 64) return zeros ? launch_w4g_wide_f<kWideGrid64Z>(pl, a, s) : launch_w4g_wide_f<kWideGrid64>(pl, a, s);
  return zeros ? launch_w4g_wide_f<kWideGridZ>(pl, a, s) : launch_w4g_wide_f<kWideGrid>(pl, a, s);
}

}  // namespace qg
