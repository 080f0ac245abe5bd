// Mixed 2/4-bit policy of the streaming GEMM (the "Enabling Fast 2-bit LLM on
// GPUs" page: only a small fraction of large-range groups keep 4-bit codes,
// stored with memory alignment in mind; dequantization overlapped with loads).
//
// Split-plane format: every group streams a dense 2-bit base plane (512 B per
// 16 columns x 128 k, one coalesced 8-byte-per-lane wave load in the same operand
// order as W4A16); the upper two bits of 4-bit groups live in a separate high
// plane of 32-byte pieces found through a per-chunk descriptor
// (slot offset, 16-bit column mask) that the workgroup stages in LDS. A lane of
// a 4-bit group loads its 8-byte quarter of the piece; the others issue the same
// load out of the resource's range and read zeros (a fixed number of memory
// operations per group keeps the driver's counted waits exact).
// Each lane then rebuilds 4-bit nibble words
//   nib_2s   = (base_s & 0x33333333) | ((high_s << 2) & 0xCCCCCCCC)
//   nib_2s+1 = ((base_s >> 2) & 0x33333333) | (high_s & 0xCCCCCCCC)
// (high = 0 for 2-bit groups) and runs the W4A16 dequantization with a per-lane
// zero point, 8 (4-bit) or 2 (2-bit): no branch on the group precision.
#include "skinny.h"

namespace qg {
namespace fmt {

struct PolicyW2W4 : Tile16 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;
  static constexpr int kFrag = 4;
  static constexpr int kAElem = 2;
  static constexpr bool kStageScales = true;   // the tile's group scales live in LDS
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows16::dma_voff(fr, lane, rows, arow);
  }

  struct Consts {
    f16x2 lo4 = splat_h2(-1032.0f), hi4 = splat_h2(-72.0f);   // zero point 8
    f16x2 lo2 = splat_h2(-1026.0f), hi2 = splat_h2(-66.0f);   // zero point 2
    uint32_t magic = 0x64006400u;
  };

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = 2 * NBW;   // base plane + high plane loads
    static constexpr int kVmemFirst = NBW;  // load_vmem: the base plane only
    u32x2 base[NBW];
    u32x2 high[NBW];
    uint32_t is4[NBW];
    uint32_t s[NBW];
  };

  // descriptors of the workgroup's chunks, [groups of the split][NB], by
  // direct loads: row i is the NB consecutive descriptors of group G0 + i
  // (NB * 8 bytes, whole 16-byte pieces)
  static constexpr bool kStageExtra = true;
  __host__ __device__ static int extra_lds(int NB, int ng, int) { return NB * ng * 8; }
  __device__ static void stage_extra(const GemmArgs& p, char* dst, const TileInfo& ti, int NB, int wave,
                                     int nwaves, int lane) {
    const int ng = ti.G1 - ti.G0;
    const int ppr = NB / 2;                         // 16-byte pieces per row
    const uint32_t srow = (uint32_t)(p.N / 16) * 8u;
    const rsrc_t r = make_rsrc(static_cast<const char*>(p.aux) + (size_t)ti.G0 * srow + (size_t)ti.b0 * 8,
                               (uint32_t)(ng - 1) * srow + (uint32_t)NB * 8u);
    dma16(r, dst, ng * ppr, [&](int q) {
      const int i = q / ppr;
      return (uint32_t)i * srow + (uint32_t)(q - i * ppr) * 16u;
    }, wave, nwaves, lane);
  }

  template <int NBW>
  struct View {
    rsrc_t rb, rh;
    uint32_t bvoff, gstep;
    const char* sl;
    const u32x2* desc;   // this wave's first block in the [ngw][NB] LDS table
    uint32_t sblk, below, hoff;
    int gw0, c8, G0, ngw, c;

    __device__ View(const GemmArgs& p, const char* lds, const SkinnyLds& L, const TileInfo& ti, int bw,
                    int gw0_, int nload, int lane)
        : gw0(gw0_), c8(ti.c8), G0(ti.G0), ngw(ti.G1 - ti.G0) {
      c = lane & 15;
      const uint32_t nbt = (uint32_t)(p.N / 16);
      gstep = nbt * 512u;
      bvoff = lane * 8u;
      rb = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 512,
                     (uint32_t)(nload - 1) * gstep + NBW * 512u);
      // High-plane slots come from the blob's own descriptors; lanes of 2-bit
      // groups address past the resource's size and read zeros.
      rh = make_rsrc(p.high, 0x7FFFFFF0u);
      sblk = ti.n8 * kScaleChunk;
      sl = lds + (bw - ti.b0) * sblk + c * 16;
      desc = reinterpret_cast<const u32x2*>(lds + L.extra_off) + (bw - ti.b0);
      below = (1u << c) - 1u;
      hoff = (lane >> 4) * 8u;
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.base[j] = load8_stream(rb, bvoff + oob, j * 512u + rel * gstep);
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>& st, int rel, uint32_t oob) const {
      const int g = gw0 + rel;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const u32x2 d = desc[(g - G0) * (4 * NBW) + j];
        const uint32_t is4 = (d[1] >> c) & 1u;
        const uint32_t off = (is4 && !oob) ? (d[0] + __builtin_popcount(d[1] & below)) * 32u + hoff : 0x7FFFFFF8u;
        st.high[j] = load8_stream(rh, off, 0);
        st.is4[j] = is4;
      }
      const int off = ((g >> 3) - c8) * kScaleChunk + (g & 7) * 2;
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.s[j] = *reinterpret_cast<const uint16_t*>(sl + j * sblk + off);
    }
  };

  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts& k, int lane) {
    f16x8 bf[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const f16x2 lo_off = cur.is4[j] ? k.lo4 : k.lo2;
      const f16x2 hi_off = cur.is4[j] ? k.hi4 : k.hi2;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t B = cur.base[j][s], H = cur.high[j][s];
        const uint32_t n0 = and_or(H << 2, 0xCCCCCCCCu, B & 0x33333333u);
        const uint32_t n1 = and_or(H, 0xCCCCCCCCu, (B >> 2) & 0x33333333u);
        bf[j][2 * s] = dequant_u4x8(n0, lo_off, hi_off, k.magic);
        bf[j][2 * s + 1] = dequant_u4x8(n1, lo_off, hi_off, k.magic);
      }
    }
    f16x8 a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[mb][t] = *reinterpret_cast<const f16x8*>(ARows16::at(aslot, mb * 16 + (lane & 15), 4 * t + (lane >> 4)));
    // the blocks' accumulation chains interleaved step by step (independent
    // consecutive MFMAs), as in the W4A16 policy
    f32x4 part[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NBW; ++j) part[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          part[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb][t], bf[j][t], part[mb][j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const float sc = valid ? half_of(cur.s[j], 0) : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][j] += sc * part[mb][j];
    }
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, float v) {
    static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)v;
  }
};

}  // namespace fmt

using namespace fmt;

size_t lds_bytes_w2w4(const Plan& pl, int G) { return skinny_lds_bytes<PolicyW2W4>(pl, G); }

hipError_t launch_w2w4(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  return dispatch_skinny<PolicyW2W4>(pl, a, s);
}

}  // namespace qg
