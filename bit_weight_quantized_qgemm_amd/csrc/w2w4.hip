// Mixed 2/4-bit policy of the streaming GEMM (the "Enabling Fast 2-bit LLM on
// GPUs" page: only a small fraction of large-range groups keep 4-bit codes,
// stored with memory alignment in mind; dequantization overlapped with loads).
//
// Split-plane format: every group streams a dense 2-bit base plane (512 B per
// 16 columns x 128 k, one coalesced 8-byte-per-lane wave load in the same operand
// order as W4A16); the upper two bits of 4-bit groups live in a separate high
// plane of 32-byte pieces found through a per-chunk descriptor
// (slot offset, 16-bit column mask) that the workgroup stages in LDS. A lane of
// a 4-bit group loads its 8-byte quarter of the piece; the others load nothing.
// Each lane then rebuilds 4-bit nibble words
//   nib_2s   = (base_s & 0x33333333) | ((high_s << 2) & 0xCCCCCCCC)
//   nib_2s+1 = ((base_s >> 2) & 0x33333333) | (high_s & 0xCCCCCCCC)
// (high = 0 for 2-bit groups) and runs the W4A16 dequantization with a per-lane
// zero point, 8 (4-bit) or 2 (2-bit): no branch on the group precision.
#include "skinny.h"

namespace qg {
namespace {

struct PolicyW2W4 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;
  static constexpr int kDepth = 2;

  struct Consts {
    f16x2 lo4 = splat_h2(-1032.0f), hi4 = splat_h2(-72.0f);   // zero point 8
    f16x2 lo2 = splat_h2(-1026.0f), hi2 = splat_h2(-66.0f);   // zero point 2
    uint32_t magic = 0x64006400u;
  };

  template <int MB, int NB>
  struct Stage {
    u32x2 base[NB];
    u32x2 high[NB];
    uint32_t is4[NB];
    u32x4 a[MB][4];
    uint32_t s[NB];
  };

  // descriptors of the workgroup's chunks, [NB][groups of the split], after the scales
  static size_t extra_lds(const Plan& pl) { return (size_t)pl.nb * pl.gps * 8 + 16; }
  static __device__ __forceinline__ size_t desc_offset(const TileInfo& ti, int NB) {
    return (size_t)NB * ti.n8 * kScaleChunk;
  }
  __device__ static void stage_extra(const GemmArgs& p, char* lds, const TileInfo& ti, int NB) {
    u32x2* dst = reinterpret_cast<u32x2*>(lds + desc_offset(ti, NB));
    const u32x2* src = static_cast<const u32x2*>(p.aux);
    const int ng = ti.G1 - ti.G0;
    for (int t = threadIdx.x; t < NB * ng; t += blockDim.x) {
      const int j = t / ng, i = t % ng;
      dst[t] = src[(size_t)(ti.b0 + j) * p.G + ti.G0 + i];
    }
  }

  template <int MB, int NB>
  struct View {
    rsrc_t rb, rh, ra;
    uint32_t bvoff, bblk;
    uint32_t avoff[MB];
    const char* sl;
    const u32x2* desc;   // [NB][ngw] in LDS
    uint32_t sblk, below, hoff;
    int gw0, c8, G0, ngw, c;

    __device__ View(const GemmArgs& p, const char* lds, const TileInfo& ti, int gw0_, int ng, int lane)
        : gw0(gw0_), c8(ti.c8), G0(ti.G0), ngw(ti.G1 - ti.G0) {
      c = lane & 15;
      const int h = lane >> 4;
      bblk = (uint32_t)p.G * 512u;
      bvoff = lane * 8u;
      rb = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)ti.b0 * p.G + gw0) * 512,
                     (NB - 1) * bblk + ng * 512u);
      rh = make_rsrc(p.high, 0x7FFFFFF0u);   // offsets come from the blob's own descriptors
      ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)ti.row0 * p.lda + (size_t)gw0 * kGroup,
                     (uint32_t)(((size_t)(ti.rows - 1) * p.lda + (size_t)ng * kGroup) * 2));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        avoff[mb] = (uint32_t)((size_t)min(mb * 16 + c, ti.rows - 1) * p.lda * 2 + h * 16);
      sblk = ti.n8 * kScaleChunk;
      sl = lds + c * 16;
      desc = reinterpret_cast<const u32x2*>(lds + desc_offset(ti, NB));
      below = (1u << c) - 1u;
      hoff = h * 8u;
    }
    __device__ __forceinline__ void load(Stage<MB, NB>& st, int rel) const {
      const int g = gw0 + rel;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        st.base[j] = load8(rb, bvoff, j * bblk + rel * 512u);
        const u32x2 d = desc[j * ngw + (g - G0)];
        const uint32_t is4 = (d[1] >> c) & 1u;
        u32x2 hv = {0u, 0u};
        if (is4) hv = load8(rh, (d[0] + __builtin_popcount(d[1] & below)) * 32u + hoff, 0);
        st.high[j] = hv;
        st.is4[j] = is4;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t) st.a[mb][t] = load16(ra, avoff[mb], rel * 256u + t * 64u);
      const int off = ((g >> 3) - c8) * kScaleChunk + (g & 7) * 2;
#pragma unroll
      for (int j = 0; j < NB; ++j) st.s[j] = *reinterpret_cast<const uint16_t*>(sl + j * sblk + off);
    }
  };

  template <int MB, int NB>
  __device__ __forceinline__ static void compute(const Stage<MB, NB>& cur, Acc (&acc)[MB][NB],
                                                 bool valid, const Consts& k, int) {
    f16x8 bf[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
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
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float sc = valid ? half_of(cur.s[j], 0) : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          part = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(cur.a[mb][t]), bf[j][t], part, 0, 0, 0);
        acc[mb][j] += sc * part;
      }
    }
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, float v) {
    static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)v;
  }
};

}  // namespace

size_t lds_bytes_w2w4(const Plan& pl, int G) { return skinny_lds_bytes<PolicyW2W4>(pl, G); }

hipError_t launch_w2w4(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  return dispatch_skinny<PolicyW2W4>(pl, a, s);
}

}  // namespace qg
