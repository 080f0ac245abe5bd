// W4A16 policy of the streaming GEMM: C[M,N] = A[M,K] (fp16) * dequant(W)[K,N],
// W = (q - 8) * s with 4-bit codes q and one fp16 scale per 128 k of a column.
//
// Per group and lane: one 16-byte weight load per 16-column block (the blob is in
// v_mfma_f32_16x16x32_f16 B-operand order, one fully coalesced 1 KB wave load),
// four 16-byte activation loads per 16-row block, and the lane's group scale
// from LDS. Dequantization: 9 VALU ops per 8 weights produce exact fp16 (q - 8)
// (dequant_u4x8); the fp32 MFMA partial of the group is scaled once
// (acc += s * partial), so the result is sum_g s[g,n] * sum_k A[m,k] (q[k,n] - 8)
// with fp32 accumulation and a single rounding of each output to fp16.
#include "skinny.h"

namespace qg {
namespace {

struct PolicyW4A16 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;   // 16 columns x 8 groups x fp16
  static constexpr int kDepth = 2;

  struct Consts {
    f16x2 lo_off = splat_h2(-1032.0f);   // -(1024 + 8)
    f16x2 hi_off = splat_h2(-72.0f);     // -(64 + 8)
    uint32_t magic = 0x64006400u;
  };

  template <int MB, int NB>
  struct Stage {
    u32x4 code[NB];
    u32x4 a[MB][4];
    uint32_t s[NB];   // fp16 scale bits in the low half
  };

  static size_t extra_lds(const Plan&) { return 0; }
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int) {}

  template <int MB, int NB>
  struct View {
    rsrc_t rc, ra;
    uint32_t cvoff, cblk;
    uint32_t avoff[MB];
    const char* sl;      // this lane's scale column in LDS
    uint32_t sblk;       // LDS bytes per column block
    int gw0, c8;

    __device__ View(const GemmArgs& p, const char* lds, const TileInfo& ti, int gw0_, int ng, int lane)
        : gw0(gw0_), c8(ti.c8) {
      const int c = lane & 15, h = lane >> 4;
      cblk = (uint32_t)p.G * 1024u;
      cvoff = lane * 16u;
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)ti.b0 * p.G + gw0) * 1024,
                     (NB - 1) * cblk + ng * 1024u);
      // Rows beyond M read a valid row: MFMA output row r depends only on A row r,
      // and those rows are never stored.
      ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)ti.row0 * p.lda + (size_t)gw0 * kGroup,
                     (uint32_t)(((size_t)(ti.rows - 1) * p.lda + (size_t)ng * kGroup) * 2));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        avoff[mb] = (uint32_t)((size_t)min(mb * 16 + c, ti.rows - 1) * p.lda * 2 + h * 16);
      sblk = ti.n8 * kScaleChunk;
      sl = lds + c * 16;
    }
    __device__ __forceinline__ void load(Stage<MB, NB>& st, int rel) const {
#pragma unroll
      for (int j = 0; j < NB; ++j) st.code[j] = load16(rc, cvoff, j * cblk + rel * 1024u);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t) st.a[mb][t] = load16(ra, avoff[mb], rel * 256u + t * 64u);
      const int g = gw0 + rel;
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
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) bf[j][t] = dequant_u4x8(cur.code[j][t], k.lo_off, k.hi_off, k.magic);
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

size_t lds_bytes_w4a16(const Plan& pl, int G) { return skinny_lds_bytes<PolicyW4A16>(pl, G); }

hipError_t launch_w4a16(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  return dispatch_skinny<PolicyW4A16>(pl, a, s);
}

}  // namespace qg
