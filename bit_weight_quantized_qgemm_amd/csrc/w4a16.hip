// W4A16 policy of the streaming GEMM: C[M,N] = A[M,K] (fp16) * dequant(W)[K,N],
// W = (q - 8) * s with 4-bit codes q and one fp16 scale per 128 k of a column.
//
// Per group and lane: one 16-byte weight load per 16-column block (the blob is in
// v_mfma_f32_16x16x32_f16 B-operand order, one fully coalesced 1 KB wave load),
// the four A operands per 16-row block from the workgroup's LDS ring, and the
// lane's group scale from LDS. Dequantization: 9 VALU ops per 8 weights produce exact fp16 (q - 8)
// (dequant_u4x8); the fp32 MFMA partial of the group is scaled once
// (acc += s * partial), so the result is sum_g s[g,n] * sum_k A[m,k] (q[k,n] - 8)
// with fp32 accumulation and a single rounding of each output to fp16.
#include "skinny.h"

namespace qg {
namespace fmt {

struct PolicyW4A16 : Tile16 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;   // 16 columns x 8 groups x fp16
  static constexpr int kFrag = 4;           // 1 KB activation loads per 16 rows and group
  static constexpr int kAElem = 2;          // bytes per activation
  static constexpr bool kStageScales = true;   // the tile's group scales live in LDS
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows16::dma_voff(fr, lane, rows, arow);
  }

  struct Consts {
    f16x2 lo_off = splat_h2(-1032.0f);   // -(1024 + 8)
    f16x2 hi_off = splat_h2(-72.0f);     // -(64 + 8)
    uint32_t magic = 0x64006400u;
  };

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = NBW;   // vector memory operations per stage
    static constexpr int kVmemFirst = NBW;   // ... issued by load_vmem
    u32x4 code[NBW];
    uint32_t s[NBW];                    // fp16 scale bits in the low half
  };

  static constexpr bool kStageExtra = false;
  __host__ __device__ static int extra_lds(int, int, int) { return 0; }
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int, int, int, int) {}

  template <int NBW>
  struct View {
    rsrc_t rc;
    uint32_t cvoff, gstep;   // gstep: bytes from a group's chunk to the next group's
    const char* sl;      // this lane's scale column of the wave's first block in LDS
    uint32_t sblk;       // LDS bytes per column block
    int gw0, c8;

    __device__ View(const GemmArgs& p, const char* lds, const SkinnyLds&, const TileInfo& ti, int bw,
                    int gw0_, int nload, int lane)
        : gw0(gw0_), c8(ti.c8) {
      const uint32_t nbt = (uint32_t)(p.N / 16);
      gstep = nbt * 1024u;
      cvoff = lane * 16u;
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 1024,
                     (uint32_t)(nload - 1) * gstep + NBW * 1024u);
      sblk = ti.n8 * kScaleChunk;
      sl = lds + (bw - ti.b0) * sblk + (lane & 15) * 16;
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.code[j] = load16_stream(rc, cvoff + oob, j * 1024u + rel * gstep);
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>& st, int rel, uint32_t) const {
      const int g = gw0 + rel;
      const int off = ((g >> 3) - c8) * kScaleChunk + (g & 7) * 2;
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.s[j] = *reinterpret_cast<const uint16_t*>(sl + j * sblk + off);
    }
  };

  // one group: exact fp16 (q - 8) weights, fp32 MFMA partial per 16x16 block,
  // scaled once in fp32
  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts& k, int lane) {
    f16x8 bf[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) bf[j][t] = dequant_u4x8(cur.code[j][t], k.lo_off, k.hi_off, k.magic);
    f16x8 a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[mb][t] = *reinterpret_cast<const f16x8*>(ARows16::at(aslot, mb * 16 + (lane & 15), 4 * t + (lane >> 4)));
    // the blocks' accumulation chains interleaved step by step, so consecutive
    // MFMAs are independent (measured on MI355X: 2-6 % at M = 8-16; splitting a
    // single block's steps over two partials, or the 32-row tile's, was slower)
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

// The 32-row x 32-column wave tile (MB = 2, NBW = 2) on v_mfma_f32_32x32x16_f16,
// which sustains about twice the rate of the 16x16x32 form on gfx950. Operand
// geometry: lane l holds A row / B column l % 32 and k = 8*(l/32) .. +7 of each
// 16-k step; result element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
// column l % 32. The blob keeps its 16-column chunks: the B operand of k-step u
// is word u/2 of blob lane 16*(2*(u%2) + l/32) + l%16 of chunk (l%32)/16, so
// each lane loads two 16-byte pieces per group (even and odd k-steps). The A
// operand of k-step u is read from the slot's whole rows (ARows16).
// The accumulator's four quarters stand in for the (mb, j) fragments of the
// shared driver.
struct PolicyW4A16M32 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;
  static constexpr int kFrag = 4;           // 2 x 4 = 8 loads of 4 whole rows per group
  static constexpr int kAElem = 2;
  // Each lane loads its own column's group scale with the weights: staging all
  // of a tall tile's scales in LDS would cost occupancy on long K ranges.
  static constexpr bool kStageScales = false;
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave

  typedef float f32x16 __attribute__((ext_vector_type(16)));

  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows16::dma_voff(fr, lane, rows, arow);
  }
  __device__ static int row_of(int mb, int j, int i, int ln) { return 8 * (mb * 2 + j) + 4 * (ln >> 5) + i; }
  __device__ static int col_of(int, int, int, int ln) { return ln & 31; }

  using Consts = PolicyW4A16::Consts;

  template <int NBW>
  struct Stage {
    static_assert(NBW == 2, "one 32-column block per wave");
    static constexpr int kVmem = 3;
    static constexpr int kVmemFirst = 3;
    u32x4 even, odd;
    uint32_t s;
  };

  static constexpr bool kStageExtra = false;
  __host__ __device__ static int extra_lds(int, int, int) { return 0; }
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int, int, int, int) {}

  template <int NBW>
  struct View {
    rsrc_t rc, rs;
    uint32_t cvoff, gstep, svoff;
    int gw0;

    __device__ View(const GemmArgs& p, const char*, const SkinnyLds&, const TileInfo&, int bw,
                    int gw0_, int nload, int lane)
        : gw0(gw0_) {
      const uint32_t nbt = (uint32_t)(p.N / 16);
      const int c32 = lane & 31;
      gstep = nbt * 1024u;
      cvoff = (uint32_t)((c32 >> 4) * 1024 + (16 * (lane >> 5) + (c32 & 15)) * 16);
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 1024,
                     (uint32_t)(nload - 1) * gstep + 2048u);
      // scales [NB][G8][16][8] fp16: this lane's column c32 of block pair bw, bw + 1
      const uint32_t sblk = (uint32_t)p.G8 * 256u;
      rs = make_rsrc(static_cast<const char*>(p.scales) + (size_t)bw * sblk, 2 * sblk);
      svoff = (uint32_t)((c32 >> 4) * sblk + (c32 & 15) * 16);
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
      st.even = load16_stream(rc, cvoff + oob, rel * gstep);
      st.odd = load16_stream(rc, cvoff + 512u + oob, rel * gstep);
      const int g = gw0 + rel;
      st.s = __builtin_amdgcn_raw_buffer_load_b16(rs, svoff + oob, (uint32_t)(g >> 3) * 256u + (uint32_t)(g & 7) * 2u, 0);
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>&, int, uint32_t) const {}
  };

  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts& k, int lane) {
    static_assert(MB == 2 && NBW == 2, "32 x 32 wave tile");
    f32x16 part;
#pragma unroll
    for (int e = 0; e < 16; ++e) part[e] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(ARows16::at(aslot, lane & 31, 2 * u + (lane >> 5)));
      const f16x8 b = dequant_u4x8((u & 1) ? cur.odd[u >> 1] : cur.even[u >> 1], k.lo_off, k.hi_off, k.magic);
      part = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, part, 0, 0, 0);
    }
    const float sc = valid ? half_of(cur.s, 0) : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q >> 1][q & 1][i] += sc * part[4 * q + i];
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, float v) {
    static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)v;
  }
};

}  // namespace fmt

using namespace fmt;

size_t lds_bytes_w4a16(const Plan& pl, int G) {
  return (pl.mb == 2 && pl.nb == 2) ? skinny_lds_bytes<PolicyW4A16M32>(pl, G) : skinny_lds_bytes<PolicyW4A16>(pl, G);
}

hipError_t launch_w4a16(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  if (pl.mb == 2 && pl.nb == 2) return dispatch_kp<PolicyW4A16M32, 2, 2>(pl, a, s);
  return dispatch_skinny<PolicyW4A16>(pl, a, s);
}

}  // namespace qg
