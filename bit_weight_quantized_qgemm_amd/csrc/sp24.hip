// 2:4 structured-sparse W4A16 on the gfx950 sparse matrix instruction (the
// MARLIN abstract extends its kernel to 2:4 sparsity for further speedups):
// at most two of every four consecutive weights along K of a column are
// nonzero, W = (q - 8) * s on the kept ones. The blob keeps only the two kept
// codes of each quad plus a 2-bit position per kept code: 3 bits per weight of
// codes and metadata instead of 4.
//
// v_smfmac_f32_16x16x64_f16 takes its SPARSE operand as the A side (rows x
// 64 k, half of each quad present), so the kernel computes the transposed
// product C^T = W^T A^T: the sparse operand is W^T (16 output columns n x 64 k)
// and the dense operand is A^T (64 k x 16 rows m). Operand geometry on gfx950
// (checked on the device with random integer operands against a CPU model):
//   * sparse: lane l holds row n = l % 16 and kept values v = 0..7 of the quads
//     4*(l/16) + v/2 of the 64-k step (k = 16*(l/16) + 4*(v/2) + position);
//   * positions: 2 bits per kept value v at bits 2v, 2v+1 of the index
//     register's 16-bit half selected by the instruction's ABID field;
//   * dense: lane l holds column m = l % 16 and k = 8*(l/16) + e for elements
//     e = 0..7 and 32 + 8*(l/16) + e - 8 for e = 8..15, i.e. the A fragments of
//     two consecutive 32-k steps of the dense 16x16x32 instruction, so the
//     activation ring of the streaming driver serves unchanged;
//   * result: lane l holds rows n = 4*(l/16) + i, column m = l % 16.
// Per 128-k chunk and 16 columns a lane makes one 12-byte load: two code words
// (the two steps' kept codes in the W4A16 nibble order, dequantized exactly to
// q - 8 by the same bit trick) and a position word (step 0 in the low half,
// step 1 in the high half, selected by ABID); codes and positions share one
// stream through the blob. The chunk's fp32 partial of each output is scaled
// once by the scale of its column n = 4*(l/16) + i.
#include "skinny.h"

namespace qg {
namespace fmt {

typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

struct PolicySP24 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 256;   // 16 columns x 8 groups x fp16 (as W4A16)
  static constexpr int kFrag = 4;           // 1 KB activation loads per 16 rows and chunk
  static constexpr int kAElem = 2;
  static constexpr bool kStageScales = true;
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows16::dma_voff(fr, lane, rows, arow);
  }
  // transposed result: element i of lane ln is column 4*(ln/16) + i, row ln % 16
  __device__ static int row_of(int mb, int, int, int ln) { return mb * 16 + (ln & 15); }
  __device__ static int col_of(int, int j, int i, int ln) { return j * 16 + 4 * (ln >> 4) + i; }

  struct Consts {
    f16x2 lo_off = splat_h2(-1032.0f);   // -(1024 + 8)
    f16x2 hi_off = splat_h2(-72.0f);     // -(64 + 8)
    uint32_t magic = 0x64006400u;
  };

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = NBW;       // one 12-byte load per column block
    static constexpr int kVmemFirst = NBW;
    u32x3 rec[NBW];                         // code words 0, 1 and the position word
    uint32_t s[NBW][2];                     // fp16 scales of columns 4h .. 4h+3 (pairs)
  };

  __host__ __device__ static int extra_lds(int, int, int) { return 0; }
  static constexpr bool kStageExtra = false;
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int, int, int, int) {}

  template <int NBW>
  struct View {
    rsrc_t rc;
    uint32_t gstep;
    const char* sl;      // scale of column 4h of the wave's first block in LDS
    uint32_t sblk;
    int gw0, c8, lane;

    __device__ View(const GemmArgs& p, const char* lds, const SkinnyLds&, const TileInfo& ti, int bw,
                    int gw0_, int nload, int lane_)
        : gw0(gw0_), c8(ti.c8), lane(lane_) {
      const uint32_t nbt = (uint32_t)(p.N / 16);
      gstep = nbt * 768u;
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 768,
                     (uint32_t)(nload - 1) * gstep + NBW * 768u);
      sblk = ti.n8 * kScaleChunk;
      sl = lds + (bw - ti.b0) * sblk + 4 * (lane >> 4) * 16;
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        st.rec[j] = __builtin_bit_cast(
            u32x3, __builtin_amdgcn_raw_buffer_load_b96(rc, lane * 12u + oob, j * 768u + rel * gstep, kStreamPolicy));
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>& st, int rel, uint32_t) const {
      const int g = gw0 + rel;
      const int off = ((g >> 3) - c8) * kScaleChunk + (g & 7) * 2;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const char* b = sl + j * sblk + off;
        const uint32_t s0 = *reinterpret_cast<const uint16_t*>(b);
        const uint32_t s1 = *reinterpret_cast<const uint16_t*>(b + 16);
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(b + 32);
        const uint32_t s3 = *reinterpret_cast<const uint16_t*>(b + 48);
        st.s[j][0] = s0 | (s1 << 16);
        st.s[j][1] = s2 | (s3 << 16);
      }
    }
  };

  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts& k, int lane) {
    f16x16 a[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r = mb * 16 + (lane & 15);
        const f16x8 lo = *reinterpret_cast<const f16x8*>(ARows16::at(aslot, r, 8 * st + (lane >> 4)));
        const f16x8 hi = *reinterpret_cast<const f16x8*>(ARows16::at(aslot, r, 8 * st + 4 + (lane >> 4)));
        a[mb][st] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const u32x3 r = cur.rec[j];
      const uint32_t c0 = r[0], c1 = r[1], pos = r[2];   // scalars first (vector-element reads)
      const f16x8 w0 = dequant_u4x8(c0, k.lo_off, k.hi_off, k.magic);
      const f16x8 w1 = dequant_u4x8(c1, k.lo_off, k.hi_off, k.magic);
      const int idx = (int)pos;
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = valid ? half_of(cur.s[j][i >> 1], i & 1) : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
        part = __builtin_amdgcn_smfmac_f32_16x16x64_f16(w0, a[mb][0], part, idx, 0, 0);
        part = __builtin_amdgcn_smfmac_f32_16x16x64_f16(w1, a[mb][1], part, idx, 0, 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][j][i] += sc[i] * part[i];
      }
    }
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, float v) {
    static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)v;
  }
};

}  // namespace fmt

using namespace fmt;

size_t lds_bytes_sp24(const Plan& pl, int G) { return skinny_lds_bytes<PolicySP24>(pl, G); }

hipError_t launch_sp24(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  return dispatch_skinny<PolicySP24>(pl, a, s);
}

}  // namespace qg
