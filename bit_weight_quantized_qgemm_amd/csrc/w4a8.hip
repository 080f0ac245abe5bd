// W4A8 policy of the streaming GEMM (the W4A8 setting of the OdysseyLLM /
// FastGEMM abstract): int8 activations with a per-row fp16 scale, signed int4
// weights with an int8 scale per group of 128 k and an fp16 scale per column.
//
//   acc[m,n] = sum_g s_g[g,n] * sum_{k in g} A[m,k] * q[k,n]     (exact int32)
//   C[m,n]   = fp16(float(acc) * a_scale[m] * s_c[n])
//
// The blob stores u = q + 8 (0..15), so one AND (plus one shift+AND) turns a
// word into eight int8 v_mfma_i32_16x16x64_i8 operand bytes with no sign work;
// the offset is removed exactly per group with the row sums of A,
//   sum_k A*q = sum_k A*u - 8 * sum_k A,
// taken from one extra MFMA against a matrix of ones per 16-row block and group
// (shared by every column block of the wave). The group scale multiplies the
// exact per-group partial with v_mul_i32_i24 (|partial| < 2^18, |s_g| <= 128).
// Split partial sums are int32, so the result is exact in any order.
#include "skinny.h"

namespace qg {
namespace fmt {

struct PolicyW4A8 : Tile16 {
  using Acc = i32x4;
  using Elem = int32_t;
  static constexpr int kScaleChunk = 128;   // 16 columns x 8 groups x int8
  static constexpr int kFrag = 2;           // 1 KB activation loads per 16 rows and group
  static constexpr int kAElem = 1;
  static constexpr bool kStageScales = true;   // the tile's group scales live in LDS
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows8::dma_voff(fr, lane, rows, arow);
  }

  struct Consts {};

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = NBW;
    static constexpr int kVmemFirst = NBW;
    u32x4 code[NBW];
    int32_t s[NBW];
  };

  __host__ __device__ static int extra_lds(int, int, int) { return 0; }
  static constexpr bool kStageExtra = false;
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int, int, int, int) {}

  template <int NBW>
  struct View {
    rsrc_t rc;
    uint32_t cvoff, gstep;   // gstep: bytes from a group's chunk to the next group's
    const char* sl;
    uint32_t sblk;
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
      sl = lds + (bw - ti.b0) * sblk + (lane & 15) * 8;
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.code[j] = load16_stream(rc, cvoff + oob, j * 1024u + rel * gstep);
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>& st, int rel, uint32_t) const {
      const int g = gw0 + rel;
      const int off = ((g >> 3) - c8) * kScaleChunk + (g & 7);
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.s[j] = *reinterpret_cast<const int8_t*>(sl + j * sblk + off);
    }
  };

  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts&, int lane) {
    const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const i32x4 zero = {0, 0, 0, 0};
    i32x4 a[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        a[mb][u] = *reinterpret_cast<const i32x4*>(ARows8::at(aslot, mb * 16 + (lane & 15), 4 * u + (lane >> 4)));
    i32x4 rsum[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      rsum[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][0], ones, zero, 0, 0, 0);
      rsum[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][1], ones, rsum[mb], 0, 0, 0);
    }
    i32x4 b[NBW][2];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const u32x4 w = cur.code[j];
      b[j][0] = i32x4{(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu),
                      (int)(w[1] & 0x0F0F0F0Fu), (int)((w[1] >> 4) & 0x0F0F0F0Fu)};
      b[j][1] = i32x4{(int)(w[2] & 0x0F0F0F0Fu), (int)((w[2] >> 4) & 0x0F0F0F0Fu),
                      (int)(w[3] & 0x0F0F0F0Fu), (int)((w[3] >> 4) & 0x0F0F0F0Fu)};
    }
    // the blocks' two-step chains interleaved (independent consecutive MFMAs)
    i32x4 part[MB][NBW];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          part[mb][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][u], b[j][u], u ? part[mb][j] : zero, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int sg = valid ? cur.s[j] : 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int corr = part[mb][j][r] - 8 * rsum[mb][r];   // sum_{k in g} A * q, |.| < 2^18
          acc[mb][j][r] += __builtin_amdgcn_sbfe(corr, 0, 24) * sg;
        }
    }
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, int32_t v) {
    if (p.acc_out) p.acc_out[(size_t)row * p.N + col] = v;
    const float as = (float)static_cast<const f16*>(p.a_scale)[row];
    const float sc = (float)static_cast<const f16*>(p.aux)[col];
    static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)((float)v * as * sc);
  }
};

}  // namespace fmt

using namespace fmt;

size_t lds_bytes_w4a8(const Plan& pl, int G) { return skinny_lds_bytes<PolicyW4A8>(pl, G); }

hipError_t launch_w4a8(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  return dispatch_skinny<PolicyW4A8>(pl, a, s);
}

}  // namespace qg
