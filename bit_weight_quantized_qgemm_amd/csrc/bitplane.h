// Bit-plane W_b A8 policy of the streaming GEMM, b = 1..8 (the arbitrary-
// precision Tensor Core page's abstract: a bipolar-INT weight format,
// symmetric, whose matrices are decomposed at the bit level and recovered after
// the products). A b-bit weight is w = sum_i 2^i (2 u_i - 1) = 2U - (2^b - 1)
// with bit planes u_i; activations are int8 with a per-row fp16 scale and each
// column has one fp16 scale:
//
//   acc[m,n] = sum_k A[m,k] * w[k,n]                  (exact int32)
//   C[m,n]   = fp16(float(acc) * a_scale[m] * s_c[n])
//
// The blob stores the planes: per 128-k chunk and 16 columns, lane l holds b
// words, word i carrying bit i of the lane's 32 weights (k = 64u + 16h + j at
// bit 16u + j). gfx950 has no 1-bit matrix instruction, so each plane becomes
// an int8 operand of 0/1 bytes - four bits spread to four bytes by one 24-bit
// multiply and a mask - and goes through v_mfma_i32_16x16x64_i8 on its own:
//   sum_k A w = 2 sum_i 2^i (A . u_i) - (2^b - 1) sum_k A,
// the per-plane products recovered with shifts in int32 and the row sums of A
// from one MFMA against ones per 16-row block. Every
// partial is an exact integer, so split-K partial sums add exactly in any
// order (|acc| <= K * 127 * 255 < 2^31 for K <= 65536).
#pragma once

#include "skinny.h"

namespace qg {
namespace fmt {

template <int B>
struct PolicyBP : Tile16 {
  static_assert(B >= 1 && B <= 8, "1..8 bit planes");
  using Acc = i32x4;
  using Elem = int32_t;
  static constexpr int kScaleChunk = 0;
  static constexpr int kFrag = 2;           // 1 KB activation loads per 16 rows and chunk
  static constexpr int kAElem = 1;
  static constexpr bool kStageScales = false;
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  static constexpr int kLoads = B > 4 ? 2 : 1;  // lane loads per chunk (4*B bytes)
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows8::dma_voff(fr, lane, rows, arow);
  }

  struct Consts {};

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = NBW * kLoads;
    static constexpr int kVmemFirst = NBW * kLoads;
    uint32_t w[NBW][B];
  };

  __host__ __device__ static int extra_lds(int, int, int) { return 0; }
  static constexpr bool kStageExtra = false;
  __device__ static void stage_extra(const GemmArgs&, char*, const TileInfo&, int, int, int, int) {}

  // 4*n bytes at (voff, soff) into w[0..n-1], n = 1..4
  template <int n>
  __device__ __forceinline__ static void load_words(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
    if constexpr (n == 1) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamPolicy);
    } else if constexpr (n == 2) {
      const u32x2 v = load8_stream(r, voff, soff);
      w[0] = v[0];
      w[1] = v[1];
    } else if constexpr (n == 3) {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, kStreamPolicy));
      w[0] = v[0];
      w[1] = v[1];
      w[2] = v[2];
    } else {
      const u32x4 v = load16_stream(r, voff, soff);
      w[0] = v[0];
      w[1] = v[1];
      w[2] = v[2];
      w[3] = v[3];
    }
  }

  template <int NBW>
  struct View {
    rsrc_t rc;
    uint32_t cvoff, gstep;

    __device__ View(const GemmArgs& p, const char*, const SkinnyLds&, const TileInfo&, int bw, int gw0,
                    int nload, int lane) {
      const uint32_t nbt = (uint32_t)(p.N / 16);
      gstep = nbt * 256u * B;
      cvoff = lane * 4u * B;
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 256 * B,
                     (uint32_t)(nload - 1) * gstep + NBW * 256u * B);
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const uint32_t soff = j * 256u * B + rel * gstep;
        load_words<(B > 4 ? 4 : B)>(rc, cvoff + oob, soff, st.w[j]);
        if constexpr (B > 4) load_words<B - 4>(rc, cvoff + 16u + oob, soff, st.w[j] + 4);
      }
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>&, int, uint32_t) const {}
  };

  // bits 4d..4d+3 of x (d = 0..3, counting from bit `off`) -> bytes 0 or 1
  __device__ __forceinline__ static i32x4 plane_bytes(uint32_t x, int off) {
    i32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t n4 = __builtin_amdgcn_ubfe(x, off + 4 * d, 4);
      // bit t of n4 -> bit 8t: the product (a 24-bit multiply: both factors
      // fit) places a copy of bit t at 8t and the others where the mask clears
      r[d] = (int)((n4 * 0x00204081u) & 0x01010101u);
    }
    return r;
  }

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
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      // sum_i 2^i (A . u_i): one product per plane, recovered by shifts
      i32x4 part[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) part[mb] = zero;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const i32x4 b0 = plane_bytes(cur.w[j][i], 0);
        const i32x4 b1 = plane_bytes(cur.w[j][i], 16);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          i32x4 p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][0], b0, zero, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][1], b1, p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) part[mb][r] += p[r] << i;
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // |row sum| <= 128 * 127 fits 24 bits: a full-rate 24-bit multiply
          const int v = 2 * part[mb][r] - __builtin_amdgcn_sbfe(rsum[mb][r], 0, 24) * ((1 << B) - 1);
          acc[mb][j][r] += valid ? v : 0;
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
}  // namespace qg
