// 4-bit weights on a general quantization grid, on the streaming driver:
//   C[M,N] = A[M,K] * W[K,N],  W[k,n] = (q[k,n] - z[g,n]) * s[g,n],  g = k / gs,
// with gs = 64 or a multiple of 128 dividing K (gs = K: one scale per column),
// z a stored 4-bit zero point per (group, column) or the implicit 8, and
// activations, scales and output all fp16 or all bf16. The 2-bit page's
// abstract and the Atom review's method section quantize weights by groups
// without fixing the group length; asymmetric grids store a zero point per
// group.
//
// The codes are the W4A16 blob's 128-k chunks. Each lane needs, per chunk, the
// grid entries of its column: the two 64-k groups of the chunk when gs = 64,
// else the one group that contains it. Two variants fetch them:
//   staged:   the workgroup copies the entries of its columns and k-split into
//             LDS once, up front, and lanes read them from there (per-lane
//             loads of a few bytes next to the 16-byte code loads cost about a
//             third of the run time at small batches on MI355X);
//   per lane: each lane loads them with its codes. Needs no LDS, which keeps
//             more workgroups resident when a k-split spans many groups.
// Every chunk
// is treated as two 64-k halves (k-steps 0-1 and 2-3 of the 16x16x32 MFMA),
// each with its own partial sum and grid entry; for gs >= 128 both halves use
// the same entry. Applying a group's scale per chunk is exact regrouping of
// the same sum, so k-splits and K-parts need not align with gs.
//
//   fp16: the magic-exponent trick gives 1024 + q (and 1024 + 16 q) exactly;
//         one packed add of -(1024 + z) (or fma with 1/16 and -(64 + z)) with
//         the lane's own zero point gives q - z exactly, so the B operand is
//         exact and each half's fp32 partial is scaled once: acc += s * part.
//   bf16: gfx950 has no packed bf16 add, so B is 128 + q (bit pattern
//         0x4300 | q, exact: the bf16 ulp at 128 is 1), and the zero point is
//         removed after the MFMA with the half's row sums of A, obtained from
//         one extra MFMA of A against ones per 16-row block and k-step:
//             acc += s * (sum_k a (128 + q) - (128 + z) * sum_k a).
//         Products of two bf16 values are exact in fp32; the subtraction
//         cancels at most a factor ~20 of magnitude, far inside fp32.
#include "skinny.h"

namespace qg {
namespace fmt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool kBF16, bool kZ, bool kStaged>
struct PolicyW4G : Tile16 {
  using Acc = f32x4;
  using Elem = float;
  static constexpr int kScaleChunk = 0;
  static constexpr int kFrag = 4;           // 1 KB activation loads per 16 rows and chunk
  static constexpr int kAElem = 2;
  static constexpr bool kStageScales = false;
  static constexpr int kWeightDepth = 2;        // weight groups in flight per wave
  static constexpr uint32_t kEntry = kZ ? 4u : 2u;   // bytes per grid entry
  __device__ static uint32_t a_voff(int fr, int lane, int rows, size_t arow) {
    return ARows16::dma_voff(fr, lane, rows, arow);
  }

  struct Consts {
    uint32_t magic = kBF16 ? 0x43004300u : 0x64006400u;
  };

  template <int NBW>
  struct Stage {
    static constexpr int kVmem = kStaged ? NBW : 2 * NBW;   // codes (+ entries when not staged)
    static constexpr int kVmemFirst = kVmem;
    u32x4 code[NBW];
    u32x2 e[NBW];                                           // entries of the chunk's two 64-k halves
  };

  // Staged variant: the workgroup's grid entries in LDS, one row per chunk of
  // its split: [chunk - G0][NB * 16 columns][per] entries, per = 2 (the
  // chunk's two 64-k groups) when gs = 64, else 1 (the group that holds the
  // chunk, repeated for each of its chunks).
  static constexpr bool kStageExtra = kStaged;
  __host__ __device__ static int extra_lds(int NB, int ng, int gs) {
    return kStaged ? ng * NB * 16 * (gs == 64 ? 2 : 1) * (int)kEntry : 0;
  }
  // the staged rows by direct loads: row r of the split is entry row (G0 + r)
  // (group length 64) or (G0 + r) / cpg of the blob, columns b0*16 .. + NB*16
  __device__ static void stage_extra(const GemmArgs& p, char* dst, const TileInfo& ti, int NB, int wave,
                                     int nwaves, int lane) {
    if constexpr (kStaged) {
      const int cpg = p.gs == 64 ? 0 : p.gs / 128;
      const int per = cpg ? 1 : 2;
      const int pieces = NB * per * (int)kEntry;      // 16-byte pieces of a staged row
      const uint32_t srow = (uint32_t)p.N * per * kEntry;
      const uint32_t nrows = (uint32_t)(cpg ? p.G / cpg : p.G);
      const rsrc_t r = make_rsrc(p.scales, nrows * srow);
      const uint32_t col0 = (uint32_t)ti.b0 * 16u * per * kEntry;
      const int ng = ti.G1 - ti.G0;
      dma16(r, dst, ng * pieces, [&](int q) {
        const int i = q / pieces;
        const int g = ti.G0 + i;
        const uint32_t row = (uint32_t)(cpg ? g / cpg : g);
        return row * srow + col0 + (uint32_t)(q - i * pieces) * 16u;
      }, wave, nwaves, lane);
    }
  }

  template <int NBW>
  struct View {
    rsrc_t rc, re;
    uint32_t cvoff, gstep;
    uint32_t evoff, rowb;   // per-lane variant: entry offset, bytes per entry row
    const char* el;         // staged variant: this lane's column of its first block
    int gw0, G0, cpg, srowb;
    bool g64;

    __device__ View(const GemmArgs& p, const char* lds, const SkinnyLds& L, const TileInfo& ti, int bw,
                    int gw0_, int nload, int lane)
        : gw0(gw0_), G0(ti.G0) {
      const uint32_t nbt = (uint32_t)(p.N / 16);
      gstep = nbt * 1024u;
      cvoff = lane * 16u;
      rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)gw0 * nbt + bw) * 1024,
                     (uint32_t)(nload - 1) * gstep + NBW * 1024u);
      g64 = p.gs == 64;
      cpg = g64 ? 0 : p.gs / 128;
      const int per = g64 ? 2 : 1;
      if constexpr (kStaged) {
        srowb = 4 * NBW * 16 * per * (int)kEntry;
        el = lds + L.extra_off + ((bw - ti.b0) * 16 + (lane & 15)) * per * (int)kEntry;
      } else {
        rowb = (uint32_t)p.N * per * kEntry;
        evoff = (uint32_t)(bw * 16 + (lane & 15)) * per * kEntry;
        re = make_rsrc(p.scales, (uint32_t)(p.K / (cpg ? p.gs : 64)) * (uint32_t)p.N * kEntry);
      }
    }
    __device__ __forceinline__ void load_vmem(Stage<NBW>& st, int rel, uint32_t oob) const {
#pragma unroll
      for (int j = 0; j < NBW; ++j) st.code[j] = load16_stream(rc, cvoff + oob, j * 1024u + rel * gstep);
      if constexpr (!kStaged) {
        const int g = gw0 + rel;
        // wave-uniform: one load per block either way
        if (g64) {
          const uint32_t soff = (uint32_t)g * rowb;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const uint32_t vo = evoff + j * 16u * 2u * kEntry + oob;
            if (kZ) {
              st.e[j] = load8(re, vo, soff);
            } else {
              const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(re, vo, soff, 0);
              st.e[j] = u32x2{w & 0xFFFFu, w >> 16};
            }
          }
        } else {
          const uint32_t soff = (uint32_t)(g / cpg) * rowb;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const uint32_t vo = evoff + j * 16u * kEntry + oob;
            const uint32_t w = kZ ? __builtin_amdgcn_raw_buffer_load_b32(re, vo, soff, 0)
                                  : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(re, vo, soff, 0);
            st.e[j] = u32x2{w, w};
          }
        }
      }
    }
    __device__ __forceinline__ void load_lds(Stage<NBW>& st, int rel, uint32_t) const {
      if constexpr (kStaged) {
        const char* row = el + (gw0 + rel - G0) * srowb;
        // wave-uniform branch
        if (g64) {
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const char* q = row + j * 16 * 2 * (int)kEntry;
            if (kZ) {
              st.e[j] = *reinterpret_cast<const u32x2*>(q);
            } else {
              const uint32_t w = *reinterpret_cast<const uint32_t*>(q);
              st.e[j] = u32x2{w & 0xFFFFu, w >> 16};
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const char* q = row + j * 16 * (int)kEntry;
            const uint32_t w = kZ ? *reinterpret_cast<const uint32_t*>(q) : (uint32_t)*reinterpret_cast<const uint16_t*>(q);
            st.e[j] = u32x2{w, w};
          }
        }
      }
    }
  };

  __device__ static float scale_of(uint32_t e) {
    const uint32_t s16 = e & 0xFFFFu;
    return kBF16 ? __builtin_bit_cast(float, s16 << 16) : (float)as_h2(s16)[0];
  }
  __device__ static uint32_t zero_of(uint32_t e) { return kZ ? (e >> 16) & 0xFu : 8u; }

  template <int MB, int NBW>
  __device__ __forceinline__ static void compute(const Stage<NBW>& cur, const char* aslot, Acc (&acc)[MB][NBW],
                                                 bool valid, const Consts& k, int lane) {
    u32x4 a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[mb][t] = *reinterpret_cast<const u32x4*>(ARows16::at(aslot, mb * 16 + (lane & 15), 4 * t + (lane >> 4)));
    if constexpr (!kBF16) {
      const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        f16x8 bf[4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t z = zero_of(cur.e[j][hf]);
          const uint32_t zz = z | (z << 16);
          const f16x2 lo_off = as_h2(zz | 0xE400E400u);            // -(1024 + z)
          const f16x2 hi_off = as_h2((zz << 4) | 0xD400D400u);     // -(64 + z)
#pragma unroll
          for (int t = 2 * hf; t < 2 * hf + 2; ++t) {
            const uint32_t w = cur.code[j][t], w8 = w >> 8;
            const f16x2 p0 = as_h2(and_or(w, 0x000F000Fu, k.magic)) + lo_off;
            const f16x2 p1 = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, k.magic)), sixteenth, hi_off);
            const f16x2 p2 = as_h2(and_or(w8, 0x000F000Fu, k.magic)) + lo_off;
            const f16x2 p3 = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, k.magic)), sixteenth, hi_off);
            bf[t] = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          }
        }
        const float s0 = valid ? scale_of(cur.e[j][0]) : 0.f;
        const float s1 = valid ? scale_of(cur.e[j][1]) : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          // the halves' chains interleaved: consecutive MFMAs are independent
          f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a[mb][0]), bf[0], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a[mb][2]), bf[2], p1, 0, 0, 0);
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a[mb][1]), bf[1], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a[mb][3]), bf[3], p1, 0, 0, 0);
          acc[mb][j] += s0 * p0 + s1 * p1;
        }
      }
    } else {
      // row sums of A per 64-k half, once for all column blocks
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      f32x4 r0[MB], r1[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        r0[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        r1[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        r0[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][0]), ones, r0[mb], 0, 0, 0);
        r1[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][2]), ones, r1[mb], 0, 0, 0);
        r0[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][1]), ones, r0[mb], 0, 0, 0);
        r1[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][3]), ones, r1[mb], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        bf16x8 bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = cur.code[j][t];
          // pairs (nibble i, nibble i + 4) land in k order: sigma-ordered words.
          // Plain C++ here, not the inline-asm and_or: these registers feed the
          // MFMA directly, and the compiler inserts the wait states an MFMA
          // operand needs after a VALU write only for instructions it generated.
          constexpr uint32_t m = 0x000F000Fu;
          const u32x4 b = {(w & m) | k.magic, ((w >> 4) & m) | k.magic, ((w >> 8) & m) | k.magic,
                           ((w >> 12) & m) | k.magic};
          bf[t] = __builtin_bit_cast(bf16x8, b);
        }
        const float s0 = valid ? scale_of(cur.e[j][0]) : 0.f;
        const float s1 = valid ? scale_of(cur.e[j][1]) : 0.f;
        const float c0 = (float)(128u + zero_of(cur.e[j][0]));
        const float c1 = (float)(128u + zero_of(cur.e[j][1]));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][0]), bf[0], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][2]), bf[2], p1, 0, 0, 0);
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][1]), bf[1], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][3]), bf[3], p1, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mb][j][i] += s0 * (p0[i] - c0 * r0[mb][i]) + s1 * (p1[i] - c1 * r1[mb][i]);
        }
      }
    }
  }

  __device__ __forceinline__ static void store(const GemmArgs& p, int row, int col, float v) {
    if constexpr (kBF16) {
      const __bf16 h = (__bf16)v;   // round to nearest even
      static_cast<uint16_t*>(p.C)[(size_t)row * p.ldc + col] = __builtin_bit_cast(uint16_t, h);
    } else {
      static_cast<f16*>(p.C)[(size_t)row * p.ldc + col] = (f16)v;
    }
  }
};

}  // namespace fmt

using namespace fmt;

size_t lds_bytes_w4g(const Plan& pl, int G, int gs, bool zeros) {
  // the layout does not depend on the activation type
  if (pl.kernel == 3) return skinny_lds_bytes<PolicyW4G<false, true, false>>(pl, G, gs);
  return zeros ? skinny_lds_bytes<PolicyW4G<false, true, true>>(pl, G, gs)
               : skinny_lds_bytes<PolicyW4G<false, false, true>>(pl, G, gs);
}

template <bool kStaged>
static hipError_t launch_w4g_v(const Plan& pl, const GemmArgs& a, bool bf16, bool zeros, hipStream_t s) {
  if (bf16) {
    return zeros ? dispatch_skinny<PolicyW4G<true, true, kStaged>>(pl, a, s)
                 : dispatch_skinny<PolicyW4G<true, false, kStaged>>(pl, a, s);
  }
  return zeros ? dispatch_skinny<PolicyW4G<false, true, kStaged>>(pl, a, s)
               : dispatch_skinny<PolicyW4G<false, false, kStaged>>(pl, a, s);
}

hipError_t launch_w4g(const Plan& pl, const GemmArgs& a, bool bf16, bool zeros, hipStream_t s) {
  return pl.kernel == 3 ? launch_w4g_v<false>(pl, a, bf16, zeros, s) : launch_w4g_v<true>(pl, a, bf16, zeros, s);
}

}  // namespace qg
