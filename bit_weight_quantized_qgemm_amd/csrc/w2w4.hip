// Mixed 2/4-bit GEMM for gfx950 (the "Enabling Fast 2-bit LLM on GPUs" page:
// only a small fraction of large-range groups keep 4-bit codes, laid out with
// memory alignment in mind, and dequantization overlapped with the loads).
//
// Split-plane format: every group streams a dense 2-bit base plane (512 B per
// 16 columns x 128 k, one coalesced 8-byte-per-lane wave load, the same operand
// order as W4A16); the upper two bits of 4-bit groups sit in a separate high
// plane of 32-byte pieces, located through a per-chunk descriptor
// (offset, 16-bit column mask) that the wave reads with scalar loads two groups
// ahead. Each lane then rebuilds 4-bit nibble words
//   nib_2s   = (base_s & 0x33333333) | ((high_s << 2) & 0xCCCCCCCC)
//   nib_2s+1 = ((base_s >> 2) & 0x33333333) | (high_s & 0xCCCCCCCC)
// (high = 0 for 2-bit groups) and runs the W4A16 dequantization with a per-lane
// zero point z = 8 (4-bit) or 2 (2-bit): no branches on the group precision.
// Scales, MFMA, split-K fix-up as in the W4A16 kernel.
#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

template <int MB, int NB>
struct StageM {
  u32x2 base[NB];
  u32x2 high[NB];
  uint32_t mask[NB];   // wave-uniform column mask of the chunk
  u32x4 a[MB][4];
};

template <int MB, int NB>
__global__ void __launch_bounds__(256) w2w4_skinny(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * kWavesPerBlock + wave;
  const int nt = item % p.nt;
  const int rest = item / p.nt;
  const int mt = rest % p.mt;
  const int split = rest / p.mt;
  if (split >= p.splits) return;
  const int g0 = split * p.gps;
  const int ng = min(p.G, g0 + p.gps) - g0;
  const int c = lane & 15;
  const int h = lane >> 4;
  const int b0 = nt * NB;
  const int row0 = mt * MB * 16;
  const int rows = min(MB * 16, p.M - row0);

  const uint32_t bblk = (uint32_t)p.G * 512u;
  const rsrc_t rb = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)b0 * p.G + g0) * 512,
                              (NB - 1) * bblk + ng * 512u);
  const uint32_t bvoff = lane * 8u;
  const uint32_t sblk = (uint32_t)p.G8 * 256u;
  const rsrc_t rs = make_rsrc(static_cast<const char*>(p.scales) + ((size_t)b0 * p.G8 + g0 / 8) * 256,
                              (NB - 1) * sblk + ((ng + 7) / 8) * 256u);
  const uint32_t svoff = c * 16u;
  const rsrc_t rh = make_rsrc(p.high, 0x7FFFFFF0u);
  const rsrc_t ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)row0 * p.lda + (size_t)g0 * kGroup,
                              (uint32_t)(((size_t)(rows - 1) * p.lda + (size_t)ng * kGroup) * 2));
  uint32_t avoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    avoff[mb] = (uint32_t)((size_t)min(mb * 16 + c, rows - 1) * p.lda * 2 + h * 64);
  // descriptors of this item's chunks: (b0 + j)*G + g0 + rel
  const u32x2* desc = static_cast<const u32x2*>(p.aux) + (size_t)b0 * p.G + g0;
  const uint32_t below = (1u << c) - 1u;

  auto load_stage = [&](StageM<MB, NB>& st, int rel, const u32x2 (&d)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      st.base[j] = load8(rb, bvoff, j * bblk + rel * 512u);
      st.mask[j] = d[j][1];
      u32x2 hv = {0u, 0u};
      if ((d[j][1] >> c) & 1u) {
        const uint32_t slot = d[j][0] + __builtin_popcount(d[j][1] & below);
        hv = load8(rh, slot * 32u + h * 8u, 0);
      }
      st.high[j] = hv;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t) st.a[mb][t] = load16(ra, avoff[mb], rel * 256u + t * 16u);
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = 0x64006400u;
  const f16x2 lo4 = splat_h2(-1032.0f), hi4 = splat_h2(-72.0f);   // zero 8
  const f16x2 lo2 = splat_h2(-1026.0f), hi2 = splat_h2(-66.0f);   // zero 2
  const int last8 = (ng - 1) >> 3;

  u32x2 d1[NB], d2[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const u32x2 d0 = desc[(size_t)j * p.G];
    d1[j] = desc[(size_t)j * p.G + min(1, ng - 1)];
    d2[j] = d0;
  }
  StageM<MB, NB> cur, nxt;
  load_stage(cur, 0, d2);
  u32x4 sv[NB], svn[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) sv[j] = load16(rs, svoff, j * sblk);

  for (int gc = 0; gc < ng; gc += 8) {
    const int n8 = min((gc >> 3) + 1, last8);
#pragma unroll
    for (int j = 0; j < NB; ++j) svn[j] = load16(rs, svoff, j * sblk + n8 * 256u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (gc + i < ng) {
        // descriptors two groups ahead; stage loads one group ahead
#pragma unroll
        for (int j = 0; j < NB; ++j) d2[j] = desc[(size_t)j * p.G + min(gc + i + 2, ng - 1)];
        load_stage(nxt, min(gc + i + 1, ng - 1), d1);
        f16x8 bf[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const bool is4 = (cur.mask[j] >> c) & 1u;
          const f16x2 lo_off = is4 ? lo4 : lo2;
          const f16x2 hi_off = is4 ? hi4 : hi2;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint32_t B = cur.base[j][s], H = cur.high[j][s];
            const uint32_t n0 = and_or(H << 2, 0xCCCCCCCCu, B & 0x33333333u);
            const uint32_t n1 = and_or(H, 0xCCCCCCCCu, (B >> 2) & 0x33333333u);
            bf[j][2 * s] = dequant_u4x8(n0, lo_off, hi_off, magic);
            bf[j][2 * s + 1] = dequant_u4x8(n1, lo_off, hi_off, magic);
          }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float sc = half_of(sv[j][i >> 1], i & 1);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              part = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(cur.a[mb][t]), bf[j][t], part, 0, 0, 0);
            acc[mb][j] += sc * part;
          }
        }
        cur = nxt;
#pragma unroll
        for (int j = 0; j < NB; ++j) d1[j] = d2[j];
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) sv[j] = svn[j];
  }

  f16* C = static_cast<f16*>(p.C);
  const int rbase = row0 + 4 * h;
  if (p.splits == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + mb * 16 + i;
          if (row < p.M) C[(size_t)row * p.ldc + (b0 + j) * 16 + c] = (f16)acc[mb][j][i];
        }
    return;
  }
  float* part = static_cast<float*>(p.partial);
  const size_t plane = (size_t)p.M * p.N;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + mb * 16 + i;
        if (row < p.M) part[split * plane + (size_t)row * p.N + (b0 + j) * 16 + c] = acc[mb][j][i];
      }
  uint32_t* counter = p.counters + (size_t)mt * p.nt + nt;
  if (!arrive_last(counter, (uint32_t)p.splits)) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + mb * 16 + i;
        if (row < p.M) {
          const size_t off = (size_t)row * p.N + (b0 + j) * 16 + c;
          float v = 0.f;
          for (int s = 0; s < p.splits; ++s) v += part[s * plane + off];
          C[(size_t)row * p.ldc + (b0 + j) * 16 + c] = (f16)v;
        }
      }
  if (lane == 0) atomicExch(counter, 0u);
}

template <int MB, int NB>
hipError_t launch_t(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  const int64_t blocks = (pl.waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((w2w4_skinny<MB, NB>), dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w2w4(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  switch (pl.mb * 10 + pl.nb) {
    case 11: return launch_t<1, 1>(pl, a, s);
    case 12: return launch_t<1, 2>(pl, a, s);
    case 14: return launch_t<1, 4>(pl, a, s);
    case 21: return launch_t<2, 1>(pl, a, s);
    case 22: return launch_t<2, 2>(pl, a, s);
    case 24: return launch_t<2, 4>(pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
