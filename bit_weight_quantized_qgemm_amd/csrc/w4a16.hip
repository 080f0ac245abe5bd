// W4A16 GEMM for gfx950: C[M,N] = A[M,K] (fp16) * dequant(W)[K,N], W 4-bit codes
// with zero point 8 and one fp16 scale per 128 k of a column.
//
// The MARLIN abstract asks for a kernel that stays practically memory-bound for
// batched decode (batch 16..32 near the full 4x speedup of 4-bit weights,
// 64..128 still ahead) through asynchronous memory access, task scheduling with
// pipelining, and bespoke quantization support. The CDNA4 design here:
//
//  * Work item = one wavefront: (m-tile of 16*MB rows, n-tile of 16*NB columns,
//    k-split of whole groups). Four waves of a workgroup take four neighbouring
//    n-tiles of the same k range, so the activation rows they read are served by
//    the CU's L1 after the first wave.
//  * Weights stream as one 1 KB, fully coalesced 128-bit wave load per 16 columns
//    x 128 k (the repacked blob is already in MFMA operand order), issued one
//    group ahead of the math (register double buffering).
//  * Dequantization in registers: 9 VALU ops per 8 weights give exact fp16
//    (q - 8); the group scale is applied once per group in fp32 on the MFMA
//    partial product (4 FMAs per 16x16 block), so each output is
//    sum_g s[g,n] * sum_{k in g} A[m,k] (q[k,n] - 8) with fp32 accumulation.
//  * v_mfma_f32_16x16x32_f16: 4 per 16x16 block per group.
//  * Split-K: each wave writes its fp32 partial tile; the last wave to arrive at
//    a tile (device-scope counter) adds all partials in split order and writes
//    fp16, so results are deterministic and no second kernel is launched.
#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

template <int MB, int NB>
struct Stage {
  u32x4 code[NB];     // 4 words = 32 codes per lane per 16-column block
  u32x4 a[MB][4];     // 32 fp16 activations per lane per 16-row block
};

// Buffer views of one work item: NB column blocks x ng groups of codes and
// scales, MB*16 activation rows from the item's first k.
template <int MB, int NB>
struct View {
  rsrc_t rc, rs, ra;
  uint32_t cvoff, cblk, svoff, sblk;
  uint32_t avoff[MB];

  __device__ __forceinline__ void load(Stage<MB, NB>& st, int rel) const {
#pragma unroll
    for (int j = 0; j < NB; ++j) st.code[j] = load16(rc, cvoff, j * cblk + rel * 1024u);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t) st.a[mb][t] = load16(ra, avoff[mb], rel * 256u + t * 16u);
  }
  __device__ __forceinline__ u32x4 scales8(int j, int g8) const {
    return load16(rs, svoff, j * sblk + g8 * 256u);
  }
};

template <int MB, int NB>
__global__ void __launch_bounds__(256) w4a16_skinny(GemmArgs p) {
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

  View<MB, NB> v;
  v.cblk = (uint32_t)p.G * 1024u;
  v.cvoff = lane * 16u;
  v.rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)b0 * p.G + g0) * 1024,
                   (NB - 1) * v.cblk + ng * 1024u);
  v.sblk = (uint32_t)p.G8 * 256u;
  v.svoff = c * 16u;
  v.rs = make_rsrc(static_cast<const char*>(p.scales) + ((size_t)b0 * p.G8 + g0 / 8) * 256,
                   (NB - 1) * v.sblk + ((ng + 7) / 8) * 256u);
  // Rows beyond M read a valid row instead: MFMA output row r depends only on
  // A row r, and those output rows are never stored.
  v.ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)row0 * p.lda + (size_t)g0 * kGroup,
                   (uint32_t)(((size_t)(rows - 1) * p.lda + (size_t)ng * kGroup) * 2));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    v.avoff[mb] = (uint32_t)((size_t)min(mb * 16 + c, rows - 1) * p.lda * 2 + h * 64);

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f16x2 lo_off = splat_h2(-1032.0f);   // -(1024 + 8)
  const f16x2 hi_off = splat_h2(-72.0f);     // -(64 + 8)
  const uint32_t magic = 0x64006400u;
  const int last8 = (ng - 1) >> 3;

  Stage<MB, NB> cur, nxt;
  v.load(cur, 0);
  u32x4 sv[NB], svn[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) sv[j] = v.scales8(j, 0);

  for (int gc = 0; gc < ng; gc += 8) {
    const int n8 = min((gc >> 3) + 1, last8);
#pragma unroll
    for (int j = 0; j < NB; ++j) svn[j] = v.scales8(j, n8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (gc + i < ng) {
        v.load(nxt, min(gc + i + 1, ng - 1));
        f16x8 bf[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) bf[j][t] = dequant_u4x8(cur.code[j][t], lo_off, hi_off, magic);
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
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) sv[j] = svn[j];
  }

  // ---- epilogue: lane (c, h) holds rows 4h..4h+3 of column c of each 16x16 block
  f16* C = static_cast<f16*>(p.C);
  const int rbase = mt * MB * 16 + 4 * h;
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
  hipLaunchKernelGGL((w4a16_skinny<MB, NB>), dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16(const Plan& pl, const GemmArgs& a, hipStream_t s) {
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
