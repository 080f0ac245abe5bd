// W4A8 GEMM for gfx950 (the W4A8 setting of the OdysseyLLM / FastGEMM abstract):
// int8 activations with a per-row fp16 scale, signed int4 weights with an int8
// scale per group of 128 k and an fp16 scale per column.
//
//   acc[m,n] = sum_g s_g[g,n] * sum_{k in g} A[m,k] * q[k,n]     (exact int32)
//   C[m,n]   = fp16(float(acc) * a_scale[m] * s_c[n])
//
// The blob stores u = q + 8 (0..15) so one AND (and one shift+AND) turns a word
// into eight int8 MFMA operand bytes with no sign handling; the offset is removed
// exactly per group with the row sums of A:
//   sum_k A*q = sum_k A*u - 8 * sum_k A,
// and the row sums come from one extra v_mfma_i32_16x16x64_i8 against a matrix
// of ones per 16-row block per group (shared by every column block of the wave).
// The group scale multiplies the exact per-group int32 partial with
// v_mul_i32_i24 (|partial| < 2^18, |s_g| <= 128). Same wave-level work items,
// buffer streaming and deterministic split-K fix-up as the W4A16 kernel; split
// partials are int32, so their sum is exact in any order.
#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

template <int MB, int NB>
struct Stage8 {
  u32x4 code[NB];   // 32 biased int4 codes per lane per 16-column block
  u32x4 a[MB][2];   // 32 int8 activations per lane per 16-row block
};

template <int MB, int NB>
struct View8 {
  rsrc_t rc, rs, ra;
  uint32_t cvoff, cblk, svoff, sblk;
  uint32_t avoff[MB];

  __device__ __forceinline__ void load(Stage8<MB, NB>& st, int rel) const {
#pragma unroll
    for (int j = 0; j < NB; ++j) st.code[j] = load16(rc, cvoff, j * cblk + rel * 1024u);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) st.a[mb][t] = load16(ra, avoff[mb], rel * 128u + t * 16u);
  }
  __device__ __forceinline__ u32x2 gscales8(int j, int g8) const {
    return load8(rs, svoff, j * sblk + g8 * 128u);
  }
};

template <int MB, int NB>
__global__ void __launch_bounds__(256) w4a8_skinny(GemmArgs p) {
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

  View8<MB, NB> v;
  v.cblk = (uint32_t)p.G * 1024u;
  v.cvoff = lane * 16u;
  v.rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)b0 * p.G + g0) * 1024,
                   (NB - 1) * v.cblk + ng * 1024u);
  v.sblk = (uint32_t)p.G8 * 128u;
  v.svoff = c * 8u;
  v.rs = make_rsrc(static_cast<const char*>(p.scales) + ((size_t)b0 * p.G8 + g0 / 8) * 128,
                   (NB - 1) * v.sblk + ((ng + 7) / 8) * 128u);
  v.ra = make_rsrc(static_cast<const int8_t*>(p.A) + (size_t)row0 * p.lda + (size_t)g0 * kGroup,
                   (uint32_t)((size_t)(rows - 1) * p.lda + (size_t)ng * kGroup));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    v.avoff[mb] = (uint32_t)((size_t)min(mb * 16 + c, rows - 1) * p.lda + h * 32);

  i32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = i32x4{0, 0, 0, 0};

  const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const int last8 = (ng - 1) >> 3;

  Stage8<MB, NB> cur, nxt;
  v.load(cur, 0);
  u32x2 sv[NB], svn[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) sv[j] = v.gscales8(j, 0);

  for (int gc = 0; gc < ng; gc += 8) {
    const int n8 = min((gc >> 3) + 1, last8);
#pragma unroll
    for (int j = 0; j < NB; ++j) svn[j] = v.gscales8(j, n8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (gc + i < ng) {
        v.load(nxt, min(gc + i + 1, ng - 1));
        i32x4 rsum[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          rsum[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i4(cur.a[mb][0]), ones, i32x4{0, 0, 0, 0}, 0, 0, 0);
          rsum[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i4(cur.a[mb][1]), ones, rsum[mb], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const u32x4 w = cur.code[j];
          const i32x4 bq0 = {(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu),
                             (int)(w[1] & 0x0F0F0F0Fu), (int)((w[1] >> 4) & 0x0F0F0F0Fu)};
          const i32x4 bq1 = {(int)(w[2] & 0x0F0F0F0Fu), (int)((w[2] >> 4) & 0x0F0F0F0Fu),
                             (int)(w[3] & 0x0F0F0F0Fu), (int)((w[3] >> 4) & 0x0F0F0F0Fu)};
          const int sg = __builtin_amdgcn_sbfe((int)sv[j][i >> 2], 8 * (i & 3), 8);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            i32x4 part = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i4(cur.a[mb][0]), bq0, i32x4{0, 0, 0, 0}, 0, 0, 0);
            part = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i4(cur.a[mb][1]), bq1, part, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int corr = part[r] - 8 * rsum[mb][r];    // sum_{k in g} A * q, |.| < 2^18
              acc[mb][j][r] += __builtin_amdgcn_sbfe(corr, 0, 24) * sg;
            }
          }
        }
        cur = nxt;
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) sv[j] = svn[j];
  }

  const int rbase = row0 + 4 * h;
  if (p.splits > 1) {
    int32_t* part = static_cast<int32_t*>(p.partial);
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
            int32_t s = 0;
            for (int q = 0; q < p.splits; ++q) s += part[q * plane + off];
            acc[mb][j][i] = s;
          }
        }
    if (lane == 0) atomicExch(counter, 0u);
  }
  // epilogue: int32 accumulators and the scaled fp16 output
  const f16* a_scale = static_cast<const f16*>(p.a_scale);
  const f16* s_c = static_cast<const f16*>(p.aux);
  f16* C = static_cast<f16*>(p.C);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = (b0 + j) * 16 + c;
    const float sc = (float)s_c[col];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + mb * 16 + i;
        if (row < p.M) {
          const int32_t a = acc[mb][j][i];
          if (p.acc_out) p.acc_out[(size_t)row * p.N + col] = a;
          C[(size_t)row * p.ldc + col] = (f16)((float)a * (float)a_scale[row] * sc);
        }
      }
  }
}

template <int MB, int NB>
hipError_t launch_t(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  const int64_t blocks = (pl.waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((w4a8_skinny<MB, NB>), dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a8(const Plan& pl, const GemmArgs& a, hipStream_t s) {
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
