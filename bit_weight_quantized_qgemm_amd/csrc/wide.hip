// W4A16 GEMM for larger batches (M > 32) on gfx950: the compute-bound end of the
// batch range of the MARLIN abstract, where its speedup shrinks with batch size
// but persists up to 64-128.
//
// Each workgroup owns a tile of 16*MBW rows (64 or 128) x 256 columns; its four
// waves each own 64 columns and every row of the tile, so every weight is
// dequantized once per tile and reused by MBW v_mfma_f32_16x16x32_f16 row blocks.
// Activations are shared by the four waves through LDS:
//   * per group of 128 k, the tile's activations arrive in MFMA A-fragment order
//     (1 KB per 16 rows x 32 k) by direct buffer-to-LDS loads, issued two groups
//     ahead into a 3-slot LDS ring, each wave fetching a quarter of the fragments;
//   * one barrier per group publishes a slot, after the wave's own loads of that
//     slot are counted complete (s_waitcnt on the in-order vector memory counter);
//   * the slot written next is the one all waves finished reading before the
//     barrier, so no second barrier is needed.
// Weights stream per wave into a register ring (two groups ahead) together with
// the lane's fp16 group scale; dequantization is exact to fp16 (q - 8), then one
// packed multiply by the scale rounds once (the scale cannot be applied after the
// MFMA here without doubling the accumulators). Accumulation is fp32.
// When a layer has too few tiles for the chip, K is also split across workgroups
// and finished with the coherent-store / arrival-counter fix-up.
#include "skinny.h"

namespace qg {
namespace {

constexpr int kWideWaves = 4;
constexpr int kWideNBW = 4;                            // 16-column blocks per wave
static_assert(kWideCols == 4 * 4 * 16, "tile width = waves x blocks x 16");
constexpr int kASlots = 3;

template <int MBW>
struct WideStage {
  u32x4 code[kWideNBW];
  uint32_t s[kWideNBW];
};

}  // namespace

template <int MBW>
__device__ __forceinline__ void wide_body(const GemmArgs& p, char* lds, int* flag) {
  constexpr int kSlotBytes = MBW * 4 * 1024;        // MBW row blocks x 4 k-steps x 1 KB
  constexpr int kAPerWave = MBW;                    // fragment loads per wave per group

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, h = lane >> 4;
  const int nt = blockIdx.x % p.nt;
  const int rest = blockIdx.x / p.nt;
  const int mt = rest % p.mt;
  const int split = rest / p.mt;
  const int G0 = split * p.gps;
  const int ng = min(p.G, G0 + p.gps) - G0;
  const int row0 = mt * MBW * 16;
  const int rows = min(MBW * 16, p.M - row0);
  const int bw = nt * (kWideCols / 16) + wave * kWideNBW;   // first block of this wave

  // activations: rows of the tile from k = 128*G0; rows beyond M re-read a valid row
  const rsrc_t ra = make_rsrc(static_cast<const f16*>(p.A) + (size_t)row0 * p.lda + (size_t)G0 * kGroup,
                              (uint32_t)(((size_t)(rows - 1) * p.lda + (size_t)ng * kGroup) * 2));
  // this wave fetches row blocks rb = wave*MBW/4 .. +MBW/4, all four k-steps
  constexpr int kRbPerWave = MBW / 4;
  uint32_t avoff[kRbPerWave];
#pragma unroll
  for (int q = 0; q < kRbPerWave; ++q) {
    const int rb = wave * kRbPerWave + q;
    avoff[q] = (uint32_t)((size_t)min(rb * 16 + c, rows - 1) * p.lda * 2 + h * 16);
  }
  auto issue_a = [&](int rel, int slot) {
#pragma unroll
    for (int q = 0; q < kRbPerWave; ++q) {
      const int rb = wave * kRbPerWave + q;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        char* dst = lds + slot * kSlotBytes + (rb * 4 + t) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)dst, 16, avoff[q], rel * 256u + t * 64u, 0, 0);
      }
    }
  };

  // weights and scales of this wave's four column blocks
  const uint32_t gstep = (uint32_t)(p.N / 16) * 1024u;   // group-major chunks
  const rsrc_t rc = make_rsrc(static_cast<const char*>(p.codes) + ((size_t)G0 * (p.N / 16) + bw) * 1024,
                              (uint32_t)(ng - 1) * gstep + kWideNBW * 1024u);
  const uint32_t sblk = (uint32_t)p.G8 * 256u;
  const rsrc_t rs = make_rsrc(static_cast<const char*>(p.scales) + (size_t)bw * p.G8 * 256,
                              kWideNBW * sblk);
  auto issue_b = [&](WideStage<MBW>& st, int rel) {
#pragma unroll
    for (int j = 0; j < kWideNBW; ++j) st.code[j] = load16(rc, lane * 16u, j * 1024u + rel * gstep);
    const int g = G0 + rel;
    const uint32_t soff = (uint32_t)(g >> 3) * 256u + (uint32_t)(g & 7) * 2u;
#pragma unroll
    for (int j = 0; j < kWideNBW; ++j)
      st.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, c * 16u, j * sblk + soff, 0);
  };

  f32x4 acc[MBW][kWideNBW];
#pragma unroll
  for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
    for (int j = 0; j < kWideNBW; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f16x2 lo_off = splat_h2(-1032.0f), hi_off = splat_h2(-72.0f);
  const uint32_t magic = 0x64006400u;

  // Prologue: activations and weights of groups 0 and 1. Each later iteration
  // issues one batch (activations, then weights and scales, of group i + 2), so
  // at the wait of iteration i exactly the weights of group i and the batch of
  // group i + 1 (MBW + 4*NBW operations) were issued after the last fragment
  // load of group i; the vector memory counter retires loads in order. Weights
  // live in a 3-stage register ring (two groups ahead); slots and stages are
  // static inside the 3-iteration body, and the iterations past the end only
  // re-issue in-bounds loads and skip the math.
  WideStage<MBW> st[kASlots];
  issue_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(st[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(min(1, ng - 1), 1);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(st[1], min(1, ng - 1));
  __builtin_amdgcn_sched_barrier(0);

  for (int base = 0; base < ng; base += kASlots) {
#pragma unroll
    for (int r = 0; r < kASlots; ++r) {
      const int i = base + r;
      // raw_barrier(): publishes only the counted completion above (see skinny.h)
      wait_vmcnt<kAPerWave + 4 * kWideNBW>();
      raw_barrier();
      issue_a(min(i + 2, ng - 1), (r + 2) % kASlots);
      issue_b(st[(r + 2) % kASlots], min(i + 2, ng - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (i < ng) {
        const WideStage<MBW>& cur = st[r];
        const char* slot = lds + r * kSlotBytes;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f16x8 bf[kWideNBW];
#pragma unroll
          for (int j = 0; j < kWideNBW; ++j) {
            const f16 sh = as_h2(cur.s[j])[0];
            const f16x8 sc8 = {sh, sh, sh, sh, sh, sh, sh, sh};
            bf[j] = dequant_u4x8(cur.code[j][t], lo_off, hi_off, magic) * sc8;
          }
#pragma unroll
          for (int rb = 0; rb < MBW; ++rb) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(slot + (rb * 4 + t) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < kWideNBW; ++j)
              acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[j], acc[rb][j], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue
  const int colw = bw * 16 + c;
  if (p.splits == 1) {
    f16* C = static_cast<f16*>(p.C);
#pragma unroll
    for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * h + i;
        if (r < rows) {
#pragma unroll
          for (int j = 0; j < kWideNBW; ++j)
            C[(size_t)(row0 + r) * p.ldc + colw + j * 16] = (f16)acc[rb][j][i];
        }
      }
    return;
  }
  // Cross-workgroup split: partials in MFMA-fragment order, one 1 KB wave
  // fragment per (wave, row block, column block), so every access is a
  // coalesced 16-byte device-coherent buffer operation. Region of (split,
  // tile): kWideWaves * MBW * NBW KB.
  constexpr int kFrag = MBW * kWideNBW;
  constexpr uint32_t kRegion = kWideWaves * kFrag * 1024;
  const size_t tile_id = (size_t)mt * p.nt + nt;
  const size_t ntiles = (size_t)p.mt * p.nt;
  auto region = [&](int q) {
    return make_rsrc(static_cast<char*>(p.partial) + ((size_t)q * ntiles + tile_id) * kRegion, kRegion);
  };
  auto voff = [&](int rb, int j) {
    return (uint32_t)(((wave * kFrag + rb * kWideNBW + j) * 64 + lane) * 16);
  };
  {
    const rsrc_t mine = region(split);
#pragma unroll
    for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
      for (int j = 0; j < kWideNBW; ++j) store16_coherent(acc[rb][j], mine, voff(rb, j));
  }
  if (!workgroup_arrive_last(p.counters + tile_id, (uint32_t)p.splits, flag)) return;
  // last arriver: sum the splits in split order (deterministic), then store fp16
#pragma unroll
  for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
    for (int j = 0; j < kWideNBW; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < p.splits; ++q) {
    const rsrc_t rq = region(q);
    f32x4 v[MBW][kWideNBW];
#pragma unroll
    for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
      for (int j = 0; j < kWideNBW; ++j) v[rb][j] = load16_coherent(rq, voff(rb, j));
#pragma unroll
    for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
      for (int j = 0; j < kWideNBW; ++j) acc[rb][j] += v[rb][j];
  }
  f16* C = static_cast<f16*>(p.C);
#pragma unroll
  for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + 4 * h + i;
      if (r < rows) {
#pragma unroll
        for (int j = 0; j < kWideNBW; ++j)
          C[(size_t)(row0 + r) * p.ldc + colw + j * 16] = (f16)acc[rb][j][i];
      }
    }
}

__global__ void __launch_bounds__(256) w4a16_wide_m64(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<4>(p, lds, &flag);
}

__global__ void __launch_bounds__(256) w4a16_wide_m128(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flag;
  wide_body<8>(p, lds, &flag);
}

namespace {

hipError_t launch_wide_k(const void* fn, void (*kernel)(GemmArgs), int mbw, const Plan& pl,
                         const GemmArgs& a, hipStream_t s) {
  const size_t lds = (size_t)kASlots * mbw * 4 * 1024;
  // the LDS size is fixed per kernel: opt in to it (above 64 KiB) once
  static bool big_lds[2] = {false, false};
  bool& done = big_lds[mbw == 8];
  if (!done) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    done = true;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)pl.workgroups), dim3(kWave * kWideWaves), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16_wide(const Plan& pl, const GemmArgs& a, hipStream_t s) {
  switch (pl.mb) {
    case 4: return launch_wide_k(reinterpret_cast<const void*>(&w4a16_wide_m64), w4a16_wide_m64, 4, pl, a, s);
    case 8: return launch_wide_k(reinterpret_cast<const void*>(&w4a16_wide_m128), w4a16_wide_m128, 8, pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
