// Achievable-peak probes on gfx950: a streaming read through raw buffer loads
// and a matrix-core loop on register operands (declared in qgemm_probes.h).
// Each kernel's work is fixed by its launch arguments alone; the host checks
// every size before a launch.
#include "qgemm_probes.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kThreads = 256;
constexpr int kInFlight = 8;   // 16-byte loads per lane per round
constexpr int kErrArg = -1, kErrHip = -6;

// Lanes past the end of the buffer read zeros (the resource's byte size bounds
// every access), so the last round needs no branch. CHUNKED = false: the eight
// 1 KB wave loads of a round lie one grid-width apart; CHUNKED = true: they are
// eight consecutive KB, and the waves of the grid take consecutive 8 KB chunks.
template <bool CHUNKED>
__global__ void __launch_bounds__(kThreads) stream_read(const void* src, uint32_t bytes, uint32_t* sink) {
  const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)bytes, 0x00020000);
  const uint32_t lane = threadIdx.x & 63, wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t grid = gridDim.x * kThreads * 16u;   // bytes of one load across the grid
  const uint32_t step = CHUNKED ? 1024u : grid;        // bytes between a lane's loads of a round
  uint32_t off = CHUNKED ? wave * (kInFlight * 1024u) + lane * 16u : (blockIdx.x * kThreads + threadIdx.x) * 16u;
  uint32_t s = 0;
  for (; off < bytes; off += kInFlight * grid) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + u * step, 0, 0));
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) s += v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  // wave sum into the wave's own slot (no atomics: thousands of them on one
  // address serialize at the end of the read and would be timed with it)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d);
  if (lane == 0) sink[wave] = s;
}

// Per-lane pseudo-random operands (xorshift32): fp16 uniform in [-1, 1) and
// int8 uniform in [-128, 127], as a GEMM on real data feeds the matrix cores.
struct LaneRandom {
  uint32_t x;
  __device__ explicit LaneRandom(uint32_t seed) : x(seed * 2654435761u + 0x9E3779B9u) {}
  __device__ uint32_t next() {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  }
  __device__ f16x8 halves() {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (f16)((float)(next() & 0xFFFF) * (1.0f / 32768.0f) - 1.0f);
    return r;
  }
  __device__ i32x4 bytes() { return i32x4{(int)next(), (int)next(), (int)next(), (int)next()}; }
};

template <int KIND>
__global__ void __launch_bounds__(kThreads) mfma_loop(uint32_t* sink, int iters) {
  const int lane = threadIdx.x & 63;
  // operands depend on the lane, so nothing folds; the values keep every
  // accumulator finite over any iteration count used here
  const f16 h = (f16)(1.0f / 4096.0f) * (f16)(lane & 7);
  const f16x8 a = {h, h, h, h, h, h, h, h};
  const i32x4 ai = {lane & 3, 1, 0, (lane >> 2) & 1};
  uint32_t out = 0;
  if constexpr (KIND == 5) {
    // random operands: four A fragments, two B fragments alternating per step
    LaneRandom g((uint32_t)(blockIdx.x * kThreads + threadIdx.x));
    f16x8 ra[4], rb[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = g.halves();
    rb[0] = g.halves();
    rb[1] = g.halves();
    f32x16 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ra[j & 3], rb[(j >> 2) & 1], acc[j & 3], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[j][0] + acc[j][15];
    out = __float_as_uint(t);
  } else if constexpr (KIND == 6) {
    LaneRandom g((uint32_t)(blockIdx.x * kThreads + threadIdx.x));
    i32x4 ra[4], rb[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = g.bytes();
    rb[0] = g.bytes();
    rb[1] = g.bytes();
    i32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[j & 3], rb[(j >> 2) & 1], acc[j & 3], 0, 0, 0);
    }
    int t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[j][0] + acc[j][3];
    out = (uint32_t)t;
  } else if constexpr (KIND == 0) {
    f32x16 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[j & 3], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[j][0] + acc[j][15];
    out = __float_as_uint(t);
  } else if constexpr (KIND == 1) {
    f32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[j & 3], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[j][0] + acc[j][3];
    out = __float_as_uint(t);
  } else {
    i32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ai, acc[j & 3], 0, 0, 0);
    }
    int t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[j][0] + acc[j][3];
    out = (uint32_t)t;
  }
  if (lane == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = out;
}

// v_mfma_f32_32x32x16_f16 with its A operand read from LDS: every 1 KB wave
// read (ds_read_b128, 16 bytes per lane) feeds USES instructions with different
// B operands, as a GEMM tile of 32 x 32*USES per wave would. The workgroup's
// 16 KB of LDS is filled once; the reads cycle through it.
template <int USES>
__global__ void __launch_bounds__(kThreads) mfma_lds_loop(uint32_t* sink, int iters) {
  __shared__ f16x8 buf[1024];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 1024; i += kThreads) {
    const f16 h = (f16)(1.0f / 4096.0f) * (f16)(i & 7);
    buf[i] = f16x8{h, h, h, h, h, h, h, h};
  }
  __syncthreads();
  const f16 hb = (f16)(1.0f / 4096.0f) * (f16)(lane & 3);
  f16x8 b[USES];
#pragma unroll
  for (int j = 0; j < USES; ++j) b[j] = f16x8{hb, hb, hb, hb, hb, hb, hb, (f16)j};
  f32x16 acc[4][USES] = {};
  const int wave = threadIdx.x >> 6;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f16x8 a = buf[(((i * 8 + u) + wave * 4) & 15) * 64 + lane];
#pragma unroll
      for (int j = 0; j < USES; ++j)
        acc[u & 3][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[j], acc[u & 3][j], 0, 0, 0);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < USES; ++j) t += acc[q][j][0] + acc[q][j][15];
  if (lane == 0) sink[blockIdx.x * (kThreads / 64) + wave] = __float_as_uint(t);
}

}  // namespace

extern "C" {

int qgemm_probe_stream_read(const void* src, int64_t bytes, void* sink, int64_t sink_words, int workgroups,
                            int chunked, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || bytes > (int64_t(3) << 30) || workgroups <= 0 ||
      workgroups > 65536 || (reinterpret_cast<uintptr_t>(src) & 15) || (chunked != 0 && chunked != 1) ||
      sink_words < (int64_t)workgroups * (kThreads / 64))
    return kErrArg;
  // every offset a lane forms (the last round's included) stays below 2^32:
  // bytes + kInFlight * grid bytes bounds them in both orders
  if (bytes + (int64_t)kInFlight * workgroups * kThreads * 16 >= (int64_t(1) << 32)) return kErrArg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (chunked)
    hipLaunchKernelGGL(stream_read<true>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, src, (uint32_t)bytes,
                       static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL(stream_read<false>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, src, (uint32_t)bytes,
                       static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : kErrHip;
}

int64_t qgemm_probe_mfma_ops(int kind) {
  switch (kind) {
    case 0: return 32LL * 32 * 16 * 2;
    case 1: return 16LL * 16 * 32 * 2;
    case 2: return 16LL * 16 * 64 * 2;
    case 3:
    case 4:
    case 5: return 32LL * 32 * 16 * 2;
    case 6: return 16LL * 16 * 64 * 2;
    default: return 0;
  }
}

int qgemm_probe_mfma(void* sink, int64_t sink_words, int workgroups, int iters, int kind, void* stream) {
  if (!sink || workgroups <= 0 || workgroups > 65536 || iters <= 0 || qgemm_probe_mfma_ops(kind) == 0 ||
      sink_words < (int64_t)workgroups * (kThreads / 64))
    return kErrArg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* out = static_cast<uint32_t*>(sink);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_loop<0>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_loop<1>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_loop<2>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    case 3: hipLaunchKernelGGL(mfma_lds_loop<1>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    case 5: hipLaunchKernelGGL(mfma_loop<5>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    case 6: hipLaunchKernelGGL(mfma_loop<6>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
    default: hipLaunchKernelGGL(mfma_lds_loop<2>, dim3((unsigned)workgroups), dim3(kThreads), 0, s, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : kErrHip;
}

}  // extern "C"
