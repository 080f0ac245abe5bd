// Per-token dynamic int8 quantization of fp16 activations, the input side of the
// W4A8 GEMM: the Atom review's method section adapts the activation
// quantization parameters to each activation matrix at inference time, and the
// OdysseyLLM abstract's W4A8 kernel consumes int8 activations with a per-token
// scale. Symmetric absmax per row:
//   a_s[m] = fp16(amax_m / 127)                  (fp32 division, one RNE rounding)
//   q[m,k] = clamp(rint(A[m,k] / a_s[m]), -127, 127)   (fp32, half to even)
// and a row whose a_s is zero quantizes to zeros.
//
// One 256-thread workgroup per row. The op moves 3 bytes per element and is
// HBM-bound; the second pass over a row (at most 2 MiB) reads it back from L2.
#include "qgemm_device.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

__global__ void __launch_bounds__(256) quantize_a8_rows(const f16* __restrict__ A, int64_t lda, int K,
                                                        int8_t* __restrict__ Q, int64_t ldq,
                                                        f16* __restrict__ S) {
  const int row = blockIdx.x;
  const f16* a = A + (size_t)row * lda;
  float amax = 0.f;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(a + k);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const f16 sh = (f16)(amax / 127.0f);
  const float s = (float)sh;
  if (threadIdx.x == 0) S[row] = sh;
  int8_t* q = Q + (size_t)row * ldq;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(a + k);
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = s > 0.f ? rintf((float)v[e] / s) : 0.f;
      r = fminf(fmaxf(r, -127.f), 127.f);
      w[e >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (e & 3));
    }
    *reinterpret_cast<u32x2*>(q + k) = w;
  }
}

}  // namespace

hipError_t launch_quantize_a8(const void* A, int64_t lda, int64_t M, int64_t K, void* Q, int64_t ldq,
                              void* S, hipStream_t s) {
  hipLaunchKernelGGL(quantize_a8_rows, dim3((unsigned)M), dim3(256), 0, s, static_cast<const f16*>(A), lda,
                     (int)K, static_cast<int8_t*>(Q), ldq, static_cast<f16*>(S));
  return hipGetLastError();
}

}  // namespace qg
