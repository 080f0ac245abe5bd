// Offline weight repacking into the order the GEMM kernels stream (the
// arbitrary-precision Tensor Core page's abstract preprocesses the matrices into
// a layout suited to the later computation; the 2-bit page's abstract stores the
// mixed 2/4-bit groups with aligned memory access in mind).
//
// Blob layout (G = K/128 groups, NB = N/16 column blocks, G8 = ceil(G/8); lane l
// of a 64-wide wave has column c = l % 16 and k-quarter h = l / 16; regions start
// on 256-byte boundaries):
//
//  W4A16 codes : chunk (b, g) of 1024 B at (g*NB + b)*1024 (group-major, so the
//                chunks of one group are adjacent for every column block and the
//                waves of a launch, advancing through K together, read
//                neighbouring kilobytes at the same time); lane l owns 16 B at
//                +16l = words t = 0..3; word t holds the 8 codes of
//                k = 128g + 32t + 8h + e (e = 0..7) of column n = 16b + c, element
//                e in nibble sigma(e) = e/2 (e even) or 4 + (e-1)/2 (e odd), so
//                that one AND/OR per nibble pair yields two fp16 lanes in k order.
//                That is exactly the v_mfma_f32_16x16x32_f16 B-operand of lane l
//                for k-step t (lanes 16h..16h+15 hold k 8h..8h+7 of the step), and
//                the matching A fragments of one step are 64 contiguous bytes per
//                row.
//  scales      : fp16 [NB][G8][16][8]: lane c loads the scales of 8 groups at once.
//  W4A8 codes  : same chunks; word t = 2u + s holds k = 128g + 64u + 16h + 8s + e
//                (v_mfma_i32_16x16x64_i8 step u: lanes 16h.. hold k 16h..16h+15),
//                element e in nibble tau(e) = 2e (e < 4) or 2(e-4) + 1 (e >= 4) so
//                that (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are the int8
//                B-operand bytes in k order; the nibble holds q + 8 (0..15).
//  W4A8 scales : int8 group scales [NB][G8][16][8], then fp16 channel scales [N].
//  W2W4 base   : chunk (b, g) of 512 B at (g*NB + b)*512; lane l owns 8 B = words s = 0, 1; bits
//                [4p, 4p+1] of word s = low 2 bits of the code at slot p of W4A16
//                word 2s, bits [4p+2, 4p+3] = same for word 2s+1.
//  W2W4 desc   : per chunk (b, g), at index g*NB + b: u32 off, u32 mask16 (bit c =
//                column 16b + c is a 4-bit group; off = 4-bit groups in all
//                earlier chunks of that order).
//  W4G codes   : as W4A16 (128-k chunks whatever the group length gs).
//  W4G entries : one per (group g = k / gs, column n): the 16-bit scale pattern
//                (fp16 or bf16), or with stored zero points a u32 = scale bits |
//                zero << 16; entry (g, n) at index ((g / P)*N + n)*P + g % P with
//                P = 2 for gs = 64 (the two groups of a 128-k chunk adjacent)
//                and P = 1 otherwise.
//  SP24 chunks : 2:4 sparse W4A16; chunk (b, g) of 768 B at (g*NB + b)*768; lane l
//                owns 12 B = code words s = 0, 1 (64-k steps) and a position word
//                (one 12-byte lane load per chunk); code word s covers
//                k = 128g + 64s + 16h + 4j + p (quads j, positions p) of column
//                16b + c; each quad keeps two positions p0 < p1 (its codes other
//                than 8, completed with the lowest other positions), kept value
//                v = 2j + i in nibble sigma(v).
//                The position word's bits 16s + 2v .. +1 hold the position of
//                kept value v of code word s.
//  SP24 status : u32 count of quads with more than two codes other than 8.
//  BP chunks   : bit-plane W_b A8; chunk (b, g) of 256*B bytes at (g*NB + b)*256*B;
//                lane l owns 4*B bytes = plane words i = 0..B-1; bit 16u + j of word
//                i is bit i of the code at k = 128g + 64u + 16h + j, column 16b + c.
//  BP cscales  : fp16 [N].
//  W2W4 high   : per 4-bit group, 32 B at 32*(off + rank(c)), quarter h at +8h,
//                the upper 2 code bits in the base-plane arrangement.
#include "qgemm_device.h"
#include "qgemm_internal.h"

#include <algorithm>

namespace qg {
namespace {

__device__ __forceinline__ int sigma(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }
__device__ __forceinline__ int sigma_inv(int p) { return p < 4 ? 2 * p : 2 * (p - 4) + 1; }
__device__ __forceinline__ int tau(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }

// canonical word (nibble e = code of k = 8r + e) -> blob word under a slot map
template <bool kTau>
__device__ __forceinline__ uint32_t permute_nibbles(uint32_t src) {
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int slot = kTau ? tau(e) : sigma(e);
    out |= ((src >> (4 * e)) & 0xFu) << (4 * slot);
  }
  return out;
}

// One thread per (chunk, lane): 4 words of W4A16 / W4A8 codes.
template <bool kW4A8>
__global__ void repack_codes_u4(const uint32_t* __restrict__ codes, uint32_t* __restrict__ out,
                                int G, int N, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  const int64_t chunk = tid >> 6;
  const int NB = N / 16;
  const int g = (int)(chunk / NB), b = (int)(chunk % NB);
  const int c = lane & 15, h = lane >> 4;
  const int n = 16 * b + c;
  u32x4 w;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // canonical word row r = k/8: W4A16 k = 128g + 32t + 8h; W4A8 k = 128g + 64u + 16h + 8s
    const int r = kW4A8 ? 16 * g + 8 * (t >> 1) + 2 * h + (t & 1) : 16 * g + 4 * t + h;
    uint32_t src = codes[(size_t)r * N + n];
    if (kW4A8) src ^= 0x88888888u;   // two's-complement q -> q + 8 in every nibble
    w[t] = permute_nibbles<kW4A8>(src);
  }
  reinterpret_cast<u32x4*>(out)[tid] = w;
}

// One thread per (block, 8-group set, column): 8 group scales of one column.
template <typename T>
__global__ void repack_scales(const T* __restrict__ s, T* __restrict__ out, int G, int G8, int N,
                              int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int c = (int)(tid % 16);
  const int64_t bg = tid / 16;
  const int b = (int)(bg / G8), g8 = (int)(bg % G8);
  const int n = 16 * b + c;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = 8 * g8 + j;
    out[tid * 8 + j] = g < G ? s[(size_t)g * N + n] : T(0);
  }
}

__global__ void copy_halves(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// One thread per (chunk, lane) of the mixed format: base words and, for 4-bit
// groups, the high words at the slot the descriptor table assigns.
__global__ void repack_w2w4_kernel(const uint8_t* __restrict__ codes, const u32x2* __restrict__ desc,
                                   u32x2* __restrict__ base, u32x2* __restrict__ high, int G, int N,
                                   int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  const int64_t chunk = tid >> 6;
  const int g = (int)(chunk / (N / 16));
  const int c = lane & 15, h = lane >> 4;
  const int n = 16 * (int)(chunk % (N / 16)) + c;
  u32x2 lo = {0u, 0u}, hi = {0u, 0u};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int e = sigma_inv(p);
      const int k0 = 128 * g + 64 * s + 8 * h + e;   // W4A16 word 2s
      const uint32_t q0 = codes[(size_t)k0 * N + n];
      const uint32_t q1 = codes[(size_t)(k0 + 32) * N + n];   // word 2s + 1
      lo[s] |= ((q0 & 3u) << (4 * p)) | ((q1 & 3u) << (4 * p + 2));
      hi[s] |= (((q0 >> 2) & 3u) << (4 * p)) | (((q1 >> 2) & 3u) << (4 * p + 2));
    }
  }
  base[tid] = lo;
  const u32x2 d = desc[chunk];
  if ((d[1] >> c) & 1u) {
    const uint32_t rank = __builtin_popcount(d[1] & ((1u << c) - 1u));
    high[(size_t)(d[0] + rank) * 4 + h] = hi;
  }
}

// One thread per (chunk, lane) of the bit-plane format: 32 codes -> B plane words.
__global__ void repack_bitplane_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ out, int N,
                                       int bits, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  const int64_t chunk = tid >> 6;
  const int NB = N / 16;
  const int g = (int)(chunk / NB), b = (int)(chunk % NB);
  const int c = lane & 15, h = lane >> 4;
  const int n = 16 * b + c;
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int t = 0; t < 32; ++t) {
    const int k = 128 * g + 64 * (t >> 4) + 16 * h + (t & 15);
    const uint32_t u = codes[(size_t)k * N + n];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] |= ((u >> i) & 1u) << t;
  }
  for (int i = 0; i < bits; ++i) out[tid * bits + i] = w[i];
}

// One thread per (chunk, lane) of the 2:4 sparse format: 16 canonical words
// (2 steps x 16 k x ... one column) -> 2 code words and 1 position word.
__global__ void repack_sp24_kernel(const uint32_t* __restrict__ codes, uint32_t* __restrict__ out,
                                   uint32_t* __restrict__ status, int N, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  const int64_t chunk = tid >> 6;
  const int NB = N / 16;
  const int g = (int)(chunk / NB), b = (int)(chunk % NB);
  const int c = lane & 15, h = lane >> 4;
  const int n = 16 * b + c;
  u32x2 w = {0u, 0u};
  uint32_t m = 0, bad = 0;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    // k = 128g + 64st + 16h + 0..15: canonical rows r = k / 8, two words
    const int r0 = 16 * g + 8 * st + 2 * h;
    const uint32_t src[2] = {codes[(size_t)r0 * N + n], codes[(size_t)(r0 + 1) * N + n]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t quad = (src[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;   // positions p at bits 4p
      int p0 = -1, p1 = -1, cnt = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (((quad >> (4 * p)) & 0xFu) != 8u) {
          ++cnt;
          if (p0 < 0) p0 = p;
          else if (p1 < 0) p1 = p;
        }
      }
      if (cnt > 2) bad = 1;
      // complete with the lowest positions not yet kept, then order
      for (int p = 0; p < 4 && p1 < 0; ++p) {
        if (p == p0) continue;
        if (p0 < 0) p0 = p;
        else p1 = p;
      }
      if (p0 > p1) { const int t = p0; p0 = p1; p1 = t; }
      const int v0 = 2 * j, v1 = 2 * j + 1;
      w[st] |= ((quad >> (4 * p0)) & 0xFu) << (4 * sigma(v0));
      w[st] |= ((quad >> (4 * p1)) & 0xFu) << (4 * sigma(v1));
      m |= ((uint32_t)p0 << (16 * st + 2 * v0)) | ((uint32_t)p1 << (16 * st + 2 * v1));
    }
  }
  out[tid * 3] = w[0];
  out[tid * 3 + 1] = w[1];
  out[tid * 3 + 2] = m;
  if (bad) __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread per (group, column) entry of the general-grid format.
__global__ void repack_w4g_entries(const uint16_t* __restrict__ s, const uint8_t* __restrict__ z,
                                   void* __restrict__ out, int N, int P, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int64_t g = tid / N, n = tid % N;
  const int64_t dst = ((g / P) * N + n) * P + g % P;
  if (z) static_cast<uint32_t*>(out)[dst] = (uint32_t)s[tid] | ((uint32_t)(z[tid] & 0xF) << 16);
  else static_cast<uint16_t*>(out)[dst] = s[tid];
}

__global__ void zero_fill16(u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

inline unsigned grid_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

}  // namespace

hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);   // blob sizes are multiples of 256
  const unsigned grid = (unsigned)std::min<int64_t>(4096, (n16 + 255) / 256);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill16, dim3(grid), dim3(256), 0, s, static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_repack_w4a16(const BlobLayout& L, const void* codes, const void* scales,
                               void* packed, hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL((repack_codes_u4<false>), dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(out + L.codes),
                     (int)L.G, (int)L.N, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = L.NB * L.G8 * 16;
  hipLaunchKernelGGL((repack_scales<uint16_t>), dim3(grid_for(ns, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), reinterpret_cast<uint16_t*>(out + L.scales),
                     (int)L.G, (int)L.G8, (int)L.N, ns);
  return hipGetLastError();
}

hipError_t launch_repack_sp24(const BlobLayout& L, const void* codes, const void* scales, void* packed,
                              hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL(repack_sp24_kernel, dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(out + L.codes),
                     reinterpret_cast<uint32_t*>(out + L.high), (int)L.N, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = L.NB * L.G8 * 16;
  hipLaunchKernelGGL((repack_scales<uint16_t>), dim3(grid_for(ns, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), reinterpret_cast<uint16_t*>(out + L.scales),
                     (int)L.G, (int)L.G8, (int)L.N, ns);
  return hipGetLastError();
}

hipError_t launch_repack_bitplane(const BlobLayout& L, int bits, const void* codes, const void* cscales,
                                  void* packed, hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL(repack_bitplane_kernel, dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(codes), reinterpret_cast<uint32_t*>(out + L.codes), (int)L.N,
                     bits, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(copy_halves, dim3(grid_for(L.N, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(cscales), reinterpret_cast<uint16_t*>(out + L.aux),
                     (int)L.N);
  return hipGetLastError();
}

hipError_t launch_repack_w4g(const BlobLayout& L, int gs, const void* codes, const void* scales,
                             const void* zeros, void* packed, hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL((repack_codes_u4<false>), dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(out + L.codes),
                     (int)L.G, (int)L.N, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ne = (L.K / gs) * L.N;
  hipLaunchKernelGGL(repack_w4g_entries, dim3(grid_for(ne, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                     static_cast<void*>(out + L.scales), (int)L.N, gs == 64 ? 2 : 1, ne);
  return hipGetLastError();
}

hipError_t launch_repack_w4a8(const BlobLayout& L, const void* codes, const void* gscales,
                              const void* cscales, void* packed, hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL((repack_codes_u4<true>), dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(out + L.codes),
                     (int)L.G, (int)L.N, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = L.NB * L.G8 * 16;
  hipLaunchKernelGGL((repack_scales<int8_t>), dim3(grid_for(ns, 256)), dim3(256), 0, s,
                     static_cast<const int8_t*>(gscales), reinterpret_cast<int8_t*>(out + L.scales),
                     (int)L.G, (int)L.G8, (int)L.N, ns);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(copy_halves, dim3(grid_for(L.N, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(cscales), reinterpret_cast<uint16_t*>(out + L.aux),
                     (int)L.N);
  return hipGetLastError();
}

hipError_t launch_repack_w2w4(const BlobLayout& L, const void* codes, const void* scales,
                              void* packed, hipStream_t s) {
  char* out = static_cast<char*>(packed);
  const int64_t nc = L.NB * L.G * 64;
  hipLaunchKernelGGL(repack_w2w4_kernel, dim3(grid_for(nc, 256)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(codes), reinterpret_cast<const u32x2*>(out + L.aux),
                     reinterpret_cast<u32x2*>(out + L.codes), reinterpret_cast<u32x2*>(out + L.high),
                     (int)L.G, (int)L.N, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = L.NB * L.G8 * 16;
  hipLaunchKernelGGL((repack_scales<uint16_t>), dim3(grid_for(ns, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), reinterpret_cast<uint16_t*>(out + L.scales),
                     (int)L.G, (int)L.G8, (int)L.N, ns);
  return hipGetLastError();
}

}  // namespace qg
