// W4A16 GEMM entry point for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same kernels and plans as qgemm_w4a16, with the split-K
// workspace (arrival counters and partial sums) taken from a fixed device
// array of this library instead of a caller-provided buffer.
//
// The array is a file-scope __device__ object: each GPU the library runs on
// holds its own copy at its own address for the life of the process. Host
// code never uses the array's name as a device address (on the host it names
// a host-side stand-in); the address comes from hipGetSymbolAddress, queried
// once per device with that device current, and is cached per device.
#include "qgemm.h"

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>

#include "qgemm_internal.h"

namespace {

// counters (64 KiB) plus partial sums: covers every automatic W4A16 plan
// (the largest, 16 MiB + 64 KiB, is the wide kernel's four k-splits at M = 65-128
// on 28672 x 8192)
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;
  bool cleared = false;   // the counter region has been cleared on some stream
};
std::mutex g_mu;
std::map<int, DeviceScratch> g_scratch;

// Device address of this device's scratch array (set up on first use).
int scratch_for_current_device(void** ptr, bool* first) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qg::fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceScratch& d = g_scratch[dev];
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return qg::fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
    d.ptr = p;
  }
  *ptr = d.ptr;
  *first = !d.cleared;
  return QGEMM_OK;
}

void mark_cleared() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_scratch[dev].cleared = true;
}

}  // namespace

extern "C" {

int qgemm_w4a16_noalloc(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
                        int64_t K, int64_t N, void* stream) {
  // shape, pointer and device checks first, exactly as qgemm_w4a16 (whose
  // validation runs again below, before any launch)
  size_t need = 0;
  int st = qgemm_workspace_bytes(QGEMM_FMT_W4A16, M, K, N, &need);
  if (st != QGEMM_OK) return st;
  if (M == 0) return QGEMM_OK;
  if (need > kScratchBytes) {
    qg::set_last_error("this call's plan needs " + std::to_string(need) + " bytes of split-K scratch; the "
                       "built-in scratch holds " + std::to_string(kScratchBytes));
    return QGEMM_ERR_WORKSPACE;
  }
  st = qg::validate_w4a16(A, lda, packed, C, ldc, M, K, N);
  if (st != QGEMM_OK) return st;
  void* ws = nullptr;
  bool first = false;
  st = scratch_for_current_device(&ws, &first);
  if (st != QGEMM_OK) return st;
  if (first) {
    // the counters must start at zero; completed calls leave them zero again
    const hipError_t e = qg::launch_zero_fill(ws, qg::kCounterBytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return qg::fail_hip(e, "scratch clear");
    mark_cleared();
  }
  return qgemm_w4a16(A, lda, packed, C, ldc, M, K, N, need ? ws : nullptr, need ? kScratchBytes : 0, stream);
}

}  // extern "C"
