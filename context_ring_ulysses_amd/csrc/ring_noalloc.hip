// cru_ring_emulate_noalloc: the ring share with its partials in a static
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Declared in include/cru.h.
//
// The array is a file-scope __device__ variable: the runtime places one copy
// on each GPU when this module is first used there, and it stays until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// the kernels receive that address as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cru.h"
#include "cru_kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)CRU_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on first use there).
cru_status current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return cru::report(CRU_EDEVICE, "no current HIP device");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return cru::report(CRU_EDEVICE, "device %d is beyond the %d the library tracks", dev,
                       kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return cru::report(CRU_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                         hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CRU_OK;
}

}  // namespace

extern "C" cru_status cru_ring_emulate_noalloc(const cru_tensor* q_share, const cru_tensor* k,
                                               const cru_tensor* v, int n_chunks, int anything,
                                               const int64_t* chunk_sizes, int fused,
                                               int convert_to_fp32, const cru_tensor* o,
                                               const cru_lse* lse, float scale,
                                               hipStream_t stream) {
  cru::clear_error();
  return cru::ring_emulate_ws(q_share, k, v, n_chunks, anything, chunk_sizes, fused,
                              convert_to_fp32, o, lse, scale, nullptr, kScratchBytes,
                              current_scratch, stream);
}
