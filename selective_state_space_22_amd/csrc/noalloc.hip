// noalloc.hip -- mamba_scan_fwd_noalloc: the forward scan for callers that
// cannot allocate device memory (code under graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The workspace that mamba_scan_fwd takes from its caller (chained-chunk
// flags and carries, split-pass aggregates) comes here from a fixed array in
// the library's device image: one copy per GPU, allocated when the code
// object is loaded and held until the process ends.  Host code never passes
// the array's name to a kernel: on the host that name is only a stand-in, so
// its device address is fetched once per device with hipGetSymbolAddress and
// that address is what the kernels get.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/mamba_mi355x.h"

namespace {

constexpr size_t kScratchBytes = MAMBA_SCAN_FWD_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on each device (nullptr if the lookup fails).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int mamba_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                                      const void* u, const void* delta, const float* delta_bias, const float* A,
                                      const void* B, const void* C, const float* Dskip, const void* z,
                                      int delta_softplus, const float* h0, void* out, float* last_state,
                                      void* stream) {
  // Shapes mamba_scan_fwd rejects report a size of 0: mamba_scan_fwd then
  // rejects them itself with the usual status.
  const size_t need = mamba_scan_fwd_workspace_size(batch, seqlen, dim, dstate, io_dtype);
  if (need > kScratchBytes) return MAMBA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return MAMBA_ERR_HIP;
  }
  return mamba_scan_fwd(batch, seqlen, dim, dstate, io_dtype, u, delta, delta_bias, A, B, C, Dskip, z,
                        delta_softplus, h0, out, last_state, ws, ws ? kScratchBytes : 0, stream);
}
