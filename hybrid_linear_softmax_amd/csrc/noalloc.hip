// hybrid_attn_group for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops): the linear layers' workspace is a
// file-scope device array of fixed size instead of a caller buffer.
//
// Each device that loads the library holds its own copy of the array until the
// process ends.  Its address on a device is taken once, with that device
// current, through hipGetSymbolAddress (in host code the array's name is only a
// host-side stand-in, never a device address) and kept per device.  All calls
// on one device share that device's array: calls that overlap on one device
// (concurrent streams, threads) race on it.  The linear layers write every
// workspace element they read within the same call, so nothing has to be
// cleared between calls.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/hybrid_attn.h"

namespace {

constexpr size_t kScratchBytes = size_t{HA_NOALLOC_SCRATCH_BYTES};
static_assert(kScratchBytes % 256 == 0, "scratch size is a multiple of the workspace alignment");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The array's device address on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

HA_API int hybrid_attn_group_noalloc(const void* Q4, const void* K4, const void* V4, const void* G4, void* O4,
                                     int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream) {
  // the size check touches no device state; an invalid or empty problem needs
  // no workspace and gets the group's own status
  const size_t need = hybrid_attn_workspace_bytes(B, H, N, d, dtype);
  if (need > kScratchBytes) return HA_EWORKSPACE;
  if (need == 0 || N == 0) return hybrid_attn_group(Q4, K4, V4, G4, O4, B, H, N, d, dtype, nullptr, 0, stream);
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return HA_EHIP;
  return hybrid_attn_group(Q4, K4, V4, G4, O4, B, H, N, d, dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
