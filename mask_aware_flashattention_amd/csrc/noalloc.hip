// Forward attention without a caller-supplied workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as flashmask_fwd; the workspace (block min/max, tile
// lists, block order) lives in a fixed file-scope device array instead.
//
// The array is a device symbol, so host code cannot use its name as an address: on first use on
// a device (with that device current) its device address is looked up once with
// hipGetSymbolAddress and kept per device; every launch receives that address.  Each device
// holds its own copy of the array for the life of the process.  Nothing in it has to start at
// zero: every kernel of the forward writes the parts it later reads.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/flashmask.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_init;

// Device address of `scratch` on the current device, looked up on the first call per device.
int32_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FM_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_init);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return FM_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FM_OK;
}

}  // namespace

extern "C" {

size_t flashmask_fwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int32_t flashmask_fwd_noalloc(const fm_shape* shape, const void* Q, const void* K, const void* V,
                              const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                              const int32_t* UTE, float scale, void* O, float* LSE,
                              void* stream) {
  if (!shape) return FM_ERR_NULL;
  const size_t need = flashmask_fwd_workspace_bytes(shape);
  if (need == 0) {
    // an invalid shape: let the checks of the workspace call report which
    return flashmask_fwd(shape, Q, K, V, LTS, LTE, UTS, UTE, scale, O, LSE, nullptr, 0, stream);
  }
  if (need > kScratchBytes) return FM_ERR_SCRATCH;
  // missing pointers are reported before the device is touched (flashmask_fwd checks the rest)
  if (!Q || !K || !V || !O || !LSE || !LTS || !LTE || !UTS || !UTE) return FM_ERR_NULL;
  void* ws = nullptr;
  const int32_t st = scratch_address(&ws);
  if (st != FM_OK) return st;
  return flashmask_fwd(shape, Q, K, V, LTS, LTE, UTS, UTE, scale, O, LSE, ws, kScratchBytes,
                       stream);
}

}  // extern "C"
