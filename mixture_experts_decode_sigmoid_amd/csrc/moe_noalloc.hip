// moe_noalloc.hip -- moe_forward for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same fused kernel, with its workspace (per-CU epoch
// flags, the error word, the tagged score slots and the mid values) in a
// file-scope device array instead of a caller-provided buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in): the first call on a device, with that
// device current, takes the device address with hipGetSymbolAddress, clears
// the words that must start at zero with a fill kernel on the call's stream,
// and keeps the address per device.  Every later call on that device passes
// that address to the kernel as its workspace.
#include "moe.h"
#include "moe_internal.h"

#include <atomic>
#include <mutex>

// Large enough for every configuration the library accepts: 64 rows, 256
// experts, top-8 and intermediates up to 4096 need 4,993,280 bytes.
static constexpr size_t kScratchBytes = 5u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct ScratchDev {
  std::atomic<int> ready{0};
  void* ptr = nullptr;
};
ScratchDev g_scratch[moe::kMaxDevices];
std::mutex g_setup;

__global__ void clear_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Bytes at the start of the workspace that must be zero before the first
// call: the flags, the error word and the score slots of the largest
// configuration (the mid values need no initial value).
size_t zero_prefix() {
  const moe::WsLayout L = moe::ws_layout(moe::kMaxRows, moe::kMaxExperts, moe::kMaxTopK, 8192, 4096, 4096);
  return L.mid;
}

// The device address of this device's scratch, set up on first use.
int scratch_ptr(int dev, hipStream_t stream, void** out) {
  ScratchDev& d = g_scratch[dev];
  if (d.ready.load(std::memory_order_acquire)) {
    *out = d.ptr;
    return MOE_OK;
  }
  std::lock_guard<std::mutex> g(g_setup);
  if (!d.ready.load(std::memory_order_relaxed)) {
    // the clearing launch must not become part of a captured graph (a
    // replay would clear the flags under later calls)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) {
      moe::set_last_hip((int)e);
      return MOE_ERR_HIP;
    }
    if (cs != hipStreamCaptureStatusNone) return MOE_ERR_WORKSPACE;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      moe::set_last_hip((int)(e != hipSuccess ? e : hipErrorInvalidSymbol));
      return MOE_ERR_HIP;
    }
    const size_t n = zero_prefix() / 4;
    hipLaunchKernelGGL(clear_words, dim3(256), dim3(256), 0, stream, (uint32_t*)ptr, n);
    e = hipGetLastError();
    if (e != hipSuccess) {
      moe::set_last_hip((int)e);
      return MOE_ERR_HIP;
    }
    d.ptr = ptr;
    d.ready.store(1, std::memory_order_release);
  }
  *out = d.ptr;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                                   uint16_t* out, void* stream) {
  size_t need = 0;
  int rc = moe_workspace_size(cfg, &need);
  if (rc) return rc;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  if (rows == 0) return MOE_OK;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= moe::kMaxDevices) {
    moe::set_last_hip((int)(e != hipSuccess ? e : hipErrorInvalidDevice));
    return MOE_ERR_HIP;
  }
  void* ws = nullptr;
  rc = scratch_ptr(dev, (hipStream_t)stream, &ws);
  if (rc) return rc;
  return moe::forward_checked(cfg, w, x, rows, nullptr, out, ws, kScratchBytes, stream);
}
