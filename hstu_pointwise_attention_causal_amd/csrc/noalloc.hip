// hstu_attn_fwd_noalloc: the attention forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). It runs exactly the kernels of
// hstu_attn_fwd, with their workspace (the clamped offsets, the work list and
// the per-block metadata) in a fixed array of device memory that the library
// itself holds, instead of a caller-passed workspace.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy until the process ends, at its own address. Host code
// never uses the array's name as an address (on the host it is only a
// stand-in symbol); the first call on a device, with that device current,
// looks the address up with hipGetSymbolAddress and keeps it per device.
//
// Every call on a GPU shares that GPU's array. The work-list builder, the
// call's first kernel, initialises everything the later kernels read
// (counters included), so nothing has to be cleared between calls; but two
// calls that overlap in time on one GPU (different streams, or different host
// threads without ordering) race on the array and may corrupt each other's
// results.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/hstu.h"
#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
hstu_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hstu::api_fail(HSTU_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return hstu::api_fail(HSTU_E_UNSUPPORTED, "device index %d beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return hstu::api_fail(HSTU_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HSTU_OK;
}

}  // namespace

extern "C" {

hstu_status_t hstu_attn_fwd_noalloc(const hstu_attn_desc_t* desc, const hstu_jagged_t* jag,
                                    const hstu_bias_t* bias, const void* q, int64_t ldq, const void* k, int64_t ldk,
                                    const void* v, int64_t ldv, void* o, int64_t ldo, void* hip_stream) {
  size_t need = 0;
  hstu_status_t st = hstu_attn_workspace_size(desc, jag, bias, 0, &need);
  if (st != HSTU_OK) return st;
  if (need > kScratchBytes)
    return hstu::api_fail(HSTU_E_UNSUPPORTED,
                          "this batch needs %zu bytes of workspace; the allocation-free entry point holds %zu "
                          "(use hstu_attn_fwd with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != HSTU_OK) return st;
  return hstu_attn_fwd(desc, jag, bias, q, ldq, k, ldk, v, ldv, o, ldo, ws, kScratchBytes, hip_stream);
}

}  // extern "C"
