// hylra_run_policy for callers that cannot allocate device memory: the
// workspace (arrival counters, split partials, block masses, the carried
// index set) is a statically sized device array of the library instead of a
// caller buffer.
//
// Each device the library runs on holds its own copy of `scratch` for the
// life of the process.  Host code never names the array directly (in host
// code its name is a host-side stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress and that
// pointer is what the launches receive.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "../../include/hylra.h"
#include "hylra_internal.h"

namespace {

constexpr size_t kScratchBytes = HYLRA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once set up

// Zero-fills `words` 32-bit words (the arrival counters at the head of the
// workspace must start at zero; every launch leaves them at zero).
__global__ void clear_words(uint32_t *p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Device address of this device's scratch array, set up on the first call
// on the device: symbol lookup, then the counter region cleared on `stream`.
int scratch_for_current_device(void *stream, void **out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return (int)err;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return (int)err;
    const size_t words = (size_t)hylra::kCounterSlots;
    hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t *>(ptr), words);
    err = hipGetLastError();
    if (err != hipSuccess) return (int)err;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace

extern "C" hylra_status hylra_run_policy_noalloc(const hylra_shape *shape, int32_t num_layers,
                                                 const int32_t *src, int32_t k,
                                                 const void *const *q, const hylra_kv *kv,
                                                 float *const *out, float *const *lse,
                                                 int32_t *idx_log, void *hip_stream) {
  size_t need = 0;
  if (hylra_status st = hylra_workspace_size(shape, k, &need)) return st;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "shape needs %zu bytes of workspace; the static scratch holds %zu "
             "(use hylra_run_policy with a caller workspace)",
             need, kScratchBytes);
    return hylra::report_error(HYLRA_E_WORKSPACE, msg);
  }
  void *ws = nullptr;
  if (int err = scratch_for_current_device(hip_stream, &ws)) {
    char msg[256];
    snprintf(msg, sizeof msg, "static scratch set-up: %s", hylra::device_error_string(err));
    return hylra::report_error(HYLRA_E_DEVICE, msg);
  }
  return hylra_run_policy(shape, num_layers, src, k, q, kv, out, lse, idx_log, ws, kScratchBytes,
                          hip_stream);
}
