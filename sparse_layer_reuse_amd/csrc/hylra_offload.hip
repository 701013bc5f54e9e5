// Index-guided gather of selected KV blocks for gfx950.
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.4 (hardware-efficient optimisations): when
// the KV cache does not fit on the device it is kept in host memory, and the
// indices a reuse layer carries name in advance the only blocks it will read,
// so just those are brought to the device instead of the whole cache.
//
// A reuse layer's blocks are known once its source reset layer has selected
// them, so the gather can run on a copy stream while the layers in between
// compute.  One workgroup copies one selected (block, KV head) pair: the
// block's K slab [128][d] and V slab [4][d][32] of that head, each contiguous
// in the pool, to staging page b * k + r.  The source is read once with
// 16-byte loads, all issued before the first store, so each workgroup keeps a
// whole slab pair in flight across the host link.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "hylra_internal.h"

namespace hylra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kMaxVecPerThread = 16;  // 65536-byte slab (float32, d = 128) / 256 threads / 16 B

__global__ __launch_bounds__(kGatherThreads) void gather_blocks(GatherArgs a) {
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int T = a.ctx[b];
  T = T < 0 ? 0 : (T > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : T);
  const int n = a.idx[((int64_t)b * a.num_kv_heads + g) * a.k + r];
  if (n < 0 || n >= (T + kBlockTokens - 1) / kBlockTokens) return;  // padding or past the context
  const int page = a.table[(int64_t)b * a.max_blocks + n];
  if (page < 0 || page >= a.num_pages) return;  // an empty block: never read
  const int64_t src = ((int64_t)page * a.num_kv_heads + g) * a.tile_bytes;
  const int64_t dst = (((int64_t)b * a.k + r) * a.num_kv_heads + g) * a.tile_bytes;
  const int nvec = a.tile_bytes / (16 * kGatherThreads);  // 4, 8 or 16
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(a.k_src + src);
  const u32x4 *vs = reinterpret_cast<const u32x4 *>(a.v_src + src);
  u32x4 *kd = reinterpret_cast<u32x4 *>(a.k_dst + dst);
  u32x4 *vd = reinterpret_cast<u32x4 *>(a.v_dst + dst);
  u32x4 kv[kMaxVecPerThread], vv[kMaxVecPerThread];
#pragma unroll
  for (int i = 0; i < kMaxVecPerThread; ++i)
    if (i < nvec) {
      kv[i] = __builtin_nontemporal_load(ks + threadIdx.x + i * kGatherThreads);
      vv[i] = __builtin_nontemporal_load(vs + threadIdx.x + i * kGatherThreads);
    }
#pragma unroll
  for (int i = 0; i < kMaxVecPerThread; ++i)
    if (i < nvec) {
      kd[threadIdx.x + i * kGatherThreads] = kv[i];
      vd[threadIdx.x + i * kGatherThreads] = vv[i];
    }
}

// Events for cross-stream waits, one pool per device, grown on demand and
// kept until the process ends.
struct EventPool {
  std::mutex mu;
  std::vector<std::vector<hipEvent_t>> per_device;
};
EventPool g_events;

hipError_t pool_event(int slot, hipEvent_t *ev) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_events.mu);
  if ((int)g_events.per_device.size() <= dev) g_events.per_device.resize(dev + 1);
  std::vector<hipEvent_t> &v = g_events.per_device[dev];
  while ((int)v.size() <= slot) {
    hipEvent_t e;
    err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return err;
    v.push_back(e);
  }
  *ev = v[slot];
  return hipSuccess;
}

}  // namespace

int launch_gather(const GatherArgs &a, int batch, void *stream) {
  void *start = nullptr, *stop = nullptr;
  timer_take(kTimerGather, &start, &stop);
  hipExtLaunchKernelGGL(gather_blocks, dim3(a.k, a.num_kv_heads, batch), dim3(kGatherThreads), 0,
                        static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start),
                        static_cast<hipEvent_t>(stop), 0, a);
  return (int)hipGetLastError();
}

int pool_readable(const void *base, size_t bytes, int *readable) {
  *readable = 0;
  const char *ends[2] = {static_cast<const char *>(base),
                         static_cast<const char *>(base) + (bytes ? bytes - 1 : 0)};
  for (const char *p : ends) {
    hipPointerAttribute_t at;
    const hipError_t err = hipPointerGetAttributes(&at, p);
    if (err != hipSuccess) {
      (void)hipGetLastError();  // an unknown pointer is an answer, not a sticky error
      return 0;
    }
    const bool dev = at.type == hipMemoryTypeDevice;
    const bool mapped_host = at.type == hipMemoryTypeHost && at.devicePointer == (void *)p;
    if (!dev && !mapped_host) return 0;
  }
  *readable = 1;
  return 0;
}

int event_record(void *stream, int slot) {
  hipEvent_t ev;
  hipError_t err = pool_event(slot, &ev);
  if (err != hipSuccess) return (int)err;
  return (int)hipEventRecord(ev, static_cast<hipStream_t>(stream));
}

int event_wait(void *stream, int slot) {
  hipEvent_t ev;
  hipError_t err = pool_event(slot, &ev);
  if (err != hipSuccess) return (int)err;
  return (int)hipStreamWaitEvent(static_cast<hipStream_t>(stream), ev, 0);
}

}  // namespace hylra
