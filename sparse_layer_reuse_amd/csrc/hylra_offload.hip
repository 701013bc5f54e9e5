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
// compute.  The unit of work is one selected (block, KV head) pair: the
// block's K slab [128][d] and V slab [4][d][32] of that head, each contiguous
// in the pool, copied to staging page b * k + r.  The source is read once
// with 16-byte loads.  The host link is saturated by a few hundred KiB in
// flight, so the gather runs as a small grid of one-wavefront workgroups
// (kGatherWorkgroups, each walking the slab pairs with a stride and keeping
// 8 KiB in flight) that use few registers: a workgroup of the kernels it
// overlaps with (the projections' GEMMs) still fits on the same compute
// unit, where a larger gather workgroup would hold it back until the
// transfer ends.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "hylra_internal.h"

namespace hylra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 64;      // one wavefront
constexpr int kGatherWorkgroups = 16;
constexpr int kGatherVec = 8;           // 16-byte loads in flight per lane (8 KiB per workgroup)

// Copies slab pair (b, g, r) if its selected block is readable: the K slab
// then the V slab, each tile_bytes, in batches of kGatherVec loads per lane
// issued before their stores.
__device__ __forceinline__ void gather_pair(const GatherArgs &a, int b, int g, int r) {
  int T = a.ctx[b];
  T = T < 0 ? 0 : (T > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : T);
  const int n = a.idx[((int64_t)b * a.num_kv_heads + g) * a.k + r];
  if (n < 0 || n >= (T + kBlockTokens - 1) / kBlockTokens) return;  // padding or past the context
  const int page = a.table[(int64_t)b * a.max_blocks + n];
  if (page < 0 || page >= a.num_pages) return;  // an empty block: never read
  const int64_t src = ((int64_t)page * a.num_kv_heads + g) * a.tile_bytes;
  const int64_t dst = (((int64_t)b * a.k + r) * a.num_kv_heads + g) * a.tile_bytes;
  const int nvec = a.tile_bytes / 16;  // per slab; a multiple of kGatherThreads * kGatherVec
  const u32x4 *srcs[2] = {reinterpret_cast<const u32x4 *>(a.k_src + src),
                          reinterpret_cast<const u32x4 *>(a.v_src + src)};
  u32x4 *dsts[2] = {reinterpret_cast<u32x4 *>(a.k_dst + dst), reinterpret_cast<u32x4 *>(a.v_dst + dst)};
#pragma unroll
  for (int t = 0; t < 2; ++t)
    for (int v0 = 0; v0 < nvec; v0 += kGatherThreads * kGatherVec) {
      u32x4 x[kGatherVec];
#pragma unroll
      for (int i = 0; i < kGatherVec; ++i)
        x[i] = __builtin_nontemporal_load(srcs[t] + v0 + i * kGatherThreads + threadIdx.x);
#pragma unroll
      for (int i = 0; i < kGatherVec; ++i) dsts[t][v0 + i * kGatherThreads + threadIdx.x] = x[i];
    }
}

// Workgroup w takes slab pairs p = w, w + gridDim.x, ... of the B * Hkv * k
// pairs, p = (b * Hkv + g) * k + r.
__global__ __launch_bounds__(kGatherThreads) void gather_blocks(GatherArgs a, int batch) {
  const int64_t pairs = (int64_t)batch * a.num_kv_heads * a.k;
  for (int64_t p = blockIdx.x; p < pairs; p += gridDim.x) {
    const int r = (int)(p % a.k);
    const int64_t bg = p / a.k;
    gather_pair(a, (int)(bg / a.num_kv_heads), (int)(bg % a.num_kv_heads), r);
  }
}

// Append of one decode step's K and V: thread (g, c) of workgroup b writes
// element c of KV head g of the new token at position pos[b] -- K row
// [page][g][slot][c] and V column [page][g][slot / 32][c][slot % 32].  The
// pools may be pinned host memory the device maps (an offloaded layer).
__global__ __launch_bounds__(256) void append_token(AppendArgs a) {
  const int b = blockIdx.x;
  const int t = a.pos[b];
  if (t < 0 || t >= a.max_blocks * kBlockTokens) return;
  const int page = a.table[(int64_t)b * a.max_blocks + t / kBlockTokens];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = t % kBlockTokens;
  const int row = a.num_kv_heads * a.head_dim;
  for (int e = threadIdx.x; e < row; e += blockDim.x) {
    const int g = e / a.head_dim, c = e % a.head_dim;
    const int64_t tile = (int64_t)page * a.num_kv_heads + g;
    const int64_t k_at = (tile * kBlockTokens + slot) * a.head_dim + c;
    const int64_t v_at = ((tile * kChunksPerBlock + slot / kChunkTokens) * a.head_dim + c) *
                             kChunkTokens + slot % kChunkTokens;
    const int64_t src = (int64_t)b * row + e;
    if (a.elt == 2) {
      reinterpret_cast<uint16_t *>(a.k_pool)[k_at] = reinterpret_cast<const uint16_t *>(a.k_new)[src];
      reinterpret_cast<uint16_t *>(a.v_pool)[v_at] = reinterpret_cast<const uint16_t *>(a.v_new)[src];
    } else {
      reinterpret_cast<uint32_t *>(a.k_pool)[k_at] = reinterpret_cast<const uint32_t *>(a.k_new)[src];
      reinterpret_cast<uint32_t *>(a.v_pool)[v_at] = reinterpret_cast<const uint32_t *>(a.v_new)[src];
    }
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
  const int64_t pairs = (int64_t)batch * a.num_kv_heads * a.k;
  const int grid = (int)(pairs < kGatherWorkgroups ? pairs : kGatherWorkgroups);
  hipExtLaunchKernelGGL(gather_blocks, dim3(grid), dim3(kGatherThreads), 0,
                        static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start),
                        static_cast<hipEvent_t>(stop), 0, a, batch);
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

int launch_append(const AppendArgs &a, int batch, void *stream) {
  hipLaunchKernelGGL(append_token, dim3(batch), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
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
