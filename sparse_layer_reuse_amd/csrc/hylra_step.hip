// Decode-step helpers for gfx950 around the hybrid attention: the rotary
// embedding of the new token's q and k fused with the append of its k and v
// into the paged cache, and the SiLU-gated product of a SwiGLU MLP.  They
// serve the end-to-end decode step (projections and MLP on the GPU BLAS),
// one launch each instead of a chain of elementwise ones.
//
// Rotary embedding in the rotate-half form (as in Llama-3): dimensions
// i < d/2 and i + d/2 of a head vector are rotated by the angle whose cosine
// and sine the caller passes per (sequence, i), in float32, rounded once to
// bf16 at the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hylra_internal.h"

namespace hylra {
namespace {

typedef unsigned short bf16_bits;

__device__ __forceinline__ float bf16_to_f32(bf16_bits x) {
  return __uint_as_float((uint32_t)x << 16);
}

// Round to nearest even (finite inputs; NaN keeps a quiet payload).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (bf16_bits)((u >> 16) | 0x40);
  return (bf16_bits)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

constexpr int kStepThreads = 256;
constexpr int kRopeThreads = 64;  // one wavefront per head vector

// Workgroup (h, b) handles head vector h of sequence b's row of qkv, all of
// whose elements are independent, so every head runs in parallel: h < Hq is
// a q head, rotated into q_out; Hq <= h < Hq + Hkv a k head, rotated into the
// page of position pos[b]; the remaining Hkv heads are v heads, copied as
// they are into the page's V sub-tile column.  A rotated pair is
// (x_i c - x_{i+d/2} s, x_{i+d/2} c + x_i s) for i < d/2.
__global__ __launch_bounds__(kRopeThreads) void rope_append(RopeAppendArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = a.head_dim, half = d / 2;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const bf16_bits *row = static_cast<const bf16_bits *>(a.qkv) + ((int64_t)b * (hq + 2 * hkv) + h) * d;
  int page = -1, slot = 0;
  if (h >= hq) {  // k and v heads go to the page of position pos[b], if it has one
    const int t = a.pos[b];
    if (t >= 0 && t < a.max_blocks * kBlockTokens) {
      const int p = a.table[(int64_t)b * a.max_blocks + t / kBlockTokens];
      if (p >= 0 && p < a.num_pages) page = p;
      slot = t % kBlockTokens;
    }
    if (page < 0) return;
  }
  if (h < hq + hkv) {
    const float *c = a.cos_tab + (int64_t)b * half;
    const float *s = a.sin_tab + (int64_t)b * half;
    bf16_bits *dst;
    if (h < hq) {
      dst = static_cast<bf16_bits *>(a.q_out) + ((int64_t)b * hq + h) * d;
    } else {
      const int64_t tile = (int64_t)page * hkv + (h - hq);
      dst = static_cast<bf16_bits *>(a.k_pool) + (tile * kBlockTokens + slot) * d;
    }
    for (int i = threadIdx.x; i < half; i += kRopeThreads) {
      const float x0 = bf16_to_f32(row[i]), x1 = bf16_to_f32(row[i + half]);
      dst[i] = f32_to_bf16(x0 * c[i] - x1 * s[i]);
      dst[i + half] = f32_to_bf16(x1 * c[i] + x0 * s[i]);
    }
  } else {
    const int64_t tile = (int64_t)page * hkv + (h - hq - hkv);
    bf16_bits *vp = static_cast<bf16_bits *>(a.v_pool) +
                    (tile * kChunksPerBlock + slot / kChunkTokens) * d * kChunkTokens + slot % kChunkTokens;
    for (int ch = threadIdx.x; ch < d; ch += kRopeThreads) vp[(int64_t)ch * kChunkTokens] = row[ch];
  }
}

// silu(gate) * up for rows of [gate | up] ([rows][2 * width] -> [rows][width]).
__global__ __launch_bounds__(kStepThreads) void silu_mul(const bf16_bits *gu, bf16_bits *out,
                                                         int64_t rows, int width) {
  const int64_t n = rows * width;
  for (int64_t e = (int64_t)blockIdx.x * kStepThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kStepThreads) {
    const int64_t r = e / width;
    const int col = (int)(e % width);
    const float g = bf16_to_f32(gu[r * 2 * width + col]);
    const float u = bf16_to_f32(gu[r * 2 * width + width + col]);
    out[e] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
  }
}

}  // namespace

int launch_rope_append(const RopeAppendArgs &a, int batch, void *stream) {
  hipLaunchKernelGGL(rope_append, dim3(a.num_q_heads + 2 * a.num_kv_heads, batch), dim3(kRopeThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_silu_mul(const void *gu, void *out, int64_t rows, int width, void *stream) {
  const int64_t n = rows * width;
  int64_t grid = (n + kStepThreads - 1) / kStepThreads;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(silu_mul, dim3((unsigned)grid), dim3(kStepThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16_bits *>(gu),
                     static_cast<bf16_bits *>(out), rows, width);
  return (int)hipGetLastError();
}

}  // namespace hylra
