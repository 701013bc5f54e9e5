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

// Workgroup b: for every head h of q and k and pair i < d/2, the rotated pair
// (x_i c - x_{i+d/2} s, x_{i+d/2} c + x_i s); q heads go to q_out, the k
// heads and the unrotated v heads to the page of position pos[b].
__global__ __launch_bounds__(kStepThreads) void rope_append(RopeAppendArgs a) {
  const int b = blockIdx.x;
  const int d = a.head_dim, half = d / 2;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const bf16_bits *row = static_cast<const bf16_bits *>(a.qkv) + (int64_t)b * (hq + 2 * hkv) * d;
  const float *c = a.cos_tab + (int64_t)b * half;
  const float *s = a.sin_tab + (int64_t)b * half;
  const int t = a.pos[b];
  int page = -1, slot = 0;
  if (t >= 0 && t < a.max_blocks * kBlockTokens) {
    const int p = a.table[(int64_t)b * a.max_blocks + t / kBlockTokens];
    if (p >= 0 && p < a.num_pages) page = p;
    slot = t % kBlockTokens;
  }
  bf16_bits *kp = static_cast<bf16_bits *>(a.k_pool);
  bf16_bits *vp = static_cast<bf16_bits *>(a.v_pool);
  bf16_bits *q_out = static_cast<bf16_bits *>(a.q_out) + (int64_t)b * hq * d;
  // rotated heads: q heads 0..hq-1, then k heads
  for (int e = threadIdx.x; e < (hq + hkv) * half; e += kStepThreads) {
    const int h = e / half, i = e % half;
    const float x0 = bf16_to_f32(row[h * d + i]), x1 = bf16_to_f32(row[h * d + i + half]);
    const bf16_bits y0 = f32_to_bf16(x0 * c[i] - x1 * s[i]);
    const bf16_bits y1 = f32_to_bf16(x1 * c[i] + x0 * s[i]);
    if (h < hq) {
      q_out[h * d + i] = y0;
      q_out[h * d + i + half] = y1;
    } else if (page >= 0) {
      const int64_t tile = (int64_t)page * hkv + (h - hq);
      kp[(tile * kBlockTokens + slot) * d + i] = y0;
      kp[(tile * kBlockTokens + slot) * d + i + half] = y1;
    }
  }
  if (page < 0) return;
  // v heads, as they are: column slot of the page's V sub-tile
  for (int e = threadIdx.x; e < hkv * d; e += kStepThreads) {
    const int g = e / d, ch = e % d;
    const int64_t tile = (int64_t)page * hkv + g;
    vp[((tile * kChunksPerBlock + slot / kChunkTokens) * d + ch) * kChunkTokens + slot % kChunkTokens] =
        row[(hq + hkv + g) * d + ch];
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
  hipLaunchKernelGGL(rope_append, dim3(batch), dim3(kStepThreads), 0, static_cast<hipStream_t>(stream), a);
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
