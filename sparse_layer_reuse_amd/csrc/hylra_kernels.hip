// HIP kernels of the HyLRA decode-phase hybrid attention for gfx950 (CDNA4).
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.3 (reset layers: full attention + top-k
// extraction; reuse layers: attention over the carried KV subset) and 2.4
// (selection over fixed 128-token blocks).
//
// Kernels
//   attn_split_bf16<D>  split-KV decode attention, bf16 K/V, MFMA
//                       (v_mfma_f32_16x16x32_bf16) for q.K and p.V; one
//                       wavefront consumes 32-token chunks, a workgroup of four
//                       wavefronts merges its partial softmax states in LDS.
//                       Full mode walks every chunk of a sequence, sparse mode
//                       the chunks of the selected blocks (through the table).
//   attn_split_f32<D>   the same contract for float32 K/V on the vector ALU.
//   merge_heads         per (sequence, query head): merges the split partials
//                       into out / lse and turns per-chunk statistics into the
//                       head's probability mass per block.
//   score_topk          per (sequence, KV head): block score = sum of the
//                       group's head masses; radix select of the top-k with the
//                       lower block id winning ties; ascending compaction.
//
// Softmax state is kept in base 2: x = s * scale * log2(e), p = 2^(x - m).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "hylra_internal.h"

namespace hylra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clamp_ctx(int t, int max_blocks) {
  return t < 0 ? 0 : (t > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : t);
}

// Number of 32-token chunk positions of (b, g) in a launch.  Full: every chunk
// of the context.  Sparse: four per selected block (k_eff = min(k, N_b)).
__device__ __forceinline__ int chunk_positions(int T, const int32_t *sel, int k) {
  if (sel == nullptr) return (T + kChunkTokens - 1) / kChunkTokens;
  const int nb = (T + kBlockTokens - 1) / kBlockTokens;
  return kChunksPerBlock * (k < nb ? k : nb);
}

// Resolves chunk position `pos` of (b, g) to its page and the valid tokens.
// Returns false when the chunk holds no token to read (past the context, a
// padding / out-of-range selected id, or a page outside the pool).
__device__ __forceinline__ bool resolve_chunk(const AttnArgs &a, int b, int g, int T, int pos,
                                              int64_t &page, int &sub, int &valid) {
  int n;
  if (a.sel == nullptr) {
    n = pos / kChunksPerBlock;
  } else {
    n = a.sel[((int64_t)b * a.num_kv_heads + g) * a.k + pos / kChunksPerBlock];
    if (n < 0 || n >= (T + kBlockTokens - 1) / kBlockTokens) return false;
  }
  sub = pos % kChunksPerBlock;
  valid = T - (n * kBlockTokens + sub * kChunkTokens);
  if (valid <= 0) return false;
  if (valid > kChunkTokens) valid = kChunkTokens;
  page = a.table[(int64_t)b * a.max_blocks + n];
  return page >= 0 && page < a.num_pages;
}

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Merges the (m, l, o) states of the four wavefronts of a workgroup (LDS) and
// writes the workgroup's partial for split `s`.  sm_o is [4][16][D].
template <int D>
__device__ __forceinline__ void write_wg_partial(const AttnArgs &a, int b, int g, int s,
                                                 const float (*sm_m)[kMaxGroup],
                                                 const float (*sm_l)[kMaxGroup],
                                                 const float (*sm_o)[kMaxGroup][D]) {
  for (int item = threadIdx.x; item < a.group * D; item += kThreads) {
    const int h = item / D, c = item % D;
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = sm_m[w][h] == kNegInf ? 0.f : fast_exp2(sm_m[w][h] - m);
      o += f * sm_o[w][h][c];
      l += f * sm_l[w][h];
    }
    const int64_t row = ((int64_t)b * a.num_q_heads + g * a.group + h) * a.nsplit + s;
    a.part_o[row * D + c] = o;
    if (c == 0) {
      a.part_ml[row * 2 + 0] = m;
      a.part_ml[row * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel.
//
// One 32-token chunk per wavefront step.  Lane i: quad q = i/16, m = i%16.
//   q.K   : two 16x16x32 tiles per k-step.  A = K rows, B = q^T (head m).
//           Tile a, row m loads token 8*(m/4) + 4a + m%4 so that the result
//           lane i holds (head m, tokens 8q .. 8q+7) -- exactly the A-operand
//           layout the p.V product needs, with no cross-lane shuffle.
//   p.V   : A = p (head m, tokens 8q..8q+7), B = V (tokens 8q..8q+7, column
//           16n+m) read as one 16-byte load from the dimension-major V page.
//           p is split into bf16 hi + lo parts (two MFMAs) so the weights
//           keep ~16 mantissa bits.
//   output: lane i holds heads 4q..4q+3, column 16n+m of each 16-column tile.
// ---------------------------------------------------------------------------
template <int D>
struct BfTile {
  u32x4 k[2][D / 32];
  u32x4 v[D / 16];
};

template <int D>
__device__ __forceinline__ void load_bf_tile(BfTile<D> &t, const uint16_t *kbase,
                                             const uint16_t *vbase, int quad, int m16) {
  const int tok = 8 * (m16 >> 2) + (m16 & 3);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      t.k[a][s] = *reinterpret_cast<const u32x4 *>(kbase + (tok + 4 * a) * D + 32 * s + 8 * quad);
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    t.v[n] = *reinterpret_cast<const u32x4 *>(vbase + (16 * n + m16) * kBlockTokens + 8 * quad);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_split_bf16(AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int C = chunk_positions(T, a.sel, a.k);
  const int c_begin = s * a.chunks_per_wg;
  if (c_begin >= C) return;
  const int c_end = min(C, c_begin + a.chunks_per_wg);

  __shared__ float sm_m[kWaves][kMaxGroup];
  __shared__ float sm_l[kWaves][kMaxGroup];
  __shared__ float sm_o[kWaves][kMaxGroup][D];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int quad = lane >> 4, m16 = lane & 15;
  const int G = a.group;

  bf16x8 qop[D / 32];
  {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                           ((int64_t)b * a.num_q_heads + g * G + m16) * D;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m16 < G) v = *reinterpret_cast<const u32x4 *>(qrow + 32 * k + 8 * quad);
      qop[k] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);
  const int Hkv = a.num_kv_heads;
  float *stats_row = a.stats ? a.stats + ((int64_t)b * a.num_q_heads + g * G + m16) *
                                             (int64_t)(kChunksPerBlock * a.max_blocks) * 2
                             : nullptr;

  auto issue = [&](BfTile<D> &t, int pos, int &valid) -> bool {
    int64_t page;
    int sub;
    if (!resolve_chunk(a, b, g, T, pos, page, sub, valid)) {
      if (stats_row != nullptr && quad == 0 && m16 < G) {  // unreadable page: no mass
        stats_row[2 * pos + 0] = kNegInf;
        stats_row[2 * pos + 1] = 0.f;
      }
      return false;
    }
    const int64_t tile = page * Hkv + g;
    load_bf_tile<D>(t, kpool + (tile * kBlockTokens + sub * kChunkTokens) * D,
                    vpool + tile * D * kBlockTokens + sub * kChunkTokens, quad, m16);
    return true;
  };

  auto consume = [&](const BfTile<D> &t, int pos, int valid) {
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[h][k]),
                                                          qop[k], sacc[h], 0, 0, 0);
    }
    // lane holds head m16, token 8*quad + 4*h + r in sacc[h][r]
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 8 * quad + j;
      x[j] = tok < valid ? sacc[j >> 2][j & 3] * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, x[j]);
    }
    mx = wave_max_xor_16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(x[j] - m_new);
      ps += p[j];
    }
    ps = wave_sum_xor_16_32(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (stats_row != nullptr && quad == 0 && m16 < G) {
      stats_row[2 * pos + 0] = m_new;
      stats_row[2 * pos + 1] = ps;
    }
    bf16x8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 hi = (__bf16)p[j];
      phi[j] = hi;
      plo[j] = (__bf16)(p[j] - (float)hi);
    }
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * quad + r);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[n][r] *= al[r];
      u32x4 v = t.v[n];
      if (valid < kChunkTokens) {
        // tokens past the context: p is 0 there, zero V so stale page bytes
        // (possibly NaN patterns) cannot leak in through 0 * NaN.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = 8 * quad + 2 * e;
          uint32_t keep = (tok < valid ? 0x0000FFFFu : 0u) | (tok + 1 < valid ? 0xFFFF0000u : 0u);
          v[e] &= keep;
        }
      }
      const bf16x8 vb = __builtin_bit_cast(bf16x8, v);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, acc[n], 0, 0, 0);
    }
  };

  // Two register tiles: the next chunk's loads are in flight while the
  // current one is consumed.
  BfTile<D> ta, tb;
  int pos = c_begin + w;
  int va = 0, vb = 0;
  bool ha = pos < c_end ? issue(ta, pos, va) : false;
  while (pos < c_end) {
    const int pn = pos + kWaves;
    bool hb = pn < c_end ? issue(tb, pn, vb) : false;
    if (ha) consume(ta, pos, va);
    pos = pn;
    if (pos >= c_end) break;
    const int pn2 = pos + kWaves;
    ha = pn2 < c_end ? issue(ta, pn2, va) : false;
    if (hb) consume(tb, pos, vb);
    pos = pn2;
  }

  if (quad == 0) {
    sm_m[w][m16] = m_run;
    sm_l[w][m16] = l_run;
  }
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[w][4 * quad + r][16 * n + m16] = acc[n][r];
  __syncthreads();
  write_wg_partial<D>(a, b, g, s, sm_m, sm_l, sm_o);
}

// ---------------------------------------------------------------------------
// float32 split kernel (vector ALU).  Lane (t = i%32, half = i/32) computes
// the logits of token t over half of the head dimension for every head of the
// group; p.V runs with lane i owning columns i and i+64.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_split_f32(AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int C = chunk_positions(T, a.sel, a.k);
  const int c_begin = s * a.chunks_per_wg;
  if (c_begin >= C) return;
  const int c_end = min(C, c_begin + a.chunks_per_wg);

  constexpr int CPL = D / 64;  // output columns per lane
  __shared__ float q_s[kMaxGroup][D];
  __shared__ float sm_m[kWaves][kMaxGroup];
  __shared__ float sm_l[kWaves][kMaxGroup];
  __shared__ float sm_o[kWaves][kMaxGroup][D];

  const int G = a.group;
  const float *qg = static_cast<const float *>(a.q) + ((int64_t)b * a.num_q_heads + g * G) * D;
  for (int i = threadIdx.x; i < G * D; i += kThreads) q_s[i / D][i % D] = qg[i];
  __syncthreads();

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = lane & 31, half = lane >> 5;
  const float *kpool = static_cast<const float *>(a.k_pool);
  const float *vpool = static_cast<const float *>(a.v_pool);
  const int Hkv = a.num_kv_heads;

  float m_run[kMaxGroup], l_run[kMaxGroup], acc[kMaxGroup][CPL];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[h][j] = 0.f;
  }

  for (int pos = c_begin + w; pos < c_end; pos += kWaves) {
    int64_t page;
    int sub, valid;
    if (!resolve_chunk(a, b, g, T, pos, page, sub, valid)) {
      if (a.stats != nullptr && lane < G) {  // unreadable page: no mass
        float *st = a.stats + ((int64_t)b * a.num_q_heads + g * G + lane) *
                                  (int64_t)(kChunksPerBlock * a.max_blocks) * 2;
        st[2 * pos + 0] = kNegInf;
        st[2 * pos + 1] = 0.f;
      }
      continue;
    }
    const int64_t tile = page * Hkv + g;
    const float *krow = kpool + (tile * kBlockTokens + sub * kChunkTokens + t) * D + half * (D / 2);
    float sc[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) sc[h] = 0.f;
    if (t < valid) {
      for (int c = 0; c < D / 2; c += 4) {
        const float4 kv = *reinterpret_cast<const float4 *>(krow + c);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            const float *qh = &q_s[h][half * (D / 2) + c];
            sc[h] += qh[0] * kv.x + qh[1] * kv.y + qh[2] * kv.z + qh[3] * kv.w;
          }
        }
      }
    }
    float p[kMaxGroup], alpha[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) continue;
      const float tot = sc[h] + __shfl_xor(sc[h], 32);
      const float x = t < valid ? tot * a.scale_log2 : kNegInf;
      float mx = x;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[h], mx);
      alpha[h] = fast_exp2(m_run[h] - m_new);
      p[h] = fast_exp2(x - m_new);
      float ps = p[h];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) ps += __shfl_xor(ps, o);
      l_run[h] = l_run[h] * alpha[h] + ps;
      m_run[h] = m_new;
      if (a.stats != nullptr && lane == 0) {
        float *st = a.stats + ((int64_t)b * a.num_q_heads + g * G + h) *
                                  (int64_t)(kChunksPerBlock * a.max_blocks) * 2;
        st[2 * pos + 0] = m_new;
        st[2 * pos + 1] = ps;
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const float *vrow = vpool + (tile * D + lane + 64 * j) * kBlockTokens + sub * kChunkTokens;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < G) acc[h][j] *= alpha[h];
      for (int tt = 0; tt < kChunkTokens; tt += 4) {
        const float4 v4 = *reinterpret_cast<const float4 *>(vrow + tt);
        const float ve[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float vv = tt + e < valid ? ve[e] : 0.f;
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < G) acc[h][j] += __shfl(p[h], tt + e) * vv;
        }
      }
    }
  }

#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    if (lane == 0) {
      sm_m[w][h] = m_run[h];
      sm_l[w][h] = l_run[h];
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) sm_o[w][h][lane + 64 * j] = acc[h][j];
  }
  __syncthreads();
  write_wg_partial<D>(a, b, g, s, sm_m, sm_l, sm_o);
}

// ---------------------------------------------------------------------------
// Block reductions / scans for 256-thread workgroups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Exclusive prefix sum over the 256 threads' values; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += tmp[i];
  total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  return base + inc - v;
}

// ---------------------------------------------------------------------------
// merge_heads: grid (Hq, B).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void merge_heads(MergeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.group, g = h / G;
  const int D = a.head_dim;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int C = chunk_positions(T, a.sel, a.k);
  const int nact = (C + a.chunks_per_wg - 1) / a.chunks_per_wg;
  const int64_t row0 = ((int64_t)b * a.num_q_heads + h) * a.nsplit;

  __shared__ float red[kWaves];
  __shared__ float ocomb[kThreads];

  float mloc = kNegInf;
  for (int s = threadIdx.x; s < nact; s += kThreads) mloc = fmaxf(mloc, a.part_ml[(row0 + s) * 2]);
  const float M = block_max(mloc, red);
  float lloc = 0.f;
  if (M != kNegInf)
    for (int s = threadIdx.x; s < nact; s += kThreads) {
      const float ms = a.part_ml[(row0 + s) * 2];
      if (ms != kNegInf) lloc += a.part_ml[(row0 + s) * 2 + 1] * fast_exp2(ms - M);
    }
  const float L = block_sum(lloc, red);

  // out: thread -> (column c, stripe of splits); stripes combined in LDS
  const int stripes = kThreads / D;
  const int c = threadIdx.x % D, stripe = threadIdx.x / D;
  float o = 0.f;
  if (L > 0.f)
    for (int s = stripe; s < nact; s += stripes) {
      const float ms = a.part_ml[(row0 + s) * 2];
      if (ms != kNegInf) o += a.part_o[(row0 + s) * D + c] * fast_exp2(ms - M);
    }
  ocomb[threadIdx.x] = o;
  __syncthreads();
  if (threadIdx.x < D) {
    float tot = 0.f;
    for (int st = 0; st < stripes; ++st) tot += ocomb[st * D + threadIdx.x];
    a.out[((int64_t)b * a.num_q_heads + h) * D + threadIdx.x] = L > 0.f ? tot / L : 0.f;
  }
  if (threadIdx.x == 0 && a.lse != nullptr)
    a.lse[(int64_t)b * a.num_q_heads + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;

  if (a.head_mass != nullptr) {
    const int nb = (T + kBlockTokens - 1) / kBlockTokens;
    const int nchunks = (T + kChunkTokens - 1) / kChunkTokens;
    const float *st = a.stats + ((int64_t)b * a.num_q_heads + h) *
                                    (int64_t)(kChunksPerBlock * a.max_blocks) * 2;
    float *hm = a.head_mass + ((int64_t)b * a.num_q_heads + h) * a.max_blocks;
    const float inv_l = L > 0.f ? 1.f / L : 0.f;
    for (int n = threadIdx.x; n < a.max_blocks; n += kThreads) {
      float mass = 0.f;
      if (n < nb && L > 0.f) {
        for (int cc = n * kChunksPerBlock; cc < (n + 1) * kChunksPerBlock && cc < nchunks; ++cc)
          mass += st[2 * cc + 1] * fast_exp2(st[2 * cc] - M);
        mass *= inv_l;
      }
      hm[n] = mass;
    }
  }
  if (a.sel_log != nullptr && h % G == 0) {
    const int64_t r0 = ((int64_t)b * a.num_kv_heads + g) * a.k;
    for (int r = threadIdx.x; r < a.k; r += kThreads) a.sel_log[r0 + r] = a.sel[r0 + r];
  }
}

// ---------------------------------------------------------------------------
// score_topk: grid (Hkv, B).  Keys are the float bits of the non-negative
// block scores (monotone as unsigned integers).  Radix select (4 x 8 bits)
// finds the k_eff-th largest key; keys above it are taken, keys equal to it
// are taken in ascending block order until k_eff are chosen.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void score_topk(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int N = (T + kBlockTokens - 1) / kBlockTokens;

  __shared__ uint32_t keys[kMaxBlocks];
  __shared__ int hist[256];
  __shared__ int scan_tmp[kWaves];
  __shared__ int pick_digit, pick_remaining;

  const float *base = a.mass + ((int64_t)b * a.num_kv_heads + g) * a.heads_per_row * a.max_blocks;
  for (int n = threadIdx.x; n < a.max_blocks; n += kThreads) {
    float sc = 0.f;
    if (n < N)
      for (int h = 0; h < a.heads_per_row; ++h) sc += base[(int64_t)h * a.max_blocks + n];
    if (a.score_out != nullptr) a.score_out[((int64_t)b * a.num_kv_heads + g) * a.max_blocks + n] = sc;
    if (n < N) keys[n] = sc > 0.f ? __float_as_uint(sc) : 0u;
  }
  if (a.idx == nullptr) return;
  int32_t *out = a.idx + ((int64_t)b * a.num_kv_heads + g) * a.k;
  const int keff = a.k < N ? a.k : N;
  if (keff == N) {  // every block is selected (also N == 0)
    for (int r = threadIdx.x; r < a.k; r += kThreads) out[r] = r < N ? r : -1;
    return;
  }
  __syncthreads();

  uint32_t prefix = 0u, mask = 0u;
  int remaining = keff;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int n = threadIdx.x; n < N; n += kThreads)
      if ((keys[n] & mask) == prefix) atomicAdd(&hist[(keys[n] >> shift) & 255u], 1);
    __syncthreads();
    // suffix count of bins >= my bin: scan over reversed bin order
    const int rb = 255 - threadIdx.x;
    const int cnt = hist[rb];
    int total;
    const int above = block_exclusive_scan(cnt, scan_tmp, total);  // bins > rb
    if (above < remaining && remaining <= above + cnt) {
      pick_digit = rb;
      pick_remaining = remaining - above;
    }
    __syncthreads();
    prefix |= (uint32_t)pick_digit << shift;
    mask |= 255u << shift;
    remaining = pick_remaining;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int need_eq = remaining;

  // contiguous element range per thread keeps index order for the scans
  const int per = (N + kThreads - 1) / kThreads;
  const int lo = threadIdx.x * per, hi = min(N, lo + per);
  int eq_cnt = 0;
  for (int n = lo; n < hi; ++n) eq_cnt += keys[n] == thr;
  int tot;
  int eq_rank = block_exclusive_scan(eq_cnt, scan_tmp, tot);
  int sel_cnt = 0;
  {
    int r = eq_rank;
    for (int n = lo; n < hi; ++n) {
      const uint32_t kv = keys[n];
      if (kv > thr) ++sel_cnt;
      else if (kv == thr) { if (r < need_eq) ++sel_cnt; ++r; }
    }
  }
  int pos = block_exclusive_scan(sel_cnt, scan_tmp, tot);
  {
    int r = eq_rank;
    for (int n = lo; n < hi; ++n) {
      const uint32_t kv = keys[n];
      bool take = false;
      if (kv > thr) take = true;
      else if (kv == thr) { take = r < need_eq; ++r; }
      if (take) out[pos++] = n;
    }
  }
  for (int r = keff + threadIdx.x; r < a.k; r += kThreads) out[r] = -1;
}

// Kernel timers: event pairs recorded around launches while running.
struct KernelTimer {
  bool running = false;
  int recorded = 0;
  std::vector<hipEvent_t> start, stop;
};
KernelTimer g_timers[kNumTimers];

struct TimerScope {
  KernelTimer *t;
  hipStream_t st;
  bool on;
  TimerScope(int kind, hipStream_t s) : t(&g_timers[kind]), st(s) {
    on = t->running && t->recorded < (int)t->start.size();
    if (on) (void)hipEventRecord(t->start[t->recorded], st);
  }
  ~TimerScope() {
    if (on) (void)hipEventRecord(t->stop[t->recorded++], st);
  }
};

}  // namespace

int timer_start(int kind, int capacity) {
  KernelTimer &t = g_timers[kind];
  hipError_t err = hipSuccess;
  while ((int)t.start.size() < capacity && err == hipSuccess) {
    hipEvent_t a, b;
    err = hipEventCreate(&a);
    if (err != hipSuccess) break;
    err = hipEventCreate(&b);
    if (err != hipSuccess) {
      (void)hipEventDestroy(a);
      break;
    }
    t.start.push_back(a);
    t.stop.push_back(b);
  }
  t.recorded = 0;
  t.running = err == hipSuccess;
  return (int)err;
}

int timer_stop(int kind, double *total_ms, int *launches) {
  KernelTimer &t = g_timers[kind];
  t.running = false;
  double sum = 0.0;
  for (int i = 0; i < t.recorded; ++i) {
    hipError_t err = hipEventSynchronize(t.stop[i]);
    if (err != hipSuccess) return (int)err;
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
    if (err != hipSuccess) return (int)err;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = t.recorded;
  t.recorded = 0;
  return 0;
}

int launch_attn(const AttnArgs &a, int dtype, int head_dim, int batch, void *stream) {
  const dim3 grid(a.nsplit, a.num_kv_heads, batch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  TimerScope timer(a.sel == nullptr ? kTimerFullAttn : kTimerSparseAttn, st);
  if (dtype == 1) {
    if (head_dim == 128) hipLaunchKernelGGL(attn_split_bf16<128>, grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(attn_split_bf16<64>, grid, dim3(kThreads), 0, st, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL(attn_split_f32<128>, grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(attn_split_f32<64>, grid, dim3(kThreads), 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_merge(const MergeArgs &a, int batch, void *stream) {
  TimerScope timer(kTimerMerge, static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(merge_heads, dim3(a.num_q_heads, batch), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_topk(const TopkArgs &a, int batch, void *stream) {
  TimerScope timer(kTimerTopk, static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(score_topk, dim3(a.num_kv_heads, batch), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

const char *device_error_string(int code) { return hipGetErrorString((hipError_t)code); }

}  // namespace hylra
