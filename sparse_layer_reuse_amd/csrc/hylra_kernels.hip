// HIP kernels of the HyLRA decode-phase hybrid attention for gfx950 (CDNA4).
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.3 (reset layers: full attention + top-k
// extraction; reuse layers: attention over the carried KV subset) and 2.4
// (selection over fixed 128-token blocks).
//
// One launch per layer.  Grid (nsplit, Hkv, B), 256 threads (4 wavefronts).
//   split pass   each wavefront consumes 32-token chunks of its workgroup's
//                range, keeping an online-softmax state for the G query heads
//                of the KV head; the four states are merged in LDS and written
//                as the workgroup's partial.  bf16 K/V: q.K and p.V on MFMA
//                (v_mfma_f32_16x16x32_bf16); float32 K/V: vector ALU.
//                Full mode walks every chunk of the sequence (and records the
//                per-chunk softmax mass for block scores); sparse mode walks
//                the chunks of the selected blocks through the block table.
//   epilogue     the last workgroup of a (sequence, KV head) to finish (device
//                scope arrival counter; partials handed over with coherent
//                device-scope stores and loads) merges them into out / lse and,
//                in full mode, turns the chunk masses into block scores and
//                selects the top-k blocks (radix select, lower id wins ties).
// A separate small kernel selects the top-k of a caller-given score array.
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 (raw 32-bit data) on gfx9

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Cross-workgroup hand-off of partials and chunk statistics: relaxed
// device-scope atomic stores / loads are coherent per location across the
// XCDs (they bypass stale cache lines), so the hand-off needs no cache-wide
// release / acquire fence.  Ordering comes from waiting for the stores to
// complete before the arrival counter is bumped, and from reading only after
// the counter shows every workgroup has arrived.
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Resolves chunk position `pos` of (b, g) to its page and the valid tokens
// (all arguments wavefront-uniform).  Returns false when the chunk holds no
// token to read: past the context, a padding / out-of-range selected id, or a
// page outside the pool.
__device__ __forceinline__ bool resolve_chunk(const AttnArgs &a, int b, int g, int T, int pos,
                                              int &page, int &sub, int &valid) {
  int n;
  if (a.sel == nullptr) {
    n = pos / kChunksPerBlock;
  } else {
    n = uniform(a.sel[((int64_t)b * a.num_kv_heads + g) * a.k + pos / kChunksPerBlock]);
    if (n < 0 || n >= (T + kBlockTokens - 1) / kBlockTokens) return false;
  }
  sub = pos % kChunksPerBlock;
  valid = T - (n * kBlockTokens + sub * kChunkTokens);
  if (valid <= 0) return false;
  if (valid > kChunkTokens) valid = kChunkTokens;
  page = uniform(a.table[(int64_t)b * a.max_blocks + n]);
  return page >= 0 && page < a.num_pages;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Exclusive prefix sum over the 256 threads' values.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp) {
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
  return base + inc - v;
}

// LDS used by the epilogue and the top-k selection.
struct EpiSmem {
  float f[kMaxGroup][kMaxSplits];  // per (head, split) rescale factor 2^(m_s - M)
  float M[kMaxGroup];
  float L[kMaxGroup];
  uint32_t keys[kMaxBlocks];
  int hist[256];
  int scan[kWaves];
  int pick_digit;
  int pick_remaining;
};

// Selects the k_eff = min(k, N) largest keys[0..N) (unsigned compare), equal
// keys going to the lower index, and writes their indices in ascending order
// to out[0..k_eff), -1 after.  keys must be in LDS and visible to all threads.
// Radix select over 4 x 8 bits finds the k_eff-th largest key `thr`; keys
// above thr are taken, keys equal to thr in index order until k_eff.
__device__ void select_topk(EpiSmem &sm, int N, int k, int32_t *out) {
  const int keff = k < N ? k : N;
  if (keff == N) {  // every block is selected (also N == 0)
    for (int r = threadIdx.x; r < k; r += kThreads) out[r] = r < N ? r : -1;
    return;
  }
  uint32_t prefix = 0u, mask = 0u;
  int remaining = keff;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    __syncthreads();
    sm.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int n = threadIdx.x; n < N; n += kThreads)
      if ((sm.keys[n] & mask) == prefix) atomicAdd(&sm.hist[(sm.keys[n] >> shift) & 255u], 1);
    __syncthreads();
    const int rb = 255 - threadIdx.x;  // bins in descending order
    const int cnt = sm.hist[rb];
    const int above = block_exclusive_scan(cnt, sm.scan);  // keys in bins > rb
    if (above < remaining && remaining <= above + cnt) {
      sm.pick_digit = rb;
      sm.pick_remaining = remaining - above;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.pick_digit << shift;
    mask |= 255u << shift;
    remaining = sm.pick_remaining;
  }
  const uint32_t thr = prefix;
  const int need_eq = remaining;

  // contiguous range per thread keeps index order for the scans
  const int per = (N + kThreads - 1) / kThreads;
  const int lo = threadIdx.x * per, hi = min(N, lo + per);
  int eq_cnt = 0;
  for (int n = lo; n < hi; ++n) eq_cnt += sm.keys[n] == thr;
  const int eq_rank = block_exclusive_scan(eq_cnt, sm.scan);
  int sel_cnt = 0;
  {
    int r = eq_rank;
    for (int n = lo; n < hi; ++n) {
      const uint32_t kv = sm.keys[n];
      if (kv > thr) {
        ++sel_cnt;
      } else if (kv == thr) {
        if (r < need_eq) ++sel_cnt;
        ++r;
      }
    }
  }
  int pos = block_exclusive_scan(sel_cnt, sm.scan);
  {
    int r = eq_rank;
    for (int n = lo; n < hi; ++n) {
      const uint32_t kv = sm.keys[n];
      bool take = false;
      if (kv > thr) {
        take = true;
      } else if (kv == thr) {
        take = r < need_eq;
        ++r;
      }
      if (take) out[pos++] = n;
    }
  }
  for (int r = keff + threadIdx.x; r < k; r += kThreads) out[r] = -1;
}

// Outputs of a (b, g) with no chunk to attend (empty context).
__device__ void write_empty(const AttnArgs &a, int b, int g, int D) {
  const int G = a.group;
  for (int i = threadIdx.x; i < G * D; i += kThreads)
    a.out[((int64_t)b * a.num_q_heads + g * G) * D + i] = 0.f;
  if (a.lse != nullptr)
    for (int h = threadIdx.x; h < G; h += kThreads)
      a.lse[(int64_t)b * a.num_q_heads + g * G + h] = kNegInf;
  if (a.score_out != nullptr)
    for (int n = threadIdx.x; n < a.max_blocks; n += kThreads)
      a.score_out[((int64_t)b * a.num_kv_heads + g) * a.max_blocks + n] = 0.f;
  if (a.idx_out != nullptr)
    for (int r = threadIdx.x; r < a.k; r += kThreads)
      a.idx_out[((int64_t)b * a.num_kv_heads + g) * a.k + r] = -1;
  if (a.sel_log != nullptr)
    for (int r = threadIdx.x; r < a.k; r += kThreads) {
      const int64_t i = ((int64_t)b * a.num_kv_heads + g) * a.k + r;
      a.sel_log[i] = a.sel[i];
    }
}

// Merges the nact split partials of (b, g) into out / lse; in full mode with
// statistics also the block scores and the top-k.  Runs in the last
// workgroup of (b, g) to finish its split pass.
template <int D>
__device__ void epilogue(const AttnArgs &a, int b, int g, int T, int nact, EpiSmem &sm) {
  const int G = a.group;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t head0 = (int64_t)b * a.num_q_heads + g * G;

  // per head: global max / sum and the per-split rescale factors
  for (int h = w; h < G; h += kWaves) {
    const float *ml = a.part_ml + (head0 + h) * a.nsplit * 2;
    float mx = kNegInf;
    for (int s = lane; s < nact; s += 64) mx = fmaxf(mx, load_agent(ml + 2 * s));
    const float M = wave_max(mx);
    float lsum = 0.f;
    for (int s = lane; s < nact; s += 64) {
      const float ms = load_agent(ml + 2 * s);
      const float f = ms == kNegInf ? 0.f : fast_exp2(ms - M);
      sm.f[h][s] = f;
      lsum += f * load_agent(ml + 2 * s + 1);
    }
    const float L = wave_sum(lsum);
    if (lane == 0) {
      sm.M[h] = M;
      sm.L[h] = L;
    }
  }
  __syncthreads();

  for (int item = threadIdx.x; item < G * D; item += kThreads) {
    const int h = item / D, c = item % D;
    const float *po = a.part_o + (head0 + h) * a.nsplit * D + c;
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < nact; ++s) acc += load_agent(po + (int64_t)s * D) * sm.f[h][s];
    const float L = sm.L[h];
    a.out[(head0 + h) * D + c] = L > 0.f ? acc / L : 0.f;
  }
  if (a.lse != nullptr && threadIdx.x < G) {
    const float L = sm.L[threadIdx.x];
    a.lse[head0 + threadIdx.x] = L > 0.f ? (sm.M[threadIdx.x] + __log2f(L)) * kLn2 : kNegInf;
  }

  if (a.sel_log != nullptr) {
    const int64_t r0 = ((int64_t)b * a.num_kv_heads + g) * a.k;
    for (int r = threadIdx.x; r < a.k; r += kThreads) a.sel_log[r0 + r] = a.sel[r0 + r];
  }
  if (a.stats == nullptr) return;

  // block score: sum over the group's heads of the softmax mass of the block
  const int N = (T + kBlockTokens - 1) / kBlockTokens;
  const int nchunks = (T + kChunkTokens - 1) / kChunkTokens;
  const int64_t stride = (int64_t)kChunksPerBlock * a.max_blocks * 2;
  for (int n = threadIdx.x; n < a.max_blocks; n += kThreads) {
    float score = 0.f;
    if (n < N) {
      for (int h = 0; h < G; ++h) {
        const float L = sm.L[h];
        if (!(L > 0.f)) continue;
        const float *st = a.stats + (head0 + h) * stride;
        float mass = 0.f;
        for (int c = n * kChunksPerBlock; c < (n + 1) * kChunksPerBlock && c < nchunks; ++c)
          mass += load_agent(st + 2 * c + 1) * fast_exp2(load_agent(st + 2 * c) - sm.M[h]);
        score += mass / L;
      }
      sm.keys[n] = score > 0.f ? __float_as_uint(score) : 0u;
    }
    if (a.score_out != nullptr)
      a.score_out[((int64_t)b * a.num_kv_heads + g) * a.max_blocks + n] = score;
  }
  if (a.idx_out != nullptr) {
    __syncthreads();
    select_topk(sm, N, a.k, a.idx_out + ((int64_t)b * a.num_kv_heads + g) * a.k);
  }
}

// Writes the workgroup partial from the four wavefront states in LDS, then
// counts the workgroup's arrival; the last of the nact workgroups of (b, g)
// runs the epilogue.  Returns true in that workgroup.
template <int D>
__device__ bool finish_split(const AttnArgs &a, int b, int g, int s, int nact,
                             const float (*sm_m)[kMaxGroup], const float (*sm_l)[kMaxGroup],
                             const float (*sm_o)[kMaxGroup][D], int *last_flag) {
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
    store_agent(a.part_o + row * D + c, o);
    if (c == 0) {
      store_agent(a.part_ml + row * 2 + 0, m);
      store_agent(a.part_ml + row * 2 + 1, l);
    }
  }
  // every store of this workgroup (partial and chunk statistics) completes
  // before the arrival is counted; the last arrival then reads everyone's.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t *cnt = a.counters + (int64_t)b * a.num_kv_heads + g;
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == nact - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = *last_flag != 0;
  __syncthreads();  // the epilogue reuses the LDS of the split pass
  return last;
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
union BfSmem {
  struct {
    float m[kWaves][kMaxGroup];
    float l[kWaves][kMaxGroup];
    float o[kWaves][kMaxGroup][D];
  } main;
  EpiSmem epi;
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_split_bf16(AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int C = chunk_positions(T, a.sel, a.k);
  __shared__ BfSmem<D> sm;
  __shared__ int last_flag;
  if (C == 0) {
    if (s == 0) write_empty(a, b, g, D);
    return;
  }
  const int c_begin = s * a.chunks_per_wg;
  if (c_begin >= C) return;
  const int c_end = min(C, c_begin + a.chunks_per_wg);
  const int nact = (C + a.chunks_per_wg - 1) / a.chunks_per_wg;

  const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
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

  const char *kpool = static_cast<const char *>(a.k_pool);
  const char *vpool = static_cast<const char *>(a.v_pool);
  const int Hkv = a.num_kv_heads;
  // per-lane byte offsets inside a chunk's K rows / V columns (chunk-invariant)
  const uint32_t k_lane = (uint32_t)(((8 * (m16 >> 2) + (m16 & 3)) * D + 8 * quad) * 2);
  const uint32_t v_lane = (uint32_t)((m16 * kBlockTokens + 8 * quad) * 2);
  float *stats_row = a.stats ? a.stats + ((int64_t)b * a.num_q_heads + g * G + m16) *
                                             (int64_t)(kChunksPerBlock * a.max_blocks) * 2
                             : nullptr;

  // Issues the 16-byte loads of chunk `pos` into t through buffer resources
  // spanning just that chunk; returns its valid token count.  A position past
  // the range or without a readable page gets an empty resource: the loads
  // return zeros without touching memory, so every path issues the same loads
  // and the register tiles never need copying.
  auto issue = [&](BfTile<D> &t, int pos) -> int {
    int page = 0, sub = 0, valid = 0;
    bool ok = false;
    if (pos < c_end) {
      ok = resolve_chunk(a, b, g, T, pos, page, sub, valid);
      if (!ok && stats_row != nullptr && quad == 0 && m16 < G) {  // unreadable page: no mass
        store_agent(stats_row + 2 * pos + 0, kNegInf);
        store_agent(stats_row + 2 * pos + 1, 0.f);
      }
    }
    if (!ok) {
      page = 0;
      sub = 0;
      valid = 0;
    }
    const int64_t tile = (int64_t)page * Hkv + g;
    const char *kb = kpool + (tile * kBlockTokens + sub * kChunkTokens) * D * 2;
    const char *vb = vpool + (tile * D * kBlockTokens + sub * kChunkTokens) * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(kb), (short)0, ok ? kChunkTokens * D * 2 : 0, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(vb), (short)0, ok ? (D - 1) * kBlockTokens * 2 + kChunkTokens * 2 : 0,
        kBufferFlags);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        t.k[h][k] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_lane, (4 * h * D + 32 * k) * 2, 0);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
      t.v[n] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_lane, n * 16 * kBlockTokens * 2, 0);
    return valid;
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
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float ps = 0.f;
    bf16x8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(x[j] - m_new);
      ps += p;
      const __bf16 hi = (__bf16)p;
      phi[j] = hi;
      plo[j] = (__bf16)(p - (float)hi);
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (stats_row != nullptr && quad == 0 && m16 < G) {
      store_agent(stats_row + 2 * pos + 0, m_new);
      store_agent(stats_row + 2 * pos + 1, ps);
    }
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * quad + r);
    // tokens past the context: p is 0 there, and V is zeroed so stale page
    // bytes (possibly NaN patterns) cannot leak in through 0 * NaN.
    u32x4 keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = 8 * quad + 2 * e;
      keep[e] = (tok < valid ? 0x0000FFFFu : 0u) | (tok + 1 < valid ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[n][r] *= al[r];
      const bf16x8 vb = __builtin_bit_cast(bf16x8, t.v[n] & keep);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, acc[n], 0, 0, 0);
    }
  };

  // Two register tiles: the next chunk's loads are in flight while the
  // current one is consumed.
  BfTile<D> ta, tb;
  int pos = c_begin + w;
  int va = issue(ta, pos);
  while (pos < c_end) {
    const int vb = issue(tb, pos + kWaves);
    if (va > 0) consume(ta, pos, va);
    pos += kWaves;
    if (pos >= c_end) break;
    va = issue(ta, pos + kWaves);
    if (vb > 0) consume(tb, pos, vb);
    pos += kWaves;
  }

  if (quad == 0) {
    sm.main.m[w][m16] = m_run;
    sm.main.l[w][m16] = l_run;
  }
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.main.o[w][4 * quad + r][16 * n + m16] = acc[n][r];
  __syncthreads();
  if (!finish_split<D>(a, b, g, s, nact, sm.main.m, sm.main.l, sm.main.o, &last_flag)) return;
  epilogue<D>(a, b, g, T, nact, sm.epi);
}

// ---------------------------------------------------------------------------
// float32 split kernel (vector ALU).  Lane (t = i%32, half = i/32) computes
// the logits of token t over half of the head dimension for every head of the
// group; p.V runs with lane i owning columns i and i+64.
// ---------------------------------------------------------------------------
template <int D>
union F32Smem {
  struct {
    float q[kMaxGroup][D];
    float m[kWaves][kMaxGroup];
    float l[kWaves][kMaxGroup];
    float o[kWaves][kMaxGroup][D];
  } main;
  EpiSmem epi;
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_split_f32(AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int C = chunk_positions(T, a.sel, a.k);
  __shared__ F32Smem<D> sm;
  __shared__ int last_flag;
  if (C == 0) {
    if (s == 0) write_empty(a, b, g, D);
    return;
  }
  const int c_begin = s * a.chunks_per_wg;
  if (c_begin >= C) return;
  const int c_end = min(C, c_begin + a.chunks_per_wg);
  const int nact = (C + a.chunks_per_wg - 1) / a.chunks_per_wg;

  constexpr int CPL = D / 64;  // output columns per lane
  const int G = a.group;
  const float *qg = static_cast<const float *>(a.q) + ((int64_t)b * a.num_q_heads + g * G) * D;
  for (int i = threadIdx.x; i < G * D; i += kThreads) sm.main.q[i / D][i % D] = qg[i];
  __syncthreads();

  const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
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
    int page, sub, valid;
    if (!resolve_chunk(a, b, g, T, pos, page, sub, valid)) {
      if (a.stats != nullptr && lane < G) {  // unreadable page: no mass
        float *st = a.stats + ((int64_t)b * a.num_q_heads + g * G + lane) *
                                  (int64_t)(kChunksPerBlock * a.max_blocks) * 2;
        store_agent(st + 2 * pos + 0, kNegInf);
        store_agent(st + 2 * pos + 1, 0.f);
      }
      continue;
    }
    const int64_t tile = (int64_t)page * Hkv + g;
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
            const float *qh = &sm.main.q[h][half * (D / 2) + c];
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
        store_agent(st + 2 * pos + 0, m_new);
        store_agent(st + 2 * pos + 1, ps);
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

  __syncthreads();  // q no longer read; the merge arrays follow it in LDS
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    if (lane == 0) {
      sm.main.m[w][h] = m_run[h];
      sm.main.l[w][h] = l_run[h];
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) sm.main.o[w][h][lane + 64 * j] = acc[h][j];
  }
  __syncthreads();
  if (!finish_split<D>(a, b, g, s, nact, sm.main.m, sm.main.l, sm.main.o, &last_flag)) return;
  epilogue<D>(a, b, g, T, nact, sm.epi);
}

// ---------------------------------------------------------------------------
// Top-k of a caller-given score array: grid (Hkv, B).  Keys are the float bits
// of the non-negative scores (monotone as unsigned integers).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void score_topk(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int N = (T + kBlockTokens - 1) / kBlockTokens;
  __shared__ EpiSmem sm;
  const float *row = a.score + ((int64_t)b * a.num_kv_heads + g) * a.max_blocks;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    const float sc = row[n];
    sm.keys[n] = sc > 0.f ? __float_as_uint(sc) : 0u;
  }
  __syncthreads();
  select_topk(sm, N, a.k, a.idx + ((int64_t)b * a.num_kv_heads + g) * a.k);
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

int launch_topk(const TopkArgs &a, int batch, void *stream) {
  TimerScope timer(kTimerTopk, static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(score_topk, dim3(a.num_kv_heads, batch), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

const char *device_error_string(int code) { return hipGetErrorString((hipError_t)code); }

}  // namespace hylra
