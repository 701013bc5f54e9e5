// HIP kernels of the HyLRA decode-phase hybrid attention for gfx950 (CDNA4).
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.3 (reset layers: full attention + top-k
// extraction; reuse layers: attention over the carried KV subset) and 2.4
// (selection over fixed 128-token blocks).
//
// One launch per layer.  Grid (nsplit, Hkv, B), 512 threads (8 wavefronts).
//   split pass   each wavefront consumes 32-token chunks of its workgroup's
//                range, keeping an online-softmax state for the G query heads
//                of the KV head; the eight states are merged in LDS and written
//                as the workgroup's partial.  bf16 K/V: q.K and p.V on MFMA
//                (v_mfma_f32_16x16x32_bf16); float32 K/V: vector ALU.
//                Full modes walk every chunk of the sequence, sparse modes the
//                chunks of the selected blocks through the block table.  The
//                chunks are dealt round-robin (wavefront w takes w, w+8, ...),
//                so the eight wavefronts stream neighbouring chunks together.
//                The scored mode records each chunk's softmax mass; a block's
//                four chunk masses are summed when the partial is written.
//   epilogue     the last workgroup of a (sequence, KV head) to finish (device
//                scope arrival counter; partials handed over with coherent
//                device-scope stores and loads) merges them into out / lse and,
//                in scored mode, turns the block masses into block scores and
//                selects the top-k blocks (one wavefront, lower id wins ties)
//                while its other wavefronts merge the output.
// The mode (full, scored, sparse, staged) is a template argument: each
// launch runs an instance holding only its own code.
// A separate small kernel selects the top-k of a caller-given score array.
//
// Softmax state is kept in base 2: x = s * scale * log2(e), p = 2^(x - m).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "hylra_internal.h"

namespace hylra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kWavesPerGroup;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 (raw 32-bit data) on gfx9
constexpr int kCoherent = 16;             // buffer instruction cache policy: sc1
constexpr int kStreaming = 2;             // buffer instruction cache policy: nt (read once)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^(m - ref) for a state with running max m (-inf: empty state -> 0).
__device__ __forceinline__ float rescale(float m, float ref) {
  return m == kNegInf ? 0.f : fast_exp2(m - ref);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wavefront-uniform read of a read-only int array through the scalar cache
// (constant address space): an s_load, counted apart from the vector loads,
// so it never waits for the K/V tiles in flight.
typedef const __attribute__((address_space(4))) int32_t *ConstI32Ptr;
__device__ __forceinline__ int scalar_load(const int32_t *p, int64_t i) {
  return ((ConstI32Ptr)(p))[i];
}

// Cross-workgroup hand-off of partials and block masses: device-scope
// coherent (sc1) stores and loads act per location across the XCDs without a
// cache-wide release / acquire fence.  Ordering comes from waiting for the
// stores to complete before the arrival counter is bumped, and from reading
// only after the counter shows that every workgroup has arrived.
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ int clamp_ctx(int t, int max_blocks) {
  return t < 0 ? 0 : (t > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : t);
}

// Launch modes of the attention kernel (compile-time, one instance each):
//   full     reset layer whose index set nobody reads: split pass + merge
//   scored   reset layer: split pass recording block masses + merge, block
//            scores and the top-k selection
//   sparse   reuse layer: the selected blocks through the block table
//   staged   reuse layer: the selected blocks from a staging pool
constexpr int kModeFull = 0;
constexpr int kModeScored = 1;
constexpr int kModeSparse = 2;
constexpr int kModeStaged = 3;
constexpr bool mode_sparse(int mode) { return mode == kModeSparse || mode == kModeStaged; }

// Number of 32-token chunk positions of (b, g) in a launch.  Full: every chunk
// of the context.  Sparse: four per selection slot, for all k slots of the row
// (a slot holding no block of the context resolves to an empty chunk), so
// the ids of a row may sit in any order with padding anywhere.
template <int kMode>
__device__ __forceinline__ int chunk_positions(int T, int k) {
  if constexpr (mode_sparse(kMode)) return T > 0 ? kChunksPerBlock * k : 0;
  return (T + kChunkTokens - 1) / kChunkTokens;
}

// Resolves chunk position `pos` of (b, g) to its page and the valid tokens
// (all arguments wavefront-uniform).  Returns false when the chunk holds no
// token to read: past the context, a padding / out-of-range selected id, or a
// page outside the pool.  Staged mode: the pools are a staging pool
// (selection slot r of sequence b in page b * k + r) and no block table is
// read.
template <int kMode>
__device__ __forceinline__ bool resolve_chunk(const AttnArgs &a, int b, int g, int T, int pos,
                                              int &page, int &sub, int &valid) {
  int n;
  if constexpr (mode_sparse(kMode)) {
    n = scalar_load(a.sel, ((int64_t)b * a.num_kv_heads + g) * a.k + pos / kChunksPerBlock);
    if (n < 0 || n >= (T + kBlockTokens - 1) / kBlockTokens) return false;
  } else {
    n = pos / kChunksPerBlock;
  }
  sub = pos % kChunksPerBlock;
  valid = T - (n * kBlockTokens + sub * kChunkTokens);
  if (valid <= 0) return false;
  if (valid > kChunkTokens) valid = kChunkTokens;
  if constexpr (kMode == kModeStaged)
    page = b * a.k + pos / kChunksPerBlock;
  else
    page = scalar_load(a.table, (int64_t)b * a.max_blocks + n);
  return page >= 0 && page < a.num_pages;
}

// Block id and page of a wavefront's first chunk (position pos), loaded at
// the start of the kernel together with the context length: neither load
// depends on it, so the first K/V loads wait for one round trip less.  Out
// of range ids give n = -1 / page = -1; resolve_first then checks them
// against the context as resolve_chunk does.
struct FirstChunk {
  int n, page;
};
template <int kMode>
__device__ __forceinline__ FirstChunk prefetch_first(const AttnArgs &a, int b, int g, int pos) {
  FirstChunk f{-1, -1};
  if constexpr (mode_sparse(kMode)) {
    if (pos < kChunksPerBlock * a.k)
      f.n = scalar_load(a.sel, ((int64_t)b * a.num_kv_heads + g) * a.k + pos / kChunksPerBlock);
  } else {
    f.n = pos / kChunksPerBlock;
  }
  if constexpr (kMode != kModeStaged) {
    if (f.n >= 0 && f.n < a.max_blocks) f.page = scalar_load(a.table, (int64_t)b * a.max_blocks + f.n);
  } else {
    f.page = b * a.k + pos / kChunksPerBlock;
  }
  return f;
}
template <int kMode>
__device__ __forceinline__ bool resolve_first(const AttnArgs &a, int T, int pos, FirstChunk f,
                                              int &page, int &sub, int &valid) {
  if (f.n < 0 || f.n >= (T + kBlockTokens - 1) / kBlockTokens) return false;
  sub = pos % kChunksPerBlock;
  valid = T - (f.n * kBlockTokens + sub * kChunkTokens);
  if (valid <= 0) return false;
  if (valid > kChunkTokens) valid = kChunkTokens;
  page = f.page;
  return page >= 0 && page < a.num_pages;
}

// The i-th chunk position of wavefront w in a workgroup range starting at
// c_begin: chunks are dealt round-robin, so at any time the wavefronts of a
// workgroup read neighbouring chunks (the four chunks of a block together).
__device__ __forceinline__ int chunk_of(int c_begin, int w, int i) {
  return c_begin + w + kWaves * i;
}
__device__ __forceinline__ bool chunk_live(int c_begin, int c_end, int w, int i) {
  return chunk_of(c_begin, w, i) < c_end;
}

// Wavefront reductions on DPP lane permutes (quad perms, row mirrors, row
// broadcasts of lanes 15 / 31): each step is a VALU op, far cheaper in
// latency than a ds_bpermute shuffle.  The result is read from lane 63.
constexpr int kDppQuad1032 = 0xb1, kDppQuad2301 = 0x4e, kDppRowHalfMirror = 0x141,
              kDppRowMirror = 0x140, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143,
              kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118;

template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, ctrl, row_mask, 0xf, false);
}
template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __builtin_bit_cast(float, dpp_u32<ctrl, row_mask>(__builtin_bit_cast(uint32_t, old),
                                                          __builtin_bit_cast(uint32_t, src)));
}
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuad1032>(v, v));
  v = fmaxf(v, dpp_f32<kDppQuad2301>(v, v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v, v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v, v));
  v = fmaxf(v, dpp_f32<kDppRowBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp_f32<kDppRowBcast31, 0xc>(v, v));
  return lane63(v);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuad1032>(0.f, v);
  v += dpp_f32<kDppQuad2301>(0.f, v);
  v += dpp_f32<kDppRowHalfMirror>(0.f, v);
  v += dpp_f32<kDppRowMirror>(0.f, v);
  v += dpp_f32<kDppRowBcast15, 0xa>(0.f, v);
  v += dpp_f32<kDppRowBcast31, 0xc>(0.f, v);
  return lane63(v);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp_u32<kDppQuad1032>(0u, v);
  v |= dpp_u32<kDppQuad2301>(0u, v);
  v |= dpp_u32<kDppRowHalfMirror>(0u, v);
  v |= dpp_u32<kDppRowMirror>(0u, v);
  v |= dpp_u32<kDppRowBcast15, 0xa>(0u, v);
  v |= dpp_u32<kDppRowBcast31, 0xc>(0u, v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  v &= dpp_u32<kDppQuad1032>(~0u, v);
  v &= dpp_u32<kDppQuad2301>(~0u, v);
  v &= dpp_u32<kDppRowHalfMirror>(~0u, v);
  v &= dpp_u32<kDppRowMirror>(~0u, v);
  v &= dpp_u32<kDppRowBcast15, 0xa>(~0u, v);
  v &= dpp_u32<kDppRowBcast31, 0xc>(~0u, v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes: DPP shifts within rows of 16, then
// the row totals (lanes 15, 31, 47) are added as scalars.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
  uint32_t x = (uint32_t)v;
  x += dpp_u32<kDppRowShr1>(0u, x) * ((lane & 15) >= 1);
  x += dpp_u32<kDppRowShr2>(0u, x) * ((lane & 15) >= 2);
  x += dpp_u32<kDppRowShr4>(0u, x) * ((lane & 15) >= 4);
  x += dpp_u32<kDppRowShr8>(0u, x) * ((lane & 15) >= 8);
  const int r0 = __builtin_amdgcn_readlane((int)x, 15);
  const int r1 = __builtin_amdgcn_readlane((int)x, 31);
  const int r2 = __builtin_amdgcn_readlane((int)x, 47);
  const int row = lane >> 4;
  const int base = row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2;
  return (int)x + base;
}

__device__ __forceinline__ bool wave_any(bool c) { return __ballot(c) != 0; }

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// The last workgroup of a reset layer splits its wavefronts in two groups
// after the per-head statistics: wavefronts [0, kScoreWaves) compute the
// block scores and wavefront 0 then selects the top-k; the others merge the
// output partials at the same time.
constexpr int kScoreWaves = 4;
constexpr int kScoreThreads = 64 * kScoreWaves;

// LDS of the split pass: the wavefront states and the chunk masses.
template <int D>
struct SplitSmem {
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float o[kWaves][kMaxGroup][D];
  float cm[kMaxWgChunks][kMaxGroup];  // chunk: running max after the chunk
  float cp[kMaxWgChunks][kMaxGroup];  // chunk: its softmax mass relative to cm
};

// LDS of the one-wavefront top-k selection.
struct alignas(16) SelectSmem {
  uint32_t cand_key[256 + 16];  // candidates of the filter, in ascending block id (+ zero pad)
  int32_t cand_id[256];
  int hist[256];                // digit histogram of the radix fallback
  uint32_t lane_max[128];       // the filter's group maxima
};

// LDS used by the epilogue.
struct EpiSmem {
  float f[kMaxGroup][kMaxSplits];  // per (head, split) rescale factor 2^(m_s - M)
  float f2[kMaxGroup][kMaxGroups]; // two-level: per (head, group) factor 2^(m_q - M)
  float M[kMaxGroup];
  float L[kMaxGroup];
  float invL[kMaxGroup];
  uint32_t keys[kMaxBlocks];       // block score bits (scores >= 0 order as unsigned)
  SelectSmem sel;
};

template <int D>
union KernelSmem {
  SplitSmem<D> split;
  EpiSmem epi;
};

// LDS written by some lanes of a wavefront and read by others: wait for the
// wavefront's LDS operations, and keep the compiler from moving accesses
// across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuad1032>(0u, v));
  v = max(v, dpp_u32<kDppQuad2301>(0u, v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(0u, v));
  v = max(v, dpp_u32<kDppRowMirror>(0u, v));
  v = max(v, dpp_u32<kDppRowBcast15, 0xa>(0u, v));
  v = max(v, dpp_u32<kDppRowBcast31, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// For each of this lane's NV values v[i]: how many of vals[0..n) are >= v[i]
// (vals in LDS, 16-byte aligned, n a wavefront-uniform multiple of 16).
// Every read is one address for the whole wavefront (a broadcast of four
// values), and the comparisons feed four independent counters: plain vector
// ALU work with no lane-to-scalar round trip per value.
//
// With these counts the kk-th largest of the values held across the lanes is
// the largest value whose count reaches kk: a value above the kk-th largest
// has fewer than kk values at or above it.
template <int NV>
__device__ __forceinline__ void count_not_below_n(const uint32_t *vals, int n,
                                                  const uint32_t (&v)[NV], int (&c)[NV]) {
  constexpr int A = NV >= 4 ? 1 : 4 / NV;  // counters per value
  int acc[NV][A];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < A; ++e) acc[i][e] = 0;
  for (int j = 0; j < n; j += 16) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u32x4 *>(&vals[j + 4 * u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i][e % A] += x[u][e] >= v[i] ? 1 : 0;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    c[i] = 0;
#pragma unroll
    for (int e = 0; e < A; ++e) c[i] += acc[i][e];
  }
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppQuad1032>(~0u, v));
  v = min(v, dpp_u32<kDppQuad2301>(~0u, v));
  v = min(v, dpp_u32<kDppRowHalfMirror>(~0u, v));
  v = min(v, dpp_u32<kDppRowMirror>(~0u, v));
  v = min(v, dpp_u32<kDppRowBcast15, 0xa>(~0u, v));
  v = min(v, dpp_u32<kDppRowBcast31, 0xc>(~0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Radix select over the keys, run by one wavefront: the threshold over 4 x 8
// bits, most significant digit first (digits shared by every key skipped,
// the passes stop once the chosen digit's bucket is taken whole), then the
// keys above it and the equal ones in id order until k_eff.  Writes the
// selected ids ascending to out[0..keff).
__device__ __forceinline__ void wave_radix_select(const uint32_t *keys, int N, int keff,
                                                  int32_t *out, SelectSmem &ss) {
  const int lane = threadIdx.x & 63;
  uint32_t kor = 0u, kand = 0xFFFFFFFFu;
  for (int n = lane; n < N; n += 64) {
    const uint32_t key = keys[n];
    kor |= key;
    kand &= key;
  }
  kor = wave_or(kor);
  kand = wave_and(kand);
  const uint32_t common = ~(kor ^ kand);
  uint32_t prefix = 0u, mask = 0u;
  int remaining = keff;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t dmask = 255u << shift;
    if ((common & dmask) == dmask) {  // every key has the same digit here
      prefix |= kand & dmask;
      mask |= dmask;
      continue;
    }
    *reinterpret_cast<u32x4 *>(&ss.hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
    for (int n = lane; n < N; n += 64) {
      const uint32_t key = keys[n];
      if ((key & mask) == prefix) atomicAdd(&ss.hist[(key >> shift) & 255u], 1);
    }
    wave_lds_sync();
    // lane l holds bins 255-4l .. 252-4l (descending) and finds the bin where
    // the count of keys from the top reaches `remaining`
    const u32x4 hv = *reinterpret_cast<const u32x4 *>(&ss.hist[252 - 4 * lane]);
    const int c[4] = {(int)hv[3], (int)hv[2], (int)hv[1], (int)hv[0]};
    const int tot = c[0] + c[1] + c[2] + c[3];
    int above = wave_inclusive_scan(tot) - tot;
    int digit = -1, rem = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above < remaining && remaining <= above + c[i]) {
        digit = 255 - 4 * lane - i;
        rem = remaining - above;
        cnt = c[i];
      }
      above += c[i];
    }
    const int leader = __builtin_ctzll(__ballot(digit >= 0));
    prefix |= (uint32_t)__builtin_amdgcn_readlane(digit, leader) << shift;
    mask |= dmask;
    remaining = __builtin_amdgcn_readlane(rem, leader);
    wave_lds_sync();  // every lane has read the histogram before the next pass clears it
    if (remaining == __builtin_amdgcn_readlane(cnt, leader)) break;  // bucket taken whole
  }
  const uint32_t thr = prefix;
  const int need_eq = remaining;
  int taken = 0, eq_before = 0;
  for (int base = 0; base < N; base += 64) {
    const int n = base + lane;
    const uint32_t kv = n < N ? keys[n] & mask : 0u;
    const bool is_gt = n < N && kv > thr;
    const bool is_eq = n < N && kv == thr;
    const uint64_t eqm = __ballot(is_eq);
    const bool sel = is_gt || (is_eq && eq_before + lanes_below(eqm) < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) out[taken + lanes_below(selm)] = n;
    taken += __builtin_popcountll(selm);
    eq_before += __builtin_popcountll(eqm);
  }
}

// k-th largest (kk >= 1) of the values v[i] of every lane (0 stands for
// none): the largest t with #{v >= t} >= kk, decided bit by bit from the top
// with ballots.
template <int NV>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t (&v)[NV], int kk) {
  uint32_t any = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) any |= v[i];
  any = wave_or(any);
  uint32_t t = 0u;
  for (int bit = any ? 31 - __builtin_clz(any) : -1; bit >= 0; --bit) {
    const uint32_t trial = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __builtin_popcountll(__ballot(v[i] >= trial));
    if (cnt >= kk) t = trial;
  }
  return t;
}

// Lower bound t0 of the k-th largest key (k <= 64).  Key n sits in lane
// n % 64; the keys of a lane form NG groups (n / 64 % NG), and t0 is the
// k-th largest of the 64 NG group maxima, found from each maximum's count
// of maxima at or above it (broadcast reads).  At least k groups hold a key
// >= t0 (or t0 = 0 and every key is >= t0), so the k largest keys, and
// every key equal to the k-th largest, are >= t0.
template <int NG>
__device__ __forceinline__ uint32_t topk_filter(const uint32_t *keys, int N, int k,
                                                SelectSmem &ss) {
  const int lane = threadIdx.x & 63;
  // four independent LDS reads per step
  uint32_t gm[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) gm[i] = 0u;
  for (int base = 0; base < N; base += 256) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = keys[base + 64 * u + lane];
#pragma unroll
    for (int u = 0; u < 4; ++u) gm[u % NG] = max(gm[u % NG], v[u]);
  }
#pragma unroll
  for (int i = 0; i < NG; ++i) ss.lane_max[64 * i + lane] = gm[i];
  wave_lds_sync();
  int c[NG];
  count_not_below_n<NG>(ss.lane_max, 64 * NG, gm, c);
  uint32_t best = 0u;
#pragma unroll
  for (int i = 0; i < NG; ++i) best = max(best, c[i] >= k ? gm[i] : 0u);
  return wave_max_u32(best);
}

// The same bound from 256 groups: group (u, lane) holds the keys n with
// n % 256 == 64 u + lane, and t0 is the k-th largest of the 256 group maxima
// (ballot bisection).  Finer groups than the lanes leave far fewer
// candidates when k or the keys per lane are large.
__device__ __forceinline__ uint32_t topk_filter256(const uint32_t *keys, int N, int k) {
  const int lane = threadIdx.x & 63;
  uint32_t gm[4] = {0u, 0u, 0u, 0u};
  for (int base = 0; base < N; base += 256) {
#pragma unroll
    for (int u = 0; u < 4; ++u) gm[u] = max(gm[u], keys[base + 64 * u + lane]);
  }
  return wave_kth_largest<4>(gm, k);
}

// Selection among C <= 64 * NV candidates, candidate p in lane p % 64 (slot
// p / 64), in ascending block id (cand_key zero past C up to a multiple of
// 16): the keff-th largest key thr from the counts of keys >= each
// candidate's, then every key above thr and the first keys equal to it, in
// id order, written in id order to out[0..keff).
template <int NV>
__device__ __forceinline__ void select_candidates_rank(const SelectSmem &ss, int C, int keff,
                                                       int32_t *out) {
  const int lane = threadIdx.x & 63;
  uint32_t ck[NV];
  int32_t ci[NV];
  bool valid[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    valid[i] = lane + 64 * i < C;
    ck[i] = valid[i] ? ss.cand_key[lane + 64 * i] : 0u;
    ci[i] = valid[i] ? ss.cand_id[lane + 64 * i] : -1;
  }
  int c[NV];
  count_not_below_n<NV>(ss.cand_key, (C + 15) & ~15, ck, c);
  // zero padding only adds to the counts of zero keys, which cannot move the
  // keff-th largest: it is zero itself if a zero key reaches count keff
  uint32_t best = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) best = max(best, valid[i] && c[i] >= keff ? ck[i] : 0u);
  const uint32_t thr = wave_max_u32(best);
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) ngt += __builtin_popcountll(__ballot(valid[i] && ck[i] > thr));
  int eq_before = 0, taken = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint64_t eqm = __ballot(valid[i] && ck[i] == thr);
    const bool sel = valid[i] && (ck[i] > thr ||
                                  (ck[i] == thr && eq_before + lanes_below(eqm) < keff - ngt));
    const uint64_t selm = __ballot(sel);
    if (sel) out[taken + lanes_below(selm)] = ci[i];
    taken += __builtin_popcountll(selm);
    eq_before += __builtin_popcountll(eqm);
  }
}

// Selection among the C (<= 64 * NV) candidates in ss, slot p = candidate p
// in ascending block id: the keff largest keys, ties to the lower slot,
// written in slot order to out[0..keff).
template <int NV>
__device__ __forceinline__ void select_candidates(const SelectSmem &ss, int C, int keff, int32_t *out) {
  const int lane = threadIdx.x & 63;
  uint32_t ck[NV];
  int32_t ci[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int p = lane + 64 * i;
    ck[i] = p < C ? ss.cand_key[p] : 0u;
    ci[i] = p < C ? ss.cand_id[p] : -1;
  }
  const uint32_t thr = wave_kth_largest<NV>(ck, keff);
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) ngt += __builtin_popcountll(__ballot(lane + 64 * i < C && ck[i] > thr));
  const int need_eq = keff - ngt;
  int taken = 0, eq_before = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool valid = lane + 64 * i < C;
    const bool is_gt = valid && ck[i] > thr;
    const bool is_eq = valid && ck[i] == thr;
    const uint64_t eqm = __ballot(is_eq);
    const bool sel = is_gt || (is_eq && eq_before + lanes_below(eqm) < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) out[taken + lanes_below(selm)] = ci[i];
    taken += __builtin_popcountll(selm);
    eq_before += __builtin_popcountll(eqm);
  }
}

// Top-k selection run by one whole wavefront: the k_eff = min(k, N) largest
// keys[0..N) (unsigned compare, equal keys going to the lower index), their
// indices written in ascending order to out[0..k_eff) and -1 after, up to k.
// keys[N..) must be zero up to the next multiple of 256.
//
// A filter bound t0 (topk_filter over 64 or 128 groups; topk_filter256 when that leaves more
// than kMaxCandidates) leaves the keys >= t0 as candidates, usually a few
// more than k; they are compacted in id order and the k-th largest among
// them is found from broadcast counts (up to 128 of them) or by ballot
// bisection (up to kMaxCandidates).  More
// candidates, or k > 64, fall back to the radix select.
// Either way the result is the exact top k under the tie rule.
constexpr int kMaxCandidates = 256;
__device__ __forceinline__ void wave_select_topk(const uint32_t *keys, int N, int k, int32_t *out,
                                                 SelectSmem &ss) {
  const int lane = threadIdx.x & 63;
  const int keff = k < N ? k : N;
  if (keff == N) {  // every block is selected (also N == 0)
    for (int r = lane; r < k; r += 64) out[r] = r < N ? r : -1;
    return;
  }
  bool done = false;
  if (k <= 64) {
    // keys >= t0 to ss in id order (the first kMaxCandidates); returns how many
    auto compact = [&](uint32_t t0) {
      int C = 0;
      for (int base = 0; base < N; base += 256) {
        uint32_t key[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = keys[base + 64 * u + lane];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int n = base + 64 * u + lane;
          const bool cand = n < N && key[u] >= t0;
          const uint64_t bm = __ballot(cand);
          const int pos = C + lanes_below(bm);
          if (cand && pos < kMaxCandidates) {
            ss.cand_key[pos] = key[u];
            ss.cand_id[pos] = n;
          }
          C += __builtin_popcountll(bm);
        }
      }
      return C;
    };
    int C = compact(k <= 32 ? topk_filter<1>(keys, N, k, ss) : topk_filter<2>(keys, N, k, ss));
    if (C > kMaxCandidates && N > 256) C = compact(topk_filter256(keys, N, k));
    if (C <= 128 && lane < 16) ss.cand_key[C + lane] = 0u;  // pad to a multiple of 16
    if (C <= kMaxCandidates) {
      wave_lds_sync();
      if (C <= 64)
        select_candidates_rank<1>(ss, C, keff, out);
      else if (C <= 128)
        select_candidates_rank<2>(ss, C, keff, out);
      else
        select_candidates<kMaxCandidates / 64>(ss, C, keff, out);
      done = true;
    }
  }
  if (!done) wave_radix_select(keys, N, keff, out, ss);
  for (int r = keff + lane; r < k; r += 64) out[r] = -1;
}

// Outputs of a (b, g) with no chunk to attend (empty context).
template <int kMode>
__device__ __forceinline__ void write_empty(const AttnArgs &a, int b, int g, int D) {
  const int G = a.group;
  for (int i = threadIdx.x; i < G * D; i += kThreads)
    a.out[((int64_t)b * a.num_q_heads + g * G) * D + i] = 0.f;
  if (a.lse != nullptr)
    for (int h = threadIdx.x; h < G; h += kThreads)
      a.lse[(int64_t)b * a.num_q_heads + g * G + h] = kNegInf;
  if constexpr (kMode == kModeScored) {
    if (a.score_out != nullptr)
      for (int n = threadIdx.x; n < a.max_blocks; n += kThreads)
        a.score_out[((int64_t)b * a.num_kv_heads + g) * a.max_blocks + n] = 0.f;
    if (a.idx_out != nullptr)
      for (int r = threadIdx.x; r < a.k; r += kThreads)
        a.idx_out[((int64_t)b * a.num_kv_heads + g) * a.k + r] = -1;
  }
  if constexpr (mode_sparse(kMode)) {
    if (a.sel_log != nullptr)
      for (int r = threadIdx.x; r < a.k; r += kThreads) {
        const int64_t i = ((int64_t)b * a.num_kv_heads + g) * a.k + r;
        a.sel_log[i] = a.sel[i];
      }
  }
}

// Two-level merge, run by the last workgroup of group q to arrive: the
// partials of its gsize splits q*kGroupSplits ... become one group partial
// (max m_q over the splits, sum and output rescaled to m_q), stored with
// coherent stores like the split partials.  Thread (h, c) handles 4 columns
// of one head; every load is issued before the first use.
template <int D>
__device__ __forceinline__ void merge_group(const AttnArgs &a, int b, int g, int q, int gsize) {
  const int G = a.group;
  if ((int)threadIdx.x >= G * (D / 4)) return;
  const int h = threadIdx.x / (D / 4), c = 4 * (threadIdx.x % (D / 4));
  const int64_t row = ((int64_t)b * a.num_q_heads + g * G + h);
  const int s0 = q * kGroupSplits;
  const __amdgpu_buffer_rsrc_t pml = buffer(a.part_ml + (row * a.nsplit + s0) * 2, (uint32_t)(gsize * 2 * 4));
  const __amdgpu_buffer_rsrc_t po = buffer(a.part_o + (row * a.nsplit + s0) * D, (uint32_t)(gsize * D * 4));
  float m[kGroupSplits], l[kGroupSplits];
  f32x4 o[kGroupSplits];
#pragma unroll
  for (int j = 0; j < kGroupSplits; ++j) {
    const uint32_t ml_off = j < gsize ? (uint32_t)(j * 2 * 4) : 0x80000000u;
    const uint32_t o_off = j < gsize ? (uint32_t)((j * D + c) * 4) : 0x80000000u;
    m[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pml, ml_off, 0, kCoherent));
    l[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pml, ml_off + 4u, 0, kCoherent));
    o[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(po, o_off, 0, kCoherent));
  }
  float mq = kNegInf;
#pragma unroll
  for (int j = 0; j < kGroupSplits; ++j)
    if (j < gsize) mq = fmaxf(mq, m[j]);
  float lq = 0.f;
  f32x4 oq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kGroupSplits; ++j) {
    const float f = j < gsize ? rescale(m[j], mq) : 0.f;
    lq += f * l[j];
    oq += f * o[j];
  }
  const __amdgpu_buffer_rsrc_t po2 = buffer(a.part_o2 + row * kMaxGroups * D, (uint32_t)(kMaxGroups * D * 4));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oq), po2, (uint32_t)((q * D + c) * 4), 0,
                                         kCoherent);
  if (c == 0) {
    store_agent(a.part_ml2 + (row * kMaxGroups + q) * 2 + 0, mq);
    store_agent(a.part_ml2 + (row * kMaxGroups + q) * 2 + 1, lq);
  }
}


// Hand-off of the workgroup partial (the eight wavefront states merged, and
// in scored mode the block masses rescaled to the partial's max) to the
// epilogue.  Every workgroup stores its partial with coherent device-scope
// stores and waits for them to complete before its arrival is counted, so
// the last arrival of (b, g) -- which returns true and runs the epilogue --
// finds every partial in memory.  Two levels: the arrival is first counted
// in the split's group; the group's last arrival merges the group and
// counts it among the groups of (b, g).
template <int D, int kMode, bool kTwoLevel>
__device__ __forceinline__ bool finish_split(const AttnArgs &a, int b, int g, int s, int nact,
                                             int c_begin, int c_end, int T, SplitSmem<D> &sm,
                                             int *last_flag) {
  const int G = a.group;
  const int64_t head0 = (int64_t)b * a.num_q_heads + g * G;
  const __amdgpu_buffer_rsrc_t po = buffer(a.part_o + head0 * a.nsplit * D,
                                           (uint32_t)(G * a.nsplit * D * 4));
  for (int item = threadIdx.x; item < G * (D / 4); item += kThreads) {
    const int h = item / (D / 4), c = 4 * (item % (D / 4));
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm.m[w][h]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = rescale(sm.m[w][h], m);
      o += f * *reinterpret_cast<const f32x4 *>(&sm.o[w][h][c]);
      l += f * sm.l[w][h];
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), po,
                                           (uint32_t)(((h * a.nsplit + s) * D + c) * 4), 0,
                                           kCoherent);
    if (c == 0) {
      const int64_t row = (head0 + h) * a.nsplit + s;
      store_agent(a.part_ml + row * 2 + 0, m);
      store_agent(a.part_ml + row * 2 + 1, l);
    }
  }
  if constexpr (kMode == kModeScored) {
    const int nb0 = c_begin / kChunksPerBlock;
    const int nblk = (c_end - c_begin + kChunksPerBlock - 1) / kChunksPerBlock;
    const int N = (T + kBlockTokens - 1) / kBlockTokens;
    for (int item = threadIdx.x; item < G * nblk; item += kThreads) {
      const int h = item / nblk, nl = item % nblk;
      float m = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm.m[w][h]);
      float v = 0.f;
      if (m != kNegInf)
#pragma unroll
        for (int j = 0; j < kChunksPerBlock; ++j) {
          const int cl = kChunksPerBlock * nl + j;  // chunk of the block, relative to c_begin
          if (c_begin + cl < c_end) v += sm.cp[cl][h] * rescale(sm.cm[cl][h], m);
        }
      if (nb0 + nl < N) store_agent(a.stats + (head0 + h) * a.max_blocks + nb0 + nl, v);
    }
  }
  // every store of this workgroup completes before the arrival is counted;
  // the last arrival then reads everyone's.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (kTwoLevel) {
    const int q = s / kGroupSplits;
    const int gsize = min(kGroupSplits, nact - q * kGroupSplits);
    if (threadIdx.x == 0) {
      int32_t *cnt = a.counters + kGroupCounterBase + ((int64_t)b * a.num_kv_heads + g) * kMaxGroups + q;
      const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev == gsize - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *last_flag = last ? 1 : 0;
    }
    __syncthreads();
    const bool group_last = *last_flag != 0;
    __syncthreads();  // every thread has read the flag before it is written again
    if (!group_last) return false;
    merge_group<D>(a, b, g, q, gsize);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int32_t *cnt = a.counters + (int64_t)b * a.num_kv_heads + g;
    const int arrivals = kTwoLevel ? (nact + kGroupSplits - 1) / kGroupSplits : nact;
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == arrivals - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = last ? 1 : 0;
  }
  __syncthreads();
  // the split LDS is no longer read: the epilogue may overwrite it at once
  return *last_flag != 0;
}

// Loads and reductions of the per-head statistics of the split partials.
// Wavefront w serves heads w and w + kWaves; lane j of it split j (and
// j + 64, ...).  Every load is issued before the first use; loads a shape
// does not need read past their buffer resource, which returns 0 without a
// memory access.
template <int HH, bool kTwoLevel>
struct HeadStats {
  float ms[HH][kMaxSplits / 64], ls[HH][kMaxSplits / 64];
  float m2[HH];

  __device__ __forceinline__ void load_ml(const AttnArgs &a, int64_t head0, int nact, int hh,
                                          int j) {
    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    const int h = w + kWaves * hh, s = lane + 64 * j;
    const bool in = h < a.group && s < nact;
    const __amdgpu_buffer_rsrc_t pml = buffer(a.part_ml + head0 * a.nsplit * 2,
                                              (uint32_t)(a.group * a.nsplit * 2 * 4));
    // two 32-bit loads: this toolchain compiles the 64-bit raw buffer load
    // builtin into a single 32-bit load whose word fills both halves
    const uint32_t off = in ? (uint32_t)((h * a.nsplit + s) * 2 * 4) : 0x80000000u;
    const uint32_t m_bits = __builtin_amdgcn_raw_buffer_load_b32(pml, off, 0, kCoherent);
    const uint32_t l_bits = __builtin_amdgcn_raw_buffer_load_b32(pml, off + 4u, 0, kCoherent);
    ms[hh][j] = in ? __builtin_bit_cast(float, m_bits) : kNegInf;
    ls[hh][j] = in ? __builtin_bit_cast(float, l_bits) : 0.f;
  }

  // The loads every shape needs: splits 0..63 of head w (and the group
  // maxima with two levels), straight-line.
  __device__ __forceinline__ void load_first(const AttnArgs &a, int64_t head0, int nact, int nparts) {
    const int G = a.group;
    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
    load_ml(a, head0, nact, 0, 0);
    if constexpr (kTwoLevel) {
      const __amdgpu_buffer_rsrc_t pml2 =
          buffer(a.part_ml2 + head0 * kMaxGroups * 2, (uint32_t)(G * kMaxGroups * 2 * 4));
#pragma unroll
      for (int hh = 0; hh < HH; ++hh) {
        const int h = w + kWaves * hh;
        const bool in = h < G && lane < nparts;
        const uint32_t off = in ? (uint32_t)((h * kMaxGroups + lane) * 2 * 4) : 0x80000000u;
        const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b32(pml2, off, 0, kCoherent);
        m2[hh] = in ? __builtin_bit_cast(float, bits) : kNegInf;
      }
    }
  }

  // The loads of larger shapes (a second head per wavefront, more than 64
  // splits), behind uniform branches: issued after every straight-line load,
  // since a branch around a load makes the compiler wait for it at the join.
  __device__ __forceinline__ void load_rest(const AttnArgs &a, int64_t head0, int nact) {
    const int w = uniform(threadIdx.x >> 6);
#pragma unroll
    for (int hh = 0; hh < HH; ++hh)
#pragma unroll
      for (int j = 0; j < kMaxSplits / 64; ++j) {
        if (hh == 0 && j == 0) continue;
        ms[hh][j] = kNegInf;
        ls[hh][j] = 0.f;
        if (w + kWaves * hh < a.group && 64 * j < nact) load_ml(a, head0, nact, hh, j);
      }
  }

  // Global max M and sum L of each head and the per-split (two levels: per
  // group) rescale factors, into LDS.
  __device__ __forceinline__ void reduce(const AttnArgs &a, int nact, int nparts, EpiSmem &sm) {
    const int G = a.group;
    const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
#pragma unroll
    for (int hh = 0; hh < HH; ++hh) {
      const int h = w + kWaves * hh;
      if (h >= G) continue;
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < kMaxSplits / 64; ++j) mx = fmaxf(mx, ms[hh][j]);
      const float M = wave_max(mx);
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxSplits / 64; ++j) {
        const int s = lane + 64 * j;
        const float f = rescale(ms[hh][j], M);
        if (s < nact) sm.f[h][s] = f;
        lsum += f * ls[hh][j];
      }
      if constexpr (kTwoLevel) {
        if (lane < nparts) sm.f2[h][lane] = rescale(m2[hh], M);
      }
      const float L = wave_sum(lsum);
      if (lane == 0) {
        sm.M[h] = M;
        sm.L[h] = L;
        sm.invL[h] = L > 0.f ? 1.f / L : 0.f;
      }
    }
  }
};

// Output merge of the partials of (b, g) into out / lse by the nw
// wavefronts [w0, w0 + nw) of the workgroup.  An item is (head h, 4
// columns); each of those wavefronts serves iw items (16, 32 or 64) with
// 64 / iw stripes of the partials per item, and the stripes are summed with
// lane shuffles, so the merge needs no barrier.  Items beyond nw * iw come
// in further passes.  The first batch of loads of the first pass is issued
// early (issue_first), before the per-head factors are known.
template <int D, int kBatch, bool kTwoLevel>
struct OutputMerge {
  __amdgpu_buffer_rsrc_t po;
  int items, iw, stripes, span, nparts, pstride, il, stripe, ow;
  f32x4 first[kBatch];

  __device__ __forceinline__ void init(const AttnArgs &a, int64_t head0, int nact, int ow_, int nw) {
    const int G = a.group;
    items = G * (D / 4);
    const int per_wave = (items + nw - 1) / nw;
    iw = per_wave > 32 ? 64 : per_wave > 16 ? 32 : 16;
    stripes = 64 / iw;
    span = nw * iw;
    const int lane = threadIdx.x & 63;
    il = lane & (iw - 1);
    stripe = lane / iw;
    ow = ow_;
    nparts = kTwoLevel ? (nact + kGroupSplits - 1) / kGroupSplits : nact;
    pstride = kTwoLevel ? kMaxGroups : a.nsplit;
    po = kTwoLevel ? buffer(a.part_o2 + head0 * kMaxGroups * D, (uint32_t)(G * kMaxGroups * D * 4))
                   : buffer(a.part_o + head0 * a.nsplit * D, (uint32_t)(G * a.nsplit * D * 4));
  }
  __device__ __forceinline__ int item(int pass) const { return pass * span + ow * iw + il; }
  // loads of partials stripe + stripes * (j0 + j), j < kBatch, of item `it`
  // (an item past the end reads nothing)
  __device__ __forceinline__ void issue(f32x4 (&v)[kBatch], int it, int j0) const {
    const int h = it / (D / 4), c = 4 * (it % (D / 4));
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = stripe + stripes * (j0 + j);
      const uint32_t off = (it < items && s < nparts)
                               ? (uint32_t)(((h * pstride + s) * D + c) * 4)
                               : 0x80000000u;
      v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(po, off, 0, kCoherent));
    }
  }
  __device__ __forceinline__ void issue_first(bool participate) {
    issue(first, participate ? item(0) : items, 0);
  }
  __device__ __forceinline__ void accumulate(f32x4 &acc, const f32x4 (&v)[kBatch], int it, int j0,
                                             const EpiSmem &sm) const {
    const int h = it / (D / 4);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = stripe + stripes * (j0 + j);
      if (it < items && s < nparts) acc += (kTwoLevel ? sm.f2[h][s] : sm.f[h][s]) * v[j];
    }
  }
  // Runs every pass and writes out (and lse from the first wavefront).
  __device__ __forceinline__ void run(const AttnArgs &a, int64_t head0, const EpiSmem &sm) {
    const int lane = threadIdx.x & 63;
    const int per_stripe = (nparts + stripes - 1) / stripes;
    for (int pass = 0; pass * span < items; ++pass) {
      const int it = item(pass);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (pass == 0) accumulate(acc, first, it, 0, sm);
      for (int j0 = pass == 0 ? kBatch : 0; j0 < per_stripe; j0 += kBatch) {
        f32x4 v[kBatch];
        issue(v, it, j0);
        accumulate(acc, v, it, j0, sm);
      }
      for (int off = iw; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off);
        acc.y += __shfl_xor(acc.y, off);
        acc.z += __shfl_xor(acc.z, off);
        acc.w += __shfl_xor(acc.w, off);
      }
      if (stripe == 0 && it < items) {
        const int h = it / (D / 4), c = 4 * (it % (D / 4));
        const float L = sm.L[h];
        const f32x4 o = L > 0.f ? acc * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4 *>(a.out + (head0 + h) * D + c) = o;
      }
    }
    if (a.lse != nullptr && ow == 0 && lane < a.group) {
      const float L = sm.L[lane];
      a.lse[head0 + lane] = L > 0.f ? (sm.M[lane] + __log2f(L)) * kLn2 : kNegInf;
    }
  }
};

// Epilogue of the full and sparse modes: every wavefront merges output.
template <int D, int kBatch, int HH, bool kTwoLevel, int kMode>
__device__ __forceinline__ void epilogue_plain(const AttnArgs &a, int b, int g, int nact, EpiSmem &sm) {
  const int w = uniform(threadIdx.x >> 6);
  const int64_t head0 = (int64_t)b * a.num_q_heads + g * a.group;
  OutputMerge<D, kBatch, kTwoLevel> mg;
  mg.init(a, head0, nact, w, kWaves);
  HeadStats<HH, kTwoLevel> hs;
  hs.load_first(a, head0, nact, mg.nparts);
  mg.issue_first(true);
  hs.load_rest(a, head0, nact);
  hs.reduce(a, nact, mg.nparts, sm);
  __syncthreads();
  mg.run(a, head0, sm);
  if constexpr (mode_sparse(kMode)) {
    if (a.sel_log != nullptr) {
      const int64_t r0 = ((int64_t)b * a.num_kv_heads + g) * a.k;
      for (int r = threadIdx.x; r < a.k; r += kThreads) a.sel_log[r0 + r] = a.sel[r0 + r];
    }
  }
}

// Epilogue of the scored mode.  After the per-head statistics, wavefronts
// [0, kScoreWaves) turn the block masses into block scores (mass stored
// relative to its split's max; f brings it to the head's max) and wavefront
// 0 selects the top-k, while the other wavefronts merge the output; the two
// groups meet at one barrier only, before the selection.  The masses of the
// first MJ blocks of each score thread and kBatch output partials per merge
// thread are loaded before the statistics are reduced.
template <int D, int GP, int kBatch, bool kTwoLevel>
__device__ __forceinline__ void epilogue_scored(const AttnArgs &a, int b, int g, int T, int nact,
                                                EpiSmem &sm) {
  constexpr int MJ = GP > 8 ? 2 : 4;
  constexpr int HH = GP > kWaves ? 2 : 1;
  const int G = a.group;
  const int w = uniform(threadIdx.x >> 6);
  const bool scorer = w < kScoreWaves;
  const int64_t head0 = (int64_t)b * a.num_q_heads + g * G;
  const int N = (T + kBlockTokens - 1) / kBlockTokens;
  const int blocks_per_split = a.chunks_per_wg / kChunksPerBlock;
  OutputMerge<D, kBatch, kTwoLevel> mg;
  mg.init(a, head0, nact, scorer ? 0 : w - kScoreWaves, kWaves - kScoreWaves);
  HeadStats<HH, kTwoLevel> hs;
  hs.load_first(a, head0, nact, mg.nparts);
  mg.issue_first(!scorer);
  const __amdgpu_buffer_rsrc_t pst = buffer(a.stats + head0 * a.max_blocks,
                                            (uint32_t)(G * a.max_blocks * 4));
  float mass[MJ][GP];
#pragma unroll
  for (int j = 0; j < MJ; ++j)
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const int n = threadIdx.x + kScoreThreads * j;
      const uint32_t off = (scorer && h < G && n < N)
                               ? (uint32_t)((h * a.max_blocks + n) * 4)
                               : 0x80000000u;
      mass[j][h] =
          __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pst, off, 0, kCoherent));
    }
  hs.load_rest(a, head0, nact);
  hs.reduce(a, nact, mg.nparts, sm);
  __syncthreads();

  if (scorer) {
    float *so = a.score_out != nullptr
                    ? a.score_out + ((int64_t)b * a.num_kv_heads + g) * a.max_blocks
                    : nullptr;
    auto score_of = [&](int n, const float (&ms)[GP]) {
      const int s = n / blocks_per_split;
      float score = 0.f;
#pragma unroll
      for (int h = 0; h < GP; ++h)
        if (h < G) score += ms[h] * sm.f[h][s] * sm.invL[h];
      return score;
    };
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int n = threadIdx.x + kScoreThreads * j;
      if (n < N) {
        const float score = score_of(n, mass[j]);
        sm.keys[n] = score > 0.f ? __float_as_uint(score) : 0u;
        if (so != nullptr) so[n] = score;
      } else if (so != nullptr && n < a.max_blocks) {
        so[n] = 0.f;
      }
    }
    for (int n = threadIdx.x + kScoreThreads * MJ; n < a.max_blocks; n += kScoreThreads) {
      if (n < N) {
        float ms[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h)
          ms[h] = h < G ? load_agent(a.stats + (head0 + h) * a.max_blocks + n) : 0.f;
        const float score = score_of(n, ms);
        sm.keys[n] = score > 0.f ? __float_as_uint(score) : 0u;
        if (so != nullptr) so[n] = score;
      } else if (so != nullptr) {
        so[n] = 0.f;
      }
    }
    // the selection reads whole rows of 256 keys: zero the keys past N
    for (int n = N + threadIdx.x; n < ((N + 255) & ~255); n += kScoreThreads) sm.keys[n] = 0u;
  }
  __syncthreads();
  // the score wavefronts return here: wavefront 0 selects (in epilogue())
  if (!scorer) mg.run(a, head0, sm);
}

// Picks the epilogue instance whose load counts fit (b, g).  Scored mode:
// group bound GP >= G (mass loads of GP heads) and the output partials each
// merge thread loads at once.  Other modes: kBatch split partials per output
// thread in a batch (more run in further batches) and heads per wavefront.
// Only the bf16 kernel with d = 128 (the large shapes) gets specialised
// instances; the others use one generic instance.
template <int D, int kMode, bool kTwoLevel, bool kSpecialise>
__device__ __forceinline__ void epilogue(const AttnArgs &a, int b, int g, int T, int nact, EpiSmem &sm) {
  if constexpr (kMode == kModeScored) {
    if constexpr (!kSpecialise) {
      epilogue_scored<D, kMaxGroup, 8, kTwoLevel>(a, b, g, T, nact, sm);
    } else {
      const int G = uniform(a.group);
      if (G <= 4)
        epilogue_scored<D, 4, 16, kTwoLevel>(a, b, g, T, nact, sm);
      else if (G <= 8)
        epilogue_scored<D, 8, 16, kTwoLevel>(a, b, g, T, nact, sm);
      else
        epilogue_scored<D, 16, 8, kTwoLevel>(a, b, g, T, nact, sm);
    }
    // one copy of the selection for every instance above (keys in LDS)
    if (uniform(threadIdx.x >> 6) == 0 && a.idx_out != nullptr) {
      const int N = (T + kBlockTokens - 1) / kBlockTokens;
      wave_select_topk(sm.keys, N, a.k, a.idx_out + ((int64_t)b * a.num_kv_heads + g) * a.k,
                       sm.sel);
    }
  } else if constexpr (!kSpecialise || kTwoLevel) {
    epilogue_plain<D, 8, 2, kTwoLevel, kMode>(a, b, g, nact, sm);
  } else {
    // partials per output thread: 8 wavefronts serve G * D / 4 items
    const int G = uniform(a.group);
    const int per_wave = (G * (D / 4) + kWaves - 1) / kWaves;
    const int stripes = per_wave > 32 ? 1 : per_wave > 16 ? 2 : 4;
    const int per = uniform((nact + stripes - 1) / stripes);
    if (G <= 8) {
      if (per <= 4)
        epilogue_plain<D, 4, 1, false, kMode>(a, b, g, nact, sm);
      else if (per <= 8)
        epilogue_plain<D, 8, 1, false, kMode>(a, b, g, nact, sm);
      else
        epilogue_plain<D, 16, 1, false, kMode>(a, b, g, nact, sm);
    } else {
      epilogue_plain<D, 8, 2, false, kMode>(a, b, g, nact, sm);
    }
  }
}

// Common prologue: range of the workgroup, early exits.  Returns false if the
// workgroup has nothing to do.
struct Range {
  int T, C, c_begin, c_end, nact;
};
template <int kMode>
__device__ __forceinline__ bool wg_range(const AttnArgs &a, int s, int g, int b, int D, int ctx_b,
                                         Range &r) {
  r.T = clamp_ctx(ctx_b, a.max_blocks);
  r.C = chunk_positions<kMode>(r.T, a.k);
  if (r.C == 0) {
    if (s == 0) write_empty<kMode>(a, b, g, D);
    return false;
  }
  r.c_begin = s * a.chunks_per_wg;
  if (r.c_begin >= r.C) return false;
  r.c_end = min(r.C, r.c_begin + a.chunks_per_wg);
  r.nact = (r.C + a.chunks_per_wg - 1) / a.chunks_per_wg;
  return true;
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

template <int D, int kMode, bool kTwoLevel = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_split_bf16(
    AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  __shared__ KernelSmem<D> sm;
  __shared__ int last_flag;
  Range r;
  // the context length and the first chunk's block id and page are loaded
  // together (prefetch_first)
  const int ctx_b = scalar_load(a.ctx, b);
  const FirstChunk first =
      prefetch_first<kMode>(a, b, g, chunk_of(s * a.chunks_per_wg, uniform(threadIdx.x >> 6), 0));
  if (!wg_range<kMode>(a, s, g, b, D, ctx_b, r)) return;
  const int T = r.T, c_begin = r.c_begin, c_end = r.c_end;
  constexpr bool want_mass = kMode == kModeScored;

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

  float m_run = kNegInf, l_run = 0.f, cmass = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const char *kpool = static_cast<const char *>(a.k_pool);
  const char *vpool = static_cast<const char *>(a.v_pool);
  const int Hkv = a.num_kv_heads;
  // per-lane byte offsets inside a chunk's K rows / V columns (chunk-invariant)
  const uint32_t k_lane = (uint32_t)(((8 * (m16 >> 2) + (m16 & 3)) * D + 8 * quad) * 2);
  const uint32_t v_lane = (uint32_t)((m16 * kChunkTokens + 8 * quad) * 2);

  // Issues the 16-byte loads of chunk `pos` into t through buffer resources
  // spanning just that chunk; returns its valid token count.  A position past
  // the range or without a readable page gets an empty resource: the loads
  // return zeros without touching memory, so every path issues the same loads
  // and the register tiles never need copying.
  auto issue = [&](BfTile<D> &t, int pos, bool live, bool is_first = false) -> int {
    int page = 0, sub = 0, valid = 0;
    const bool ok = live && pos < c_end &&
                    (is_first ? resolve_first<kMode>(a, T, pos, first, page, sub, valid)
                              : resolve_chunk<kMode>(a, b, g, T, pos, page, sub, valid));
    if (!ok) {
      page = 0;
      sub = 0;
      valid = 0;
    }
    const int64_t tile = (int64_t)page * Hkv + g;
    // K chunk: 32 token rows of d; V sub-tile: d rows of 32 tokens (8 KiB each at d = 128)
    const char *kb = kpool + (tile * kBlockTokens + sub * kChunkTokens) * D * 2;
    const char *vb = vpool + (tile * kChunksPerBlock + sub) * D * kChunkTokens * 2;
    const __amdgpu_buffer_rsrc_t krs = buffer(kb, ok ? kChunkTokens * D * 2 : 0);
    const __amdgpu_buffer_rsrc_t vrs = buffer(vb, ok ? kChunkTokens * D * 2 : 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        t.k[h][k] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_lane, (4 * h * D + 32 * k) * 2,
                                                          kStreaming);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
      t.v[n] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_lane, n * 16 * kChunkTokens * 2,
                                                     kStreaming);
    return valid;
  };

  auto consume = [&](const BfTile<D> &t, int valid) {
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
    cmass = ps;
    m_run = m_new;
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

  // consumes the i-th chunk of the wavefront and, in full mode with scores,
  // records its softmax mass (0 for a chunk without tokens)
  auto step = [&](const BfTile<D> &t, int i, int valid) {
    cmass = 0.f;
    if (valid > 0) consume(t, valid);
    if (want_mass && quad == 0 && m16 < G) {
      const int cl = w + kWaves * i;
      sm.split.cm[cl][m16] = m_run;
      sm.split.cp[cl][m16] = cmass;
    }
  };

  // Two register tiles: the next chunk's loads are in flight while the
  // current one is consumed.
  BfTile<D> ta, tb;
  int i = 0;
  bool live = chunk_live(c_begin, c_end, w, 0);
  int va = issue(ta, chunk_of(c_begin, w, 0), live, true);
  while (live) {
    const bool live_b = chunk_live(c_begin, c_end, w, i + 1);
    const int vb = issue(tb, chunk_of(c_begin, w, i + 1), live_b);
    step(ta, i, va);
    ++i;
    if (!live_b) break;
    const bool live_a = chunk_live(c_begin, c_end, w, i + 1);
    va = issue(ta, chunk_of(c_begin, w, i + 1), live_a);
    step(tb, i, vb);
    ++i;
    live = live_a;
  }

  if (quad == 0) {
    sm.split.m[w][m16] = m_run;
    sm.split.l[w][m16] = l_run;
  }
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.split.o[w][4 * quad + r][16 * n + m16] = acc[n][r];
  __syncthreads();
  if (!finish_split<D, kMode, kTwoLevel>(a, b, g, s, r.nact, c_begin, c_end, T, sm.split,
                                         &last_flag))
    return;
  epilogue<D, kMode, kTwoLevel, D == 128 && kMode != kModeStaged>(a, b, g, T, r.nact, sm.epi);
}

// ---------------------------------------------------------------------------
// float32 split kernel (vector ALU).  Lane (t = i%32, half = i/32) computes
// the logits of token t over half of the head dimension for every head of the
// group; p.V runs with lane i owning columns i and i+64.
// ---------------------------------------------------------------------------
template <int D, int kMode>
__global__ __launch_bounds__(kThreads) void attn_split_f32(AttnArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  __shared__ KernelSmem<D> sm;
  __shared__ float q_s[kMaxGroup][D];
  __shared__ int last_flag;
  Range r;
  if (!wg_range<kMode>(a, s, g, b, D, scalar_load(a.ctx, b), r)) return;
  const int T = r.T, c_begin = r.c_begin, c_end = r.c_end;
  constexpr bool want_mass = kMode == kModeScored;

  constexpr int CPL = D / 64;  // output columns per lane
  const int G = a.group;
  const float *qg = static_cast<const float *>(a.q) + ((int64_t)b * a.num_q_heads + g * G) * D;
  for (int i = threadIdx.x; i < G * D; i += kThreads) q_s[i / D][i % D] = qg[i];
  __syncthreads();

  const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
  const int t = lane & 31, half = lane >> 5;
  const float *kpool = static_cast<const float *>(a.k_pool);
  const float *vpool = static_cast<const float *>(a.v_pool);
  const int Hkv = a.num_kv_heads;

  float m_run[kMaxGroup], l_run[kMaxGroup], cmass[kMaxGroup], acc[kMaxGroup][CPL];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
    cmass[h] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[h][j] = 0.f;
  }

  for (int i = 0; chunk_live(c_begin, c_end, w, i); ++i) {
    const int pos = chunk_of(c_begin, w, i);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) cmass[h] = 0.f;
    int page, sub, valid;
    if (pos < c_end && resolve_chunk<kMode>(a, b, g, T, pos, page, sub, valid)) {
      const int64_t tile = (int64_t)page * Hkv + g;
      const float *krow =
          kpool + (tile * kBlockTokens + sub * kChunkTokens + t) * D + half * (D / 2);
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
        cmass[h] = ps;
        m_run[h] = m_new;
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float *vrow = vpool + ((tile * kChunksPerBlock + sub) * D + lane + 64 * j) * kChunkTokens;
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
    if (want_mass && lane == 0) {
      const int cl = w + kWaves * i;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < G) {
          sm.split.cm[cl][h] = m_run[h];
          sm.split.cp[cl][h] = cmass[h];
        }
    }
  }

#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    if (lane == 0) {
      sm.split.m[w][h] = m_run[h];
      sm.split.l[w][h] = l_run[h];
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) sm.split.o[w][h][lane + 64 * j] = acc[h][j];
  }
  __syncthreads();
  if (!finish_split<D, kMode, false>(a, b, g, s, r.nact, c_begin, c_end, T, sm.split, &last_flag))
    return;
  epilogue<D, kMode, false, false>(a, b, g, T, r.nact, sm.epi);
}

// ---------------------------------------------------------------------------
// Top-k of a caller-given score array: grid (Hkv, B).  Every thread loads
// keys (the float bits of the non-negative scores, monotone as unsigned
// integers) into LDS; wavefront 0 then selects.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void score_topk(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int T = clamp_ctx(a.ctx[b], a.max_blocks);
  const int N = (T + kBlockTokens - 1) / kBlockTokens;
  __shared__ uint32_t keys[kMaxBlocks];
  __shared__ SelectSmem ss;
  const float *row = a.score + ((int64_t)b * a.num_kv_heads + g) * a.max_blocks;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    const float sc = row[n];
    keys[n] = sc > 0.f ? __float_as_uint(sc) : 0u;
  }
  for (int n = N + threadIdx.x; n < ((N + 255) & ~255); n += kThreads) keys[n] = 0u;
  __syncthreads();
  if (uniform(threadIdx.x >> 6) == 0)
    wave_select_topk(keys, N, a.k, a.idx + ((int64_t)b * a.num_kv_heads + g) * a.k, ss);
}

// Kernel timers: while a timer runs, each launch of its kind takes an event
// pair that the launch itself records (hipExtLaunchKernel stamps the events
// with the dispatch's own start and end), so the elapsed time is the kernel's
// execution without the separate event packets' overhead.
struct KernelTimer {
  bool running = false;
  int recorded = 0;
  std::vector<hipEvent_t> start, stop;
};
KernelTimer g_timers[kNumTimers];

struct TimerScope {
  hipEvent_t start = nullptr, stop = nullptr;
  explicit TimerScope(int kind) {
    KernelTimer &t = g_timers[kind];
    if (t.running && t.recorded < (int)t.start.size()) {
      start = t.start[t.recorded];
      stop = t.stop[t.recorded];
      ++t.recorded;
    }
  }
};

}  // namespace

void timer_take(int kind, void **start, void **stop) {
  const TimerScope tm(kind);
  *start = tm.start;
  *stop = tm.stop;
}

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
  const int mode = a.sel != nullptr ? (a.staged ? kModeStaged : kModeSparse)
                                    : (a.stats != nullptr ? kModeScored : kModeFull);
  const TimerScope tm(mode_sparse(mode) ? kTimerSparseAttn
                      : mode == kModeScored ? kTimerFullScored : kTimerFullAttn);
  const dim3 block(kThreads);
#define HYLRA_LAUNCH(K) hipExtLaunchKernelGGL(K, grid, block, 0, st, tm.start, tm.stop, 0, a)
  if (dtype == 1 && head_dim == 128) {
    switch (mode) {
      case kModeFull:
        if (a.two_level) HYLRA_LAUNCH((attn_split_bf16<128, kModeFull, true>));
        else HYLRA_LAUNCH((attn_split_bf16<128, kModeFull, false>));
        break;
      case kModeScored:
        if (a.two_level) HYLRA_LAUNCH((attn_split_bf16<128, kModeScored, true>));
        else HYLRA_LAUNCH((attn_split_bf16<128, kModeScored, false>));
        break;
      case kModeSparse: HYLRA_LAUNCH((attn_split_bf16<128, kModeSparse>)); break;
      default: HYLRA_LAUNCH((attn_split_bf16<128, kModeStaged>)); break;
    }
  } else if (dtype == 1) {
    switch (mode) {
      case kModeFull: HYLRA_LAUNCH((attn_split_bf16<64, kModeFull>)); break;
      case kModeScored: HYLRA_LAUNCH((attn_split_bf16<64, kModeScored>)); break;
      case kModeSparse: HYLRA_LAUNCH((attn_split_bf16<64, kModeSparse>)); break;
      default: HYLRA_LAUNCH((attn_split_bf16<64, kModeStaged>)); break;
    }
  } else if (head_dim == 128) {
    switch (mode) {
      case kModeFull: HYLRA_LAUNCH((attn_split_f32<128, kModeFull>)); break;
      case kModeScored: HYLRA_LAUNCH((attn_split_f32<128, kModeScored>)); break;
      case kModeSparse: HYLRA_LAUNCH((attn_split_f32<128, kModeSparse>)); break;
      default: HYLRA_LAUNCH((attn_split_f32<128, kModeStaged>)); break;
    }
  } else {
    switch (mode) {
      case kModeFull: HYLRA_LAUNCH((attn_split_f32<64, kModeFull>)); break;
      case kModeScored: HYLRA_LAUNCH((attn_split_f32<64, kModeScored>)); break;
      case kModeSparse: HYLRA_LAUNCH((attn_split_f32<64, kModeSparse>)); break;
      default: HYLRA_LAUNCH((attn_split_f32<64, kModeStaged>)); break;
    }
  }
#undef HYLRA_LAUNCH
  return (int)hipGetLastError();
}

// Read probe: each workgroup streams a contiguous range with the K/V loads
// of the attention kernels (16-byte non-temporal buffer loads, four in
// flight per lane) and folds them into one word that is stored only if the
// fold hits a value the probe's callers never place in memory.
constexpr uint32_t kProbeBytesPerWg = 2u << 20;
__global__ __launch_bounds__(kThreads) void read_probe(const char *base, uint64_t bytes,
                                                       uint32_t *sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * kProbeBytesPerWg;
  const uint64_t left = bytes - begin;
  const uint32_t span = left < kProbeBytesPerWg ? (uint32_t)left : kProbeBytesPerWg;
  const __amdgpu_buffer_rsrc_t r = buffer(base + begin, span);
  u32x4 acc = {0u, 0u, 0u, 0u};
  constexpr uint32_t kStep = kThreads * 16 * 4;
  for (uint32_t off = threadIdx.x * 16; off < span; off += kStep) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off + u * kThreads * 16, 0, kStreaming);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = blockIdx.x;
}

int launch_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, void *stream) {
  const unsigned grid = (unsigned)((bytes + kProbeBytesPerWg - 1) / kProbeBytesPerWg);
  hipLaunchKernelGGL(read_probe, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char *>(buf), bytes, sink);
  return (int)hipGetLastError();
}

int launch_topk(const TopkArgs &a, int batch, void *stream) {
  const TimerScope tm(kTimerTopk);
  hipExtLaunchKernelGGL(score_topk, dim3(a.num_kv_heads, batch), dim3(kThreads), 0,
                        static_cast<hipStream_t>(stream), tm.start, tm.stop, 0, a);
  return (int)hipGetLastError();
}

const char *device_error_string(int code) { return hipGetErrorString((hipError_t)code); }

}  // namespace hylra
