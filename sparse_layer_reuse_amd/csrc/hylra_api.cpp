// C ABI of libhylra: argument validation, workspace layout, launch sequencing
// of the decode attention kernels, and the host-side policy dynamic program.
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.2 (offline policy DP) and 2.3 (hybrid
// execution of the policy during decoding).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/hylra.h"
#include "hylra_internal.h"

namespace {

thread_local std::string g_last_error;

hylra_status fail(hylra_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hylra_status ok() {
  g_last_error.clear();
  return HYLRA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hylra_status check_shape(const hylra_shape *s) {
  if (s == nullptr) return fail(HYLRA_E_INVALID_ARG, "shape is NULL");
  if (s->batch < 1) return fail(HYLRA_E_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
  if (s->num_kv_heads < 1 || s->num_q_heads < s->num_kv_heads ||
      s->num_q_heads % s->num_kv_heads != 0)
    return fail(HYLRA_E_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads / s->num_kv_heads > hylra::kMaxGroup)
    return fail(HYLRA_E_UNSUPPORTED, "group size %d exceeds %d query heads per KV head",
                s->num_q_heads / s->num_kv_heads, hylra::kMaxGroup);
  if (s->num_kv_heads > 65535 || s->batch > 65535 ||
      (long)s->batch * s->num_kv_heads > hylra::kCounterSlots)
    return fail(HYLRA_E_UNSUPPORTED, "batch and num_kv_heads must be <= 65535 and their product <= %d",
                hylra::kCounterSlots);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(HYLRA_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->block_size != HYLRA_BLOCK_TOKENS)
    return fail(HYLRA_E_UNSUPPORTED, "block_size must be 128 (got %d)", s->block_size);
  if (s->dtype != HYLRA_F32 && s->dtype != HYLRA_BF16)
    return fail(HYLRA_E_INVALID_ARG, "dtype must be HYLRA_F32 or HYLRA_BF16 (got %d)", s->dtype);
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > hylra::kMaxBlocks)
    return fail(HYLRA_E_UNSUPPORTED, "max_blocks_per_seq must be in [1, %d] (got %d)",
                hylra::kMaxBlocks, s->max_blocks_per_seq);
  if (!(s->scale >= 0.f) || isinf(s->scale))
    return fail(HYLRA_E_INVALID_ARG, "scale must be finite and >= 0");
  return HYLRA_OK;
}

hylra_status check_kv(const hylra_kv *kv) {
  if (kv == nullptr) return fail(HYLRA_E_INVALID_ARG, "kv is NULL");
  if (kv->k_pool == nullptr || kv->v_pool == nullptr || kv->block_table == nullptr ||
      kv->ctx_lens == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "kv has a NULL pointer");
  if (!aligned16(kv->k_pool) || !aligned16(kv->v_pool))
    return fail(HYLRA_E_INVALID_ARG, "K/V pools must be 16-byte aligned");
  if (kv->num_pages < 1) return fail(HYLRA_E_INVALID_ARG, "num_pages must be >= 1");
  return HYLRA_OK;
}

// Length of a selection row: 1 <= k <= kMaxBlocks (every slot of a row is
// walked, so k also bounds the work of a launch).
hylra_status check_k(int k) {
  if (k < 1) return fail(HYLRA_E_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > hylra::kMaxBlocks)
    return fail(HYLRA_E_UNSUPPORTED, "k must be <= %d (got %d)", hylra::kMaxBlocks, k);
  return HYLRA_OK;
}

float logit_scale_log2(const hylra_shape *s) {
  const float scale = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  return scale * 1.4426950408889634f;
}

// Workspace carve-up shared by every entry point.
struct Workspace {
  float *part_ml;
  float *part_o;
  float *stats;
  int32_t *counters;
  int32_t *idx;
  float *part_ml2;  // two-level merge of the full plan only, else null
  float *part_o2;
  size_t bytes;
};

// Whether a full-mode launch of this shape merges its split partials in two
// levels: one merging workgroup per (sequence, KV head) would read more than
// kOneLevelMergeBytes of partials (~90 GB/s through one compute unit).  Only
// the bf16, d = 128 kernel has the two-level instance; its group counters
// must fit the upper half of the counter region.
bool two_level_merge(const hylra_shape *s, const hylra::SplitPlan &p) {
  const long part_bytes = (long)(s->num_q_heads / s->num_kv_heads) * s->head_dim * 4;
  return s->dtype == HYLRA_BF16 && s->head_dim == 128 &&
         (long)p.nsplit * part_bytes > hylra::kOneLevelMergeBytes &&
         (long)s->batch * s->num_kv_heads * hylra::kMaxGroups <=
             hylra::kCounterSlots - hylra::kGroupCounterBase;
}

int max_nsplit(const hylra_shape *s, int k) {
  const hylra::SplitPlan f = hylra::plan_full(s->batch, s->num_kv_heads, s->max_blocks_per_seq);
  int n = f.nsplit;
  if (k > 0) {
    const hylra::SplitPlan p =
        hylra::plan_sparse(s->batch, s->num_kv_heads, s->max_blocks_per_seq, k,
                           s->num_q_heads / s->num_kv_heads, s->head_dim);
    if (p.nsplit > n) n = p.nsplit;
  }
  return n;
}

Workspace layout(const hylra_shape *s, int k, void *base) {
  const size_t B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, D = s->head_dim;
  const size_t mb = s->max_blocks_per_seq;
  const size_t ns = max_nsplit(s, k);
  const size_t a = 256;
  size_t off = 0;
  Workspace w{};
  char *p = static_cast<char *>(base);
  auto take = [&](size_t bytes) -> char * {
    char *r = p ? p + off : nullptr;
    off = round_up(off + bytes, a);
    return r;
  };
  // counters first, in a fixed-size region: every shape finds them at the same
  // place, so a workspace reused across shapes keeps them zero between calls
  w.counters = reinterpret_cast<int32_t *>(take(hylra::kCounterSlots * sizeof(int32_t)));
  w.part_ml = reinterpret_cast<float *>(take(B * Hq * ns * 2 * sizeof(float)));
  w.part_o = reinterpret_cast<float *>(take(B * Hq * ns * D * sizeof(float)));
  w.stats = reinterpret_cast<float *>(take(B * Hq * mb * sizeof(float)));
  w.idx = reinterpret_cast<int32_t *>(take(B * Hkv * (size_t)(k > 0 ? k : 1) * sizeof(int32_t)));
  if (two_level_merge(s, hylra::plan_full(s->batch, s->num_kv_heads, s->max_blocks_per_seq))) {
    w.part_ml2 = reinterpret_cast<float *>(take(B * Hq * hylra::kMaxGroups * 2 * sizeof(float)));
    w.part_o2 = reinterpret_cast<float *>(take(B * Hq * hylra::kMaxGroups * D * sizeof(float)));
  }
  w.bytes = off;
  return w;
}

hylra_status check_ws(const hylra_shape *s, int k, void *ws, size_t ws_bytes, Workspace &w) {
  w = layout(s, k, ws);
  if (ws == nullptr || ws_bytes < w.bytes)
    return fail(HYLRA_E_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", w.bytes, ws_bytes,
                ws == nullptr ? ", NULL" : "");
  if (!aligned16(ws)) return fail(HYLRA_E_INVALID_ARG, "workspace must be 16-byte aligned");
  return HYLRA_OK;
}

hylra_status device_status(int code, const char *what) {
  if (code == 0) return HYLRA_OK;
  return fail(HYLRA_E_DEVICE, "%s: %s", what, hylra::device_error_string(code));
}

hylra::AttnArgs attn_args(const hylra_shape *s, const void *q, const hylra_kv *kv,
                          const int32_t *sel, int k, const hylra::SplitPlan &plan,
                          const Workspace &w) {
  hylra::AttnArgs a{};
  a.q = q;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.num_pages = kv->num_pages;
  a.table = kv->block_table;
  a.ctx = kv->ctx_lens;
  a.sel = sel;
  a.k = k;
  a.max_blocks = s->max_blocks_per_seq;
  a.num_q_heads = s->num_q_heads;
  a.num_kv_heads = s->num_kv_heads;
  a.group = s->num_q_heads / s->num_kv_heads;
  a.scale_log2 = logit_scale_log2(s);
  a.chunks_per_wg = plan.chunks_per_wg;
  a.nsplit = plan.nsplit;
  a.part_ml = w.part_ml;
  a.part_o = w.part_o;
  a.counters = w.counters;
  a.part_ml2 = w.part_ml2;
  a.part_o2 = w.part_o2;
  return a;
}

// Reset layer: one launch -- full attention, merge, and (when asked) block
// scores and the top-k index set.
hylra_status run_full(const hylra_shape *s, const void *q, const hylra_kv *kv, float *out,
                      float *lse, float *block_score, int32_t *idx, int k, const Workspace &w,
                      void *stream) {
  const hylra::SplitPlan plan = hylra::plan_full(s->batch, s->num_kv_heads, s->max_blocks_per_seq);
  hylra::AttnArgs a = attn_args(s, q, kv, nullptr, k, plan, w);
  a.stats = (block_score != nullptr || idx != nullptr) ? w.stats : nullptr;
  a.two_level = two_level_merge(s, plan) ? 1 : 0;
  a.out = out;
  a.lse = lse;
  a.score_out = block_score;
  a.idx_out = idx;
  return device_status(hylra::launch_attn(a, s->dtype, s->head_dim, s->batch, stream),
                       "attention launch");
}

// Reuse layer: one launch -- attention over the selected blocks and merge.
// staged: kv holds staging pools (selection slot r of sequence b in page
// b * k + r) instead of the layer's pools and block table.
hylra_status run_sparse(const hylra_shape *s, const void *q, const hylra_kv *kv,
                        const int32_t *idx, int k, float *out, float *lse, int32_t *log,
                        const Workspace &w, void *stream, bool staged = false) {
  const hylra::SplitPlan plan =
      hylra::plan_sparse(s->batch, s->num_kv_heads, s->max_blocks_per_seq, k,
                         s->num_q_heads / s->num_kv_heads, s->head_dim);
  hylra::AttnArgs a = attn_args(s, q, kv, idx, k, plan, w);
  a.staged = staged ? 1 : 0;
  a.out = out;
  a.lse = lse;
  a.sel_log = log;
  return device_status(hylra::launch_attn(a, s->dtype, s->head_dim, s->batch, stream),
                       "attention launch");
}

size_t elt_bytes(const hylra_shape *s) { return s->dtype == HYLRA_BF16 ? 2 : 4; }

// Gather of the selected blocks of one layer into staging pools.
hylra_status run_gather(const hylra_shape *s, const hylra_kv *kv, const int32_t *idx, int k,
                        void *dst_k, void *dst_v, void *stream) {
  hylra::GatherArgs g{};
  g.k_src = static_cast<const char *>(kv->k_pool);
  g.v_src = static_cast<const char *>(kv->v_pool);
  g.num_pages = kv->num_pages;
  g.table = kv->block_table;
  g.ctx = kv->ctx_lens;
  g.idx = idx;
  g.k = k;
  g.max_blocks = s->max_blocks_per_seq;
  g.num_kv_heads = s->num_kv_heads;
  g.tile_bytes = (int)(hylra::kBlockTokens * s->head_dim * elt_bytes(s));
  g.k_dst = static_cast<char *>(dst_k);
  g.v_dst = static_cast<char *>(dst_v);
  return device_status(hylra::launch_gather(g, s->batch, stream), "gather launch");
}

// A staging-pool view for the attention kernel: the block table is not read.
hylra_kv staged_kv(const hylra_shape *s, const void *k_pool, const void *v_pool, int k,
                   const int32_t *ctx_lens) {
  hylra_kv v{};
  v.k_pool = k_pool;
  v.v_pool = v_pool;
  v.num_pages = (int64_t)s->batch * k;
  v.block_table = nullptr;
  v.ctx_lens = ctx_lens;
  return v;
}

// The gather reads the source pools through the addresses the caller passes:
// both pools must be device memory or pinned host memory mapped at the same
// address over their whole extent (num_pages pages).
hylra_status check_gather_source(const hylra_shape *s, const hylra_kv *kv) {
  const size_t bytes = (size_t)kv->num_pages * s->num_kv_heads * hylra::kBlockTokens *
                       s->head_dim * elt_bytes(s);
  for (const void *p : {kv->k_pool, kv->v_pool}) {
    int readable = 0;
    if (hylra_status st = device_status(hylra::pool_readable(p, bytes, &readable), "pointer query"))
      return st;
    if (!readable)
      return fail(HYLRA_E_INVALID_ARG,
                  "K/V pools must be device memory or pinned host memory "
                  "(hipHostMalloc) the device maps at the same address, over %zu bytes", bytes);
  }
  return HYLRA_OK;
}

hylra_status check_staging(const void *k_pool, const void *v_pool) {
  if (k_pool == nullptr || v_pool == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "staging pools must be non-NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return fail(HYLRA_E_INVALID_ARG, "staging pools must be 16-byte aligned");
  return HYLRA_OK;
}

}  // namespace

namespace hylra {

int report_error(int status, const char *message) {
  return fail(status, "%s", message);
}

// Split plans: whole waves of 256 workgroups (one 8-wavefront workgroup
// resident per compute unit on a 256-CU part) -- the fewest waves whose
// chunks per workgroup fit kMaxWgChunks -- with the same number of splits
// for every (sequence, KV head) row, so rows * nsplit never exceeds the
// waves' slots: a partly filled extra wave would run its few workgroups on a
// few compute units after the others have finished.  Full mode: a multiple
// of 8 chunks per workgroup (one per wavefront, and whole 128-token blocks,
// so a block's mass never straddles two workgroups), at most kMaxSplits
// workgroups per row.  Sparse mode: a multiple of 4 chunks, so a small
// selection spreads over more compute units with one busy wavefront per
// SIMD (two wavefronts on one SIMD share its vector issue), but at most as
// many splits as the merge reads with one batch of 8 partial loads per
// thread (8 * 512 / (G * d / 4)).
static_assert(kWavesPerGroup % kChunksPerBlock == 0, "a workgroup unit must hold whole blocks");
constexpr long kTargetWorkgroups = 256;

static SplitPlan make_plan(long chunks_per_seq, long rows, long unit, long max_splits) {
  const long min_cpw = (chunks_per_seq + max_splits - 1) / max_splits;
  long cpw = 0;
  for (long waves = 1;; ++waves) {
    long splits = waves * kTargetWorkgroups / rows;
    if (splits < 1) splits = 1;
    if (splits > max_splits) splits = max_splits;
    cpw = (chunks_per_seq + splits - 1) / splits;
    if (cpw < min_cpw) cpw = min_cpw;
    cpw = (cpw + unit - 1) / unit * unit;
    if (cpw <= kMaxWgChunks || splits == max_splits) break;
  }
  // a sparse merge bound below kMaxSplits can leave more chunks per split
  // than kMaxWgChunks: then the splits grow past it (nsplit <= 4 * 8192 / 256)
  if (cpw > kMaxWgChunks) cpw = kMaxWgChunks;
  SplitPlan p;
  p.chunks_per_wg = (int)cpw;
  p.nsplit = (int)((chunks_per_seq + cpw - 1) / cpw);
  return p;
}

SplitPlan plan_full(int batch, int num_kv_heads, int max_blocks) {
  return make_plan((long)kChunksPerBlock * max_blocks, (long)batch * num_kv_heads,
                   (long)kWavesPerGroup, (long)kMaxSplits);
}

SplitPlan plan_sparse(int batch, int num_kv_heads, int max_blocks, int k, int group,
                      int head_dim) {
  (void)max_blocks;  // every one of the k selection slots is walked
  const long items = (long)group * head_dim / 4;  // merge threads per split
  long max_splits = 8 * (items < 512 ? 512 / items : 1);
  if (max_splits > kMaxSplits) max_splits = kMaxSplits;
  return make_plan((long)kChunksPerBlock * (k > 0 ? k : 1), (long)batch * num_kv_heads,
                   (long)kChunksPerBlock, max_splits);
}

}  // namespace hylra

extern "C" {

hylra_status hylra_workspace_size(const hylra_shape *shape, int32_t k, size_t *bytes) {
  if (hylra_status st = check_shape(shape)) return st;
  if (bytes == nullptr) return fail(HYLRA_E_INVALID_ARG, "bytes is NULL");
  *bytes = layout(shape, k, nullptr).bytes;
  return ok();
}

hylra_status hylra_decode_full(const hylra_shape *shape, const void *q, const hylra_kv *kv,
                               float *out, float *lse, float *block_score, void *workspace,
                               size_t workspace_bytes, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (hylra_status st = check_kv(kv)) return st;
  if (q == nullptr || out == nullptr) return fail(HYLRA_E_INVALID_ARG, "q and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(HYLRA_E_INVALID_ARG, "q and out must be 16-byte aligned");
  Workspace w;
  if (hylra_status st = check_ws(shape, 0, workspace, workspace_bytes, w)) return st;
  if (hylra_status st = run_full(shape, q, kv, out, lse, block_score, nullptr, 0, w, hip_stream))
    return st;
  return ok();
}

hylra_status hylra_block_topk(const hylra_shape *shape, const float *block_score,
                              const int32_t *ctx_lens, int32_t k, int32_t *idx, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (block_score == nullptr || ctx_lens == nullptr || idx == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "block_score, ctx_lens and idx must be non-NULL");
  if (k < 1) return fail(HYLRA_E_INVALID_ARG, "k must be >= 1 (got %d)", k);
  hylra::TopkArgs t{};
  t.score = block_score;
  t.ctx = ctx_lens;
  t.max_blocks = shape->max_blocks_per_seq;
  t.num_kv_heads = shape->num_kv_heads;
  t.idx = idx;
  t.k = k;
  if (hylra_status st = device_status(hylra::launch_topk(t, shape->batch, hip_stream), "top-k launch"))
    return st;
  return ok();
}

hylra_status hylra_decode_sparse(const hylra_shape *shape, const void *q, const hylra_kv *kv,
                                 const int32_t *idx, int32_t k, float *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (hylra_status st = check_kv(kv)) return st;
  if (q == nullptr || out == nullptr || idx == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "q, idx and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(HYLRA_E_INVALID_ARG, "q and out must be 16-byte aligned");
  if (hylra_status st = check_k(k)) return st;
  Workspace w;
  if (hylra_status st = check_ws(shape, k, workspace, workspace_bytes, w)) return st;
  if (hylra_status st = run_sparse(shape, q, kv, idx, k, out, lse, nullptr, w, hip_stream))
    return st;
  return ok();
}

hylra_status hylra_run_policy(const hylra_shape *shape, int32_t num_layers, const int32_t *src,
                              int32_t k, const void *const *q, const hylra_kv *kv,
                              float *const *out, float *const *lse, int32_t *idx_log,
                              void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (num_layers < 1) return fail(HYLRA_E_INVALID_ARG, "num_layers must be >= 1");
  if (src == nullptr || q == nullptr || kv == nullptr || out == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "src, q, kv and out must be non-NULL");
  if (hylra_status st = check_k(k)) return st;
  if (src[0] != 0) return fail(HYLRA_E_BAD_POLICY, "layer 0 must reset (src[0] = %d)", src[0]);
  for (int j = 1; j < num_layers; ++j)
    if (src[j] != j && src[j] != src[j - 1])
      return fail(HYLRA_E_BAD_POLICY, "src[%d] = %d is neither %d nor src[%d] = %d", j, src[j], j,
                  j - 1, src[j - 1]);
  for (int j = 0; j < num_layers; ++j) {
    if (hylra_status st = check_kv(&kv[j])) return fail(st, "layer %d: %s", j, hylra_last_error());
    if (q[j] == nullptr || out[j] == nullptr || !aligned16(q[j]) || !aligned16(out[j]))
      return fail(HYLRA_E_INVALID_ARG, "layer %d: q and out must be non-NULL and 16-byte aligned", j);
  }
  Workspace w;
  if (hylra_status st = check_ws(shape, k, workspace, workspace_bytes, w)) return st;
  const size_t row = (size_t)shape->batch * shape->num_kv_heads * k;
  for (int j = 0; j < num_layers; ++j) {
    float *lj = lse ? lse[j] : nullptr;
    hylra_status st;
    if (src[j] == j) {
      // the index set of a reset layer is needed only if the next layer
      // reuses it, or the caller logs it
      const bool used = idx_log != nullptr || (j + 1 < num_layers && src[j + 1] == j);
      int32_t *dst = used ? (idx_log ? idx_log + (size_t)j * row : w.idx) : nullptr;
      st = run_full(shape, q[j], &kv[j], out[j], lj, nullptr, dst, k, w, hip_stream);
    } else {
      const int32_t *carried = idx_log ? idx_log + (size_t)src[j] * row : w.idx;
      int32_t *log = idx_log ? idx_log + (size_t)j * row : nullptr;
      st = run_sparse(shape, q[j], &kv[j], carried, k, out[j], lj, log, w, hip_stream);
    }
    if (st) return fail(st, "layer %d: %s", j, hylra_last_error());
  }
  return ok();
}

hylra_status hylra_gather_blocks(const hylra_shape *shape, const hylra_kv *kv, const int32_t *idx,
                                 int32_t k, void *staged_k, void *staged_v, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (hylra_status st = check_kv(kv)) return st;
  if (idx == nullptr) return fail(HYLRA_E_INVALID_ARG, "idx must be non-NULL");
  if (hylra_status st = check_k(k)) return st;
  if ((long)shape->batch * k > (1L << 30))
    return fail(HYLRA_E_UNSUPPORTED, "batch * k = %ld exceeds 2^30 staging pages", (long)shape->batch * k);
  if (hylra_status st = check_staging(staged_k, staged_v)) return st;
  if (hylra_status st = check_gather_source(shape, kv)) return st;
  if (hylra_status st = run_gather(shape, kv, idx, k, staged_k, staged_v, hip_stream)) return st;
  return ok();
}

hylra_status hylra_append_kv(const hylra_shape *shape, const hylra_kv *kv, const void *k_new,
                             const void *v_new, const int32_t *pos, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (hylra_status st = check_kv(kv)) return st;
  if (k_new == nullptr || v_new == nullptr || pos == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "k_new, v_new and pos must be non-NULL");
  if (hylra_status st = check_gather_source(shape, kv)) return st;
  hylra::AppendArgs a{};
  a.k_pool = const_cast<void *>(kv->k_pool);
  a.v_pool = const_cast<void *>(kv->v_pool);
  a.num_pages = kv->num_pages;
  a.table = kv->block_table;
  a.pos = pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.max_blocks = shape->max_blocks_per_seq;
  a.num_kv_heads = shape->num_kv_heads;
  a.head_dim = shape->head_dim;
  a.elt = (int)elt_bytes(shape);
  if (hylra_status st = device_status(hylra::launch_append(a, shape->batch, hip_stream), "append launch"))
    return st;
  return ok();
}

hylra_status hylra_rope_append(const hylra_shape *shape, const hylra_kv *kv, const void *qkv,
                               const float *cos_tab, const float *sin_tab, const int32_t *pos,
                               void *q_out, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (shape->dtype != HYLRA_BF16)
    return fail(HYLRA_E_UNSUPPORTED, "rope_append takes bf16 activations and pools");
  if (hylra_status st = check_kv(kv)) return st;
  if (qkv == nullptr || cos_tab == nullptr || sin_tab == nullptr || pos == nullptr || q_out == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "qkv, cos_tab, sin_tab, pos and q_out must be non-NULL");
  if (hylra_status st = check_gather_source(shape, kv)) return st;
  hylra::RopeAppendArgs a{};
  a.qkv = qkv;
  a.cos_tab = cos_tab;
  a.sin_tab = sin_tab;
  a.pos = pos;
  a.table = kv->block_table;
  a.q_out = q_out;
  a.k_pool = const_cast<void *>(kv->k_pool);
  a.v_pool = const_cast<void *>(kv->v_pool);
  a.num_pages = kv->num_pages;
  a.max_blocks = shape->max_blocks_per_seq;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.head_dim = shape->head_dim;
  if (hylra_status st = device_status(hylra::launch_rope_append(a, shape->batch, hip_stream),
                                      "rope_append launch"))
    return st;
  return ok();
}

hylra_status hylra_silu_mul(const void *gate_up, void *out, int64_t rows, int32_t width,
                            void *hip_stream) {
  if (gate_up == nullptr || out == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "gate_up and out must be non-NULL");
  if (rows < 1 || width < 1) return fail(HYLRA_E_INVALID_ARG, "rows and width must be >= 1");
  if (hylra_status st = device_status(hylra::launch_silu_mul(gate_up, out, rows, width, hip_stream),
                                      "silu_mul launch"))
    return st;
  return ok();
}

hylra_status hylra_decode_staged(const hylra_shape *shape, const void *q, const void *staged_k,
                                 const void *staged_v, const int32_t *ctx_lens, const int32_t *idx,
                                 int32_t k, float *out, float *lse, void *workspace,
                                 size_t workspace_bytes, void *hip_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (hylra_status st = check_staging(staged_k, staged_v)) return st;
  if (q == nullptr || out == nullptr || idx == nullptr || ctx_lens == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "q, ctx_lens, idx and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(HYLRA_E_INVALID_ARG, "q and out must be 16-byte aligned");
  if (hylra_status st = check_k(k)) return st;
  if ((long)shape->batch * k > (1L << 30))
    return fail(HYLRA_E_UNSUPPORTED, "batch * k = %ld exceeds 2^30 staging pages", (long)shape->batch * k);
  Workspace w;
  if (hylra_status st = check_ws(shape, k, workspace, workspace_bytes, w)) return st;
  const hylra_kv kv = staged_kv(shape, staged_k, staged_v, k, ctx_lens);
  if (hylra_status st = run_sparse(shape, q, &kv, idx, k, out, lse, nullptr, w, hip_stream, true))
    return st;
  return ok();
}

hylra_status hylra_run_policy_offload(const hylra_shape *shape, int32_t num_layers,
                                      const int32_t *src, int32_t k, const void *const *q,
                                      const hylra_kv *kv, const uint8_t *offloaded,
                                      void *const *staged_k, void *const *staged_v,
                                      float *const *out, float *const *lse, int32_t *idx_log,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *copy_stream) {
  if (hylra_status st = check_shape(shape)) return st;
  if (num_layers < 1) return fail(HYLRA_E_INVALID_ARG, "num_layers must be >= 1");
  if (src == nullptr || q == nullptr || kv == nullptr || out == nullptr || offloaded == nullptr)
    return fail(HYLRA_E_INVALID_ARG, "src, q, kv, offloaded and out must be non-NULL");
  if (hylra_status st = check_k(k)) return st;
  if ((long)shape->batch * k > (1L << 30))
    return fail(HYLRA_E_UNSUPPORTED, "batch * k = %ld exceeds 2^30 staging pages", (long)shape->batch * k);
  if (src[0] != 0) return fail(HYLRA_E_BAD_POLICY, "layer 0 must reset (src[0] = %d)", src[0]);
  for (int j = 1; j < num_layers; ++j)
    if (src[j] != j && src[j] != src[j - 1])
      return fail(HYLRA_E_BAD_POLICY, "src[%d] = %d is neither %d nor src[%d] = %d", j, src[j], j,
                  j - 1, src[j - 1]);
  bool any = false;
  for (int j = 0; j < num_layers; ++j) any = any || offloaded[j];
  if (any && copy_stream == hip_stream)
    return fail(HYLRA_E_INVALID_ARG, "copy_stream must differ from hip_stream");
  for (int j = 0; j < num_layers; ++j) {
    if (hylra_status st = check_kv(&kv[j])) return fail(st, "layer %d: %s", j, hylra_last_error());
    if (q[j] == nullptr || out[j] == nullptr || !aligned16(q[j]) || !aligned16(out[j]))
      return fail(HYLRA_E_INVALID_ARG, "layer %d: q and out must be non-NULL and 16-byte aligned", j);
    if (offloaded[j]) {
      if (src[j] == j)
        return fail(HYLRA_E_BAD_POLICY,
                    "layer %d resets and needs its whole KV cache on the device; only reuse "
                    "layers may be offloaded", j);
      if (staged_k == nullptr || staged_v == nullptr)
        return fail(HYLRA_E_INVALID_ARG, "staged_k and staged_v must be non-NULL");
      if (hylra_status st = check_staging(staged_k[j], staged_v[j]))
        return fail(st, "layer %d: %s", j, hylra_last_error());
      if (hylra_status st = check_gather_source(shape, &kv[j]))
        return fail(st, "layer %d: %s", j, hylra_last_error());
    }
  }
  Workspace w;
  if (hylra_status st = check_ws(shape, k, workspace, workspace_bytes, w)) return st;
  const size_t row = (size_t)shape->batch * shape->num_kv_heads * k;
  // event slots: slot j marks the end of layer j's gather on the copy
  // stream; slot num_layers marks the index set of the latest reset
  const int fork_slot = num_layers;
  for (int j = 0; j < num_layers; ++j) {
    float *lj = lse ? lse[j] : nullptr;
    hylra_status st;
    if (src[j] == j) {
      bool gathers = false;
      for (int i = j + 1; i < num_layers && src[i] == j; ++i) gathers = gathers || offloaded[i];
      const bool used = idx_log != nullptr || (j + 1 < num_layers && src[j + 1] == j);
      int32_t *dst = used ? (idx_log ? idx_log + (size_t)j * row : w.idx) : nullptr;
      st = run_full(shape, q[j], &kv[j], out[j], lj, nullptr, dst, k, w, hip_stream);
      if (st) return fail(st, "layer %d: %s", j, hylra_last_error());
      if (gathers) {
        // fork: once the index set exists, the copy stream brings in every
        // offloaded reuse layer's blocks, in layer order, while the compute
        // stream runs the layers in between
        if (hylra_status e = device_status(hylra::event_record(hip_stream, fork_slot), "event record"))
          return e;
        if (hylra_status e = device_status(hylra::event_wait(copy_stream, fork_slot), "event wait"))
          return e;
        for (int i = j + 1; i < num_layers && src[i] == j; ++i) {
          if (!offloaded[i]) continue;
          st = run_gather(shape, &kv[i], dst, k, staged_k[i], staged_v[i], copy_stream);
          if (st) return fail(st, "layer %d gather: %s", i, hylra_last_error());
          if (hylra_status e = device_status(hylra::event_record(copy_stream, i), "event record"))
            return e;
        }
      }
    } else {
      const int32_t *carried = idx_log ? idx_log + (size_t)src[j] * row : w.idx;
      int32_t *log = idx_log ? idx_log + (size_t)j * row : nullptr;
      if (offloaded[j]) {
        // join: this layer's staged blocks are complete.  The next reset,
        // which overwrites the carried set, runs after every reuse layer of
        // this source, so after all of the gathers that read the set.
        if (hylra_status e = device_status(hylra::event_wait(hip_stream, j), "event wait")) return e;
        const hylra_kv skv = staged_kv(shape, staged_k[j], staged_v[j], k, kv[j].ctx_lens);
        st = run_sparse(shape, q[j], &skv, carried, k, out[j], lj, log, w, hip_stream, true);
      } else {
        st = run_sparse(shape, q[j], &kv[j], carried, k, out[j], lj, log, w, hip_stream);
      }
    }
    if (st) return fail(st, "layer %d: %s", j, hylra_last_error());
  }
  return ok();
}

hylra_status hylra_policy_dp(int32_t num_layers, const float *M, float theta,
                             const uint8_t *force_reset, int32_t *src_out, int32_t *num_resets,
                             double *sim_sum) {
  const int L = num_layers;
  if (L < 1 || L > 1024) return fail(HYLRA_E_INVALID_ARG, "num_layers must be in [1, 1024] (got %d)", L);
  if (M == nullptr || src_out == nullptr) return fail(HYLRA_E_INVALID_ARG, "M and src_out must be non-NULL");
  if (isnan(theta)) return fail(HYLRA_E_INVALID_ARG, "theta is NaN");
  for (int j = 0; j < L; ++j)
    for (int i = 0; i < j; ++i)
      if (isnan(M[(size_t)j * L + i])) return fail(HYLRA_E_INVALID_ARG, "M[%d][%d] is NaN", j, i);

  auto reusable = [&](int i, int j) {  // layer j may reuse the indices of reset layer i
    return !(force_reset && force_reset[j]) && (double)M[(size_t)j * L + i] > (double)theta;
  };
  // best (resets, similarity) of layers j+1 .. L-1 from state (i, j), i <= j
  std::vector<int> br((size_t)L * L, 0);
  std::vector<double> bs((size_t)L * L, 0.0);
  auto at = [L](int i, int j) { return (size_t)i * L + j; };
  for (int j = L - 2; j >= 0; --j) {
    for (int i = 0; i <= j; ++i) {
      int r = br[at(j + 1, j + 1)] + 1;
      double s = bs[at(j + 1, j + 1)];
      if (reusable(i, j + 1)) {
        const int r2 = br[at(i, j + 1)];
        const double s2 = bs[at(i, j + 1)] + (double)M[(size_t)(j + 1) * L + i];
        if (r2 < r || (r2 == r && s2 > s)) {
          r = r2;
          s = s2;
        }
      }
      br[at(i, j)] = r;
      bs[at(i, j)] = s;
    }
  }
  const int r_opt = 1 + br[at(0, 0)];
  const double s_opt = bs[at(0, 0)];
  // forward pass: reuse whenever a reuse continuation is still optimal
  int i = 0, acc_r = 1;
  double acc_s = 0.0;
  src_out[0] = 0;
  for (int j = 0; j + 1 < L; ++j) {
    bool reuse = false;
    if (reusable(i, j + 1)) {
      const double gain = (double)M[(size_t)(j + 1) * L + i];
      reuse = acc_r + br[at(i, j + 1)] == r_opt && acc_s + gain + bs[at(i, j + 1)] >= s_opt - 1e-12;
      if (reuse) acc_s += gain;
    }
    if (!reuse) {
      ++acc_r;
      i = j + 1;
    }
    src_out[j + 1] = i;
  }
  if (num_resets) *num_resets = acc_r;
  if (sim_sum) *sim_sum = acc_s;
  return ok();
}

hylra_status hylra_timer_start(int32_t kind, int32_t capacity) {
  if (kind < 0 || kind >= hylra::kNumTimers) return fail(HYLRA_E_INVALID_ARG, "unknown timer kind %d", kind);
  if (capacity < 1 || capacity > (1 << 20))
    return fail(HYLRA_E_INVALID_ARG, "timer capacity must be in [1, 2^20] (got %d)", capacity);
  if (hylra_status st = device_status(hylra::timer_start(kind, capacity), "timer start")) return st;
  return ok();
}

hylra_status hylra_overlap_matrix(int32_t steps, int32_t num_layers, int32_t slices, int32_t k,
                                  const int32_t *idx_log, float *M, void *hip_stream) {
  if (idx_log == nullptr || M == nullptr) return fail(HYLRA_E_INVALID_ARG, "overlap: null pointer");
  if (steps < 1 || slices < 1 || k < 1 || num_layers < 1 || num_layers > 1024)
    return fail(HYLRA_E_INVALID_ARG,
                "overlap: need steps >= 1, 1 <= layers <= 1024, slices >= 1, k >= 1 "
                "(got %d, %d, %d, %d)", steps, num_layers, slices, k);
  if (hylra::overlap_smem_bytes(num_layers, k) > 65536)
    return fail(HYLRA_E_UNSUPPORTED, "overlap: layers * k = %lld exceeds 16000",
                (long long)num_layers * k);
  if ((reinterpret_cast<uintptr_t>(idx_log) & 3u) || (reinterpret_cast<uintptr_t>(M) & 3u))
    return fail(HYLRA_E_INVALID_ARG, "overlap: pointers must be 4-byte aligned");
  hylra::OverlapArgs a{idx_log, steps, num_layers, slices, k, M};
  return device_status(hylra::launch_overlap(a, hip_stream), "overlap launch");
}

hylra_status hylra_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *hip_stream) {
  if (buf == nullptr || sink == nullptr) return fail(HYLRA_E_INVALID_ARG, "read probe: null pointer");
  if (!aligned16(buf)) return fail(HYLRA_E_INVALID_ARG, "read probe: buffer must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
    return fail(HYLRA_E_INVALID_ARG, "read probe: bytes must be a positive multiple of 16 (got %zu)",
                bytes);
  return device_status(hylra::launch_read_probe(buf, bytes, sink, hip_stream), "read probe launch");
}

hylra_status hylra_timer_stop(int32_t kind, double *total_ms, int32_t *launches) {
  if (kind < 0 || kind >= hylra::kNumTimers) return fail(HYLRA_E_INVALID_ARG, "unknown timer kind %d", kind);
  int n = 0;
  if (hylra_status st = device_status(hylra::timer_stop(kind, total_ms, &n), "timer stop")) return st;
  if (launches) *launches = n;
  return ok();
}

const char *hylra_status_str(hylra_status status) {
  switch (status) {
    case HYLRA_OK: return "ok";
    case HYLRA_E_INVALID_ARG: return "invalid argument";
    case HYLRA_E_UNSUPPORTED: return "unsupported";
    case HYLRA_E_BAD_POLICY: return "malformed policy";
    case HYLRA_E_WORKSPACE: return "workspace too small";
    case HYLRA_E_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char *hylra_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
