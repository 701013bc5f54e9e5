/*
 * hylra.h -- C ABI of the MI355X (gfx950) HyLRA decode-phase hybrid attention.
 *
 * Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
 * Inference" (technical summary).  Sensitive ("reset") layers run standard
 * full attention and extract the top-k indices, which are passed forward
 * (section 2.3, Sensitive Layers); tolerant ("reuse") layers attend only to
 * the KV subset named by the carried indices (section 2.3, Tolerant Layers);
 * selection works on fixed 128-token blocks (section 2.4, Block-level
 * Sparsity); the per-layer reset/reuse policy comes from an offline dynamic
 * program over a lower-triangular similarity matrix M with a fidelity
 * threshold theta (section 2.2).
 *
 * Conventions shared by every entry point
 *   - All device pointers are HIP device memory owned by the caller (the
 *     offloading entry points below also read K/V pools in pinned host
 *     memory).  The
 *     library never allocates, frees, copies device-to-host or synchronises;
 *     device work is enqueued on `hip_stream` (a hipStream_t, NULL = the
 *     default stream) and is asynchronous.
 *   - Element type of q / K / V: HYLRA_F32 (IEEE float32) or HYLRA_BF16
 *     (bfloat16).  Outputs and scores are float32.
 *   - Layouts (row-major, innermost last):
 *       q            [B][Hq][d]
 *       K pool       [num_pages][Hkv][128][d]   token-major page tile
 *       V pool       [num_pages][Hkv][4][d][32] a page as four 32-token
 *                                               sub-tiles, each dimension-major
 *       block_table  [B][max_blocks_per_seq] int32, logical block -> page
 *       ctx_lens     [B] int32, tokens of each sequence (device memory)
 *       out          [B][Hq][d] float32, lse [B][Hq] float32 (natural log)
 *       block_score  [B][Hkv][max_blocks_per_seq] float32
 *       idx          [B][Hkv][k] int32 selection rows.  Rows the library
 *                    writes (top-k) hold ascending block ids, -1 padded.
 *                    Rows it reads (sparse, staged, gather) may hold the
 *                    ids in any order with padding anywhere: every slot
 *                    is read, and a slot outside [0, ceil(T_b/128)) names
 *                    no block.  The ids of a row must be distinct: a
 *                    repeated id is attended once per repeat.
 *     Query head h uses KV head h / (Hq / Hkv).  Pointers must be 16-byte
 *     aligned.  Every page named by the table holds 128 tokens of storage.
 *   - ctx_lens values are clamped to [0, 128 * max_blocks_per_seq].  A
 *     sequence with no tokens gets out = 0, lse = -inf, idx = -1.
 *   - A block-table entry outside [0, num_pages) makes that block empty
 *     (never read); a selected block id outside [0, ceil(T/128)) is skipped.
 *   - Return values: HYLRA_OK or an error code; argument checks run on the
 *     host before anything is enqueued, and a failed check enqueues nothing.
 *     hylra_last_error() gives a thread-local message for the last failure.
 */
#ifndef HYLRA_H
#define HYLRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hylra_status;
#define HYLRA_OK 0
#define HYLRA_E_INVALID_ARG 1 /* null pointer, bad size, inconsistent shape */
#define HYLRA_E_UNSUPPORTED 2 /* valid but not implemented (head_dim, group size, ...) */
#define HYLRA_E_BAD_POLICY 3  /* malformed per-layer source list */
#define HYLRA_E_WORKSPACE 4   /* workspace missing or smaller than required */
#define HYLRA_E_DEVICE 5      /* HIP launch / runtime error (message in hylra_last_error) */

#define HYLRA_F32 0
#define HYLRA_BF16 1
#define HYLRA_BLOCK_TOKENS 128

typedef struct {
  int32_t batch;              /* B >= 1; B * num_kv_heads <= 65536 */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* must be 128 (section 2.4 block granularity) */
  int32_t dtype;              /* HYLRA_F32 or HYLRA_BF16 */
  int32_t max_blocks_per_seq; /* block_table row stride, 1 .. 8192 */
  float scale;                /* logit scale; 0 selects 1/sqrt(head_dim) */
} hylra_shape;

typedef struct {
  const void *k_pool;         /* [num_pages][Hkv][128][d] */
  const void *v_pool;         /* [num_pages][Hkv][4][d][32] */
  int64_t num_pages;          /* >= 1 */
  const int32_t *block_table; /* [B][max_blocks_per_seq] */
  const int32_t *ctx_lens;    /* [B] */
} hylra_kv;

/* Bytes of device workspace that every entry point below needs for `shape`
 * and top-k `k` (k <= 0 allowed when no sparse/top-k call is made).  The
 * caller allocates it once, zero-fills it before its first use, and may reuse
 * it across calls on one stream: it holds per-(sequence, KV head) arrival
 * counters that every launch leaves at zero when it completes.  Calls that
 * share one workspace must not overlap (use one workspace per stream). */
hylra_status hylra_workspace_size(const hylra_shape *shape, int32_t k, size_t *bytes);

/* Full decode attention of one layer (section 2.3, sensitive layers):
 *   s_t = scale * q_h . K_t, p = softmax over all t < T_b,
 *   out_h = sum_t p_t V_t, lse_h = ln sum_t exp(s_t),
 * and, when block_score is non-NULL, the block score of every 128-token
 * block n < ceil(T_b/128) of KV head g:
 *   score[b][g][n] = sum over query heads h of group g of sum_{t in n} p_t,
 * entries n >= ceil(T_b/128) set to 0.  lse may be NULL. */
hylra_status hylra_decode_full(const hylra_shape *shape, const void *q, const hylra_kv *kv,
                               float *out, float *lse, float *block_score, void *workspace,
                               size_t workspace_bytes, void *hip_stream);

/* Top-k blocks of a score array (section 2.3: the top-k indices extracted at
 * sensitive layers).  Per (b, g): the k_eff = min(k, ceil(T_b/128)) blocks
 * with the largest score, ties going to the lower block id, written in
 * ascending id order to idx[b][g][0..k_eff) and -1 after.  Scores must be
 * finite and >= 0.  k >= 1. */
hylra_status hylra_block_topk(const hylra_shape *shape, const float *block_score,
                              const int32_t *ctx_lens, int32_t k, int32_t *idx,
                              void *hip_stream);

/* Decode attention restricted to the selected blocks (section 2.3, tolerant
 * layers): U = tokens t < T_b whose block id is one of idx[b][g][0..k), in
 * any slot (entries outside [0, ceil(T_b/128)), negative ones included, are
 * padding); softmax and output over U only.  The ids of a row must be
 * distinct (see the idx layout above).  An empty U gives out = 0 and
 * lse = -inf.  lse may be NULL.  1 <= k <= 8192 (HYLRA_E_UNSUPPORTED above). */
hylra_status hylra_decode_sparse(const hylra_shape *shape, const void *q, const hylra_kv *kv,
                                 const int32_t *idx, int32_t k, float *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *hip_stream);

/* One decode step of the hybrid policy over num_layers layers (section 2.3):
 * layer j with src[j] == j resets (full attention, block scores, top-k, the
 * result becomes the carried index set); a layer with src[j] == src[j-1]
 * reuses the carried set (sparse attention).  src is a host array and must
 * satisfy src[0] == 0 and src[j] in {j, src[j-1]} (HYLRA_E_BAD_POLICY
 * otherwise).  q, kv, out and lse are host arrays of num_layers entries (lse
 * may be NULL, or hold NULL entries).  idx_log (device, nullable)
 * [num_layers][B][Hkv][k] receives the index set each layer computed or
 * reused.  With idx_log NULL, a reset layer whose indices the next layer does
 * not reuse skips the block scores and top-k (nothing would read them).
 * Everything is enqueued on one stream with no host synchronisation.
 * 1 <= k <= 8192 (HYLRA_E_UNSUPPORTED above). */
hylra_status hylra_run_policy(const hylra_shape *shape, int32_t num_layers, const int32_t *src,
                              int32_t k, const void *const *q, const hylra_kv *kv,
                              float *const *out, float *const *lse, int32_t *idx_log,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/* hylra_run_policy for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, with the workspace taken from a static device
 * array of HYLRA_NOALLOC_SCRATCH_BYTES inside the library instead of a
 * caller buffer.  The caller still passes inputs and outputs.  Each device
 * holds its own array from its first call until the process ends; the first
 * call on a device looks the array up and clears its counters on hip_stream.
 * The entry point allocates and frees nothing.  A shape whose
 * hylra_workspace_size exceeds the array returns HYLRA_E_WORKSPACE (nothing
 * enqueued).  Every call on one device shares that device's array, so calls
 * that overlap on one device (several streams or host threads) race; run
 * them in order on one stream. */
#define HYLRA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
hylra_status hylra_run_policy_noalloc(const hylra_shape *shape, int32_t num_layers,
                                      const int32_t *src, int32_t k, const void *const *q,
                                      const hylra_kv *kv, float *const *out, float *const *lse,
                                      int32_t *idx_log, void *hip_stream);

/* Index-guided offloading (section 2.4, hardware-efficient optimisations):
 * the indices a reuse layer carries name, before it runs, the only blocks it
 * reads, so its KV cache can stay in host memory and just those blocks cross
 * the host link.
 *
 * hylra_gather_blocks: for every (b, g, r) with n = idx[b][g][r] in
 * [0, ceil(T_b/128)) and page = block_table[b][n] in [0, num_pages), copies
 * the K slab [128][d] and the V slab [4][d][32] of (page, KV head g) from
 * kv's pools into staging page b*k + r: staged_k [B*k][Hkv][128][d] and
 * staged_v [B*k][Hkv][4][d][32], same element type.  Other staging slots
 * are left as they are.  kv's pools may be pinned host memory that the device
 * maps at the same address (hipHostMalloc) or device memory, over their whole
 * extent (num_pages pages); anything else, pageable host memory included, is
 * HYLRA_E_INVALID_ARG.  block_table, ctx_lens, idx and the staging pools are
 * device memory.  Every slot r < k of a row is read (idx layout above).
 * 1 <= k <= 8192, B*k <= 2^30. */
hylra_status hylra_gather_blocks(const hylra_shape *shape, const hylra_kv *kv, const int32_t *idx,
                                 int32_t k, void *staged_k, void *staged_v, void *hip_stream);

/* Decode-step bookkeeping for a cache that may live in host memory: writes
 * the new token's k_new and v_new ([B][Hkv][d] device arrays, the pools'
 * element type) at position pos[b] (device [B]) of each sequence -- K row
 * [page][g][slot][:] and V column [page][g][slot/32][:][slot%32] with page =
 * block_table[b][pos/128], slot = pos % 128.  A position outside
 * [0, 128*max_blocks_per_seq) or a page outside [0, num_pages) writes
 * nothing.  kv's pools may be device memory or pinned host memory mapped at
 * the same address (HYLRA_E_INVALID_ARG otherwise); ctx_lens is not read. */
hylra_status hylra_append_kv(const hylra_shape *shape, const hylra_kv *kv, const void *k_new,
                             const void *v_new, const int32_t *pos, void *hip_stream);

/* Decode-step helpers around the attention (the end-to-end step puts the
 * GPU BLAS projections and MLP around this library; these replace chains of
 * elementwise launches).  bf16 only.
 *
 * hylra_rope_append: qkv [B][(Hq + 2 Hkv) d] holds each sequence's new q,
 * k and v heads in that order.  The q and k heads get the rotary embedding
 * in the rotate-half form: for i < d/2, (x_i, x_{i+d/2}) becomes
 * (x_i c - x_{i+d/2} s, x_{i+d/2} c + x_i s) with c = cos_tab[b][i],
 * s = sin_tab[b][i] (float32 [B][d/2], the cosine and sine of the angle of
 * position pos[b] for pair i), computed in float32 and rounded to bf16.
 * Rotated q goes to q_out [B][Hq][d]; rotated k and the v heads are written
 * at position pos[b] of kv's pages as hylra_append_kv does (same bounds
 * rule; pools on the device or pinned in host memory).  hylra_silu_mul:
 * out[r][c] = silu(g) * u with g = gate_up[r][c], u = gate_up[r][width + c]
 * (gate_up [rows][2 width], out [rows][width], bf16, computed in float32). */
hylra_status hylra_rope_append(const hylra_shape *shape, const hylra_kv *kv, const void *qkv,
                               const float *cos_tab, const float *sin_tab, const int32_t *pos,
                               void *q_out, void *hip_stream);
hylra_status hylra_silu_mul(const void *gate_up, void *out, int64_t rows, int32_t width,
                            void *hip_stream);

/* Attention over staged blocks: the result of hylra_decode_sparse on the
 * layer's own pools with the same idx (bit for bit: the same kernel reads the
 * same values in the same order), reading selection slot r of sequence b
 * from staging page b*k + r as hylra_gather_blocks fills it.  ctx_lens [B]
 * is the layer's context lengths; no block table is read.  1 <= k <= 8192. */
hylra_status hylra_decode_staged(const hylra_shape *shape, const void *q, const void *staged_k,
                                 const void *staged_v, const int32_t *ctx_lens, const int32_t *idx,
                                 int32_t k, float *out, float *lse, void *workspace,
                                 size_t workspace_bytes, void *hip_stream);

/* hylra_run_policy with offloaded reuse layers.  offloaded (host [L]):
 * nonzero marks a reuse layer whose kv[j] pools may be in host memory; its
 * staging pools are staged_k[j] / staged_v[j] (host arrays of device
 * pointers, read only for offloaded layers; each [B*k][Hkv][...] as above).
 * A reset layer reads its whole cache and must not be offloaded
 * (HYLRA_E_BAD_POLICY).  After each reset layer, copy_stream waits for it and
 * then gathers the blocks of that layer's offloaded reuse layers in layer
 * order, recording an event after each; the compute stream (hip_stream)
 * waits for a layer's event just before that layer's attention.  The gathers
 * thus overlap with the layers in between.  Outputs, lse and idx_log are
 * those of hylra_run_policy.  copy_stream must differ from hip_stream when a
 * layer is offloaded.  The events come from a per-device pool of the
 * library (slots 0..L), so calls on one device must not run concurrently
 * from several host threads; the sequence can be captured into a graph from
 * hip_stream (the copy stream forks from and joins back into it). */
hylra_status hylra_run_policy_offload(const hylra_shape *shape, int32_t num_layers,
                                      const int32_t *src, int32_t k, const void *const *q,
                                      const hylra_kv *kv, const uint8_t *offloaded,
                                      void *const *staged_k, void *const *staged_v,
                                      float *const *out, float *const *lse, int32_t *idx_log,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *copy_stream);

/* Offline policy dynamic program (section 2.2), host only, synchronous.
 * M: host [L][L] float32, row = target layer, column = source layer
 * (M[j*L + i] = similarity of reusing layer i's indices at layer j, i <= j;
 * the upper triangle and the diagonal are not read).  A reuse move of layer
 * j from source i is allowed when force_reset[j] == 0 and M[j][i] > theta.
 * Objective: fewest resets, then the largest summed similarity of the reuse
 * moves; among optima (equal resets, sums within 1e-12) the policy that
 * reuses at the earliest layer where they differ.  Layer 0 always resets.
 * Writes src_out[L]; num_resets and sim_sum may be NULL.  1 <= L <= 1024;
 * M entries and theta must not be NaN. */
hylra_status hylra_policy_dp(int32_t num_layers, const float *M, float theta,
                             const uint8_t *force_reset, int32_t *src_out, int32_t *num_resets,
                             double *sim_sum);

/* Kernel timer (instrumentation).  While the timer of a kernel kind runs,
 * every launch of that kind (the first `capacity` launches) carries a pair
 * of HIP events that the dispatch itself stamps at its start and end
 * (hipExtLaunchKernel), so the time is the kernel's own execution on the
 * launch stream.  Timers must not run while the stream is being captured
 * into a graph.  hylra_timer_stop waits
 * for the recorded events and returns the summed kernel time in milliseconds
 * and the number of timed launches (both pointers nullable).  Timers are
 * process-global and not thread-safe; starting a running timer restarts it. */
#define HYLRA_KERNEL_FULL_ATTN 0   /* full attention layer without block scores: split pass + merge */
#define HYLRA_KERNEL_SPARSE_ATTN 1 /* selected-block attention layer: split pass + merge */
#define HYLRA_KERNEL_TOPK 2        /* top-k of a given score array (hylra_block_topk) */
#define HYLRA_KERNEL_GATHER 3      /* selected-block gather (hylra_gather_blocks, offloading) */
#define HYLRA_KERNEL_FULL_ATTN_SCORED 4 /* full attention layer with block scores, and the
                                           top-k when the index set is used: split pass +
                                           merge, scores, top-k */
hylra_status hylra_timer_start(int32_t kind, int32_t capacity);
hylra_status hylra_timer_stop(int32_t kind, double *total_ms, int32_t *launches);

/* Offline similarity matrix for the policy program (section 2.2: M is built
 * from the overlap ratio of the layers' top-k indices on profiling data).
 * idx_log: device [steps][num_layers][slices][k] int32, each row a layer's
 * selected block ids in ascending order, -1 padded (for example the idx_log
 * of hylra_run_policy with every layer resetting, slices = B * Hkv, one
 * entry per profiling step).  M: device [num_layers][num_layers] float32,
 * row = target layer j, column = source layer i: for i <= j the mean over
 * the slices (step, sequence, KV head) whose target set is not empty of
 * |I_i n I_j| / |I_j|, summed in float64 in slice order; 0 if every target
 * set is empty, and 0 above the diagonal.  1 <= num_layers <= 1024,
 * num_layers * k <= 16000 (HYLRA_E_UNSUPPORTED beyond).  Asynchronous on
 * `hip_stream`; hylra_policy_dp takes M once copied to the host. */
hylra_status hylra_overlap_matrix(int32_t steps, int32_t num_layers, int32_t slices, int32_t k,
                                  const int32_t *idx_log, float *M, void *hip_stream);

/* Diagnostic: reads `bytes` (a positive multiple of 16) of device memory at
 * `buf` (16-byte aligned) once, with the loads and cache policy of the
 * attention kernels' K/V stream (16-byte non-temporal buffer loads, 512-thread
 * workgroups each reading a contiguous 2 MiB range), and folds the data into
 * a value stored to the device word `sink` only when it equals a constant the
 * callers never produce.  Timing it gives the practical HBM read ceiling
 * against which the attention kernels' bandwidth is set.  Asynchronous on
 * `hip_stream`. */
hylra_status hylra_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *hip_stream);

/* Static string for a status code. */
const char *hylra_status_str(hylra_status status);

/* Message of the last failure on the calling thread ("" if none). */
const char *hylra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HYLRA_H */
