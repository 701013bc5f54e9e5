// Internal interface between the C-ABI host code and the HIP kernels of
// libhylra.  Not installed; the public interface is include/hylra.h.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace hylra {

constexpr int kBlockTokens = 128;  // selection granularity (128-token blocks)
constexpr int kChunkTokens = 32;   // tokens one wavefront consumes per step
constexpr int kChunksPerBlock = kBlockTokens / kChunkTokens;
constexpr int kMaxGroup = 16;      // query heads per KV head handled by one tile
constexpr int kMaxBlocks = 8192;   // blocks per sequence (1M tokens)
constexpr int kMaxSplits = 256;    // workgroups per (sequence, KV head)
constexpr int kCounterSlots = 65536;  // (sequence, KV head) arrival counters in a workspace
constexpr int kMaxWgChunks = 256;     // chunk positions per workgroup (64 blocks)
constexpr int kWavesPerGroup = 8;     // wavefronts per workgroup (one workgroup per CU)
// Two-level merge (full mode, many splits): the last arrival of each group of
// kGroupSplits consecutive splits merges the group into one partial, and the
// last group to finish merges the group partials.  Group arrival counters
// sit in the upper half of the counter region.
constexpr int kGroupSplits = 16;
constexpr int kMaxGroups = kMaxSplits / kGroupSplits;
constexpr int kGroupCounterBase = kCounterSlots / 2;
constexpr long kOneLevelMergeBytes = 512l << 10;  // above this many partial bytes per
                                                  // (sequence, KV head): two levels

// Work split of one attention launch: each workgroup (8 wavefronts) takes
// `chunks_per_wg` consecutive 32-token chunk positions of one (sequence, KV
// head); `nsplit` workgroups cover the longest sequence.
struct SplitPlan {
  int chunks_per_wg;
  int nsplit;
};

SplitPlan plan_full(int batch, int num_kv_heads, int max_blocks);
SplitPlan plan_sparse(int batch, int num_kv_heads, int max_blocks, int k, int group, int head_dim);

// Arguments of the attention kernels (split pass + fused epilogue).
struct AttnArgs {
  const void *q;
  const void *k_pool;
  const void *v_pool;
  int64_t num_pages;
  const int32_t *table;
  const int32_t *ctx;
  const int32_t *sel;  // nullptr: every block (full); else [B][Hkv][k] block ids
  int staged;          // sparse mode: selection slot r of sequence b sits in page b * k + r
                       // of a staging pool (table not read); runs a kernel instance of its own
  int k;
  int max_blocks;
  int num_q_heads;
  int num_kv_heads;
  int group;
  float scale_log2;  // logit scale * log2(e)
  int chunks_per_wg;
  int nsplit;
  // workspace
  float *part_ml;      // [B][Hq][nsplit][2]  running max (log2 units) and sum
  float *part_o;       // [B][Hq][nsplit][d]  unnormalised output
  float *stats;        // full mode with scores: [B][Hq][max_blocks] block mass, relative to
                       // the running max of the block's workgroup partial
  int two_level;       // split partials merged in groups first (bf16, d = 128 only)
  float *part_ml2;     // two-level: [B][Hq][kMaxGroups][2]  group max (log2 units) and sum
  float *part_o2;      // two-level: [B][Hq][kMaxGroups][d]  group output, relative to its max
  int32_t *counters;   // [B][Hkv] arrival counters, zero between launches
  // outputs
  float *out;          // [B][Hq][d]
  float *lse;          // nullable [B][Hq]
  float *score_out;    // nullable [B][Hkv][max_blocks]  (full mode)
  int32_t *idx_out;    // nullable [B][Hkv][k]           (full mode: top-k)
  int32_t *sel_log;    // nullable [B][Hkv][k]           (sparse mode: copy of sel)
};

// Arguments of the standalone top-k kernel over a given score array.
struct TopkArgs {
  const float *score;  // [B][Hkv][max_blocks]
  const int32_t *ctx;
  int max_blocks;
  int num_kv_heads;
  int32_t *idx;        // [B][Hkv][k]
  int k;
};

// Index-guided gather (hylra_offload.hip): the K and V tiles of the selected
// blocks, (page, KV head) slabs of tile_bytes each, copied from pools the
// device can read (host or device memory) into staging pools
// [B * k][Hkv][...] at page b * k + r.
struct GatherArgs {
  const char *k_src, *v_src;
  int64_t num_pages;
  const int32_t *table, *ctx, *idx;
  int k, max_blocks, num_kv_heads, tile_bytes;
  char *k_dst, *v_dst;
};

// Append of one decode step's token (hylra_offload.hip): k_new / v_new
// [B][Hkv][d] written at position pos[b] of each sequence.
struct AppendArgs {
  void *k_pool, *v_pool;
  int64_t num_pages;
  const int32_t *table, *pos;
  const void *k_new, *v_new;
  int max_blocks, num_kv_heads, head_dim, elt;
};

// Rotary embedding of one decode step's q and k fused with the append of k
// and v (hylra_step.hip); bf16 only.
struct RopeAppendArgs {
  const void *qkv;                 // [B][(Hq + 2 Hkv) d]: q heads, k heads, v heads
  const float *cos_tab, *sin_tab;  // [B][d / 2]
  const int32_t *pos, *table;
  void *q_out;                     // [B][Hq][d]
  void *k_pool, *v_pool;
  int64_t num_pages;
  int max_blocks, num_q_heads, num_kv_heads, head_dim;
};

// Launchers: return 0 on success or the hipError_t code of the launch.
int launch_attn(const AttnArgs &a, int dtype, int head_dim, int batch, void *stream);
int launch_gather(const GatherArgs &a, int batch, void *stream);
int launch_append(const AppendArgs &a, int batch, void *stream);
int launch_rope_append(const RopeAppendArgs &a, int batch, void *stream);
int launch_silu_mul(const void *gu, void *out, int64_t rows, int width, void *stream);
// Cross-stream ordering through a per-device pool of events: event_record
// records event `slot` on `stream` (after the work enqueued so far),
// event_wait makes `stream` wait for the last recording of `slot`.
int event_record(void *stream, int slot);
// Sets *readable to 1 when both the first and the last byte of [base,
// base + bytes) are device memory or pinned host memory that the device maps
// at the same address (what the gather kernel dereferences), else 0.
int pool_readable(const void *base, size_t bytes, int *readable);
int event_wait(void *stream, int slot);
int launch_topk(const TopkArgs &a, int batch, void *stream);
int launch_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, void *stream);

// Offline similarity matrix of logged top-k index sets (hylra_profile.hip).
struct OverlapArgs {
  const int32_t *idx;  // [steps][layers][slices][k], ascending ids, -1 padded
  int steps, layers, slices, k;
  float *M;  // [layers][layers], row = target layer
};
size_t overlap_smem_bytes(int layers, int k);
int launch_overlap(const OverlapArgs &a, void *stream);
const char *device_error_string(int code);
// Records `message` as the calling thread's last error (hylra_last_error) and
// returns `status`.
int report_error(int status, const char *message);

// Kernel timers (see hylra_timer_start in hylra.h).
enum TimerKind {
  kTimerFullAttn = 0,    // full attention, no block scores
  kTimerSparseAttn = 1,
  kTimerTopk = 2,
  kTimerGather = 3,
  kTimerFullScored = 4,  // full attention with block scores (and the top-k when asked)
  kNumTimers = 5
};
int timer_start(int kind, int capacity);
int timer_stop(int kind, double *total_ms, int *launches);
// The event pair of the next timed launch of `kind` (both NULL when the timer
// is not running or full); the launch records them (hipExtLaunchKernel).
void timer_take(int kind, void **start, void **stop);

}  // namespace hylra
