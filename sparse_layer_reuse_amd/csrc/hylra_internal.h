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

// Work split of one attention launch: each workgroup (4 wavefronts) takes
// `chunks_per_wg` consecutive 32-token chunk positions of one (sequence, KV head).
struct SplitPlan {
  int chunks_per_wg;
  int nsplit;
};

SplitPlan plan_full(int batch, int num_kv_heads, int max_blocks);
SplitPlan plan_sparse(int batch, int num_kv_heads, int max_blocks, int k);

// Arguments of the split (partial) attention kernels.
struct AttnArgs {
  const void *q;
  const void *k_pool;
  const void *v_pool;
  int64_t num_pages;
  const int32_t *table;
  const int32_t *ctx;
  const int32_t *sel;  // nullptr: every block (full); else [B][Hkv][k] block ids
  int k;
  int max_blocks;
  int num_q_heads;
  int num_kv_heads;
  int group;
  float scale_log2;  // logit scale * log2(e)
  int chunks_per_wg;
  int nsplit;
  float *part_ml;    // [B][Hq][nsplit][2]  running max (log2 units) and sum
  float *part_o;     // [B][Hq][nsplit][d]  unnormalised output
  float *stats;      // nullable [B][Hq][4*max_blocks][2] per chunk (max, mass)
};

// Arguments of the per-head merge kernel.
struct MergeArgs {
  const float *part_ml;
  const float *part_o;
  const float *stats;      // nullable: per-chunk statistics -> per-head block mass
  const int32_t *ctx;
  const int32_t *sel;      // sparse launches: the index set (chunk count, log copy)
  int32_t *sel_log;        // nullable: copy of sel for this layer
  int k;
  int max_blocks;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int head_dim;
  int chunks_per_wg;
  int nsplit;
  float *out;              // [B][Hq][d]
  float *lse;              // nullable [B][Hq]
  float *head_mass;        // nullable [B][Hq][max_blocks] probability mass per block
};

// Arguments of the block score / top-k kernel.
struct TopkArgs {
  const float *mass;       // [B][Hkv*heads_per_row][max_blocks]
  int heads_per_row;       // rows summed per (b, g): group size, or 1 for given scores
  const int32_t *ctx;
  int max_blocks;
  int num_kv_heads;
  float *score_out;        // nullable [B][Hkv][max_blocks]
  int32_t *idx;            // nullable [B][Hkv][k]
  int k;
};

// Launchers: return 0 on success or the hipError_t code of the launch.
int launch_attn(const AttnArgs &a, int dtype, int head_dim, int batch, void *stream);
int launch_merge(const MergeArgs &a, int batch, void *stream);
int launch_topk(const TopkArgs &a, int batch, void *stream);
const char *device_error_string(int code);

// Kernel timers (see hylra_timer_start in hylra.h).
enum TimerKind { kTimerFullAttn = 0, kTimerSparseAttn = 1, kTimerMerge = 2, kTimerTopk = 3,
                 kNumTimers = 4 };
int timer_start(int kind, int capacity);
int timer_stop(int kind, double *total_ms, int *launches);

}  // namespace hylra
