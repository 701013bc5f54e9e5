// Host stand-ins for the device side of libhylra, for the sanitizer build of
// the C-ABI host code (hylra_api.cpp) on the CPU.  Nothing here launches
// anything: each launcher checks the launch it is handed (grid and split
// plan within the kernels' limits) and then touches, on the host, every byte
// of every buffer the kernel would read or write for that launch.  The test
// driver allocates those buffers on the host at exactly the sizes the ABI
// documents (the workspace at hylra_workspace_size bytes), so AddressSanitizer
// reports any launch whose footprint leaves its buffers.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../sparse_layer_reuse_amd/csrc/hylra_internal.h"

namespace {

volatile unsigned char g_sink;

void die(const char *what) {
  fprintf(stderr, "device stub: %s\n", what);
  abort();
}

void touch_read(const void *p, size_t bytes) {
  if (bytes == 0) return;
  if (p == nullptr) die("read through a NULL pointer");
  const unsigned char *c = static_cast<const unsigned char *>(p);
  unsigned char acc = 0;
  for (size_t i = 0; i < bytes; ++i) acc ^= c[i];
  g_sink = acc;
}

void touch_write(void *p, size_t bytes) {
  if (bytes == 0) return;
  if (p == nullptr) die("write through a NULL pointer");
  unsigned char *c = static_cast<unsigned char *>(p);
  for (size_t i = 0; i < bytes; ++i) c[i] = (unsigned char)(c[i] + 0);
}

size_t elt(int dtype) { return dtype == 1 ? 2 : 4; }

}  // namespace

namespace hylra {

int launch_attn(const AttnArgs &a, int dtype, int head_dim, int batch, void *) {
  const size_t B = batch, Hq = a.num_q_heads, Hkv = a.num_kv_heads, D = head_dim;
  const size_t mb = a.max_blocks, ns = a.nsplit, k = a.k;
  if (a.nsplit < 1 || a.nsplit > kMaxSplits) die("nsplit outside [1, kMaxSplits]");
  if (a.chunks_per_wg < 1 || a.chunks_per_wg > kMaxWgChunks) die("chunks per workgroup out of range");
  const long need = a.sel == nullptr ? (long)kChunksPerBlock * a.max_blocks : (long)kChunksPerBlock * a.k;
  if ((long)a.nsplit * a.chunks_per_wg < need) die("split plan does not cover every chunk position");
  if ((long)a.nsplit * a.chunks_per_wg - a.chunks_per_wg >= need) die("split plan has an empty split");
  if (a.group * a.num_kv_heads != a.num_q_heads || a.group > kMaxGroup) die("bad group size");
  if (B * Hkv > (size_t)kCounterSlots) die("more rows than arrival counters");
  touch_read(a.q, B * Hq * D * elt(dtype));
  touch_read(a.ctx, B * sizeof(int32_t));
  if (!a.staged) touch_read(a.table, B * mb * sizeof(int32_t));
  touch_read(a.k_pool, (size_t)a.num_pages * Hkv * kBlockTokens * D * elt(dtype));
  touch_read(a.v_pool, (size_t)a.num_pages * Hkv * kBlockTokens * D * elt(dtype));
  if (a.sel != nullptr) touch_read(a.sel, B * Hkv * k * sizeof(int32_t));
  touch_write(a.counters, B * Hkv * sizeof(int32_t));
  touch_write(a.part_ml, B * Hq * ns * 2 * sizeof(float));
  touch_write(a.part_o, B * Hq * ns * D * sizeof(float));
  if (a.stats != nullptr) touch_write(a.stats, B * Hq * mb * sizeof(float));
  if (a.two_level) {
    if (a.sel != nullptr) die("two-level merge in sparse mode");
    touch_write(a.counters + kGroupCounterBase, B * Hkv * kMaxGroups * sizeof(int32_t));
    touch_write(a.part_ml2, B * Hq * kMaxGroups * 2 * sizeof(float));
    touch_write(a.part_o2, B * Hq * kMaxGroups * D * sizeof(float));
  }
  touch_write(a.out, B * Hq * D * sizeof(float));
  if (a.lse != nullptr) touch_write(a.lse, B * Hq * sizeof(float));
  if (a.score_out != nullptr) touch_write(a.score_out, B * Hkv * mb * sizeof(float));
  if (a.idx_out != nullptr) touch_write(a.idx_out, B * Hkv * k * sizeof(int32_t));
  if (a.sel_log != nullptr) touch_write(a.sel_log, B * Hkv * k * sizeof(int32_t));
  return 0;
}

int launch_topk(const TopkArgs &a, int batch, void *) {
  touch_read(a.score, (size_t)batch * a.num_kv_heads * a.max_blocks * sizeof(float));
  touch_read(a.ctx, (size_t)batch * sizeof(int32_t));
  touch_write(a.idx, (size_t)batch * a.num_kv_heads * a.k * sizeof(int32_t));
  return 0;
}

int launch_gather(const GatherArgs &a, int batch, void *) {
  const size_t slabs = (size_t)batch * a.k * a.num_kv_heads;
  touch_read(a.idx, slabs * sizeof(int32_t));
  touch_read(a.ctx, (size_t)batch * sizeof(int32_t));
  touch_read(a.table, (size_t)batch * a.max_blocks * sizeof(int32_t));
  touch_read(a.k_src, (size_t)a.num_pages * a.num_kv_heads * a.tile_bytes);
  touch_read(a.v_src, (size_t)a.num_pages * a.num_kv_heads * a.tile_bytes);
  touch_write(a.k_dst, slabs * a.tile_bytes);
  touch_write(a.v_dst, slabs * a.tile_bytes);
  return 0;
}

int launch_append(const AppendArgs &a, int batch, void *) {
  const size_t row = (size_t)a.num_kv_heads * a.head_dim * a.elt;
  touch_read(a.k_new, batch * row);
  touch_read(a.v_new, batch * row);
  touch_read(a.pos, (size_t)batch * sizeof(int32_t));
  touch_read(a.table, (size_t)batch * a.max_blocks * sizeof(int32_t));
  touch_write(a.k_pool, (size_t)a.num_pages * kBlockTokens * row);
  touch_write(a.v_pool, (size_t)a.num_pages * kBlockTokens * row);
  return 0;
}

int launch_rope_append(const RopeAppendArgs &a, int batch, void *) {
  const size_t d = a.head_dim;
  touch_read(a.qkv, (size_t)batch * (a.num_q_heads + 2 * a.num_kv_heads) * d * 2);
  touch_read(a.cos_tab, (size_t)batch * (d / 2) * sizeof(float));
  touch_read(a.sin_tab, (size_t)batch * (d / 2) * sizeof(float));
  touch_read(a.pos, (size_t)batch * sizeof(int32_t));
  touch_read(a.table, (size_t)batch * a.max_blocks * sizeof(int32_t));
  touch_write(a.q_out, (size_t)batch * a.num_q_heads * d * 2);
  touch_write(a.k_pool, (size_t)a.num_pages * a.num_kv_heads * kBlockTokens * d * 2);
  touch_write(a.v_pool, (size_t)a.num_pages * a.num_kv_heads * kBlockTokens * d * 2);
  return 0;
}

int launch_silu_mul(const void *gu, void *out, int64_t rows, int width, void *) {
  touch_read(gu, (size_t)rows * 2 * width * 2);
  touch_write(out, (size_t)rows * width * 2);
  return 0;
}

int launch_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, void *) {
  touch_read(buf, bytes);
  touch_write(sink, sizeof(uint32_t));
  return 0;
}

size_t overlap_smem_bytes(int layers, int k) {
  return (size_t)8 * layers + (size_t)4 * layers * k;
}

int launch_overlap(const OverlapArgs &a, void *) {
  touch_read(a.idx, (size_t)a.steps * a.layers * a.slices * a.k * sizeof(int32_t));
  touch_write(a.M, (size_t)a.layers * a.layers * sizeof(float));
  return 0;
}

int event_record(void *, int slot) { return slot < 0 ? 1 : 0; }
int event_wait(void *, int slot) { return slot < 0 ? 1 : 0; }

int pool_readable(const void *base, size_t bytes, int *readable) {
  touch_read(base, bytes);
  *readable = 1;
  return 0;
}

int timer_start(int, int) { return 0; }
int timer_stop(int, double *total_ms, int *launches) {
  if (total_ms) *total_ms = 0.0;
  if (launches) *launches = 0;
  return 0;
}

const char *device_error_string(int) { return "device stub error"; }

}  // namespace hylra
