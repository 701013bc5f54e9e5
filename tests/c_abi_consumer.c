/*
 * A plain C consumer of libhylra's C ABI (include/hylra.h): no Python, no
 * torch.  Built by the tests with gcc against the header and the shared
 * library.
 *
 *   c_abi_consumer host
 *       host-only calls: workspace sizing, the policy DP on a banded
 *       similarity matrix (resets exactly every w layers), status strings
 *       and the failure paths of a few entry points.  Exit status 0 if all
 *       checks hold.
 *
 *   c_abi_consumer gpu <problem.bin> <result.bin>
 *       one decode step of a policy through hylra_run_policy on device
 *       buffers allocated with hipMalloc.  problem.bin (written by the test):
 *         int32 B, Hq, Hkv, d, dtype, max_blocks, num_pages, L, k
 *         int32 src[L], table[B][max_blocks], ctx[B]
 *         per layer: q bytes, K pool bytes, V pool bytes (element type dtype)
 *       result.bin: float32 out[L][B][Hq][d], lse[L][B][Hq], int32
 *       idx_log[L][B][Hkv][k].
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hylra.h"

static int failures = 0;

#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static int host_checks(void) {
  hylra_shape s = {2, 8, 2, 128, 128, HYLRA_BF16, 16, 0.0f};
  size_t a = 0, b = 0;
  EXPECT(hylra_workspace_size(&s, 4, &a) == HYLRA_OK && a > 0);
  EXPECT(hylra_workspace_size(&s, 64, &b) == HYLRA_OK && b >= a);
  s.head_dim = 96;
  EXPECT(hylra_workspace_size(&s, 4, &a) == HYLRA_E_UNSUPPORTED);
  EXPECT(strlen(hylra_last_error()) > 0);
  s.head_dim = 128;

  /* banded similarity: layer j reuses source i with similarity 1 when
   * j - i < w, else 0; at theta 0.5 the fewest resets are every w layers */
  enum { L = 12, W = 3 };
  float M[L * L];
  for (int j = 0; j < L; ++j)
    for (int i = 0; i < L; ++i) M[j * L + i] = (i <= j && j - i < W) ? 1.0f : 0.0f;
  int32_t src[L], nres = 0;
  double sim = 0.0;
  EXPECT(hylra_policy_dp(L, M, 0.5f, NULL, src, &nres, &sim) == HYLRA_OK);
  EXPECT(nres == (L + W - 1) / W);
  for (int j = 0; j < L; ++j) EXPECT(src[j] == j - j % W);
  EXPECT(hylra_policy_dp(0, M, 0.5f, NULL, src, NULL, NULL) == HYLRA_E_INVALID_ARG);

  /* a malformed policy is refused before anything is enqueued */
  const int32_t bad[2] = {0, 2};
  const void *qs[2] = {(const void *)0x10000, (const void *)0x10000};
  hylra_kv kvs[2];
  for (int j = 0; j < 2; ++j) {
    kvs[j].k_pool = (const void *)0x20000;
    kvs[j].v_pool = (const void *)0x30000;
    kvs[j].num_pages = 4;
    kvs[j].block_table = (const int32_t *)0x40000;
    kvs[j].ctx_lens = (const int32_t *)0x50000;
  }
  float *outs[2] = {(float *)0x60000, (float *)0x60000};
  EXPECT(hylra_run_policy(&s, 2, bad, 4, qs, kvs, outs, NULL, NULL, (void *)0x70000,
                          (size_t)1 << 30, NULL) == HYLRA_E_BAD_POLICY);
  EXPECT(strcmp(hylra_status_str(HYLRA_OK), hylra_status_str(HYLRA_E_DEVICE)) != 0);
  if (failures == 0) printf("host checks ok\n");
  return failures ? 1 : 0;
}

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                            \
    }                                                                      \
  } while (0)

static void *read_all(FILE *f, size_t n) {
  void *p = malloc(n ? n : 1);
  if (p && n && fread(p, 1, n, f) != n) {
    free(p);
    return NULL;
  }
  return p;
}

static int gpu_run(const char *in_path, const char *out_path) {
  FILE *f = fopen(in_path, "rb");
  if (!f) return 3;
  int32_t h[9];
  if (fread(h, sizeof h, 1, f) != 1) return 3;
  const int B = h[0], Hq = h[1], Hkv = h[2], d = h[3], dtype = h[4], mb = h[5], P = h[6];
  const int L = h[7], k = h[8];
  const size_t elt = dtype == HYLRA_BF16 ? 2 : 4;
  int32_t *src = read_all(f, sizeof(int32_t) * L);
  int32_t *table = read_all(f, sizeof(int32_t) * B * mb);
  int32_t *ctx = read_all(f, sizeof(int32_t) * B);
  const size_t q_bytes = (size_t)B * Hq * d * elt, pool_bytes = (size_t)P * Hkv * 128 * d * elt;
  if (!src || !table || !ctx) return 3;

  hylra_shape s = {B, Hq, Hkv, d, 128, dtype, mb, 0.0f};
  int32_t *d_table, *d_ctx, *d_idx;
  HIP_OK(hipMalloc((void **)&d_table, sizeof(int32_t) * B * mb));
  HIP_OK(hipMalloc((void **)&d_ctx, sizeof(int32_t) * B));
  HIP_OK(hipMalloc((void **)&d_idx, sizeof(int32_t) * L * B * Hkv * k));
  HIP_OK(hipMemcpy(d_table, table, sizeof(int32_t) * B * mb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_ctx, ctx, sizeof(int32_t) * B, hipMemcpyHostToDevice));
  const void **qs = calloc(L, sizeof(void *));
  hylra_kv *kvs = calloc(L, sizeof(hylra_kv));
  float **outs = calloc(L, sizeof(float *)), **lses = calloc(L, sizeof(float *));
  for (int j = 0; j < L; ++j) {
    void *hq = read_all(f, q_bytes), *hk = read_all(f, pool_bytes), *hv = read_all(f, pool_bytes);
    if (!hq || !hk || !hv) return 3;
    void *dq, *dk, *dv;
    HIP_OK(hipMalloc(&dq, q_bytes));
    HIP_OK(hipMalloc(&dk, pool_bytes));
    HIP_OK(hipMalloc(&dv, pool_bytes));
    HIP_OK(hipMemcpy(dq, hq, q_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, hk, pool_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, hv, pool_bytes, hipMemcpyHostToDevice));
    free(hq);
    free(hk);
    free(hv);
    qs[j] = dq;
    kvs[j].k_pool = dk;
    kvs[j].v_pool = dv;
    kvs[j].num_pages = P;
    kvs[j].block_table = d_table;
    kvs[j].ctx_lens = d_ctx;
    HIP_OK(hipMalloc((void **)&outs[j], sizeof(float) * B * Hq * d));
    HIP_OK(hipMalloc((void **)&lses[j], sizeof(float) * B * Hq));
  }
  fclose(f);
  size_t ws_bytes = 0;
  if (hylra_workspace_size(&s, k, &ws_bytes) != HYLRA_OK) return 4;
  void *ws;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemset(ws, 0, ws_bytes));
  const hylra_status st = hylra_run_policy(&s, L, src, k, qs, kvs, (float *const *)outs,
                                           (float *const *)lses, d_idx, ws, ws_bytes, NULL);
  if (st != HYLRA_OK) {
    fprintf(stderr, "hylra_run_policy: %s: %s\n", hylra_status_str(st), hylra_last_error());
    return 5;
  }
  HIP_OK(hipDeviceSynchronize());
  FILE *o = fopen(out_path, "wb");
  if (!o) return 3;
  float *hbuf = malloc(sizeof(float) * B * Hq * d);
  for (int j = 0; j < L; ++j) {
    HIP_OK(hipMemcpy(hbuf, outs[j], sizeof(float) * B * Hq * d, hipMemcpyDeviceToHost));
    fwrite(hbuf, sizeof(float), (size_t)B * Hq * d, o);
  }
  for (int j = 0; j < L; ++j) {
    HIP_OK(hipMemcpy(hbuf, lses[j], sizeof(float) * B * Hq, hipMemcpyDeviceToHost));
    fwrite(hbuf, sizeof(float), (size_t)B * Hq, o);
  }
  int32_t *hidx = malloc(sizeof(int32_t) * L * B * Hkv * k);
  HIP_OK(hipMemcpy(hidx, d_idx, sizeof(int32_t) * L * B * Hkv * k, hipMemcpyDeviceToHost));
  fwrite(hidx, sizeof(int32_t), (size_t)L * B * Hkv * k, o);
  fclose(o);
  printf("gpu run ok\n");
  return 0;
}

int main(int argc, char **argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 4 && strcmp(argv[1], "gpu") == 0) return gpu_run(argv[2], argv[3]);
  fprintf(stderr, "usage: %s host | gpu <problem.bin> <result.bin>\n", argv[0]);
  return 64;
}
