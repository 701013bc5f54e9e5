/*
 * Driver of the host sanitizer build (AddressSanitizer + UndefinedBehavior-
 * Sanitizer, CPU only): calls every entry point of include/hylra.h with host
 * buffers of exactly the documented sizes (the device side is replaced by
 * stubs that touch each launch's whole footprint), checks the argument
 * validation, runs the policy DP on random matrices, and runs the C oracle on
 * small inputs.  Exits 0 when every check holds; a sanitizer report aborts.
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/hylra.h"

/* the oracle's entry points (oracle/hylra_oracle.c) */
int oracle_attend(int B, int Hq, int Hkv, int d, int dtype, double scale, const void *q,
                  const void *kpool, const void *vpool, int64_t num_pages, const int32_t *table,
                  int max_blocks, const int32_t *ctx, const int32_t *sel, int k, double *out,
                  double *lse, double *probs);
void oracle_block_score(int B, int Hq, int Hkv, int max_blocks, const int32_t *ctx,
                        const double *probs, double *score);
void oracle_topk(int B, int Hkv, int max_blocks, const int32_t *ctx, const double *score,
                 int k, int32_t *idx, double *margin);

static int g_fail = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
              hylra_last_error());                                               \
      g_fail = 1;                                                                \
    }                                                                            \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)(g_rng >> 11);
}
static double urand(void) { return (rnd() & 0xFFFFFF) / (double)0x1000000; }

/* exact-size, 16-byte aligned, zero-filled host buffer */
static void *buf(size_t bytes) {
  void *p = NULL;
  if (bytes == 0) bytes = 1;
  if (posix_memalign(&p, 16, bytes) != 0) abort();
  memset(p, 0, bytes);
  return p;
}

typedef struct {
  hylra_shape s;
  int64_t pages;
  size_t elt;
  void *q, *kp, *vp;
  int32_t *table, *ctx;
  hylra_kv kv;
} layer_t;

static void make_layer(layer_t *L, int B, int Hq, int Hkv, int d, int dtype, int mb) {
  memset(L, 0, sizeof *L);
  L->s.batch = B;
  L->s.num_q_heads = Hq;
  L->s.num_kv_heads = Hkv;
  L->s.head_dim = d;
  L->s.block_size = HYLRA_BLOCK_TOKENS;
  L->s.dtype = dtype;
  L->s.max_blocks_per_seq = mb;
  L->s.scale = 0.f;
  L->elt = dtype == HYLRA_BF16 ? 2 : 4;
  L->pages = (int64_t)B * mb;
  L->q = buf((size_t)B * Hq * d * L->elt);
  L->kp = buf((size_t)L->pages * Hkv * 128 * d * L->elt);
  L->vp = buf((size_t)L->pages * Hkv * 128 * d * L->elt);
  L->table = (int32_t *)buf(sizeof(int32_t) * B * mb);
  L->ctx = (int32_t *)buf(sizeof(int32_t) * B);
  for (int i = 0; i < B * mb; ++i) L->table[i] = (int32_t)(((int64_t)i * 7 + 3) % L->pages);
  for (int b = 0; b < B; ++b) L->ctx[b] = (int32_t)(rnd() % (128 * mb + 1));
  L->kv.k_pool = L->kp;
  L->kv.v_pool = L->vp;
  L->kv.num_pages = L->pages;
  L->kv.block_table = L->table;
  L->kv.ctx_lens = L->ctx;
}

static void free_layer(layer_t *L) {
  free(L->q);
  free(L->kp);
  free(L->vp);
  free(L->table);
  free(L->ctx);
}

/* Every entry point on one shape, buffers at their documented sizes. */
static void run_shape(int B, int Hq, int Hkv, int d, int dtype, int mb, int k) {
  enum { NL = 5 };
  layer_t lay[NL];
  for (int j = 0; j < NL; ++j) make_layer(&lay[j], B, Hq, Hkv, d, dtype, mb);
  const hylra_shape *s = &lay[0].s;
  size_t wsb = 0;
  CHECK(hylra_workspace_size(s, k, &wsb) == HYLRA_OK);
  void *ws = buf(wsb);
  size_t ws0 = 0;
  CHECK(hylra_workspace_size(s, 0, &ws0) == HYLRA_OK);
  void *wsf = buf(ws0);
  float *out[NL], *lse[NL];
  for (int j = 0; j < NL; ++j) {
    out[j] = (float *)buf(sizeof(float) * B * Hq * d);
    lse[j] = (float *)buf(sizeof(float) * B * Hq);
  }
  float *score = (float *)buf(sizeof(float) * B * Hkv * mb);
  int32_t *idx = (int32_t *)buf(sizeof(int32_t) * B * Hkv * k);
  int32_t *log = (int32_t *)buf(sizeof(int32_t) * NL * B * Hkv * k);

  CHECK(hylra_decode_full(s, lay[0].q, &lay[0].kv, out[0], lse[0], score, wsf, ws0, NULL) == HYLRA_OK);
  CHECK(hylra_decode_full(s, lay[0].q, &lay[0].kv, out[0], NULL, NULL, wsf, ws0, NULL) == HYLRA_OK);
  CHECK(hylra_decode_full(s, lay[0].q, &lay[0].kv, out[0], lse[0], score, wsf, ws0 - 1, NULL) ==
        HYLRA_E_WORKSPACE);
  CHECK(hylra_block_topk(s, score, lay[0].ctx, k, idx, NULL) == HYLRA_OK);
  CHECK(hylra_decode_sparse(s, lay[1].q, &lay[1].kv, idx, k, out[1], lse[1], ws, wsb, NULL) ==
        HYLRA_OK);

  const void *qs[NL];
  hylra_kv kvs[NL];
  for (int j = 0; j < NL; ++j) {
    qs[j] = lay[j].q;
    kvs[j] = lay[j].kv;
  }
  const int32_t src[NL] = {0, 0, 2, 2, 2};
  CHECK(hylra_run_policy(s, NL, src, k, qs, kvs, out, lse, NULL, ws, wsb, NULL) == HYLRA_OK);
  CHECK(hylra_run_policy(s, NL, src, k, qs, kvs, out, NULL, log, ws, wsb, NULL) == HYLRA_OK);
  const int32_t bad[NL] = {0, 0, 1, 2, 2};
  CHECK(hylra_run_policy(s, NL, bad, k, qs, kvs, out, lse, NULL, ws, wsb, NULL) ==
        HYLRA_E_BAD_POLICY);

  /* offloading: staging pools of B*k pages */
  const size_t slab = (size_t)Hkv * 128 * d * lay[0].elt;
  void *sk = buf((size_t)B * k * slab), *sv = buf((size_t)B * k * slab);
  CHECK(hylra_gather_blocks(s, &lay[2].kv, idx, k, sk, sv, NULL) == HYLRA_OK);
  CHECK(hylra_decode_staged(s, lay[2].q, sk, sv, lay[2].ctx, idx, k, out[2], lse[2], ws, wsb,
                            NULL) == HYLRA_OK);
  void *sks[NL] = {0}, *svs[NL] = {0};
  uint8_t off[NL] = {0, 1, 0, 1, 1};
  for (int j = 0; j < NL; ++j)
    if (off[j]) {
      sks[j] = buf((size_t)B * k * slab);
      svs[j] = buf((size_t)B * k * slab);
    }
  int copy_stream_tag;
  CHECK(hylra_run_policy_offload(s, NL, src, k, qs, kvs, off, sks, svs, out, lse, log, ws, wsb,
                                 NULL, &copy_stream_tag) == HYLRA_OK);
  off[0] = 1; /* a reset layer may not be offloaded */
  CHECK(hylra_run_policy_offload(s, NL, src, k, qs, kvs, off, sks, svs, out, lse, log, ws, wsb,
                                 NULL, &copy_stream_tag) == HYLRA_E_BAD_POLICY);
  for (int j = 0; j < NL; ++j) {
    free(sks[j]);
    free(svs[j]);
  }
  free(sk);
  free(sv);

  /* per-step helpers */
  int32_t *pos = (int32_t *)buf(sizeof(int32_t) * B);
  void *kn = buf((size_t)B * Hkv * d * lay[0].elt), *vn = buf((size_t)B * Hkv * d * lay[0].elt);
  CHECK(hylra_append_kv(s, &lay[3].kv, kn, vn, pos, NULL) == HYLRA_OK);
  if (dtype == HYLRA_BF16) {
    void *qkv = buf((size_t)B * (Hq + 2 * Hkv) * d * 2);
    float *ct = (float *)buf(sizeof(float) * B * (d / 2)), *st = (float *)buf(sizeof(float) * B * (d / 2));
    void *qo = buf((size_t)B * Hq * d * 2);
    CHECK(hylra_rope_append(s, &lay[4].kv, qkv, ct, st, pos, qo, NULL) == HYLRA_OK);
    free(qkv);
    free(ct);
    free(st);
    free(qo);
  }
  free(pos);
  free(kn);
  free(vn);

  /* argument validation: nothing is launched on these */
  hylra_shape t = *s;
  t.head_dim = 96;
  CHECK(hylra_decode_full(&t, lay[0].q, &lay[0].kv, out[0], lse[0], NULL, wsf, ws0, NULL) ==
        HYLRA_E_UNSUPPORTED);
  CHECK(hylra_decode_sparse(s, lay[1].q, &lay[1].kv, idx, 0, out[1], lse[1], ws, wsb, NULL) ==
        HYLRA_E_INVALID_ARG);
  CHECK(hylra_decode_sparse(s, lay[1].q, &lay[1].kv, idx, 8193, out[1], lse[1], ws, wsb, NULL) ==
        HYLRA_E_UNSUPPORTED);
  CHECK(hylra_decode_sparse(s, lay[1].q, &lay[1].kv, NULL, k, out[1], lse[1], ws, wsb, NULL) ==
        HYLRA_E_INVALID_ARG);
  CHECK(hylra_decode_full(NULL, lay[0].q, &lay[0].kv, out[0], lse[0], NULL, wsf, ws0, NULL) ==
        HYLRA_E_INVALID_ARG);
  CHECK(hylra_decode_full(s, (const char *)lay[0].q + 4, &lay[0].kv, out[0], lse[0], NULL, wsf,
                          ws0, NULL) == HYLRA_E_INVALID_ARG);

  free(ws);
  free(wsf);
  for (int j = 0; j < NL; ++j) {
    free(out[j]);
    free(lse[j]);
    free_layer(&lay[j]);
  }
  free(score);
  free(idx);
  free(log);
}

/* The DP's policy is valid: layer 0 and forced layers reset, every reuse
 * keeps the previous source and clears the threshold; counts agree. */
static void check_dp(int L, float theta, int with_force) {
  float *M = (float *)buf(sizeof(float) * L * L);
  uint8_t *force = (uint8_t *)buf((size_t)L);
  int32_t *src = (int32_t *)buf(sizeof(int32_t) * L);
  for (int j = 0; j < L; ++j) {
    for (int i = 0; i <= j; ++i) M[j * L + i] = (float)urand();
    force[j] = with_force && (rnd() % 5 == 0);
  }
  int nres = -1;
  double sim = -1.0;
  CHECK(hylra_policy_dp(L, M, theta, with_force ? force : NULL, src, &nres, &sim) == HYLRA_OK);
  int r = 0;
  double acc = 0.0;
  CHECK(src[0] == 0);
  for (int j = 0; j < L; ++j) {
    if (src[j] == j) {
      ++r;
    } else {
      CHECK(j > 0 && src[j] == src[j - 1]);
      CHECK(!(with_force && force[j]));
      CHECK(M[j * L + src[j]] > theta);
      acc += M[j * L + src[j]];
    }
  }
  CHECK(r == nres);
  CHECK(fabs(acc - sim) <= 1e-9 * (1.0 + fabs(acc)));
  M[(L - 1) * L] = NAN;
  if (L > 1) CHECK(hylra_policy_dp(L, M, theta, NULL, src, NULL, NULL) == HYLRA_E_INVALID_ARG);
  free(M);
  free(force);
  free(src);
}

/* The oracle on small ragged inputs, both element types, odd selections. */
static void run_oracle(int dtype) {
  enum { B = 3, Hq = 6, Hkv = 2, d = 64, mb = 4, k = 5 };
  const size_t elt = dtype ? 2 : 4;
  const int64_t pages = B * mb;
  void *q = buf((size_t)B * Hq * d * elt);
  void *kp = buf((size_t)pages * Hkv * 128 * d * elt), *vp = buf((size_t)pages * Hkv * 128 * d * elt);
  if (dtype) {
    uint16_t *a = (uint16_t *)q, *b = (uint16_t *)kp, *c = (uint16_t *)vp;
    for (int i = 0; i < B * Hq * d; ++i) a[i] = (uint16_t)(0x3E00 + rnd() % 0x200);
    for (int64_t i = 0; i < pages * Hkv * 128 * d; ++i) {
      b[i] = (uint16_t)(0x3E00 + rnd() % 0x200);
      c[i] = (uint16_t)(0xBE00 + rnd() % 0x200);
    }
  } else {
    float *a = (float *)q, *b = (float *)kp, *c = (float *)vp;
    for (int i = 0; i < B * Hq * d; ++i) a[i] = (float)urand() - 0.5f;
    for (int64_t i = 0; i < pages * Hkv * 128 * d; ++i) {
      b[i] = (float)urand() - 0.5f;
      c[i] = (float)urand() - 0.5f;
    }
  }
  int32_t table[B * mb], ctx[B] = {0, 300, 512};
  for (int i = 0; i < B * mb; ++i) table[i] = (i * 5 + 1) % (int)pages;
  int32_t sel[B * Hkv * k];
  for (int i = 0; i < B * Hkv * k; ++i) sel[i] = (int32_t)(rnd() % 9) - 3; /* -3 .. 5 */
  double *out = (double *)buf(sizeof(double) * B * Hq * d), *lse = (double *)buf(sizeof(double) * B * Hq);
  double *probs = (double *)buf(sizeof(double) * B * Hq * mb * 128);
  double *score = (double *)buf(sizeof(double) * B * Hkv * mb);
  int32_t idx[B * Hkv * k];
  double margin[B * Hkv];
  CHECK(oracle_attend(B, Hq, Hkv, d, dtype, 0.125, q, kp, vp, pages, table, mb, ctx, NULL, 0,
                      out, lse, probs) == 0);
  oracle_block_score(B, Hq, Hkv, mb, ctx, probs, score);
  oracle_topk(B, Hkv, mb, ctx, score, k, idx, margin);
  CHECK(oracle_attend(B, Hq, Hkv, d, dtype, 0.125, q, kp, vp, pages, table, mb, ctx, sel, k, out,
                      lse, NULL) == 0);
  table[2 * mb + 1] = (int32_t)pages; /* a page outside the pool is reported */
  CHECK(oracle_attend(B, Hq, Hkv, d, dtype, 0.125, q, kp, vp, pages, table, mb, ctx, NULL, 0,
                      out, lse, NULL) == -1);
  free(q);
  free(kp);
  free(vp);
  free(out);
  free(lse);
  free(probs);
  free(score);
}

int main(void) {
  run_shape(2, 8, 2, 64, HYLRA_F32, 5, 3);
  run_shape(3, 32, 8, 128, HYLRA_BF16, 40, 16);
  run_shape(1, 16, 1, 128, HYLRA_BF16, 1024, 64); /* two-level merge plan */
  run_shape(2, 4, 4, 64, HYLRA_BF16, 3, 9);       /* k larger than the table row */
  for (int L = 1; L <= 40; ++L) check_dp(L, 0.3f + 0.015f * L, L % 2);
  check_dp(1024, 0.5f, 1);
  run_oracle(0);
  run_oracle(1);
  if (g_fail) return 1;
  printf("host sanitizer driver: all checks passed\n");
  return 0;
}
