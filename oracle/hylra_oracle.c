/*
 * HyLRA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct double-precision implementation of what
 * the hybrid decode attention path computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the
 * product library never links, loads or calls it, and it shares no source,
 * header or helper with the HIP path.
 *
 * Sources (all from "HyLRA: Hybrid Layer Reuse Attention for Efficient
 * Long-Context Inference", technical summary):
 *   - section 2.3 "Sensitive Layers": full (standard) attention over the whole
 *     context, after which the top-k indices are extracted and passed on;
 *   - section 2.3 "Tolerant Layers": attention restricted to the subset of the
 *     KV cache named by the reused indices;
 *   - section 2.4 "Block-level Sparsity": selection works on fixed blocks of
 *     128 tokens.
 * The block score (sum over the query heads of a KV group of the softmax
 * probabilities of the block's tokens), the tie rule (lower block index wins)
 * and the ascending output order are fixed by the project specification, the
 * summary leaves them open.
 *
 * Memory layout read here (the same bits the GPU path reads):
 *   q      [B][Hq][d]                      element type `dtype`
 *   K pool [pages][Hkv][128][d]            token-major page tile
 *   V pool [pages][Hkv][4][d][32]          a page as four 32-token sub-tiles,
 *                                          each dimension-major
 *   table  [B][max_blocks]                 logical block -> physical page
 *   ctx    [B]                             context length T_b in tokens
 * dtype 0 = IEEE float32, 1 = bfloat16 (upper 16 bits of a float32).
 * Query head h belongs to KV group g = h / (Hq / Hkv).
 *
 * Everything is accumulated in double; no blocking or reordering beyond the
 * definitions.  OpenMP only runs independent (sequence, head) rows side by
 * side.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 128
#define ORACLE_SUBTILE 32

/* One element of a q / K / V buffer as an exact double. */
static double elem(const void *base, int64_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t k_index(int64_t page, int Hkv, int g, int tok, int d, int c) {
  return ((page * Hkv + g) * ORACLE_BLOCK + tok) * d + c;
}

static int64_t v_index(int64_t page, int Hkv, int g, int tok, int d, int c) {
  const int64_t sub = tok / ORACLE_SUBTILE;
  return (((page * Hkv + g) * (ORACLE_BLOCK / ORACLE_SUBTILE) + sub) * d + c) * ORACLE_SUBTILE +
         tok % ORACLE_SUBTILE;
}

static int clamp_ctx(int t, int max_blocks) {
  if (t < 0) return 0;
  if (t > max_blocks * ORACLE_BLOCK) return max_blocks * ORACLE_BLOCK;
  return t;
}

/*
 * Attention of every query head of every sequence over a token set U.
 *   sel == NULL : U = all tokens t < T_b            (full attention, 2.3)
 *   sel != NULL : U = tokens t < T_b whose block n = t/128 appears in
 *                 sel[b][g][0..k)  (entries < 0 are padding)   (subset, 2.3)
 * For each (b, h):
 *   s_t   = scale * sum_c q[h,c] K[g,t,c]
 *   m     = max_{t in U} s_t,  l = sum_{t in U} exp(s_t - m)
 *   p_t   = exp(s_t - m) / l
 *   out   = sum_{t in U} p_t V[g,t,:],   lse = m + ln l
 * An empty U gives out = 0 and lse = -inf.
 * probs (nullable) receives p as [B][Hq][max_blocks*128] (0 outside U).
 * Returns 0, or -1 if a page index is outside [0, num_pages).
 */
int oracle_attend(int B, int Hq, int Hkv, int d, int dtype, double scale,
                  const void *q, const void *kpool, const void *vpool,
                  int64_t num_pages, const int32_t *table, int max_blocks,
                  const int32_t *ctx, const int32_t *sel, int k,
                  double *out, double *lse, double *probs) {
  const int G = Hq / Hkv;
  const int64_t tmax = (int64_t)max_blocks * ORACLE_BLOCK;
  int bad = 0;
  if (probs) memset(probs, 0, sizeof(double) * (size_t)B * Hq * tmax);
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int row = 0; row < B * Hq; ++row) {
    const int b = row / Hq, h = row % Hq, g = h / G;
    const int T = clamp_ctx(ctx[b], max_blocks);
    double *s = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
    char *in = (char *)calloc(T > 0 ? T : 1, 1);
    /* membership of each token in U */
    for (int t = 0; t < T; ++t) {
      if (!sel) { in[t] = 1; continue; }
      const int n = t / ORACLE_BLOCK;
      for (int r = 0; r < k; ++r)
        if (sel[((int64_t)b * Hkv + g) * k + r] == n) in[t] = 1;
    }
    double m = -INFINITY;
    for (int t = 0; t < T; ++t) {
      if (!in[t]) continue;
      const int64_t page = table[(int64_t)b * max_blocks + t / ORACLE_BLOCK];
      if (page < 0 || page >= num_pages) { bad = 1; in[t] = 0; continue; }
      double acc = 0.0;
      for (int c = 0; c < d; ++c)
        acc += elem(q, ((int64_t)b * Hq + h) * d + c, dtype) *
               elem(kpool, k_index(page, Hkv, g, t % ORACLE_BLOCK, d, c), dtype);
      s[t] = scale * acc;
      if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int t = 0; t < T; ++t)
      if (in[t]) l += exp(s[t] - m);
    double *o = out + (int64_t)row * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (l > 0.0) {
      for (int t = 0; t < T; ++t) {
        if (!in[t]) continue;
        const int64_t page = table[(int64_t)b * max_blocks + t / ORACLE_BLOCK];
        const double p = exp(s[t] - m) / l;
        if (probs) probs[(int64_t)row * tmax + t] = p;
        for (int c = 0; c < d; ++c)
          o[c] += p * elem(vpool, v_index(page, Hkv, g, t % ORACLE_BLOCK, d, c), dtype);
      }
      lse[row] = m + log(l);
    } else {
      lse[row] = -INFINITY;
    }
    free(s);
    free(in);
  }
  return bad ? -1 : 0;
}

/*
 * Block score from explicit probabilities:
 *   score[b][g][n] = sum_{h in group g} sum_{t in block n, t < T_b} p[b][h][t]
 * for n < ceil(T_b/128); entries for n >= ceil(T_b/128) are set to 0.
 */
void oracle_block_score(int B, int Hq, int Hkv, int max_blocks, const int32_t *ctx,
                        const double *probs, double *score) {
  const int G = Hq / Hkv;
  const int64_t tmax = (int64_t)max_blocks * ORACLE_BLOCK;
  for (int b = 0; b < B; ++b) {
    const int T = clamp_ctx(ctx[b], max_blocks);
    for (int g = 0; g < Hkv; ++g) {
      for (int n = 0; n < max_blocks; ++n) {
        double acc = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h)
          for (int t = n * ORACLE_BLOCK; t < (n + 1) * ORACLE_BLOCK && t < T; ++t)
            acc += probs[((int64_t)b * Hq + h) * tmax + t];
        score[((int64_t)b * Hkv + g) * max_blocks + n] = acc;
      }
    }
  }
}

/* qsort helper: order block ids by (score descending, id ascending). */
static const double *g_sort_score;
static int by_score_then_id(const void *pa, const void *pb) {
  const int a = *(const int *)pa, b = *(const int *)pb;
  if (g_sort_score[a] > g_sort_score[b]) return -1;
  if (g_sort_score[a] < g_sort_score[b]) return 1;
  return (a > b) - (a < b);
}
static int ascending_int(const void *pa, const void *pb) {
  const int a = *(const int *)pa, b = *(const int *)pb;
  return (a > b) - (a < b);
}

/*
 * Top-k blocks of one (b, g) row: sort the N_b = ceil(T_b/128) blocks by
 * (score descending, block id ascending), keep the first k_eff = min(k, N_b),
 * emit them in ascending id order, pad with -1 up to k.
 * margin[b][g] = (score of k_eff-th - score of (k_eff+1)-th) / score of
 * k_eff-th when k_eff < N_b, else +inf (how close the cut is to a tie).
 * Not thread safe (qsort comparator state).
 */
void oracle_topk(int B, int Hkv, int max_blocks, const int32_t *ctx, const double *score,
                 int k, int32_t *idx, double *margin) {
  int *order = (int *)malloc(sizeof(int) * (max_blocks > 0 ? max_blocks : 1));
  for (int b = 0; b < B; ++b) {
    const int T = clamp_ctx(ctx[b], max_blocks);
    const int N = (T + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    const int keff = k < N ? k : N;
    for (int g = 0; g < Hkv; ++g) {
      const double *row = score + ((int64_t)b * Hkv + g) * max_blocks;
      for (int n = 0; n < N; ++n) order[n] = n;
      g_sort_score = row;
      qsort(order, N, sizeof(int), by_score_then_id);
      int32_t *dst = idx + ((int64_t)b * Hkv + g) * k;
      qsort(order, keff, sizeof(int), ascending_int);
      for (int r = 0; r < k; ++r) dst[r] = r < keff ? order[r] : -1;
      if (margin) {
        double mg = INFINITY;
        if (keff > 0 && keff < N) {
          /* order[0..keff) was re-sorted by id; recompute the cut values. */
          double kth = INFINITY, next = -INFINITY;
          for (int r = 0; r < keff; ++r)
            if (row[order[r]] < kth) kth = row[order[r]];
          for (int r = keff; r < N; ++r)
            if (row[order[r]] > next) next = row[order[r]];
          mg = kth > 0.0 ? (kth - next) / kth : 0.0;
        }
        margin[(int64_t)b * Hkv + g] = mg;
      }
    }
  }
  free(order);
}
