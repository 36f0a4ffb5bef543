/*
 * CPU oracle for prefill block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg call this file; the product library (libspa.so) never
 * does, and the two share no code, header or table.
 *
 * Source: the LServe write-up at bqwf.cn ("LServe长序列LLM服务系统"), section
 * "3.1 预填充阶段优化": during prefill, the importance of each block of text is
 * estimated with a low-rank approximation, Score(Q, K_i) ~ (Q W_q)(K_i W_k)^T
 * / sqrt(d), where W_q and W_k project d dimensions down to d/8; exact
 * attention is then computed only for the most important blocks; the
 * approximate scores of all blocks come first, the selected blocks are then
 * processed; sequences shorter than 32K fall back to dense attention (no
 * selection). Streaming heads keep their sink + local window (section "2.1
 * 混合稀疏注意力机制"). The long-context survey (xllm-io.github.io,
 * "2.3 分组查询注意力 (GQA)") gives the scaled softmax and the head mapping.
 *
 * Readings (the page leaves these open; each is the plainest one the rest
 * supports):
 *   - A block is `b` consecutive tokens (query blocks and key blocks alike);
 *     the last block of a sequence may be shorter.
 *   - The score of query block j against key block i is the mean, over the
 *     block pair, of the approximate logits (q_t W_q)(k_s W_k)^T / sqrt(d).
 *     By linearity that is (qbar_j W_q) . (kbar_i W_k) / sqrt(d) with qbar_j,
 *     kbar_i the mean query / key of each block; it is computed in fp64 in
 *     that order (mean, projection, dot product) and rounded once to fp32.
 *   - Selection is per KV head, for its whole group of G query heads
 *     (grouped-query attention; the decode path selects per KV head too):
 *     the score averages the low-rank logits over the group's G heads as
 *     well, i.e. qbar_j is the mean query of block j over the G heads and
 *     the block's tokens. One W_q, W_k pair per layer, shared by the heads.
 *     Query block j always attends its own block j
 *     (causally, so every query sees at least itself) and, of the earlier
 *     blocks 0..j-1, the min(j, kb - 1) best ones in the order (score
 *     descending, block id ascending), kb = max(1, budget / b) blocks per
 *     query block in all.
 *   - Within the attended blocks attention is exact and causal: query t
 *     attends key s when s <= t and block(s) is selected for block(t).
 *   - Dense mode (L < dense_below): a dynamic head attends every s <= t.
 *     Streaming heads attend s in [0, min(sink, t + 1)) U [max(sink, t + 1 -
 *     window), t + 1) in both modes (their pattern needs no selection).
 * Attention is fp64 throughout: out_t = sum_s softmax_s(q_t . k_s / sqrt(d))
 * v_s, lse_t = natural log of the softmax denominator.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PF_OK 0
#define PF_ERR_ARG 1

static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Mean of rows [t0, t1) of X [L][D] (bf16), fp64. */
static void block_mean(const uint16_t* X, int32_t D, int64_t t0, int64_t t1, double* m) {
  for (int32_t c = 0; c < D; c++) m[c] = 0.0;
  for (int64_t t = t0; t < t1; t++)
    for (int32_t c = 0; c < D; c++) m[c] += bf(X[t * D + c]);
  for (int32_t c = 0; c < D; c++) m[c] /= (double)(t1 - t0);
}

/* y[r] = sum_c x[c] W[c][r], W bf16 [D][R], fp64, c ascending. */
static void project(const double* x, const uint16_t* W, int32_t D, int32_t R, double* y) {
  for (int32_t r = 0; r < R; r++) {
    double s = 0.0;
    for (int32_t c = 0; c < D; c++) s += x[c] * bf(W[(int64_t)c * R + r]);
    y[r] = s;
  }
}

/* Block scores of one KV head for its group of G query heads: S[j][i] for
 * 0 <= i < j < nb (other entries NaN), nb = ceil(L / b). Q: [G][L][D] (the
 * group's queries), K: [L][D]. */
int orc_prefill_block_scores(const uint16_t* Q, int32_t G, const uint16_t* K, const uint16_t* Wq,
                             const uint16_t* Wk, int64_t L, int32_t D, int32_t R, int32_t b, float* S) {
  if (!Q || !K || !Wq || !Wk || !S || G < 1 || L < 1 || D < 1 || R < 1 || b < 1) return PF_ERR_ARG;
  const int64_t nb = (L + b - 1) / b;
  double* qp = malloc(sizeof(double) * nb * R);
  double* kp = malloc(sizeof(double) * nb * R);
  double* m = malloc(sizeof(double) * D);
  double* mg = malloc(sizeof(double) * D);
  if (!qp || !kp || !m || !mg) { free(qp); free(kp); free(m); free(mg); return PF_ERR_ARG; }
  for (int64_t j = 0; j < nb; j++) {
    const int64_t t0 = j * b, t1 = t0 + b < L ? t0 + b : L;
    for (int32_t c = 0; c < D; c++) mg[c] = 0.0;
    for (int32_t g = 0; g < G; g++) {                    /* the group's mean query of the block */
      block_mean(Q + (int64_t)g * L * D, D, t0, t1, m);
      for (int32_t c = 0; c < D; c++) mg[c] += m[c];
    }
    for (int32_t c = 0; c < D; c++) mg[c] /= (double)G;
    project(mg, Wq, D, R, qp + j * R);
    block_mean(K, D, t0, t1, m);
    project(m, Wk, D, R, kp + j * R);
  }
  const double scale = 1.0 / sqrt((double)D);
  for (int64_t j = 0; j < nb; j++)
    for (int64_t i = 0; i < nb; i++) {
      if (i >= j) { S[j * nb + i] = NAN; continue; }
      double s = 0.0;
      for (int32_t r = 0; r < R; r++) s += qp[j * R + r] * kp[i * R + r];
      S[j * nb + i] = (float)(s * scale);
    }
  free(qp);
  free(kp);
  free(m);
  free(mg);
  return PF_OK;
}

/* Selected key blocks of every query block from the scores above: block j
 * itself plus the min(j, kb - 1) best of blocks 0..j-1 (score descending,
 * id ascending), written ascending to sel[j][0..cnt[j]) (sel is [nb][cap]). */
int orc_prefill_select(const float* S, int64_t nb, int64_t kb, int32_t* sel, int32_t* cnt, int64_t cap) {
  if (!S || !sel || !cnt || nb < 1 || kb < 1 || cap < 1) return PF_ERR_ARG;
  int32_t* order = malloc(sizeof(int32_t) * nb);
  if (!order) return PF_ERR_ARG;
  for (int64_t j = 0; j < nb; j++) {
    const int64_t k = j < kb - 1 ? j : kb - 1;            /* earlier blocks kept */
    if (k + 1 > cap) { free(order); return PF_ERR_ARG; }
    for (int64_t i = 0; i < j; i++) order[i] = (int32_t)i;
    /* selection sort of the first k places by (score desc, id asc) */
    for (int64_t a = 0; a < k; a++) {
      int64_t best = a;
      for (int64_t c = a + 1; c < j; c++) {
        const float x = S[j * nb + order[c]], y = S[j * nb + order[best]];
        if (x > y || (x == y && order[c] < order[best])) best = c;
      }
      const int32_t t = order[a];
      order[a] = order[best];
      order[best] = t;
    }
    /* the kept ids ascending, then the diagonal block (the largest id) */
    for (int64_t a = 1; a < k; a++)
      for (int64_t c = a; c > 0 && order[c - 1] > order[c]; c--) {
        const int32_t t = order[c];
        order[c] = order[c - 1];
        order[c - 1] = t;
      }
    for (int64_t a = 0; a < k; a++) sel[j * cap + a] = order[a];
    sel[j * cap + k] = (int32_t)j;
    cnt[j] = (int32_t)(k + 1);
  }
  free(order);
  return PF_OK;
}

/* Attention of one query head. mode 0: streaming (sink + window); mode 1:
 * dynamic, dense (every s <= t); mode 2: dynamic, the selected blocks
 * sel[j][0..cnt[j]) (cap per row). out [L][D], lse [L], fp64. */
int orc_prefill_attend(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t L, int32_t D,
                       int32_t b, int32_t mode, int32_t sink, int32_t window, const int32_t* sel,
                       const int32_t* cnt, int64_t cap, double* out, double* lse) {
  if (!Q || !K || !V || !out || !lse || L < 1 || D < 1 || b < 1 || mode < 0 || mode > 2) return PF_ERR_ARG;
  if (mode == 0 && (sink < 0 || window < 1)) return PF_ERR_ARG;
  if (mode == 2 && (!sel || !cnt || cap < 1)) return PF_ERR_ARG;
  const int64_t nb = (L + b - 1) / b;
  uint8_t* use = malloc(nb);
  double* x = malloc(sizeof(double) * L);
  if (!use || !x) { free(use); free(x); return PF_ERR_ARG; }
  const double scale = 1.0 / sqrt((double)D);
  for (int64_t t = 0; t < L; t++) {
    const int64_t j = t / b;
    if (mode == 2) {
      memset(use, 0, nb);
      for (int32_t a = 0; a < cnt[j]; a++) {
        const int32_t i = sel[j * cap + a];
        if (i < 0 || i > j) { free(use); free(x); return PF_ERR_ARG; }
        use[i] = 1;
      }
    }
    double mx = -INFINITY;
    for (int64_t s = 0; s <= t; s++) {
      int keep;
      if (mode == 0) keep = s < sink || s >= t + 1 - window;
      else if (mode == 1) keep = 1;
      else keep = use[s / b];
      if (!keep) { x[s] = -INFINITY; continue; }
      double d = 0.0;
      for (int32_t c = 0; c < D; c++) d += bf(Q[t * D + c]) * bf(K[s * D + c]);
      x[s] = d * scale;
      if (x[s] > mx) mx = x[s];
    }
    double den = 0.0;
    for (int32_t c = 0; c < D; c++) out[t * D + c] = 0.0;
    for (int64_t s = 0; s <= t; s++) {
      if (x[s] == -INFINITY) continue;
      const double w = exp(x[s] - mx);
      den += w;
      for (int32_t c = 0; c < D; c++) out[t * D + c] += w * bf(V[s * D + c]);
    }
    for (int32_t c = 0; c < D; c++) out[t * D + c] /= den;
    lse[t] = mx + log(den);
  }
  free(use);
  free(x);
  return PF_OK;
}

/* Independent query rows: the same as orc_prefill_attend but only for the
 * positions rows[0..nrows) (out [nrows][D], lse [nrows]); for checks of very
 * long sequences on sampled rows. */
int orc_prefill_attend_rows(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t L, int32_t D,
                            int32_t b, int32_t mode, int32_t sink, int32_t window, const int32_t* sel,
                            const int32_t* cnt, int64_t cap, const int64_t* rows, int64_t nrows, double* out,
                            double* lse) {
  if (!rows || nrows < 0) return PF_ERR_ARG;
  if (!Q || !K || !V || !out || !lse || L < 1 || D < 1 || b < 1 || mode < 0 || mode > 2) return PF_ERR_ARG;
  const int64_t nb = (L + b - 1) / b;
  int rc = PF_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
  for (int64_t n = 0; n < nrows; n++) {
    const int64_t t = rows[n];
    if (t < 0 || t >= L) { rc |= PF_ERR_ARG; continue; }
    const int64_t j = t / b;
    uint8_t* use = calloc(nb, 1);
    double* x = malloc(sizeof(double) * (t + 1));
    if (!use || !x) { free(use); free(x); rc |= PF_ERR_ARG; continue; }
    if (mode == 2)
      for (int32_t a = 0; a < cnt[j]; a++) {
        const int32_t i = sel[j * cap + a];
        if (i >= 0 && i <= j) use[i] = 1;
      }
    const double scale = 1.0 / sqrt((double)D);
    double mx = -INFINITY;
    for (int64_t s = 0; s <= t; s++) {
      int keep = mode == 0 ? (s < sink || s >= t + 1 - window) : mode == 1 ? 1 : use[s / b];
      if (!keep) { x[s] = -INFINITY; continue; }
      double d = 0.0;
      for (int32_t c = 0; c < D; c++) d += bf(Q[t * D + c]) * bf(K[s * D + c]);
      x[s] = d * scale;
      if (x[s] > mx) mx = x[s];
    }
    double den = 0.0;
    for (int32_t c = 0; c < D; c++) out[n * D + c] = 0.0;
    for (int64_t s = 0; s <= t; s++) {
      if (x[s] == -INFINITY) continue;
      const double w = exp(x[s] - mx);
      den += w;
      for (int32_t c = 0; c < D; c++) out[n * D + c] += w * bf(V[s * D + c]);
    }
    for (int32_t c = 0; c < D; c++) out[n * D + c] /= den;
    lse[n] = mx + log(den);
    free(use);
    free(x);
  }
  return rc ? PF_ERR_ARG : PF_OK;
}
