/*
 * CPU oracle for sparse paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
 * CPU-baseline leg call this file; the product library (libspa.so) never
 * does, and the two share no code, header or table.
 *
 * Everything here works on plain logical-order arrays: a head's keys and
 * values are K[t][c], V[t][c] for positions t = 0..L-1 -- no pool, no page
 * table. bf16 numbers are passed as their 16-bit patterns.
 *
 * Precision: attention is computed in fp64. A page score is the correctly
 * rounded fp32 value of an exactly computed sum (integer arithmetic), which is
 * the definition the GPU approximates with fp64 accumulation.
 *
 * Sources (page title and section; PAGE = the LServe write-up at bqwf.cn,
 * "LServe长序列LLM服务系统"; LCI = the long-context inference survey at
 * xllm-io.github.io, "大语言模型长上下文推理优化"):
 *   PAGE "2.1 混合稀疏注意力机制": streaming heads keep local context; dynamic
 *       heads keep a token budget chosen by query-to-(min-max pooled block)
 *       similarity.
 *   PAGE "2.2 分层分页KV缓存": logical pages (selection unit) inside physical
 *       pages (allocation unit).
 *   PAGE "3.2 解码阶段加速": reuse the page selection for C steps; budget =
 *       min(4096, L/32).
 *   LCI "2.3 分组查询注意力 (GQA)": query head i uses KV head i/G; logits are
 *       divided by sqrt(head_dim); softmax over the keys.
 *   LCI sparse-method table (StreamingLLM row): attention sink + local window.
 *   PAGE "5.2 参数调优指南" and the long-text article at lshu.cn, "4.2 KV Cache
 *       Quantization（INT8/FP8）": K and V kept in fp8 (E4M3); the scale
 *       convention is this file's reading (see the fp8 section).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1      /* bad argument */
#define ORC_ERR_NONFINITE 2/* an input is Inf or NaN */
#define ORC_ERR_RANGE 3    /* exact score sum outside what this code handles */

/* ------------------------------------------------------------------ bf16 */

/* Value of a bf16 bit pattern: the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int bf16_finite(uint16_t b) { return ((b >> 7) & 0xFF) != 0xFF; }

/* a < b in IEEE totalOrder restricted to finite values: by value, and
 * -0 before +0. */
static int bf16_less(uint16_t a, uint16_t b) {
  double x = orc_bf16_value(a), y = orc_bf16_value(b);
  if (x != y) return x < y;
  return (a & 0x8000) && !(b & 0x8000);
}

/* --------------------------------------------------------- budget rule */

/* PAGE "3.2": dynamic budget = min(4096, sequence length / 32). */
int32_t orc_budget_tokens(int64_t L) {
  int64_t b = L / 32;
  return (int32_t)(b < 4096 ? b : 4096);
}

/* Pages a dynamic head keeps: the budget in tokens divided by the logical
 * page size, at least one page, at most all n pages. */
int64_t orc_pages_to_select(int64_t n, int64_t budget, int32_t p) {
  int64_t k = budget / p;
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

/* ------------------------------------------------------- page summaries */

/* PAGE "2.1": min-max pooling of each block. Logical page j covers positions
 * [j*p, min(j*p + p, L)); kmin/kmax[j][c] are the channel-wise min and max of
 * the keys there. K is [L][D]; kmin, kmax are [ceil(L/p)][D]. */
int orc_page_summary(const uint16_t* K, int64_t L, int32_t D, int32_t p,
                     uint16_t* kmin, uint16_t* kmax) {
  if (!K || !kmin || !kmax || L < 0 || D < 1 || p < 1) return ORC_ERR_ARG;
  int64_t n = (L + p - 1) / p;
  for (int64_t j = 0; j < n; j++) {
    int64_t t0 = j * p, t1 = t0 + p < L ? t0 + p : L;
    for (int32_t c = 0; c < D; c++) {
      uint16_t lo = K[t0 * D + c], hi = lo;
      if (!bf16_finite(lo)) return ORC_ERR_NONFINITE;
      for (int64_t t = t0 + 1; t < t1; t++) {
        uint16_t v = K[t * D + c];
        if (!bf16_finite(v)) return ORC_ERR_NONFINITE;
        if (bf16_less(v, lo)) lo = v;
        if (bf16_less(hi, v)) hi = v;
      }
      kmin[j * D + c] = lo;
      kmax[j * D + c] = hi;
    }
  }
  return ORC_OK;
}

/* -------------------------------------------------------- exact scores */

/* A finite bf16 value as sig * 2^ex with sig an integer, |sig| < 256. */
static void bf16_split(uint16_t b, int32_t* sig, int32_t* ex) {
  int32_t e = (b >> 7) & 0xFF, m = b & 0x7F;
  if (e == 0) { *sig = m; *ex = -133; }          /* subnormal: m * 2^-133 */
  else { *sig = 128 + m; *ex = e - 134; }        /* (1 + m/128) * 2^(e-127) */
  if (b & 0x8000) *sig = -*sig;
}

/* Round sig * 2^ex (sig an exact integer) to the nearest binary32, ties to
 * even. Only results in the normal binary32 range (or exactly zero) are
 * handled; anything else is reported. */
static int round_to_f32(__int128 sig, int32_t ex, float* out) {
  if (sig == 0) { *out = 0.0f; return ORC_OK; }
  int neg = sig < 0;
  unsigned __int128 a = neg ? (unsigned __int128)(-sig) : (unsigned __int128)sig;
  int nb = 0;
  for (unsigned __int128 t = a; t; t >>= 1) nb++;         /* a in [2^(nb-1), 2^nb) */
  if (nb > 24) {
    int sh = nb - 24;
    unsigned __int128 q = a >> sh;
    unsigned __int128 r = a - (q << sh);
    unsigned __int128 half = (unsigned __int128)1 << (sh - 1);
    if (r > half || (r == half && (q & 1))) q++;
    if (q == ((unsigned __int128)1 << 24)) { q >>= 1; sh++; }
    a = q;
    ex += sh;
  }
  /* a < 2^24 is exact in binary32; value = a * 2^ex */
  int top = ex + (nb > 24 ? 23 : nb - 1);                   /* exponent of the leading bit */
  if (top < -126 || top > 127) return ORC_ERR_RANGE;
  float f = ldexpf((float)a, ex);
  *out = neg ? -f : f;
  return ORC_OK;
}

/* RN32 of sum_c max(q[c] * kmax[c], q[c] * kmin[c]), the sum taken exactly. */
static int exact_bound_score(const uint16_t* q, const uint16_t* kmin,
                             const uint16_t* kmax, int32_t D, float* out) {
  int32_t sig[512], ex[512];
  if (D > 512) return ORC_ERR_ARG;
  int32_t emin = INT32_MAX, emax = INT32_MIN;
  for (int32_t c = 0; c < D; c++) {
    int32_t qs, qe, as, ae, bs, be;
    bf16_split(q[c], &qs, &qe);
    bf16_split(kmax[c], &as, &ae);
    bf16_split(kmin[c], &bs, &be);
    /* both products are exact in fp64 (16-bit significands), so comparing
       them as doubles is exact */
    double pa = ldexp((double)qs * as, qe + ae);
    double pb = ldexp((double)qs * bs, qe + be);
    if (pa >= pb) { sig[c] = qs * as; ex[c] = qe + ae; }
    else { sig[c] = qs * bs; ex[c] = qe + be; }
    if (sig[c] != 0) {
      if (ex[c] < emin) emin = ex[c];
      if (ex[c] > emax) emax = ex[c];
    }
  }
  if (emin == INT32_MAX) { *out = 0.0f; return ORC_OK; }
  /* |sig| < 2^16 and at most 512 terms: shifts up to 100 keep the sum below
     2^125 */
  if (emax - emin > 100) return ORC_ERR_RANGE;
  __int128 acc = 0;
  for (int32_t c = 0; c < D; c++)
    if (sig[c] != 0) acc += (__int128)sig[c] * ((__int128)1 << (ex[c] - emin));
  return round_to_f32(acc, emin, out);
}

/* PAGE "2.1": query-aware page importance from the min-max summaries, taken
 * as the largest q.k any key inside the page's min/max box can reach; with a
 * query group (GQA) the page keeps the largest of its queries' scores.
 *   q: [G][D]; kmin, kmax: [n][D]; scores: [n]. */
int orc_page_scores(const uint16_t* q, int32_t G, int32_t D,
                    const uint16_t* kmin, const uint16_t* kmax, int64_t n,
                    float* scores) {
  if (!q || !kmin || !kmax || !scores || G < 1 || D < 1 || n < 0) return ORC_ERR_ARG;
  for (int64_t i = 0; i < (int64_t)G * D; i++)
    if (!bf16_finite(q[i])) return ORC_ERR_NONFINITE;
  for (int64_t j = 0; j < n; j++) {
    float best = 0.0f;
    for (int32_t g = 0; g < G; g++) {
      float s;
      int rc = exact_bound_score(q + (int64_t)g * D, kmin + j * D, kmax + j * D, D, &s);
      if (rc) return rc;
      if (g == 0 || s > best) best = s;
    }
    scores[j] = best;
  }
  return ORC_OK;
}

/* ----------------------------------------------------------------- top-k */

typedef struct { float score; int32_t id; } scored_page;

/* (score descending, page id ascending) */
static int better_first(const void* pa, const void* pb) {
  const scored_page* a = (const scored_page*)pa;
  const scored_page* b = (const scored_page*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->id > b->id) - (a->id < b->id);
}
static int ascending(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* The k pages first in the order (score descending, page id ascending),
 * written in ascending page id. */
int orc_topk(const float* scores, int64_t n, int64_t k, int32_t* ids_out) {
  if (!scores || !ids_out || n < 0 || k < 0 || k > n) return ORC_ERR_ARG;
  scored_page* order = (scored_page*)malloc(sizeof(scored_page) * (size_t)(n ? n : 1));
  if (!order) return ORC_ERR_ARG;
  for (int64_t j = 0; j < n; j++) { order[j].score = scores[j]; order[j].id = (int32_t)j; }
  qsort(order, (size_t)n, sizeof(scored_page), better_first);
  for (int64_t i = 0; i < k; i++) ids_out[i] = order[i].id;
  qsort(ids_out, (size_t)k, sizeof(int32_t), ascending);
  free(order);
  return ORC_OK;
}

/* -------------------------------------------------------- attended sets */

/* mask[t] = 1 for every position t < L the head attends, else 0; returns
 * the number of attended positions.
 *   streaming (dynamic == 0): [0, min(sink, L)) U [max(sink, L - window), L)
 *   dynamic: positions in the selected logical pages, plus every position
 *            appended since the selection was made, [Ls, L). */
int64_t orc_attended_set(int32_t dynamic, int64_t L, int32_t sink, int32_t window,
                         int32_t p, const int32_t* sel, int64_t nsel, int64_t Ls,
                         uint8_t* mask) {
  if (!mask || L < 0) return -1;
  memset(mask, 0, (size_t)L);
  if (!dynamic) {
    int64_t s = sink < L ? sink : L;
    int64_t w0 = L - window > sink ? L - window : sink;
    for (int64_t t = 0; t < s; t++) mask[t] = 1;
    for (int64_t t = w0; t < L; t++) mask[t] = 1;
  } else {
    for (int64_t i = 0; i < nsel; i++)
      for (int64_t t = (int64_t)sel[i] * p; t < (int64_t)sel[i] * p + p && t < L; t++)
        if (t >= 0) mask[t] = 1;
    for (int64_t t = Ls < 0 ? 0 : Ls; t < L; t++) mask[t] = 1;
  }
  int64_t cnt = 0;
  for (int64_t t = 0; t < L; t++) cnt += mask[t];
  return cnt;
}

/* ------------------------------------------------------------- attention */

/* LCI "2.3": softmax over q.K_t / sqrt(D), weights applied to V_t; only the
 * masked positions take part. out[D] and lse (natural log of the softmax
 * denominator) in fp64. An empty set gives out = 0, lse = -inf. */
int orc_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V,
               int64_t L, int32_t D, const uint8_t* mask, double* out, double* lse) {
  if (!q || !K || !V || !mask || !out || !lse || L < 0 || D < 1) return ORC_ERR_ARG;
  double* x = (double*)malloc(sizeof(double) * (size_t)(L ? L : 1));
  if (!x) return ORC_ERR_ARG;
  double m = -INFINITY;
  for (int64_t t = 0; t < L; t++) {
    if (!mask[t]) continue;
    double dot = 0.0;
    for (int32_t c = 0; c < D; c++) dot += orc_bf16_value(q[c]) * orc_bf16_value(K[t * D + c]);
    x[t] = dot / sqrt((double)D);
    if (x[t] > m) m = x[t];
  }
  for (int32_t c = 0; c < D; c++) out[c] = 0.0;
  if (m == -INFINITY) { *lse = -INFINITY; free(x); return ORC_OK; }
  double den = 0.0;
  for (int64_t t = 0; t < L; t++) {
    if (!mask[t]) continue;
    double w = exp(x[t] - m);
    den += w;
    for (int32_t c = 0; c < D; c++) out[c] += w * orc_bf16_value(V[t * D + c]);
  }
  for (int32_t c = 0; c < D; c++) out[c] /= den;
  *lse = m + log(den);
  free(x);
  return ORC_OK;
}

/* ------------------------------------------------------ one head, one step */

/* One decode step of one (sequence, KV head) pair, in the method's order:
 *   dynamic head and do_select: page summaries -> page scores -> keep the
 *   top pages under the budget, remember L as the selection length Ls;
 *   dynamic head otherwise: keep sel / nsel / Ls from the previous step
 *   (PAGE "3.2", selector reuse);
 *   then attend each of the G query heads over the head's token set.
 * Arguments
 *   K, V [L][D]; q [G][D]
 *   sel: in/out, capacity sel_cap; nsel, Ls: in/out
 *   scores: NULL or [ceil(L/p)], receives the page scores on selection
 *   out [G][D], lse [G]: fp64 results */
int orc_decode_head(const uint16_t* K, const uint16_t* V, const uint16_t* q,
                    int64_t L, int32_t D, int32_t G, int32_t dynamic,
                    int32_t sink, int32_t window, int32_t p, int64_t budget,
                    int32_t do_select, int32_t* sel, int64_t sel_cap,
                    int64_t* nsel, int64_t* Ls, float* scores,
                    double* out, double* lse) {
  if (!K || !V || !q || !out || !lse || L < 1 || D < 1 || G < 1 || p < 1) return ORC_ERR_ARG;
  int rc = ORC_OK;
  if (dynamic && do_select) {
    if (!sel || !nsel || !Ls) return ORC_ERR_ARG;
    int64_t n = (L + p - 1) / p;
    uint16_t* kmin = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * D));
    uint16_t* kmax = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * D));
    float* s = scores ? scores : (float*)malloc(sizeof(float) * (size_t)n);
    if (!kmin || !kmax || !s) rc = ORC_ERR_ARG;
    if (!rc) rc = orc_page_summary(K, L, D, p, kmin, kmax);
    if (!rc) rc = orc_page_scores(q, G, D, kmin, kmax, n, s);
    int64_t k = orc_pages_to_select(n, budget, p);
    if (!rc && k > sel_cap) rc = ORC_ERR_ARG;
    if (!rc) rc = orc_topk(s, n, k, sel);
    if (!rc) { *nsel = k; *Ls = L; }
    free(kmin);
    free(kmax);
    if (!scores) free(s);
    if (rc) return rc;
  }
  uint8_t* mask = (uint8_t*)malloc((size_t)L);
  if (!mask) return ORC_ERR_ARG;
  if (orc_attended_set(dynamic, L, sink, window, p, sel, dynamic ? *nsel : 0,
                       dynamic ? *Ls : L, mask) < 0) rc = ORC_ERR_ARG;
  for (int32_t g = 0; g < G && !rc; g++)
    rc = orc_attend(q + (int64_t)g * D, K, V, L, D, mask, out + (int64_t)g * D, lse + g);
  free(mask);
  return rc;
}

/* ------------------------------------------------------------ fp8 pages */

/* PAGE "5.2 参数调优指南" sets the KV cache precision to fp8, and the
 * long-text article at lshu.cn ("4.2 KV Cache Quantization（INT8/FP8）")
 * keeps K and V in the FP8 E4M3 format; neither fixes the scale. The reading
 * taken here: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities, S.1111.111 is NaN, largest finite 448), one fp32 scale
 * per (token, head) row, scale = amax / 448 in fp32, code = the value x / scale
 * (fp32 division) rounded to the nearest E4M3 value, ties to even, saturating
 * at +-448. A row of zeros has scale 0 and all codes +0. The dequantized value
 * is code value x scale. */

/* Value of an E4M3 code (NaN for the two NaN codes). */
double orc_e4m3_value(uint8_t code) {
  int32_t e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);          /* subnormal: m/8 * 2^-6 */
  else v = ldexp((double)(8 + m), e - 10);      /* (1 + m/8) * 2^(e-7) */
  return (code & 0x80) ? -v : v;
}

/* Nearest E4M3 code of a finite x, ties to even, saturating. */
static uint8_t e4m3_encode(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: integer multiples of 2^-9; 8 * 2^-9 is the smallest
     * normal, whose code is also 8 */
    return sign | (uint8_t)nearbyint(ldexp(a, 9));
  }
  int32_t k;
  frexp(a, &k);                                  /* a = f * 2^k, f in [0.5, 1) */
  int32_t E = k - 1;                             /* a in [2^E, 2^(E+1)) */
  int32_t m = (int32_t)nearbyint((ldexp(a, -E) - 1.0) * 8.0);
  if (m == 8) { E += 1; m = 0; }
  return sign | (uint8_t)(((E + 7) << 3) | m);
}

/* Codes of n fp32 values; a non-finite value is an error. */
int orc_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
  if (!x || !out || n < 0) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; i++) {
    if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
    out[i] = e4m3_encode((double)x[i]);
  }
  return ORC_OK;
}

/* Quantizes L rows of D bf16 values (X [L][D]) into codes [L][D] and one
 * scale per row, as stated above. */
int orc_quantize_rows(const uint16_t* X, int64_t L, int32_t D, uint8_t* codes,
                      float* scales) {
  if (!X || !codes || !scales || L < 0 || D < 1) return ORC_ERR_ARG;
  for (int64_t t = 0; t < L; t++) {
    float amax = 0.0f;
    for (int32_t c = 0; c < D; c++) {
      uint16_t b = X[t * D + c];
      if (!bf16_finite(b)) return ORC_ERR_NONFINITE;
      float a = (float)fabs(orc_bf16_value(b));  /* exact: a bf16 is an fp32 */
      if (a > amax) amax = a;
    }
    volatile float s = amax / 448.0f;            /* one fp32 division */
    scales[t] = s;
    for (int32_t c = 0; c < D; c++) {
      if (s == 0.0f) { codes[t * D + c] = 0; continue; }
      volatile float y = (float)orc_bf16_value(X[t * D + c]) / s;
      codes[t * D + c] = e4m3_encode((double)y);
    }
  }
  return ORC_OK;
}

/* Largest bf16 <= x (x finite, within the bf16 range). */
static uint16_t bf16_down(double x) {
  float f = (float)x;
  if ((double)f > x) f = nextafterf(f, -INFINITY);   /* largest fp32 <= x */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t b = (uint16_t)(u >> 16);                  /* toward zero */
  if ((u & 0xFFFF) && (u & 0x80000000u)) b += 1;     /* negative: one more step down */
  return b;
}

/* Smallest bf16 >= x. */
static uint16_t bf16_up(double x) { return bf16_down(-x) ^ 0x8000; }

/* Bit patterns of bf16_down / bf16_up of n doubles (dir < 0: down, else up). */
int orc_bf16_round_outward(const double* x, int64_t n, int32_t dir, uint16_t* out) {
  if (!x || !out || n < 0) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; i++) {
    if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
    out[i] = dir < 0 ? bf16_down(x[i]) : bf16_up(x[i]);
  }
  return ORC_OK;
}

/* Dequantized element t, c of a code matrix [L][D] with row scales. */
static double q8_value(const uint8_t* codes, const float* scales, int64_t t, int32_t D,
                       int32_t c) {
  return orc_e4m3_value(codes[t * D + c]) * (double)scales[t];   /* exact in fp64 */
}

/* PAGE "2.1" min-max pooling over the dequantized keys of fp8 pages: the
 * channel-wise min and max of each logical page, computed exactly in IEEE
 * totalOrder (-0 below +0, the order of the bf16 summaries), then rounded
 * outward to bf16 (min down, max up), so that a bf16 summary still bounds
 * every key of its page. Rounding outward is monotone in that order, so a
 * page's summary after one more key is the min / max of its summary before
 * and the new key rounded outward. */
int orc_page_summary_q8(const uint8_t* Kc, const float* Ks, int64_t L, int32_t D,
                        int32_t p, uint16_t* kmin, uint16_t* kmax) {
  if (!Kc || !Ks || !kmin || !kmax || L < 0 || D < 1 || p < 1) return ORC_ERR_ARG;
  int64_t n = (L + p - 1) / p;
  for (int64_t j = 0; j < n; j++) {
    int64_t t0 = j * p, t1 = t0 + p < L ? t0 + p : L;
    for (int32_t c = 0; c < D; c++) {
      double lo = INFINITY, hi = -INFINITY;
      for (int64_t t = t0; t < t1; t++) {
        double v = q8_value(Kc, Ks, t, D, c);
        if (!isfinite(v)) return ORC_ERR_NONFINITE;
        if (v < lo || (v == lo && signbit(v))) lo = v;        /* -0 below +0 */
        if (v > hi || (v == hi && !signbit(v))) hi = v;
      }
      kmin[j * D + c] = bf16_down(lo);
      kmax[j * D + c] = bf16_up(hi);
    }
  }
  return ORC_OK;
}

/* orc_attend over fp8 pages: the same softmax attention, with K_t and V_t the
 * dequantized rows. */
int orc_attend_q8(const uint16_t* q, const uint8_t* Kc, const float* Ks,
                  const uint8_t* Vc, const float* Vs, int64_t L, int32_t D,
                  const uint8_t* mask, double* out, double* lse) {
  if (!q || !Kc || !Ks || !Vc || !Vs || !mask || !out || !lse || L < 0 || D < 1)
    return ORC_ERR_ARG;
  double* x = (double*)malloc(sizeof(double) * (size_t)(L ? L : 1));
  if (!x) return ORC_ERR_ARG;
  double m = -INFINITY;
  for (int64_t t = 0; t < L; t++) {
    if (!mask[t]) continue;
    double dot = 0.0;
    for (int32_t c = 0; c < D; c++) dot += orc_bf16_value(q[c]) * q8_value(Kc, Ks, t, D, c);
    x[t] = dot / sqrt((double)D);
    if (x[t] > m) m = x[t];
  }
  for (int32_t c = 0; c < D; c++) out[c] = 0.0;
  if (m == -INFINITY) { *lse = -INFINITY; free(x); return ORC_OK; }
  double den = 0.0;
  for (int64_t t = 0; t < L; t++) {
    if (!mask[t]) continue;
    double w = exp(x[t] - m);
    den += w;
    for (int32_t c = 0; c < D; c++) out[c] += w * q8_value(Vc, Vs, t, D, c);
  }
  for (int32_t c = 0; c < D; c++) out[c] /= den;
  *lse = m + log(den);
  free(x);
  return ORC_OK;
}

/* orc_decode_head over fp8 pages: summaries from orc_page_summary_q8, then the
 * same scores, top-k, token set and attention (orc_attend_q8). */
int orc_decode_head_q8(const uint8_t* Kc, const float* Ks, const uint8_t* Vc,
                       const float* Vs, const uint16_t* q, int64_t L, int32_t D,
                       int32_t G, int32_t dynamic, int32_t sink, int32_t window,
                       int32_t p, int64_t budget, int32_t do_select, int32_t* sel,
                       int64_t sel_cap, int64_t* nsel, int64_t* Ls, float* scores,
                       double* out, double* lse) {
  if (!Kc || !Ks || !Vc || !Vs || !q || !out || !lse || L < 1 || D < 1 || G < 1 || p < 1)
    return ORC_ERR_ARG;
  int rc = ORC_OK;
  if (dynamic && do_select) {
    if (!sel || !nsel || !Ls) return ORC_ERR_ARG;
    int64_t n = (L + p - 1) / p;
    uint16_t* kmin = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * D));
    uint16_t* kmax = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * D));
    float* s = scores ? scores : (float*)malloc(sizeof(float) * (size_t)n);
    if (!kmin || !kmax || !s) rc = ORC_ERR_ARG;
    if (!rc) rc = orc_page_summary_q8(Kc, Ks, L, D, p, kmin, kmax);
    if (!rc) rc = orc_page_scores(q, G, D, kmin, kmax, n, s);
    int64_t k = orc_pages_to_select(n, budget, p);
    if (!rc && k > sel_cap) rc = ORC_ERR_ARG;
    if (!rc) rc = orc_topk(s, n, k, sel);
    if (!rc) { *nsel = k; *Ls = L; }
    free(kmin);
    free(kmax);
    if (!scores) free(s);
    if (rc) return rc;
  }
  uint8_t* mask = (uint8_t*)malloc((size_t)L);
  if (!mask) return ORC_ERR_ARG;
  if (orc_attended_set(dynamic, L, sink, window, p, sel, dynamic ? *nsel : 0,
                       dynamic ? *Ls : L, mask) < 0) rc = ORC_ERR_ARG;
  for (int32_t g = 0; g < G && !rc; g++)
    rc = orc_attend_q8(q + (int64_t)g * D, Kc, Ks, Vc, Vs, L, D, mask,
                       out + (int64_t)g * D, lse + g);
  free(mask);
  return rc;
}

/* ------------------------------------------------------ many heads at once */

/* One orc_decode_head call; rc receives its status. */
typedef struct orc_job {
  const uint16_t *K, *V, *q;
  int64_t L;
  int32_t D, G, dynamic, sink, window, p;
  int64_t budget;
  int32_t do_select;
  int32_t* sel;
  int64_t sel_cap;
  int64_t* nsel;
  int64_t* Ls;
  float* scores;
  double* out;
  double* lse;
  int32_t rc;
} orc_job;

/* Runs independent jobs, in parallel over the host's cores when built with
 * OpenMP. Returns the number of jobs that failed. */
int32_t orc_decode_heads(int32_t njobs, orc_job* jobs) {
  int32_t failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : failed)
  for (int32_t i = 0; i < njobs; i++) {
    orc_job* j = &jobs[i];
    j->rc = orc_decode_head(j->K, j->V, j->q, j->L, j->D, j->G, j->dynamic, j->sink,
                            j->window, j->p, j->budget, j->do_select, j->sel, j->sel_cap,
                            j->nsel, j->Ls, j->scores, j->out, j->lse);
    failed += j->rc != 0;
  }
  return failed;
}

/* Threads the parallel loop above uses (1 without OpenMP). */
int32_t orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
