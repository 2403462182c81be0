/*
 * Plain CPU oracle for one RTPurbo decode step.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no code, header or constant
 * with the HIP library: it is written from the method's definitions, single
 * threaded, with plain loops and no blocking, fusion or reordering.
 *
 * Source: "Full Attention Strikes Back: Transferring Full Attention into Sparse
 * within Hundred Training Steps" (xllm-io.github.io paper review), section 三
 * 技术架构:
 *   - 核心公式 / 自适应稀疏注意力, first equation: the indexer score
 *     s_h(m,n) = (W^Q_h q^pre)^T (W^K_h k^pre), computed on projected 16-dim
 *     features before RoPE;
 *   - same paragraph, second equation: O_h(m) is the softmax-weighted sum of v_n
 *     over n in S_h(m) = Top-P(s_h(m,.), p), logits q^T k_n / sqrt(d_h);
 *   - 硬件感知解码内核: top-p without sorting, through a 256-bin histogram of
 *     1 KB per head, independent of the sequence length.
 * The gist.science technical summary (section 3, "Dynamic Top-p Selection")
 * states the top-p semantics: mass is accumulated until the cumulative
 * threshold p is reached.
 *
 * The pages leave the histogram's bins open.  The reading implemented here
 * (fixed-width logit cells of width w anchored at the top occupied cell, a
 * catch-all last bin, softmax mass per bin, the whole threshold bin kept) is
 * the one the rest of the pages support: it returns a superset of exact top-p
 * whose mass is at least p.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math, no contraction:
 * every fused multiply-add below is an explicit fmaf call).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_NBINS 256

/* IEEE 754 binary16 bit pattern -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double rtpo_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);   /* (1024 + m) * 2^(e - 15 - 10) */
  return sign ? -v : v;
}

static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F16) return rtpo_half_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* Indexer score for one query head over L cached tokens.
 *   a_n = fp32 fused-multiply-add chain over i = 0..r-1, starting from +0:
 *         a <- fmaf(q_idx[i], k_idx[n][i], a)
 *   z_n = fl32(scale * a_n)
 * k_idx values (fp16 or fp32) convert to fp32 exactly. */
void rtpo_index_score(const float* q_idx, const void* k_idx, int k_dtype, int64_t L, int r,
                      float scale, float* z) {
  for (int64_t n = 0; n < L; n++) {
    float a = 0.0f;
    for (int i = 0; i < r; i++) {
      float k = (float)elem(k_idx, k_dtype, n * r + i);
      a = fmaf(q_idx[i], k, a);
    }
    z[n] = scale * a;
  }
}

/* Indexer projection of one head's pre-RoPE feature vector (section 三, 核心公式: the
 * indexer compares W^Q_h q^pre with W^K_h k^pre, projected to r dims before RoPE).
 * W is stored [d][r] (column i maps x to feature i):
 *   out[i] = fp32 fused-multiply-add chain over c = 0..d-1, starting from +0:
 *            a <- fmaf(x[c], W[c][i], a)                                          */
void rtpo_project(const float* x, const float* W, int d, int r, float* out) {
  for (int i = 0; i < r; i++) {
    float a = 0.0f;
    for (int c = 0; c < d; c++) a = fmaf(x[c], W[c * r + i], a);
    out[i] = a;
  }
}

/* bfloat16 rounding, from the format: 8 significant bits (7 stored) with fp32's exponent
 * range, round to nearest with ties to even; below 2^-126 the spacing is fixed at 2^-133
 * (subnormals).  Returns the rounded value. */
double rtpo_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  const double ax = fabs(x);
  double r;
  if (ax < ldexp(1.0, -126)) {
    r = nearbyint(ax * ldexp(1.0, 133)) * ldexp(1.0, -133);
  } else {
    int e;
    const double m = frexp(ax, &e);          /* ax = m 2^e, m in [0.5, 1) */
    r = ldexp(nearbyint(ldexp(m, 8)), e - 8); /* 8 significant bits, ties to even */
  }
  return x < 0 ? -r : r;
}

/* Cell of a logit on the global grid of width w (w a power of two). */
static int64_t cell_of(float z, double w) { return (int64_t)floor((double)z / w); }

/* Histogram top-p rule for one query head.
 *   g_n = floor(z_n / w);  A = max_n g_n;  j_n = min(A - g_n, 255)
 *   mu_j = sum over n with j_n = j of exp(z_n - (A + 1) w)        (fp64)
 *   Z = sum_j mu_j;  b* = 255 if p >= 1, else the least j with mu_0 + .. + mu_j >= p Z
 *   S = { n : j_n <= b* }, ascending.
 * Writes hist[256], *A_out, *bstar_out and sel[0 .. |S|-1]; returns |S|. */
int64_t rtpo_topp_select(const float* z, int64_t L, double p, double w, int32_t* sel,
                         double* hist, int64_t* A_out, int32_t* bstar_out) {
  int64_t A = INT64_MIN;
  for (int64_t n = 0; n < L; n++) {
    int64_t g = cell_of(z[n], w);
    if (g > A) A = g;
  }
  for (int j = 0; j < ORACLE_NBINS; j++) hist[j] = 0.0;
  double ref = (double)(A + 1) * w;
  for (int64_t n = 0; n < L; n++) {
    int64_t j = A - cell_of(z[n], w);
    if (j > ORACLE_NBINS - 1) j = ORACLE_NBINS - 1;
    hist[j] += exp((double)z[n] - ref);
  }
  double Zsum = 0.0;
  for (int j = 0; j < ORACLE_NBINS; j++) Zsum += hist[j];
  int32_t b = ORACLE_NBINS - 1;
  if (p < 1.0) {
    double c = 0.0;
    for (int j = 0; j < ORACLE_NBINS; j++) {
      c += hist[j];
      if (c >= p * Zsum) { b = j; break; }
    }
  }
  int64_t cnt = 0;
  for (int64_t n = 0; n < L; n++) {
    int64_t j = A - cell_of(z[n], w);
    if (j > ORACLE_NBINS - 1) j = ORACLE_NBINS - 1;
    if (j <= b) sel[cnt++] = (int32_t)n;
  }
  *A_out = A;
  *bstar_out = b;
  return cnt;
}

/* Fixed top-k through the same histogram (the pages' comparison of fixed budgets with
 * top-p: section 三, insight 3 and its top-k vs top-p table).  The bins are those of
 * rtpo_topp_select; each token weighs one instead of its softmax mass:
 *   c_j = #{ n : j_n = j };  b* = the least j with c_0 + .. + c_j >= k, or 255 when the
 *   whole sequence holds fewer than k tokens;  S = { n : j_n <= b* }, ascending.
 * S holds at least min(k, L) tokens and contains the k highest logits (ties at the k-th
 * value included), because the bins are whole cells in logit order.
 * Writes hist[256] (the counts), *A_out, *bstar_out and sel; returns |S|. */
int64_t rtpo_topk_select(const float* z, int64_t L, int64_t k, double w, int32_t* sel,
                         double* hist, int64_t* A_out, int32_t* bstar_out) {
  int64_t A = INT64_MIN;
  for (int64_t n = 0; n < L; n++) {
    int64_t g = cell_of(z[n], w);
    if (g > A) A = g;
  }
  for (int j = 0; j < ORACLE_NBINS; j++) hist[j] = 0.0;
  for (int64_t n = 0; n < L; n++) {
    int64_t j = A - cell_of(z[n], w);
    if (j > ORACLE_NBINS - 1) j = ORACLE_NBINS - 1;
    hist[j] += 1.0;
  }
  int32_t b = ORACLE_NBINS - 1;
  double c = 0.0;
  for (int j = 0; j < ORACLE_NBINS; j++) {
    c += hist[j];
    if (c >= (double)k) { b = j; break; }
  }
  int64_t cnt = 0;
  for (int64_t n = 0; n < L; n++) {
    int64_t j = A - cell_of(z[n], w);
    if (j > ORACLE_NBINS - 1) j = ORACLE_NBINS - 1;
    if (j <= b) sel[cnt++] = (int32_t)n;
  }
  *A_out = A;
  *bstar_out = b;
  return cnt;
}

/* Exact softmax attention over a list of rows, in fp64.
 *   s_i = scale * sum_c q[c] K[row_i][c];  m = max_i s_i
 *   out[c] = sum_i e^{s_i - m} V[row_i][c] / sum_i e^{s_i - m};  lse = m + log(sum_i e^{s_i - m})
 * K and V point at the first row of the head (row stride d elements). */
void rtpo_attention(const double* q, const void* K, const void* V, int kv_dtype, int d,
                    const int64_t* rows, int64_t n, double scale, double* out, double* lse) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double m = -INFINITY;
  for (int64_t i = 0; i < n; i++) {
    double acc = 0.0;
    for (int c = 0; c < d; c++) acc += q[c] * elem(K, kv_dtype, rows[i] * d + c);
    s[i] = scale * acc;
    if (s[i] > m) m = s[i];
  }
  double den = 0.0;
  for (int c = 0; c < d; c++) out[c] = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double e = exp(s[i] - m);
    den += e;
    for (int c = 0; c < d; c++) out[c] += e * elem(V, kv_dtype, rows[i] * d + c);
  }
  for (int c = 0; c < d; c++) out[c] /= den;
  *lse = m + log(den);
  free(s);
}
