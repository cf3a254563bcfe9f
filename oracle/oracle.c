/*
 * CPU oracle of the routed MoE FFN layer — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this; the product path never does.  It shares no code, header, table
 * or constant with the HIP library.
 *
 * Plain loops, fp64 throughout, fixed ascending reduction order, built with
 * -ffp-contract=off so no multiply-add is fused (the pages' kimi-k3-in-c
 * engine pins its bits the same way: fixed summation order, no BLAS, no FMA
 * contraction — translated README, "why no BLAS" and build-flags sections).
 * OpenMP splits only independent outputs across threads; each output is
 * reduced by one thread in one order, so the thread count changes no bit.
 *
 * What is computed (one MoE FFN layer; the pages' routed experts are MXFP4,
 * "multiplied directly without dequantizing", 16 of 896 chosen per token,
 * plus 2 always-on shared experts — review page "KDA/MLA/MoE" table and
 * "at a glance" table; README "shard census"):
 *   logits[t][e] = sum_i x[t][i] * Wr[e][i]
 *   S_t          = the k experts with the largest logits (ties: lower id)
 *   w[t][e]      = exp(l_e - m) / sum_{j in S_t} exp(l_j - m), m = max over S_t
 *   per chosen (t, e):  g = Wg x,  u = Wu x,  h = silu(g) * u,  y = Wd h
 *   shared:      s = sum over shared experts in order of the same FFN (bf16 W)
 *   out[t]       = s[t] + sum over S_t in ascending expert id (w != 0) of w * y
 *
 * MXFP4 (the pages: 0.5 byte per E2M1 nibble + 1/32 byte of shared E8M0 scale
 * per weight, README "shard census"): element value = E2M1(code) * 2^(s-127).
 * Byte i of a packed row holds element 2i in its low nibble, 2i+1 in its high.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads an OpenMP region of the oracle uses. */
int oracle_threads(void) { return omp_get_max_threads(); }

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: 0.m * 2^0 = m * 0.5; otherwise
 * 2^(e-1) * (1 + m/2). */
double oracle_e2m1(int code) {
  int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* E8M0 (OCP MX v1.0): 2^(s-127); the all-ones byte encodes NaN. */
double oracle_e8m0(int s) {
  if (s == 255) return NAN;
  return ldexp(1.0, s - 127);
}

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Element (r, i) of a packed MXFP4 matrix with `cols` columns. */
static double mx_elem(const uint8_t* q, const uint8_t* s, int cols, int64_t r, int i) {
  uint8_t byte = q[r * (cols / 2) + i / 2];
  int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  return oracle_e2m1(code) * oracle_e8m0(s[r * (cols / 32) + i / 32]);
}

/* Decode rows [r0, r0 + nr) of a packed MXFP4 matrix to fp64 (exact). */
void oracle_mxfp4_decode(int64_t r0, int64_t nr, int cols, const uint8_t* q, const uint8_t* s,
                         double* out) {
  for (int64_t r = 0; r < nr; ++r)
    for (int i = 0; i < cols; ++i) out[r * cols + i] = mx_elem(q, s, cols, r0 + r, i);
}

/* logits[t][e] = sum_{i ascending} x[t][i] * Wr[e][i]; x is fp64 (exact copy of
 * bf16/fp32 inputs), Wr bf16. */
void oracle_router_logits(int64_t T, int d, int E, const double* x, const uint16_t* wr,
                          double* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += x[t * d + i] * bf16_value(wr[(int64_t)e * d + i]);
      logits[t * E + e] = acc;
    }
}

/* a ranks before b: larger logit first, equal logits by lower id. */
static int ranks_before(double la, int a, double lb, int b) {
  return la > lb || (la == lb && a < b);
}

/* Top-k by (logit desc, id asc); idx rows in ascending expert id; w aligned. */
void oracle_topk_softmax(int64_t T, int E, int k, const double* logits, int32_t* idx,
                         double* w) {
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)E);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double* l = logits + t * E;
      memset(taken, 0, (size_t)E);
      for (int r = 0; r < k; ++r) { /* r-th best among the not yet taken */
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || ranks_before(l[e], e, l[best], best))) best = e;
        taken[best] = 1;
        sel[r] = best;
      }
      double m = l[sel[0]];
      int pos = 0;
      for (int e = 0; e < E; ++e) /* ascending id */
        if (taken[e]) idx[t * k + pos++] = e;
      double z = 0.0;
      for (int r = 0; r < k; ++r) z += exp(l[idx[t * k + r]] - m);
      for (int r = 0; r < k; ++r) w[t * k + r] = exp(l[idx[t * k + r]] - m) / z;
    }
    free(taken);
    free(sel);
  }
}

/* The pages' K3 router (kimi-k3-in-c review page, "KDA/MLA/MoE" table: the
 * routing bias only bends the selection; the combine weights come from the
 * unbiased sigmoid scores):
 *   s[e]   = 1 / (1 + exp(-l[e]))                      (sigmoid score)
 *   S_t    = the k experts with the largest s[e] + bias[e] (ties: lower id)
 *   w[t][e] = s[e]                 (norm == 0), or
 *           = s[e] / sum_{j in S_t} s[j]   (norm != 0; the pages do not say
 *             whether the weights are renormalised, so both are offered)
 * bias may be NULL (no bias).  idx rows ascending, w aligned. */
static double sigmoid_score(double l) { return 1.0 / (1.0 + exp(-l)); }

void oracle_topk_sigmoid(int64_t T, int E, int k, const double* logits, const float* bias,
                         int norm, int32_t* idx, double* w) {
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)E);
    double* sel = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double* l = logits + t * E;
      for (int e = 0; e < E; ++e) sel[e] = sigmoid_score(l[e]) + (bias ? (double)bias[e] : 0.0);
      memset(taken, 0, (size_t)E);
      for (int r = 0; r < k; ++r) { /* r-th best selection score among the not taken */
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || ranks_before(sel[e], e, sel[best], best))) best = e;
        taken[best] = 1;
      }
      int pos = 0;
      for (int e = 0; e < E; ++e)
        if (taken[e]) idx[t * k + pos++] = e;
      double z = 0.0;
      for (int r = 0; r < k; ++r) z += sigmoid_score(l[idx[t * k + r]]);
      for (int r = 0; r < k; ++r) {
        double s = sigmoid_score(l[idx[t * k + r]]);
        w[t * k + r] = norm ? s / z : s;
      }
    }
    free(taken);
    free(sel);
  }
}

/* Counting sort of the T*k (token, slot) pairs by expert, stable in pair
 * order: counts[e], offsets[e] = sum_{e' < e} counts[e'] (E+1 entries),
 * sorted_pair[p] = t*k + slot of the p-th pair, pair_pos its inverse. */
void oracle_permute(int64_t T, int E, int k, const int32_t* idx, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos) {
  int64_t P = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[idx[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < P; ++p) {
    int e = idx[p];
    int32_t pos = offsets[e] + fill[e]++;
    sorted_pair[pos] = (int32_t)p;
    pair_pos[p] = pos;
  }
  free(fill);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One MXFP4 expert over n activation rows x [n][d]:
 *   g_j = sum_i Wg[j][i] x_i, u_j = sum_i Wu[j][i] x_i   (i ascending)
 *   h_j = silu(g_j) u_j
 *   y_o = sum_j Wd[o][j] h_j                             (j ascending)
 * w13 [2f][d/2] codes with w13s [2f][d/32] (rows 0..f-1 gate, f..2f-1 up);
 * w2 [d][f/2] with w2s [d][f/32].  h (optional, [n][f]) receives h. */
void oracle_mxfp4_ffn(int d, int f, const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                      const uint8_t* w2s, int64_t n, const double* x, double* y, double* h_out) {
  double* g = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* u = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* h = (double*)malloc(sizeof(double) * (size_t)(n * f));
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(d > f ? d : f));
#pragma omp for schedule(static)
    for (int j = 0; j < 2 * f; ++j) {
      oracle_mxfp4_decode(j, 1, d, w13, w13s, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += row[i] * x[r * d + i];
        if (j < f) g[r * f + j] = acc;
        else u[r * f + (j - f)] = acc;
      }
    }
#pragma omp for schedule(static)
    for (int64_t q = 0; q < n * f; ++q) h[q] = silu(g[q]) * u[q];
#pragma omp for schedule(static)
    for (int o = 0; o < d; ++o) {
      oracle_mxfp4_decode(o, 1, f, w2, w2s, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int j = 0; j < f; ++j) acc += row[j] * h[r * f + j];
        y[r * d + o] = acc;
      }
    }
    free(row);
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(n * f));
  free(g);
  free(u);
  free(h);
}

/* ---------------------------------------------------------------------------
 * Quantised-activation mode (not a method of the pages: they never quantise
 * activations — review page, "KDA/MLA/MoE" table; explainer page, "reduction
 * one".  It is the single-pass MXFP4 x MXFP4 form of the same FFN, checked
 * apart from the exact layer).  The quantiser is OCP MX v1.0's for MXFP4:
 *   X = max |v| over a 32-element block;
 *   shared exponent E = floor(log2 X) - 2   (2: exponent of E2M1's largest
 *     value, 6 = 1.5 * 2^2), so X / 2^E lies in [4, 8);
 *   scale byte = E + 127, clamped to [0, 254]; X = 0 gives byte 0;
 *   each element: the E2M1 value nearest to v / 2^s (s = byte - 127), ties
 *     to the code with an even mantissa bit, magnitudes above 6 saturating
 *     to 6; the sign is kept (a zero keeps its sign);
 *   a block holding a NaN or an infinity: scale byte 255 (NaN), codes 0.
 * Codes are packed as the weights are: byte i = element 2i (low nibble),
 * element 2i+1 (high nibble).
 * ------------------------------------------------------------------------- */
void oracle_quantize_mxfp4(int64_t nblk, const double* v, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < nblk; ++b) {
    const double* vb = v + b * 32;
    double X = 0.0;
    int bad = 0;
    for (int i = 0; i < 32; ++i) {
      if (!isfinite(vb[i])) bad = 1;
      else if (fabs(vb[i]) > X) X = fabs(vb[i]);
    }
    uint8_t* cb = codes + b * 16;
    if (bad) {
      scales[b] = 255;
      for (int i = 0; i < 16; ++i) cb[i] = 0;
      continue;
    }
    int byte = 0;
    if (X > 0.0) {
      int E = (int)floor(log2(X)) - 2;
      byte = E + 127;
      if (byte < 0) byte = 0;
      if (byte > 254) byte = 254;
    }
    scales[b] = (uint8_t)byte;
    double unit = ldexp(1.0, byte - 127);
    for (int i = 0; i < 32; ++i) {
      double a = fabs(vb[i]) / unit;
      int best = 0; /* code of the nearest magnitude (codes 0..7 are the magnitudes) */
      for (int c = 1; c < 8; ++c) {
        double dc = fabs(a - oracle_e2m1(c)), db = fabs(a - oracle_e2m1(best));
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
      }
      int code = best | (signbit(vb[i]) ? 8 : 0);
      if (i % 2 == 0) cb[i / 2] = (uint8_t)code;
      else cb[i / 2] |= (uint8_t)(code << 4);
    }
  }
}

/* Values of n rows of `cols` elements after MXFP4 quantisation (in place). */
static void quantize_rows(int64_t n, int cols, double* v) {
  int64_t nblk = n * (cols / 32);
  uint8_t* codes = (uint8_t*)malloc((size_t)nblk * 16);
  uint8_t* scales = (uint8_t*)malloc((size_t)nblk);
  oracle_quantize_mxfp4(nblk, v, codes, scales);
  for (int64_t b = 0; b < nblk; ++b)
    for (int i = 0; i < 32; ++i) {
      uint8_t byte = codes[b * 16 + i / 2];
      int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      v[b * 32 + i] = oracle_e2m1(code) * oracle_e8m0(scales[b]);
    }
  free(codes);
  free(scales);
}

/* The MXFP4 expert with quantised activations: x rows quantised to MXFP4,
 * g = Wg xq, u = Wu xq, h = silu(g) u, h rows quantised to MXFP4, y = Wd hq;
 * sums in fp64 in ascending order.  h_out (optional) receives hq. */
void oracle_mxfp4_ffn_qact(int d, int f, const uint8_t* w13, const uint8_t* w13s,
                           const uint8_t* w2, const uint8_t* w2s, int64_t n, const double* x,
                           double* y, double* h_out) {
  double* xq = (double*)malloc(sizeof(double) * (size_t)(n * d));
  memcpy(xq, x, sizeof(double) * (size_t)(n * d));
  quantize_rows(n, d, xq);
  double* g = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* u = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* h = (double*)malloc(sizeof(double) * (size_t)(n * f));
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(d > f ? d : f));
#pragma omp for schedule(static)
    for (int j = 0; j < 2 * f; ++j) {
      oracle_mxfp4_decode(j, 1, d, w13, w13s, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += row[i] * xq[r * d + i];
        if (j < f) g[r * f + j] = acc;
        else u[r * f + (j - f)] = acc;
      }
    }
    free(row);
  }
  for (int64_t q = 0; q < n * f; ++q) h[q] = silu(g[q]) * u[q];
  quantize_rows(n, f, h);
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(d > f ? d : f));
#pragma omp for schedule(static)
    for (int o = 0; o < d; ++o) {
      oracle_mxfp4_decode(o, 1, f, w2, w2s, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int j = 0; j < f; ++j) acc += row[j] * h[r * f + j];
        y[r * d + o] = acc;
      }
    }
    free(row);
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(n * f));
  free(xq);
  free(g);
  free(u);
  free(h);
}

/* ---------------------------------------------------------------------------
 * RVQ3 experts (WASTE article page, section "정확성 검증과 양자화": expert
 * weights in residual vector quantisation at 3.00 bits per weight, three
 * stages of 256-entry codebooks per 8-dimensional vector).  A matrix of
 * rows x cols has, for every row r and group g of 8 columns, three 8-bit
 * indices i_s[r][g]; its weights are
 *   W[r][8g + j] = C_0[i_0[r][g]][j] + C_1[i_1[r][g]][j] + C_2[i_2[r][g]][j]
 * with C_s [256][8] fp32 codebooks of the matrix.  Index layout (this
 * library's): idx[s][cols/128][rows][16], i.e. per stage, per slice of 16
 * groups, every row's 16 indices contiguous; codebooks cb[s][256][8].
 * ------------------------------------------------------------------------- */
static double rvq_elem(const uint8_t* idx, const float* cb, int64_t rows, int cols, int64_t r,
                       int c) {
  int g = c / 8, j = c % 8, sl = g / 16, gi = g % 16;
  double w = 0.0;
  for (int s = 0; s < 3; ++s) {
    uint8_t i = idx[(((int64_t)s * (cols / 128) + sl) * rows + r) * 16 + gi];
    w += (double)cb[((int64_t)s * 256 + i) * 8 + j];
  }
  return w;
}

/* Decode rows [r0, r0 + nr) of an RVQ3 matrix to fp64 (codeword sums in fp64). */
void oracle_rvq_decode(int64_t r0, int64_t nr, int64_t rows, int cols, const uint8_t* idx,
                       const float* cb, double* out) {
  for (int64_t r = 0; r < nr; ++r)
    for (int c = 0; c < cols; ++c) out[r * cols + c] = rvq_elem(idx, cb, rows, cols, r0 + r, c);
}

/* One RVQ3 expert over n activation rows: the same FFN as the MXFP4 expert,
 * g, u from w13 (rows 0..f-1 gate, f..2f-1 up), y from w2, fp64, ascending. */
void oracle_rvq_ffn(int d, int f, const uint8_t* w13i, const float* w13c, const uint8_t* w2i,
                    const float* w2c, int64_t n, const double* x, double* y, double* h_out) {
  double* g = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* u = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* h = (double*)malloc(sizeof(double) * (size_t)(n * f));
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(d > f ? d : f));
#pragma omp for schedule(static)
    for (int j = 0; j < 2 * f; ++j) {
      oracle_rvq_decode(j, 1, 2 * f, d, w13i, w13c, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += row[i] * x[r * d + i];
        if (j < f) g[r * f + j] = acc;
        else u[r * f + (j - f)] = acc;
      }
    }
#pragma omp for schedule(static)
    for (int64_t q = 0; q < n * f; ++q) h[q] = silu(g[q]) * u[q];
#pragma omp for schedule(static)
    for (int o = 0; o < d; ++o) {
      oracle_rvq_decode(o, 1, d, f, w2i, w2c, row);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int j = 0; j < f; ++j) acc += row[j] * h[r * f + j];
        y[r * d + o] = acc;
      }
    }
    free(row);
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(n * f));
  free(g);
  free(u);
  free(h);
}

/* One bf16 expert (the always-on shared experts): same FFN with
 * w13 [2f][d] and w2 [d][f] bf16. */
void oracle_bf16_ffn(int d, int f, const uint16_t* w13, const uint16_t* w2, int64_t n,
                     const double* x, double* y) {
  double* g = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* u = (double*)malloc(sizeof(double) * (size_t)(n * f));
  double* h = (double*)malloc(sizeof(double) * (size_t)(n * f));
#pragma omp parallel for schedule(static)
  for (int j = 0; j < 2 * f; ++j)
    for (int64_t r = 0; r < n; ++r) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += bf16_value(w13[(int64_t)j * d + i]) * x[r * d + i];
      if (j < f) g[r * f + j] = acc;
      else u[r * f + (j - f)] = acc;
    }
  for (int64_t q = 0; q < n * f; ++q) h[q] = silu(g[q]) * u[q];
#pragma omp parallel for schedule(static)
  for (int o = 0; o < d; ++o)
    for (int64_t r = 0; r < n; ++r) {
      double acc = 0.0;
      for (int j = 0; j < f; ++j) acc += bf16_value(w2[(int64_t)o * f + j]) * h[r * f + j];
      y[r * d + o] = acc;
    }
  free(g);
  free(u);
  free(h);
}

/* out[t][o] = shared[t][o] (or 0 when shared is NULL), then for slots in
 * order (ascending expert id) with w != 0: += w * y_perm[pair_pos[t*k+slot]][o]. */
void oracle_combine(int64_t T, int d, int k, const double* y_perm, const int32_t* pair_pos,
                    const double* w, const double* shared, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int o = 0; o < d; ++o) {
      double acc = shared ? shared[t * d + o] : 0.0;
      for (int s = 0; s < k; ++s) {
        double ws = w[t * k + s];
        if (ws != 0.0) acc += ws * y_perm[(int64_t)pair_pos[t * k + s] * d + o];
      }
      out[t * d + o] = acc;
    }
}
