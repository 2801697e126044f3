/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, deliberately slow fp64 CPU implementation of the mixture-of-experts
 * FFN block, written from the archdiff.com architecture-comparison pages:
 *   - "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component table, router row
 *     (Qwen3.5 cell: one linear map gives a logit per expert, then softmax,
 *     the k largest kept and renormalised, no selection bias; DeepSeek-V4-Pro
 *     cell: sqrt-softplus scores, a per-expert bias that only affects which k
 *     are picked, the picked scores normalised and multiplied by 2.5),
 *   - the same page's blueprint diagram, Mixture-of-experts group (router box:
 *     sigma or sqrt-softplus scores balanced by a bias; routed experts: 6 to 22
 *     of 256 to 896 SwiGLU experts; shared experts: one or two, used by every
 *     token; training box: FP8 with block scales),
 *   - "Qwen3.5-397B-A17B vs Gemma 4 31B", component table, routed-experts row
 *     (SwiGLU experts) and shared-expert row (shared output added to the
 *     routed sum).
 *
 * Only tests/, the package's smoke entry and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header or table with the GPU path.
 * Every routine below is the definition written out in fp64 loops; the only
 * rounding to fp32 is where the path's definition fixes an fp32 value (the
 * selection key and the block-scaled FP8 scales), as noted at each site.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2
#define ORC_MXFP4 3

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1
#define ORC_SQRT_SOFTPLUS 2

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3 "FN" (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448).  The diagram's
 * training box names block-scaled FP8 without fixing the variant; E4M3FN is
 * the reading taken. */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6); /* subnormal */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Round v to the nearest E4M3FN value, ties to even, saturating at +-448. */
double orc_e4m3_round(double v) {
  double a = fabs(v), q, r;
  int ex, e;
  if (a == 0.0) return v;
  (void)frexp(a, &ex); /* a = f * 2^ex with f in [0.5, 1) */
  e = ex - 1;          /* a in [2^e, 2^(e+1)) */
  if (e < -6) e = -6;  /* below the normal range the spacing stays 2^-9 */
  q = ldexp(1.0, e - 3);
  r = nearbyint(a / q) * q; /* default rounding mode: to nearest, ties even */
  if (r > 448.0) r = 448.0;
  return copysign(r, v);
}

/* Code of the E4M3FN value nearest to v (same rounding as above). */
uint8_t orc_e4m3_encode(double v) {
  double r = orc_e4m3_round(v);
  double a = fabs(r);
  uint8_t sign = signbit(r) ? 0x80 : 0x00;
  int ex, e, m;
  if (a == 0.0) return sign;
  (void)frexp(a, &ex);
  e = ex - 1;
  if (e < -6) { /* subnormal: exponent field 0, value m * 2^-9 */
    m = (int)(a / ldexp(1.0, -9));
    return (uint8_t)(sign | m);
  }
  m = (int)((a / ldexp(1.0, e) - 1.0) * 8.0);
  return (uint8_t)(sign | ((e + 7) << 3) | m);
}

/* OCP MX E2M1 element (MXFP4's 4-bit element: 1 sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; exponent field 0 is subnormal, 0.5 * mantissa).
 * The training box of the blueprint names MXFP4. */
double orc_e2m1_value(uint8_t code) {
  int e = (code >> 1) & 3, m = code & 1;
  double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
  return (code & 8) ? -mag : mag;
}

/* OCP MX E8M0 shared scale: 2^(code - 127); code 255 is NaN. */
double orc_e8m0_value(uint8_t code) {
  return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

/* Block-scaled FP8 quantisation of one group of n values (the diagram's
 * training box): the scale is the group's largest magnitude over 448,
 * held in fp32 (1 when the group is all zero); each value divided by that
 * scale, held in fp32, is rounded to E4M3FN.  Writes the codes, the scale and
 * the dequantised values q*s.  The fp64 division followed by one rounding to
 * fp32 equals the correctly rounded fp32 division, since 53 >= 2*24 + 2. */
void orc_quant_group(const double* x, int n, uint8_t* codes, float* scale, double* xdq) {
  double amax = 0.0;
  float s;
  int i;
  for (i = 0; i < n; ++i)
    if (fabs(x[i]) > amax) amax = fabs(x[i]);
  s = amax == 0.0 ? 1.0f : (float)(amax / 448.0);
  for (i = 0; i < n; ++i) {
    float r = (float)(x[i] / (double)s);
    double q = orc_e4m3_round((double)r);
    if (codes) codes[i] = orc_e4m3_encode(q);
    if (xdq) xdq[i] = q * (double)s;
  }
  if (scale) *scale = s;
}

/* Rows x groups: x is [rows, cols] with cols a multiple of g. */
void orc_quant_rows(const double* x, int rows, int cols, int g, uint8_t* codes, float* scales,
                    double* xdq) {
  int r, b;
  for (r = 0; r < rows; ++r)
    for (b = 0; b < cols / g; ++b)
      orc_quant_group(x + (size_t)r * cols + (size_t)b * g, g,
                      codes ? codes + (size_t)r * cols + (size_t)b * g : NULL,
                      scales ? scales + (size_t)r * (cols / g) + b : NULL,
                      xdq ? xdq + (size_t)r * cols + (size_t)b * g : NULL);
}

/* One element (r, c) of a stored matrix of logical shape [rows, cols] as fp64.
 * F32 / BF16 / E4M3: row-major [rows, cols]; E4M3 carries one fp32 scale per
 * 128 x 128 block, laid out [rows/128, cols/128].  MXFP4: stored transposed,
 * [cols, rows/2] bytes with two E2M1 codes per byte (the lower row index in
 * the low nibble), and one E8M0 byte per 32 consecutive rows of a column,
 * [cols, rows/32] -- the MX blocks run along the reduction axis (rows). */
static double orc_elem(int dtype, const void* w, const void* scales, int rows, int cols,
                       int block, size_t r, size_t c) {
  size_t i = r * (size_t)cols + c;
  if (dtype == ORC_F32) return (double)((const float*)w)[i];
  if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t*)w)[i]);
  if (dtype == ORC_MXFP4) {
    uint8_t byte = ((const uint8_t*)w)[c * (size_t)(rows / 2) + r / 2];
    uint8_t code = (r & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    return orc_e2m1_value(code) *
           orc_e8m0_value(((const uint8_t*)scales)[c * (size_t)(rows / 32) + r / 32]);
  }
  return orc_e4m3_value(((const uint8_t*)w)[i]) *
         (double)((const float*)scales)[(r / block) * (size_t)(cols / block) + c / block];
}

/* ------------------------------------------------------------------------- */
/* Router                                                                     */
/* ------------------------------------------------------------------------- */

/* Router logits (router row, Qwen3.5 cell: one linear map of the token gives
 * a logit for every expert):
 * l[t,e] = sum_i x[t,i] * W_r[i,e] (+ z_e, a per-expert logit bias used to
 * skew load in the synthetic workloads).  W_r is [d, E]. */
void orc_router_logits(int T, int d, int E, const double* x, int wr_dtype, const void* wr,
                       const float* logit_bias, double* logits) {
  int t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    int e, i;
    for (e = 0; e < E; ++e) {
      double acc = 0.0;
      for (i = 0; i < d; ++i)
        acc += x[(size_t)t * d + i] * orc_elem(wr_dtype, wr, NULL, d, E, 1, (size_t)i, (size_t)e);
      if (logit_bias) acc += (double)logit_bias[e];
      logits[(size_t)t * E + e] = acc;
    }
  }
}

/* Scores of the sigma-family router (blueprint router box: sigma or
 * sqrt-softplus; DeepSeek-V4-Pro router cell: sqrt-softplus). */
double orc_score(int score, double l) {
  if (score == ORC_SIGMOID) return 1.0 / (1.0 + exp(-l));
  /* softplus(l) = log(1 + e^l) = max(l, 0) + log1p(e^-|l|) */
  return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
}

/* Combine weights of one token's selected experts sel[k] (slot order kept).
 * Softmax, renormalised (Qwen3.5 router cell, k = 10 there): softmax over the
 * selected logits; not renormalised: the full softmax probability.
 * sigma / sqrt-softplus (DeepSeek-V4-Pro router cell: picked scores
 * normalised, then multiplied by 2.5): the selected unbiased scores divided by
 * their sum; not renormalised: the score itself.  Either way the result is
 * multiplied by gamma (2.5 in that cell, 1 for softmax).  l: the token's E
 * logits; s: their unbiased scores (softmax: the logits). */
static void orc_weights(int E, int k, int score, int renorm, double gamma, const double* l,
                        const double* s, const int32_t* sel, double* w) {
  int j, e;
  double denom = 0.0, mx;
  if (score == ORC_SOFTMAX) {
    if (renorm) {
      mx = l[sel[0]];
      for (j = 1; j < k; ++j) mx = fmax(mx, l[sel[j]]);
      for (j = 0; j < k; ++j) denom += exp(l[sel[j]] - mx);
    } else {
      mx = l[0];
      for (e = 1; e < E; ++e) mx = fmax(mx, l[e]);
      for (e = 0; e < E; ++e) denom += exp(l[e] - mx);
    }
    for (j = 0; j < k; ++j) w[j] = gamma * exp(l[sel[j]] - mx) / denom;
  } else {
    if (renorm)
      for (j = 0; j < k; ++j) denom += s[sel[j]];
    else
      denom = 1.0;
    for (j = 0; j < k; ++j) w[j] = gamma * s[sel[j]] / denom;
  }
}

/* Top-k selection and combine weights for each token.
 *
 * Keys.  Softmax router: the logit itself (softmax is monotone, so the top-k
 * of the probabilities is the top-k of the logits).  sigma / sqrt-softplus
 * router: score plus the per-expert selection bias, the bias being used only
 * to pick (DeepSeek-V4-Pro router cell); the score is rounded once to fp32 and
 * the bias added in fp32, so that the key is one fixed fp32 number.
 * Order: key descending, equal keys broken by the lower expert index.
 * Weights: orc_weights on the selection.
 *
 * scores_out, if non-NULL, receives the unbiased score (softmax: logit) of each
 * selected slot.  Returns 0, or -1 for invalid k. */
int orc_route(int T, int E, int k, int score, int renorm, double gamma, const double* logits,
              const float* select_bias, int32_t* ids, double* w, double* scores_out) {
  int t;
  if (k < 1 || k > E) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    const double* l = logits + (size_t)t * E;
    double* key = (double*)malloc(sizeof(double) * (size_t)E);
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)calloc((size_t)E, 1);
    int j, e;
    for (e = 0; e < E; ++e) {
      if (score == ORC_SOFTMAX) {
        s[e] = l[e];
        key[e] = l[e];
      } else {
        float s32, b32 = select_bias ? select_bias[e] : 0.0f;
        s[e] = orc_score(score, l[e]);
        s32 = (float)s[e];
        key[e] = (double)(float)(s32 + b32); /* fp32 add, fp32 result */
      }
    }
    /* k rounds of "largest key, lower index on ties" */
    for (j = 0; j < k; ++j) {
      int best = -1;
      for (e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || key[e] > key[best]) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    if (scores_out)
      for (j = 0; j < k; ++j) scores_out[(size_t)t * k + j] = s[ids[(size_t)t * k + j]];
    orc_weights(E, k, score, renorm, gamma, l, s, ids + (size_t)t * k, w + (size_t)t * k);
    free(key);
    free(s);
    free(taken);
  }
  return 0;
}

/* Routing by a fixed token-id hash (router row, DeepSeek-V4-Pro cell: the first
 * three MoE layers choose their experts by a fixed hash of the token id).  The
 * hash is a table of k expert ids per token id, applied as given: ids[t] =
 * table[token_ids[t]].  Only the choice changes; the combine weights are the
 * router's, orc_weights on the table's experts in the table's slot order.
 * Returns -1 if a token id is outside [0, vocab) or a table row does not hold
 * k distinct ids in [0, E). */
int orc_route_hashed(int T, int E, int k, int score, int renorm, double gamma,
                     const double* logits, const int32_t* token_ids, int vocab,
                     const int32_t* table, int32_t* ids, double* w) {
  int t;
  if (k < 1 || k > E) return -1;
  for (t = 0; t < T; ++t) {
    int j, i;
    const int32_t* row;
    if (token_ids[t] < 0 || token_ids[t] >= vocab) return -1;
    row = table + (size_t)token_ids[t] * k;
    for (j = 0; j < k; ++j) {
      if (row[j] < 0 || row[j] >= E) return -1;
      for (i = 0; i < j; ++i)
        if (row[i] == row[j]) return -1;
    }
  }
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    const double* l = logits + (size_t)t * E;
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    int j, e;
    for (e = 0; e < E; ++e) s[e] = score == ORC_SOFTMAX ? l[e] : orc_score(score, l[e]);
    for (j = 0; j < k; ++j) ids[(size_t)t * k + j] = table[(size_t)token_ids[t] * k + j];
    orc_weights(E, k, score, renorm, gamma, l, s, ids + (size_t)t * k, w + (size_t)t * k);
    free(s);
  }
  return 0;
}

/* Auxiliary-loss-free balancing step (router row, DeepSeek-V4-Pro cell: bias
 * balancing with speed 0.001; the update is the published sign rule of that
 * method): every expert's selection bias moves by `speed` towards balance,
 *   b_e <- b_e + speed * sign(mean load - load_e),
 * load_e = number of the batch's T*k assignments routed to e, mean load =
 * T*k / E.  The sign is decided exactly in integers, sign(T*k - E*load_e), and
 * the step is one fp32 add (the bias is fp32); an expert exactly at the mean
 * load keeps its bias bit for bit (no add, so a -0 stays -0).  Returns -1 for
 * an id outside [0, E). */
int orc_bias_update(int T, int k, int E, const int32_t* ids, float speed, float* bias) {
  int64_t* load = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t A = (int64_t)T * k, a;
  int e;
  for (a = 0; a < A; ++a) {
    if (ids[a] < 0 || ids[a] >= E) {
      free(load);
      return -1;
    }
    load[ids[a]] += 1;
  }
  for (e = 0; e < E; ++e) {
    int64_t diff = A - (int64_t)E * load[e];
    if (diff != 0) bias[e] = bias[e] + (diff > 0 ? speed : -speed); /* fp32 add */
  }
  free(load);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Permutation into expert-contiguous order                                   */
/* ------------------------------------------------------------------------- */

/* Counting sort of the T*k (token, slot) assignments by expert, stable in
 * token order: off[e] is the exclusive prefix sum of the per-expert counts
 * (off[E] = T*k); perm_token[r] is the token of row r of the expert-contiguous
 * order; inv_perm[t*k + j] is the row that holds (t, j).  Returns -1 if an id
 * is out of range. */
int orc_permute(int T, int k, int E, const int32_t* ids, int32_t* off, int32_t* perm_token,
                int32_t* inv_perm) {
  size_t A = (size_t)T * (size_t)k, a;
  int32_t* cursor = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  int e;
  for (e = 0; e <= E; ++e) off[e] = 0;
  for (a = 0; a < A; ++a) {
    if (ids[a] < 0 || ids[a] >= E) {
      free(cursor);
      return -1;
    }
    off[ids[a] + 1] += 1;
  }
  for (e = 0; e < E; ++e) off[e + 1] += off[e];
  for (a = 0; a < A; ++a) {
    int32_t ex = ids[a];
    int32_t r = off[ex] + cursor[ex]++;
    perm_token[r] = (int32_t)(a / (size_t)k);
    inv_perm[a] = r;
  }
  free(cursor);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Experts                                                                    */
/* ------------------------------------------------------------------------- */

typedef struct {
  int dtype;                        /* ORC_F32, ORC_BF16, ORC_E4M3 or ORC_MXFP4 */
  int n;                            /* number of experts in the set */
  const void* const* gate;          /* n pointers to logical [d, f] (NULL: not supplied) */
  const void* const* up;            /* n pointers to logical [d, f] */
  const void* const* down;          /* n pointers to logical [f, d] */
  const void* const* gate_scales;   /* E4M3: fp32 [d/128, f/128]; MXFP4: E8M0 [f, d/32] */
  const void* const* up_scales;     /* likewise */
  const void* const* down_scales;   /* E4M3: fp32 [f/128, d/128]; MXFP4: E8M0 [d, f/32] */
} orc_expert_set;

typedef struct {
  int d;          /* model width */
  int f;          /* routed-expert intermediate size */
  int k;          /* experts per token */
  int f_shared;   /* shared-expert intermediate size */
  int quant;      /* 1: block-scaled FP8 activations (x and h) */
  int block;      /* quantisation group / block edge (128) */
  const double* shared_gate;  /* [d] gate vector w of the shared output, or NULL (ungated) */
} orc_ffn_cfg;

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert on one (already dequantised) token row xr[d]:
 * g = xr W_gate, u = xr W_up, h = SiLU(g) * u, (FP8: h re-quantised per group
 * of `block`), y += wgt * (h W_down).  SwiGLU experts (routed-experts row,
 * Qwen3.5 cell).  Returns -1 if the expert was not supplied. */
static int orc_swiglu(const orc_ffn_cfg* c, int f, const orc_expert_set* s, int e,
                      const double* xr, double wgt, double* y, double* h, double* g,
                      double* u) {
  int i, j;
  const void* wg = s->gate[e];
  const void* wu = s->up[e];
  const void* wd = s->down[e];
  const int scaled = s->dtype == ORC_E4M3 || s->dtype == ORC_MXFP4;
  const void* sg = scaled ? s->gate_scales[e] : NULL;
  const void* su = scaled ? s->up_scales[e] : NULL;
  const void* sd = scaled ? s->down_scales[e] : NULL;
  if (!wg || !wu || !wd) return -1;
  if (scaled && (!sg || !su || !sd)) return -1;
  for (j = 0; j < f; ++j) g[j] = u[j] = 0.0;
  for (i = 0; i < c->d; ++i) {
    double xi = xr[i];
    for (j = 0; j < f; ++j) {
      g[j] += xi * orc_elem(s->dtype, wg, sg, c->d, f, c->block, (size_t)i, (size_t)j);
      u[j] += xi * orc_elem(s->dtype, wu, su, c->d, f, c->block, (size_t)i, (size_t)j);
    }
  }
  for (j = 0; j < f; ++j) h[j] = orc_silu(g[j]) * u[j];
  if (c->quant) orc_quant_rows(h, 1, f, c->block, NULL, NULL, h);
  for (j = 0; j < f; ++j) {
    double hj = h[j] * wgt;
    for (i = 0; i < c->d; ++i)
      y[i] += hj * orc_elem(s->dtype, wd, sd, f, c->d, c->block, (size_t)j, (size_t)i);
  }
  return 0;
}

/* The block output for n tokens:
 * out[t] = G(t) * sum_s SharedSwiGLU_s(x~[t]) + sum_j w[t,j] * SwiGLU_{ids[t,j]}(x~[t]),
 * with x~ = x, or for FP8 the dequantised block-scaled x.  Shared experts are
 * always active (blueprint shared-expert box: one or two, used by every
 * token); ungated,
 * G = 1 (DeepSeek-style), or with a gate vector w_g the per-token sigmoid gate
 * G(t) = sigma(x~[t] . w_g) of the Qwen3.5 cell of the shared-expert row of
 * "Qwen3.5-397B-A17B vs Gemma 4 31B" (it scales the shared output before the
 * routed sum is added).  The routed sum is weighted by the router weights.  The
 * residual add outside the block is not part of it.  x is [n, d] fp64 (exact
 * values of the stored inputs), ids/w are [n, k], out is [n, d].  Returns 0,
 * or -1 if a needed expert was not supplied. */
int orc_moe_tokens(const orc_ffn_cfg* c, int n, const double* x, const int32_t* ids,
                   const double* w, const orc_expert_set* routed, const orc_expert_set* shared,
                   double* out) {
  int t, bad = 0;
  int fmax_ = c->f > c->f_shared ? c->f : c->f_shared;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (t = 0; t < n; ++t) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)c->d);
    double* h = (double*)malloc(sizeof(double) * (size_t)fmax_);
    double* g = (double*)malloc(sizeof(double) * (size_t)fmax_);
    double* u = (double*)malloc(sizeof(double) * (size_t)fmax_);
    double* y = out + (size_t)t * c->d;
    int i, j, s;
    memcpy(xr, x + (size_t)t * c->d, sizeof(double) * (size_t)c->d);
    if (c->quant) orc_quant_rows(xr, 1, c->d, c->block, NULL, NULL, xr);
    for (i = 0; i < c->d; ++i) y[i] = 0.0;
    if (shared) {
      double gate = 1.0;
      if (c->shared_gate) {
        double z = 0.0;
        for (i = 0; i < c->d; ++i) z += xr[i] * c->shared_gate[i];
        gate = 1.0 / (1.0 + exp(-z));
      }
      for (s = 0; s < shared->n; ++s)
        if (orc_swiglu(c, c->f_shared, shared, s, xr, gate, y, h, g, u)) bad = 1;
    }
    for (j = 0; j < c->k; ++j) {
      int e = ids[(size_t)t * c->k + j];
      if (e < 0 || e >= routed->n) {
        bad = 1;
        continue;
      }
      if (orc_swiglu(c, c->f, routed, e, xr, w[(size_t)t * c->k + j], y, h, g, u)) bad = 1;
    }
    free(xr);
    free(h);
    free(g);
    free(u);
  }
  return bad ? -1 : 0;
}

/* Number of threads an OpenMP region of this library runs with. */
int orc_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
