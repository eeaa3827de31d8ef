/*
 * CPU ORACLE for the Grok-1 mixture-of-experts feed-forward layer.
 *
 * Test infrastructure only: the parity tests, the smoke check and the bench's
 * CPU-baseline leg call it. The GPU library never links, loads or calls it,
 * and it shares no code, header or table with the GPU library.
 *
 * Plain and slow on purpose: every result is accumulated in double precision
 * in the order the definition reads, one token and one expert at a time, with
 * no blocking, fusion or reordering. Threads only split independent tokens or
 * (token, expert) assignments.
 *
 * What the layer computes (Grok-1 field guide, "MoE 子层" section; Grok-1
 * book ch. 10 "与其他 MoE 对比", section 10.3.1, the Grok-1 routing code;
 * section 10.4, the GeGLU box):
 *   1. router: logit[t][e] = sum_i x[t][i] * Wr[e][i]           (no bias)
 *   2. p[t] = softmax(logit[t]) over all E experts
 *   3. the k largest p (ties: lower expert index first) are the selected
 *      experts; their gates are those p values, NOT renormalised
 *   4. expert e (gated FFN, no biases):
 *        a[j] = sum_i x[i] Wg[e][j][i],  b[j] = sum_i x[i] Wu[e][j][i]
 *        h[j] = GELU(a[j]) * b[j],  GELU(z) = z * Phi(z) = z (1 + erf(z/sqrt2)) / 2
 *        y[i] = sum_j h[j] Wd[e][i][j]
 *   5. out[t] = sum over selected slots s (in slot order) of gate[t][s] * y_s
 * Plus the expert-contiguous permutation the sparse dispatch needs (book ch.
 * 11, section 11.3.1: sparse reorder + grouped GEMM instead of running all
 * experts densely).
 *
 * Storage layouts: x [T][d]; Wr [E][d]; Wg, Wu [E][f][d]; Wd [E][d][f].
 * Element types: ORC_F64, ORC_F32, ORC_BF16 (uint16 bit patterns) and
 * ORC_I8 (int8 values q; the weight is q * scale with one fp32 scale per
 * output channel, packed [gate: E*f | up: E*f | down: E*d]).
 *
 * Readings where the pages are silent (also listed in the design notes):
 * exact-erf GELU on the gate branch; fp64 logits; ties to the lower index;
 * gates in slot order with slot 0 the larger; segment rows in ascending token
 * order.
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * closed forms, invariants, brute force or independent library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2, ORC_I8 = 3 };
enum { ORC_MAXE = 512 }; /* experts a router may have */

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

static double elem(const void* p, int dt, int64_t i) {
  switch (dt) {
    case ORC_F64: return ((const double*)p)[i];
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: {
      uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
      float f;
      memcpy(&f, &u, 4);
      return (double)f;
    }
    case ORC_I8: return (double)((const int8_t*)p)[i];
  }
  return NAN;
}

static int valid_dt(int dt) { return dt >= ORC_F64 && dt <= ORC_I8; }

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_num_procs();
  return nthreads;
#else
  (void)nthreads;
  return 1;
#endif
}

/* GELU with the exact Gaussian CDF: z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2
 * (book ch. 10, section 10.4, GeGLU vs SwiGLU box). */
double oracle_gelu(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

/* SiLU: z * sigmoid(z), the activation of the SwiGLU experts that Mixtral and
 * the later MoEs use in place of GELU (book ch. 10, section 10.4 table and
 * the GeGLU vs SwiGLU box). */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Steps 1-3 for one token: logits, softmax over all experts, top-k without
 * renormalisation (book ch. 10, section 10.3.1, the Grok-1 code). With a
 * selection bias b (nullable; the per-expert bias of DeepSeek-V3's
 * aux-loss-free routing, book ch. 10, section 10.3.2), experts are chosen by
 * p[e] + b[e] while the gates stay p[e]. */
static void route_token(const void* x, int xdt, const void* wr, int rdt, int64_t t, int64_t d, int E,
                        int k, const float* bias, double* p, int32_t* idx, double* gate) {
  double logit[ORC_MAXE];
  for (int e = 0; e < E; ++e) {
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += elem(x, xdt, t * d + i) * elem(wr, rdt, (int64_t)e * d + i);
    logit[e] = s;
  }
  double mx = logit[0];
  for (int e = 1; e < E; ++e)
    if (logit[e] > mx) mx = logit[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp(logit[e] - mx);
  for (int e = 0; e < E; ++e) p[e] = exp(logit[e] - mx) / z;
  /* selection by the key (-(p + b), e): largest score first, lower index on ties */
  double key[ORC_MAXE];
  for (int e = 0; e < E; ++e) key[e] = bias ? p[e] + (double)bias[e] : p[e];
  int taken[ORC_MAXE] = {0};
  for (int s = 0; s < k; ++s) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e;
    }
    taken[best] = 1;
    idx[s] = best;
    gate[s] = p[best];
  }
}

/* probs [T][E] (nullable), idx [T][k], gate [T][k]. */
int oracle_route(const void* x, int xdt, const void* router_w, int rdt, int64_t T, int64_t d, int E, int k,
                 double* probs, int32_t* idx, double* gate, int nthreads) {
  if (T < 0 || d < 1 || E < 1 || E > ORC_MAXE || k < 1 || k > E || !valid_dt(xdt) || !valid_dt(rdt))
    return ORC_EINVAL;
  if (T > 0 && (!x || !router_w || !idx || !gate)) return ORC_EINVAL;
  int nt = set_threads(nthreads);
  (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int64_t t = 0; t < T; ++t) {
    double p[ORC_MAXE];
    route_token(x, xdt, router_w, rdt, t, d, E, k, NULL, p, idx + t * k, gate + t * k);
    if (probs)
      for (int e = 0; e < E; ++e) probs[t * E + e] = p[e];
  }
  return ORC_OK;
}

/* Expert-contiguous permutation of the k*T assignments (sparse reorder, book
 * ch. 11, section 11.3.1). counts[e] = #assignments to e; offsets = exclusive
 * scan (E+1 entries); segment e lists its tokens in ascending token order;
 * perm[row] = token; pos[t][s] = the row of assignment (t, s). */
int oracle_permute(const int32_t* idx, int64_t T, int E, int k, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* pos) {
  if (T < 0 || E < 1 || k < 1 || k > E || !counts || !offsets) return ORC_EINVAL;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < T * k; ++a) {
    int e = idx[a];
    if (e < 0 || e >= E) return ORC_EINVAL;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!fill) return ORC_ENOMEM;
  for (int64_t t = 0; t < T; ++t) {
    for (int s = 0; s < k; ++s) {
      int e = idx[t * k + s];
      int32_t row = offsets[e] + fill[e];
      fill[e] += 1;
      perm[row] = (int32_t)t;
      pos[t * k + s] = row;
    }
  }
  free(fill);
  return ORC_OK;
}

/* Weight element readers with the per-output-channel scale of 8-bit weights. */
typedef struct {
  const void *wg, *wu, *wd;
  int wdt;
  const float* scales;
  int64_t d, f;
  int E;
  int act; /* 0: GELU (Grok-1), 1: SiLU (the SwiGLU variant) */
} weights_t;

static double w_gate(const weights_t* w, int e, int64_t j, int64_t i) {
  double v = elem(w->wg, w->wdt, ((int64_t)e * w->f + j) * w->d + i);
  if (w->wdt == ORC_I8) v *= (double)w->scales[(int64_t)e * w->f + j];
  return v;
}
static double w_up(const weights_t* w, int e, int64_t j, int64_t i) {
  double v = elem(w->wu, w->wdt, ((int64_t)e * w->f + j) * w->d + i);
  if (w->wdt == ORC_I8) v *= (double)w->scales[(int64_t)w->E * w->f + (int64_t)e * w->f + j];
  return v;
}
static double w_down(const weights_t* w, int e, int64_t i, int64_t j) {
  double v = elem(w->wd, w->wdt, ((int64_t)e * w->d + i) * w->f + j);
  if (w->wdt == ORC_I8) v *= (double)w->scales[2 * (int64_t)w->E * w->f + (int64_t)e * w->d + i];
  return v;
}

/* Step 4: token row x (d values) through expert e; y gets d values; h (f values) is scratch. */
static void expert_ffn(const weights_t* w, const double* x, int e, double* h, double* y) {
  const int64_t d = w->d, f = w->f;
  for (int64_t j = 0; j < f; ++j) {
    double a = 0.0, b = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      a += x[i] * w_gate(w, e, j, i);
      b += x[i] * w_up(w, e, j, i);
    }
    h[j] = (w->act ? oracle_silu(a) : oracle_gelu(a)) * b;
  }
  for (int64_t i = 0; i < d; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < f; ++j) s += h[j] * w_down(w, e, i, j);
    y[i] = s;
  }
}

static int check_weights(int wdt, const float* scales) {
  if (!valid_dt(wdt)) return 0;
  if (wdt == ORC_I8 && !scales) return 0;
  return 1;
}

/* Single expert output for one token (used by tests for per-expert checks). */
int oracle_expert(const void* x, int xdt, int64_t t, const void* wg, const void* wu, const void* wd, int wdt,
                  const float* scales, int64_t d, int64_t f, int E, int e, double* y) {
  if (!check_weights(wdt, scales) || !valid_dt(xdt) || e < 0 || e >= E || d < 1 || f < 1) return ORC_EINVAL;
  weights_t w = {wg, wu, wd, wdt, scales, d, f, E, 0};
  double* xr = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)f);
  if (!xr || !h) { free(xr); free(h); return ORC_ENOMEM; }
  for (int64_t i = 0; i < d; ++i) xr[i] = elem(x, xdt, t * d + i);
  expert_ffn(&w, xr, e, h, y);
  free(xr);
  free(h);
  return ORC_OK;
}

/* Steps 4-5 for a list of tokens, given the routing (idx [T][k], gate [T][k]).
 * out has ntok rows of d values: row r is token tokens[r] (all T tokens when
 * tokens is NULL, then ntok must equal T). */
int oracle_forward_given_routing(const void* x, int xdt, const void* wg, const void* wu, const void* wd, int wdt,
                                 const float* scales, const int32_t* idx, const double* gate, int64_t T,
                                 int64_t d, int64_t f, int E, int k, const int64_t* tokens, int64_t ntok,
                                 double* out, int nthreads) {
  if (!check_weights(wdt, scales) || !valid_dt(xdt) || T < 0 || d < 1 || f < 1 || E < 1 || k < 1 || k > E)
    return ORC_EINVAL;
  if (!tokens && ntok != T) return ORC_EINVAL;
  if (ntok == 0) return ORC_OK;
  for (int64_t r = 0; r < ntok; ++r) {
    int64_t t = tokens ? tokens[r] : r;
    if (t < 0 || t >= T) return ORC_EINVAL;
    for (int s = 0; s < k; ++s)
      if (idx[t * k + s] < 0 || idx[t * k + s] >= E) return ORC_EINVAL;
  }
  weights_t w = {wg, wu, wd, wdt, scales, d, f, E, 0};
  /* y[r][s][:] = output of the expert in slot s for token tokens[r] */
  double* y = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d));
  if (!y) return ORC_ENOMEM;
  int nt = set_threads(nthreads);
  (void)nt;
  int fail = 0;
#pragma omp parallel num_threads(nt)
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    if (!xr || !h) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t a = 0; a < ntok * k; ++a) {
        int64_t r = a / k;
        int s = (int)(a % k);
        int64_t t = tokens ? tokens[r] : r;
        for (int64_t i = 0; i < d; ++i) xr[i] = elem(x, xdt, t * d + i);
        expert_ffn(&w, xr, idx[t * k + s], h, y + a * d);
      }
    }
    free(xr);
    free(h);
  }
  if (fail) { free(y); return ORC_ENOMEM; }
  for (int64_t r = 0; r < ntok; ++r) {
    int64_t t = tokens ? tokens[r] : r;
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int s = 0; s < k; ++s) acc += gate[t * k + s] * y[(r * k + s) * d + i];
      out[r * d + i] = acc;
    }
  }
  free(y);
  return ORC_OK;
}

/* The whole layer: route every token, then steps 4-5 for every token.
 * idx/gate (nullable) receive the routing. */
int oracle_forward(const void* x, int xdt, const void* router_w, int rdt, const void* wg, const void* wu,
                   const void* wd, int wdt, const float* scales, int64_t T, int64_t d, int64_t f, int E, int k,
                   double* out, int32_t* idx_out, double* gate_out, int nthreads) {
  if (T < 0 || E < 1 || E > ORC_MAXE || k < 1 || k > E) return ORC_EINVAL;
  if (T == 0) return ORC_OK;
  int32_t* idx = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  double* gate = gate_out ? gate_out : (double*)malloc(sizeof(double) * (size_t)(T * k));
  int rc = ORC_ENOMEM;
  if (idx && gate) {
    rc = oracle_route(x, xdt, router_w, rdt, T, d, E, k, NULL, idx, gate, nthreads);
    if (rc == ORC_OK)
      rc = oracle_forward_given_routing(x, xdt, wg, wu, wd, wdt, scales, idx, gate, T, d, f, E, k, NULL, T, out,
                                        nthreads);
  }
  if (!idx_out) free(idx);
  if (!gate_out) free(gate);
  return rc;
}

/* Brute force in the pages' own dense formulation (book ch. 11, section
 * 11.3.1 and 11.5.2: every expert runs on every token, then a one-hot mask of
 * the top-k keeps the selected outputs, each times its gate). The expert math
 * is written out again here, with different loop nesting, so that this path
 * shares no helper with the sparse one above except the element reader, GELU
 * and the router. */
int oracle_dense_onehot(const void* x, int xdt, const void* router_w, int rdt, const void* wg, const void* wu,
                        const void* wd, int wdt, const float* scales, int64_t T, int64_t d, int64_t f, int E,
                        int k, double* out, int nthreads) {
  if (!check_weights(wdt, scales) || !valid_dt(xdt) || T < 0 || d < 1 || f < 1 || E < 1 || E > ORC_MAXE || k < 1 ||
      k > E)
    return ORC_EINVAL;
  weights_t w = {wg, wu, wd, wdt, scales, d, f, E, 0};
  int nt = set_threads(nthreads);
  (void)nt;
  int fail = 0;
#pragma omp parallel num_threads(nt)
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)f);
    double* b = (double*)malloc(sizeof(double) * (size_t)f);
    double* ye = (double*)malloc(sizeof(double) * (size_t)d);
    if (!a || !b || !ye) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < T; ++t) {
        double p[ORC_MAXE], g[ORC_MAXE], mask[ORC_MAXE];
        int32_t id[ORC_MAXE];
        route_token(x, xdt, router_w, rdt, t, d, E, k, NULL, p, id, g);
        for (int e = 0; e < E; ++e) mask[e] = 0.0;
        for (int s = 0; s < k; ++s) mask[id[s]] = g[s];
        for (int64_t i = 0; i < d; ++i) out[t * d + i] = 0.0;
        for (int e = 0; e < E; ++e) {
          /* up-projections accumulated input-feature-outer */
          for (int64_t j = 0; j < f; ++j) a[j] = b[j] = 0.0;
          for (int64_t i = 0; i < d; ++i) {
            double xi = elem(x, xdt, t * d + i);
            for (int64_t j = 0; j < f; ++j) {
              a[j] += xi * w_gate(&w, e, j, i);
              b[j] += xi * w_up(&w, e, j, i);
            }
          }
          /* down-projection as a sum of columns h[j] * Wd[:, j] */
          for (int64_t i = 0; i < d; ++i) ye[i] = 0.0;
          for (int64_t j = 0; j < f; ++j) {
            double hj = oracle_gelu(a[j]) * b[j];
            for (int64_t i = 0; i < d; ++i) ye[i] += hj * w_down(&w, e, i, j);
          }
          for (int64_t i = 0; i < d; ++i) out[t * d + i] += mask[e] * ye[i];
        }
      }
    }
    free(a);
    free(b);
    free(ye);
  }
  return fail ? ORC_ENOMEM : ORC_OK;
}

/* ==================================================================== variants
 * Layer variants the pages describe beside the Grok-1 default. Every knob at
 * zero gives the Grok-1 layer above.
 *  - act = 1: SiLU experts (SwiGLU; book ch. 10, section 10.4).
 *  - renormalize: the k selected gates are divided by their sum, as Mixtral
 *    does after its top-k (book ch. 10, section 10.3.1, the Mixtral code).
 *  - capacity_factor c > 0: each expert takes at most c * k * T / E of the
 *    k * T assignments, the rest are dropped and contribute nothing (book
 *    ch. 10, section 10.3.2, the capacity factor box). The pages do not say
 *    which assignments overflow; here an expert keeps those of its lowest
 *    token indices (first come, first served in token order), and "at most
 *    c*k*T/E" is the integer floor of that bound.
 *  - norm_pre and norm_post: the sandwich sub-layer (field guide, "数据怎样流
 *    过 64 层": the sub-layer normalises, runs the MoE, and adds the gated sum
 *    back to the trunk; book ch. 11, list of what Grok-1 left behind: two
 *    norms per sub-layer; book ch. 10, section 10.3.1: the post-norm bounds
 *    the output that un-normalised gates leave unscaled):
 *        u   = RMSNorm(x; norm_pre), stored in the activation type
 *        out = x + RMSNorm(MoE(u); norm_post)
 *    with RMSNorm(v; g)[i] = g[i] * v[i] / sqrt(mean_j v[j]^2 + eps). u is
 *    rounded to the activation type (bf16 or fp32, round to nearest even)
 *    because the router and the experts consume it as a stored tensor of a
 *    bf16 forward pass; MoE(u) and the post-norm stay in double.
 *  - the fine-grained layout of DeepSeek-V3 (book ch. 10, section 10.1 table
 *    and the shared-expert box; section 10.11.4): many small routed experts
 *    plus n_shared shared experts that every token runs with gate 1, their
 *    weights stored after the E routed experts' (E + n_shared experts in
 *    w_gate/w_up/w_down and in the scales); and router_bias, a per-expert
 *    bias of the aux-loss-free routing (section 10.3.2) that the pages say
 *    shifts which experts are chosen: here it is added to the softmax
 *    probabilities for the top-k choice only, the gates remain the
 *    probabilities (then renormalised when asked). The capacity cap applies
 *    to the routed experts only. */

/* Round to the nearest bf16 value (8 significant bits), ties to even; returns
 * the bit pattern. Normal range only (|v| in [2^-126, 2^128)) and zero. */
uint16_t oracle_bf16_rne(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
  int e;
  double m = frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
  double r = nearbyint(ldexp(m, 8));      /* 8 significant bits, ties to even */
  float q = (float)ldexp(r, e - 8);       /* exact: 8 significant bits */
  uint32_t u;
  memcpy(&u, &q, 4);
  return (uint16_t)((u >> 16) | (v < 0.0 ? 0x8000u : 0u));
}

/* Rows per expert under capacity factor c, or -1 (no cap) when c <= 0. */
int64_t oracle_capacity(double c, int64_t T, int E, int k) {
  if (!(c > 0.0)) return -1;
  return (int64_t)floor(c * (double)(k * T) / (double)E);
}

/* Routing with the optional selection bias (nullable, E values) and the
 * optional renormalisation: gates divided by their sum over the k slots
 * (summed in slot order). */
int oracle_route_v(const void* x, int xdt, const void* router_w, int rdt, int64_t T, int64_t d, int E, int k,
                   int renormalize, const float* bias, double* probs, int32_t* idx, double* gate, int nthreads) {
  if (T < 0 || d < 1 || E < 1 || E > ORC_MAXE || k < 1 || k > E || !valid_dt(xdt) || !valid_dt(rdt))
    return ORC_EINVAL;
  if (T > 0 && (!x || !router_w || !idx || !gate)) return ORC_EINVAL;
  int nt = set_threads(nthreads);
  (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int64_t t = 0; t < T; ++t) {
    double p[ORC_MAXE];
    route_token(x, xdt, router_w, rdt, t, d, E, k, bias, p, idx + t * k, gate + t * k);
    if (probs)
      for (int e = 0; e < E; ++e) probs[t * E + e] = p[e];
  }
  if (!renormalize) return ORC_OK;
  for (int64_t t = 0; t < T; ++t) {
    double sum = 0.0;
    for (int s = 0; s < k; ++s) sum += gate[t * k + s];
    for (int s = 0; s < k; ++s) gate[t * k + s] /= sum;
  }
  return ORC_OK;
}

/* Permutation with a per-expert cap (cap < 0: none) on the experts e <
 * E_cap (the routed ones; shared experts are never capped). For every capped
 * expert, its assignments are ranked by token index; those of rank >= cap
 * are dropped (pos = -1, no row). counts are the kept assignments, offsets
 * their exclusive scan, and segment e lists its kept tokens in ascending
 * order. */
int oracle_permute_cap(const int32_t* idx, int64_t T, int E, int k, int64_t cap, int E_cap, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* pos) {
  if (T < 0 || E < 1 || k < 1 || k > E || !counts || !offsets) return ORC_EINVAL;
  int64_t* seen = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!seen) return ORC_ENOMEM;
  /* pass 1: how many assignments each expert has, and how many it keeps */
  for (int64_t a = 0; a < T * k; ++a) {
    int e = idx[a];
    if (e < 0 || e >= E) { free(seen); return ORC_EINVAL; }
    seen[e] += 1;
  }
  for (int e = 0; e < E; ++e) counts[e] = (int32_t)((cap >= 0 && e < E_cap && seen[e] > cap) ? cap : seen[e]);
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* pass 2: walk the tokens in order; an expert's rank-th assignment gets row
   * offsets[e] + rank while rank < counts[e] */
  for (int e = 0; e < E; ++e) seen[e] = 0;
  for (int64_t t = 0; t < T; ++t) {
    for (int s = 0; s < k; ++s) {
      int e = idx[t * k + s];
      int64_t rank = seen[e]++;
      if (rank < counts[e]) {
        int32_t row = (int32_t)(offsets[e] + rank);
        perm[row] = (int32_t)t;
        pos[t * k + s] = row;
      } else {
        pos[t * k + s] = -1;
      }
    }
  }
  free(seen);
  return ORC_OK;
}

/* RMSNorm of each of the T rows of v (d values): out[t][i] = g[i] * v[t][i] *
 * r_t, r_t = 1 / sqrt(mean_i v[t][i]^2 + eps), all in double. */
int oracle_rmsnorm(const void* v, int vdt, int64_t T, int64_t d, const void* g, int gdt, double eps, double* out) {
  if (T < 0 || d < 1 || !valid_dt(vdt) || !valid_dt(gdt) || !(eps >= 0.0)) return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      double a = elem(v, vdt, t * d + i);
      ss += a * a;
    }
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int64_t i = 0; i < d; ++i) out[t * d + i] = (elem(v, vdt, t * d + i) * r) * elem(g, gdt, i);
  }
  return ORC_OK;
}

/* Every input of one layer call, with the variant knobs. */
typedef struct {
  const void* x;
  int xdt; /* ORC_BF16 or ORC_F32: also the type u is stored in */
  const void* router_w;
  int rdt;
  const void *wg, *wu, *wd;
  int wdt;
  const float* scales;
  int64_t T, d, f;
  int E, k; /* routed experts and how many each token picks */
  int act;
  int renormalize;
  double capacity_factor;
  const void* norm_pre; /* both NULL, or both [d] of type norm_dt */
  const void* norm_post;
  int norm_dt;
  double norm_eps;
  int n_shared;            /* experts E .. E + n_shared - 1 of the weights run on every token, gate 1 */
  const float* router_bias; /* nullable, E values: added to p for the top-k choice only */
} orc_layer;

/* The layer with its variants: routing and permutation for all T tokens, then
 * the outputs of the listed tokens (all T when tokens is NULL; ntok rows of d
 * values in out). Optional outputs: idx/gate/pos [T][K] with K = k + n_shared
 * (slots k.. are the shared experts; pos -1 = dropped), u (T*d values of type
 * xdt, the stored pre-norm output). */
int oracle_layer(const orc_layer* L, const int64_t* tokens, int64_t ntok, double* out, int32_t* idx_out,
                 double* gate_out, int32_t* pos_out, void* u_out, int nthreads) {
  if (!L || L->T < 0 || L->d < 1 || L->f < 1 || L->E < 1 || L->E > ORC_MAXE || L->k < 1 || L->k > L->E) return ORC_EINVAL;
  if (L->n_shared < 0 || L->n_shared > 64) return ORC_EINVAL;
  if (L->xdt != ORC_BF16 && L->xdt != ORC_F32) return ORC_EINVAL;
  if (!check_weights(L->wdt, L->scales) || (L->act != 0 && L->act != 1)) return ORC_EINVAL;
  if ((L->norm_pre == NULL) != (L->norm_post == NULL)) return ORC_EINVAL;
  const int sandwich = L->norm_pre != NULL;
  if (sandwich && (!valid_dt(L->norm_dt) || !(L->norm_eps >= 0.0))) return ORC_EINVAL;
  if (!tokens && ntok != L->T) return ORC_EINVAL;
  const int64_t T = L->T, d = L->d, f = L->f;
  const int E = L->E, kr = L->k;            /* routed experts, routed slots */
  const int Et = E + L->n_shared, k = kr + L->n_shared; /* all experts, all slots */
  if (T == 0) return ORC_OK;
  for (int64_t r = 0; r < ntok; ++r)
    if (tokens && (tokens[r] < 0 || tokens[r] >= T)) return ORC_EINVAL;

  const size_t esz = L->xdt == ORC_BF16 ? 2 : 4;
  void* u = NULL;
  double* tmp = NULL;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  double* gate = (double*)malloc(sizeof(double) * (size_t)(T * k));
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)Et);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Et + 1));
  int32_t* ridx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * kr));
  double* rgate = (double*)malloc(sizeof(double) * (size_t)(T * kr));
  double* y = (double*)malloc(sizeof(double) * (size_t)(ntok * k * d + 1));
  int rc = ORC_ENOMEM;
  if (!idx || !gate || !pos || !perm || !y || !counts || !offsets || !ridx || !rgate) goto done;

  /* 1. the MoE input: x, or the pre-norm of x stored in the activation type */
  const void* a = L->x;
  if (sandwich) {
    u = malloc(esz * (size_t)(T * d));
    tmp = (double*)malloc(sizeof(double) * (size_t)d);
    if (!u || !tmp) goto done;
    for (int64_t t = 0; t < T; ++t) {
      rc = oracle_rmsnorm((const char*)L->x + esz * (size_t)(t * d), L->xdt, 1, d, L->norm_pre, L->norm_dt,
                          L->norm_eps, tmp);
      if (rc != ORC_OK) goto done;
      for (int64_t i = 0; i < d; ++i) {
        if (L->xdt == ORC_BF16) ((uint16_t*)u)[t * d + i] = oracle_bf16_rne(tmp[i]);
        else ((float*)u)[t * d + i] = (float)tmp[i];
      }
    }
    a = u;
  }
  /* 2. routing over the routed experts (softmax, top-k by p + bias, optional
   *    renormalisation), then the shared experts' slots with gate 1 */
  rc = oracle_route_v(a, L->xdt, L->router_w, L->rdt, T, d, E, kr, L->renormalize, L->router_bias, NULL, ridx,
                      rgate, nthreads);
  if (rc != ORC_OK) goto done;
  for (int64_t t = 0; t < T; ++t) {
    for (int s = 0; s < kr; ++s) {
      idx[t * k + s] = ridx[t * kr + s];
      gate[t * k + s] = rgate[t * kr + s];
    }
    for (int j = 0; j < L->n_shared; ++j) {
      idx[t * k + kr + j] = E + j;
      gate[t * k + kr + j] = 1.0;
    }
  }
  /* 3. permutation with the capacity cap on the routed experts: decides which
   *    assignments run */
  rc = oracle_permute_cap(idx, T, Et, k, oracle_capacity(L->capacity_factor, T, E, kr), E, counts, offsets, perm,
                          pos);
  if (rc != ORC_OK) goto done;
  /* 4. expert outputs of the kept assignments of the listed tokens */
  {
    weights_t w = {L->wg, L->wu, L->wd, L->wdt, L->scales, d, f, Et, L->act};
    int nt = set_threads(nthreads);
    (void)nt;
    int fail = 0;
#pragma omp parallel num_threads(nt)
    {
      double* xr = (double*)malloc(sizeof(double) * (size_t)d);
      double* h = (double*)malloc(sizeof(double) * (size_t)f);
      if (!xr || !h) {
#pragma omp atomic write
        fail = 1;
      } else {
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < ntok * k; ++q) {
          int64_t r = q / k;
          int s = (int)(q % k);
          int64_t t = tokens ? tokens[r] : r;
          if (pos[t * k + s] < 0) {
            for (int64_t i = 0; i < d; ++i) y[q * d + i] = 0.0;
            continue;
          }
          for (int64_t i = 0; i < d; ++i) xr[i] = elem(a, L->xdt, t * d + i);
          expert_ffn(&w, xr, idx[t * k + s], h, y + q * d);
        }
      }
      free(xr);
      free(h);
    }
    if (fail) { rc = ORC_ENOMEM; goto done; }
  }
  /* 5. gated sum over the kept slots, then the post-norm and the residual */
  for (int64_t r = 0; r < ntok; ++r) {
    int64_t t = tokens ? tokens[r] : r;
    double* o = out + r * d;
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int s = 0; s < k; ++s)
        if (pos[t * k + s] >= 0) acc += gate[t * k + s] * y[(r * k + s) * d + i];
      o[i] = acc;
    }
    if (sandwich) {
      rc = oracle_rmsnorm(o, ORC_F64, 1, d, L->norm_post, L->norm_dt, L->norm_eps, tmp);
      if (rc != ORC_OK) goto done;
      for (int64_t i = 0; i < d; ++i) o[i] = elem(L->x, L->xdt, t * d + i) + tmp[i];
    }
  }
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)(T * k));
  if (gate_out) memcpy(gate_out, gate, sizeof(double) * (size_t)(T * k));
  if (pos_out) memcpy(pos_out, pos, sizeof(int32_t) * (size_t)(T * k));
  if (u_out && u) memcpy(u_out, u, esz * (size_t)(T * d));
  rc = ORC_OK;
done:
  free(idx);
  free(gate);
  free(pos);
  free(perm);
  free(y);
  free(u);
  free(tmp);
  free(counts);
  free(offsets);
  free(ridx);
  free(rgate);
  return rc;
}
