/*
 * moe_oracle.c -- plain fp64 CPU oracle of the small-batch decode MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): used by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark; never by the product.
 *
 * Everything is written as the definition, in the order the definition
 * states, with no blocking or fusion.  Sums run over ascending index.  Each
 * product of a decoded weight, its scale and a bf16 activation is exact in
 * fp64 (at most 4 + 24 + 8 significant bits), so only the sums round.
 *
 * Parity pins (tests/test_oracle_*.py): every decoder against torch's casts
 * or an exact embedding into E4M3; round-trip of the seeded quantiser;
 * brute-force routing by full sorts and group-subset enumeration; one-hot
 * closed forms for gate/up/SwiGLU/down; zero routed scale giving exactly the
 * shared expert; row-permutation equivariance; bf16 rounding by exhaustive
 * neighbour search.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Format decode.                                                            */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_dec_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 448; exponent field 0 is
 * subnormal with value m * 2^-9.  Normal value (1 + m/8) * 2^(e-7). */
double oracle_dec_e4m3(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* OCP MX v1.0 FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; no
 * NaN or infinity; exponent field 0 is subnormal, value 0.5 * m.  Normal
 * value (1 + m/2) * 2^(e-1). */
double oracle_dec_e2m1(uint8_t nibble) {
  int sign = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 0x3;
  int m = nibble & 0x1;
  double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + (double)m / 2.0, e - 1);
  return sign ? -v : v;
}

/* OCP MX v1.0 E8M0 scale: 2^(c-127); code 0xFF is NaN. */
double oracle_dec_e8m0(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* fp64 -> bf16 with round-to-nearest, ties to even, straight from fp64.
 * bf16 has 8 significant bits and binary32's exponent range: in the binade
 * [2^(E-1), 2^E) its spacing is 2^(E-8); below 2^-126 (subnormal) it is
 * 2^-133.  Values that round to 2^128 or more become infinity. */
uint16_t oracle_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int E;
  (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
  int ulp_exp = (E - 1 >= -126) ? E - 8 : -133;
  double q = ldexp(a, -ulp_exp);   /* exact: scaling by a power of two */
  double n = nearbyint(q);         /* default mode: nearest, ties to even */
  double r = ldexp(n, ulp_exp);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

/* One element of a dequantised [N,K] weight stored K-contiguous.
 *  FP8_B128: fp32 scale per 128x128 block, scale grid [N/128, K/128],
 *            W[n,k] = e4m3(q[n,k]) * s[n/128, k/128]   (scales multiply).
 *  MXFP4:    two E2M1 codes per byte, element k in the low nibble when k is
 *            even; one E8M0 scale per 32 consecutive k, grid [N, K/32],
 *            W[n,k] = e2m1(q[n,k]) * 2^(s[n,k/32]-127). */
double oracle_weight(int fmt, const uint8_t* q, const void* scale, int N, int K,
                     int n, int k) {
  (void)N;
  if (fmt == ORACLE_FMT_FP8_B128) {
    const float* s = (const float*)scale;
    double code = oracle_dec_e4m3(q[(size_t)n * K + k]);
    return code * (double)s[(size_t)(n / 128) * (K / 128) + k / 128];
  } else {
    const uint8_t* s = (const uint8_t*)scale;
    uint8_t byte = q[(size_t)n * (K / 2) + k / 2];
    uint8_t nib = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    return oracle_dec_e2m1(nib) * oracle_dec_e8m0(s[(size_t)n * (K / 32) + k / 32]);
  }
}

/* ------------------------------------------------------------------------ */
/* Configuration checks.                                                     */
/* ------------------------------------------------------------------------ */

static int cfg_ok(const oracle_cfg* c) {
  if (!c) return 0;
  if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0) return 0;
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts) return 0;
  if (c->n_group < 1 || c->n_experts % c->n_group) return 0;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return 0;
  if (c->n_group > 1 && c->n_experts / c->n_group < 2) return 0;
  if (c->n_group > 1 && c->topk_group * (c->n_experts / c->n_group) < c->top_k) return 0;
  if (c->n_shared != 0 && c->n_shared != 1) return 0;
  if (c->expert_first < 0 || c->expert_count < 0 || c->expert_first + c->expert_count > c->n_experts) return 0;
  if (c->expert_count == 0 && c->expert_first != 0) return 0;
  if (c->n_shared && (c->shared_inter <= 0 || c->shared_inter % 128 || c->hidden % 128)) return 0;
  if (c->routed_fmt == ORACLE_FMT_FP8_B128) {
    if (c->hidden % 128 || c->inter % 128) return 0;
  } else if (c->routed_fmt == ORACLE_FMT_MXFP4) {
    if (c->hidden % 32 || c->inter % 32) return 0;
  } else {
    return 0;
  }
  return 1;
}

/* ------------------------------------------------------------------------ */
/* Routing.                                                                  */
/* ------------------------------------------------------------------------ */

static double bias_of(const oracle_cfg* c, const void* bias, int e) {
  if (c->bias_bf16) return oracle_dec_bf16(((const uint16_t*)bias)[e]);
  return (double)((const float*)bias)[e];
}

/* Router logit l[e] = sum_h x[h] * Wr[e,h] (Wr is [E,H] bf16), summed over
 * ascending h; score s = sigmoid(l) = 1/(1+exp(-l)); selection key
 * b = s + bias[e].  The bias only steers selection (the correction bias the
 * hotspot page says may be bf16). */
void oracle_scores(const oracle_cfg* cfg, const uint16_t* x_row,
                   const uint16_t* router_w, const void* bias,
                   double* logits, double* s, double* b) {
  const int H = cfg->hidden, E = cfg->n_experts;
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int h = 0; h < H; ++h)
      acc += oracle_dec_bf16(x_row[h]) * oracle_dec_bf16(router_w[(size_t)e * H + h]);
    logits[e] = acc;
    s[e] = 1.0 / (1.0 + exp(-acc));
    b[e] = s[e] + bias_of(cfg, bias, e);
  }
}

/* True when (va, a) ranks before (vb, b): larger value first, lower index on
 * an exact tie. */
static int ranks_before(double va, int a, double vb, int b) {
  return va > vb || (va == vb && a < b);
}

/* Routes one row from its scores.  Group stage (n_group > 1): group j holds
 * experts [j*E/n_g, (j+1)*E/n_g); its score is the sum of its two largest b;
 * the k_g groups ranked first by (score desc, j asc) are kept.  Then the K
 * experts of kept groups ranked first by (b desc, e asc) are picked, in
 * that order.  Weights use the unbiased scores: w_p = s[id_p] / sum_q
 * s[id_q] * routed_scale, the sum over q ascending. */
static void route_row(const oracle_cfg* cfg, const double* s, const double* b,
                      int32_t* ids, double* w, double* gap_expert, double* gap_group) {
  const int E = cfg->n_experts, K = cfg->top_k, ng = cfg->n_group, kg = cfg->topk_group;
  int kept_expert[1024];
  int chosen[1024];
  double gs[1024];
  int gkept[1024];
  for (int e = 0; e < E; ++e) { kept_expert[e] = 1; chosen[e] = 0; }
  double ggap = INFINITY;
  if (ng > 1) {
    const int gsz = E / ng;
    for (int j = 0; j < ng; ++j) {
      /* two largest b of the group */
      int i1 = -1, i2 = -1;
      for (int e = j * gsz; e < (j + 1) * gsz; ++e)
        if (i1 < 0 || ranks_before(b[e], e, b[i1], i1)) i1 = e;
      for (int e = j * gsz; e < (j + 1) * gsz; ++e)
        if (e != i1 && (i2 < 0 || ranks_before(b[e], e, b[i2], i2))) i2 = e;
      gs[j] = b[i1] + b[i2];
      gkept[j] = 0;
    }
    for (int t = 0; t < kg; ++t) {
      int best = -1;
      for (int j = 0; j < ng; ++j)
        if (!gkept[j] && (best < 0 || ranks_before(gs[j], j, gs[best], best))) best = j;
      gkept[best] = 1;
    }
    double worst_kept = INFINITY, best_dropped = -INFINITY;
    for (int j = 0; j < ng; ++j) {
      if (gkept[j] && gs[j] < worst_kept) worst_kept = gs[j];
      if (!gkept[j] && gs[j] > best_dropped) best_dropped = gs[j];
    }
    ggap = (kg < ng) ? worst_kept - best_dropped : INFINITY;
    for (int e = 0; e < E; ++e) kept_expert[e] = gkept[e / gsz];
  }
  for (int p = 0; p < K; ++p) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (kept_expert[e] && !chosen[e] && (best < 0 || ranks_before(b[e], e, b[best], best)))
        best = e;
    chosen[best] = 1;
    ids[p] = best;
  }
  double best_left = -INFINITY;
  int any_left = 0;
  for (int e = 0; e < E; ++e)
    if (kept_expert[e] && !chosen[e]) {
      any_left = 1;
      if (b[e] > best_left) best_left = b[e];
    }
  double sum = 0.0;
  for (int p = 0; p < K; ++p) sum += s[ids[p]];
  for (int p = 0; p < K; ++p) w[p] = s[ids[p]] / sum * cfg->routed_scale;
  if (gap_expert) *gap_expert = any_left ? b[ids[K - 1]] - best_left : INFINITY;
  if (gap_group) *gap_group = ggap;
}

int oracle_route(const oracle_cfg* cfg, const uint16_t* x, int T,
                 const uint16_t* router_w, const void* bias,
                 int32_t* ids, double* w, double* gap_expert, double* gap_group) {
  if (!cfg_ok(cfg) || cfg->n_experts > 1024 || T < 0) return -1;
  const int E = cfg->n_experts, H = cfg->hidden, K = cfg->top_k;
  double* l = (double*)malloc(sizeof(double) * 3 * (size_t)E);
  if (!l) return -1;
  double *s = l + E, *b = l + 2 * E;
  for (int r = 0; r < T; ++r) {
    oracle_scores(cfg, x + (size_t)r * H, router_w, bias, l, s, b);
    route_row(cfg, s, b, ids + (size_t)r * K, w + (size_t)r * K,
              gap_expert ? gap_expert + r : NULL, gap_group ? gap_group + r : NULL);
  }
  free(l);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Distinct-expert grouping (PR #27, Modifications, commit 1: each expert the */
/* step uses streams once, the shared expert and every distinct routed one,  */
/* in order of first use, each with every row that picked it).               */
/* ------------------------------------------------------------------------ */

int oracle_groups(const oracle_cfg* cfg, int T, const int32_t* ids,
                  int32_t* n_groups, int32_t* group_expert, int32_t* group_ncols,
                  int32_t* group_col_start, int32_t* cols, int32_t* use_group) {
  if (!cfg_ok(cfg) || T < 0) return -1;
  const int E = cfg->n_experts, K = cfg->top_k;
  int* gof = (int*)malloc(sizeof(int) * (size_t)E);
  if (!gof) return -1;
  for (int e = 0; e < E; ++e) gof[e] = -1;
  int G = 0;
  if (cfg->n_shared) {
    group_expert[G] = -1;
    group_ncols[G] = T;
    ++G;
  }
  for (int u = 0; u < T * K; ++u) {
    int e = ids[u];
    if (e < 0 || e >= E) { free(gof); return -1; }
    if (gof[e] < 0) {
      gof[e] = G;
      group_expert[G] = e;
      group_ncols[G] = 0;
      ++G;
    }
    use_group[u] = gof[e];
    group_ncols[gof[e]] += 1;
  }
  int start = 0;
  for (int g = 0; g < G; ++g) {
    group_col_start[g] = start;
    start += group_ncols[g];
  }
  int* fill = (int*)calloc((size_t)(G > 0 ? G : 1), sizeof(int));
  if (!fill) { free(gof); return -1; }
  if (cfg->n_shared)
    for (int r = 0; r < T; ++r) cols[group_col_start[0] + fill[0]++] = r * 16 + K;
  for (int u = 0; u < T * K; ++u) {
    int g = use_group[u];
    cols[group_col_start[g] + fill[g]++] = (u / K) * 16 + (u % K);
  }
  *n_groups = G;
  free(fill);
  free(gof);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN: gate/up, SwiGLU, down.                                        */
/* ------------------------------------------------------------------------ */

/* W_gate_up is [2I, H]: rows 0..I-1 are the gate projection, rows I..2I-1
 * the up projection.  W_down is [H, I].
 *   g_i = sum_h Wgu[i,h] x_h,  u_i = sum_h Wgu[I+i,h] x_h,
 *   m_i = silu(g_i) * u_i = g_i / (1 + exp(-g_i)) * u_i,
 *   y_h = sum_i Wd[h,i] m_i. */
void oracle_expert_ffn(int fmt, int H, int Iexp,
                       const uint8_t* w_gate_up, const void* s_gate_up,
                       const uint8_t* w_down, const void* s_down,
                       const double* x, double* y, double* mid_out) {
  double* mid = (double*)malloc(sizeof(double) * (size_t)Iexp);
  if (!mid) abort();
#pragma omp parallel for schedule(static)
  for (int i = 0; i < Iexp; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) g += oracle_weight(fmt, w_gate_up, s_gate_up, 2 * Iexp, H, i, h) * x[h];
    for (int h = 0; h < H; ++h) u += oracle_weight(fmt, w_gate_up, s_gate_up, 2 * Iexp, H, Iexp + i, h) * x[h];
    mid[i] = g / (1.0 + exp(-g)) * u;
  }
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    double acc = 0.0;
    for (int i = 0; i < Iexp; ++i) acc += oracle_weight(fmt, w_down, s_down, H, Iexp, h, i) * mid[i];
    y[h] = acc;
  }
  if (mid_out) memcpy(mid_out, mid, sizeof(double) * (size_t)Iexp);
  free(mid);
}

/* ------------------------------------------------------------------------ */
/* The layer.                                                                */
/* ------------------------------------------------------------------------ */

/* out[r,:] = y_shared(x_r) + sum_{p=0..K-1} w[r,p] * y_{ids[r,p]}(x_r), in
 * fp64 with the shared term first, then rounded once to bf16 (the hotspot
 * page: fp32-or-better accumulation, bf16 written once; the shared expert is
 * applied to every token with weight 1).
 * Expert parallelism (the expert-parallel all-to-all backends the hotspot
 * page mentions): with a range of held experts, the sum runs over the picks
 * inside it only, in the same order; the full layer is the sum of the
 * shares of a partition of the experts, the shared term counted in one. */
int oracle_forward_rows(const oracle_cfg* cfg, const uint16_t* x, int T,
                        const int32_t* rows, int nrows,
                        const uint16_t* router_w, const void* bias,
                        const uint8_t* const* w_gate_up, const void* const* s_gate_up,
                        const uint8_t* const* w_down, const void* const* s_down,
                        const uint8_t* sh_w_gate_up, const float* sh_s_gate_up,
                        const uint8_t* sh_w_down, const float* sh_s_down,
                        double* out64, uint16_t* out_bf16, int nthreads) {
  if (!cfg_ok(cfg) || T < 0) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int H = cfg->hidden, K = cfg->top_k, I = cfg->inter;
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  double* acc = (double*)malloc(sizeof(double) * (size_t)H);
  if (!xr || !y || !acc) return -1;
  int rc = 0;
  for (int ri = 0; ri < nrows && rc == 0; ++ri) {
    const int r = rows[ri];
    if (r < 0 || r >= T) { rc = -1; break; }
    int32_t ids[8];
    double w[8];
    if (oracle_route(cfg, x + (size_t)r * H, 1, router_w, bias, ids, w, NULL, NULL)) { rc = -1; break; }
    for (int h = 0; h < H; ++h) {
      xr[h] = oracle_dec_bf16(x[(size_t)r * H + h]);
      acc[h] = 0.0;
    }
    if (cfg->n_shared) {
      oracle_expert_ffn(ORACLE_FMT_FP8_B128, H, cfg->shared_inter, sh_w_gate_up, sh_s_gate_up,
                        sh_w_down, sh_s_down, xr, y, NULL);
      for (int h = 0; h < H; ++h) acc[h] = y[h];
    }
    const int e_lo = cfg->expert_first;
    const int e_hi = cfg->expert_count ? cfg->expert_first + cfg->expert_count : cfg->n_experts;
    for (int p = 0; p < K; ++p) {
      const int e = ids[p];
      if (e < e_lo || e >= e_hi) continue; /* another device's expert */
      if (!w_gate_up[e] || !s_gate_up[e] || !w_down[e] || !s_down[e]) { rc = -2; break; }
      oracle_expert_ffn(cfg->routed_fmt, H, I, w_gate_up[e], s_gate_up[e], w_down[e], s_down[e],
                        xr, y, NULL);
      for (int h = 0; h < H; ++h) acc[h] += w[p] * y[h];
    }
    for (int h = 0; h < H; ++h) {
      if (out64) out64[(size_t)r * H + h] = acc[h];
      if (out_bf16) out_bf16[(size_t)r * H + h] = oracle_bf16_rne(acc[h]);
    }
  }
  free(xr);
  free(y);
  free(acc);
  return rc;
}

int oracle_forward(const oracle_cfg* cfg, const uint16_t* x, int T,
                   const uint16_t* router_w, const void* bias,
                   const uint8_t* const* w_gate_up, const void* const* s_gate_up,
                   const uint8_t* const* w_down, const void* const* s_down,
                   const uint8_t* sh_w_gate_up, const float* sh_s_gate_up,
                   const uint8_t* sh_w_down, const float* sh_s_down,
                   double* out64, uint16_t* out_bf16,
                   int32_t* ids, double* w, int nthreads) {
  if (!cfg_ok(cfg) || T < 0) return -1;
  if (ids && w) {
    if (oracle_route(cfg, x, T, router_w, bias, ids, w, NULL, NULL)) return -1;
  }
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!rows) return -1;
  for (int r = 0; r < T; ++r) rows[r] = r;
  int rc = oracle_forward_rows(cfg, x, T, rows, T, router_w, bias, w_gate_up, s_gate_up,
                               w_down, s_down, sh_w_gate_up, sh_s_gate_up, sh_w_down,
                               sh_s_down, out64, out_bf16, nthreads);
  free(rows);
  return rc;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
