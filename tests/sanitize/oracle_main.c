/* The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: routing,
 * grouping and the whole layer on small seeded cases (FP8 and MXFP4 routed
 * experts, grouped and plain routing, an expert range), every output
 * finite.  Prints "ok". */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) {
  st ^= st << 13; st ^= st >> 7; st ^= st << 17;
  return (uint32_t)(st >> 11);
}
/* a bf16 near N(0, sd): a uniform sum, enough for a finite, varied input */
static uint16_t bf16_of(double v) { return oracle_bf16_rne(v); }
static double unif(void) { return (rnd() & 0xffffff) / 16777216.0 - 0.5; }
static uint8_t fp8_code(void) {
  uint8_t c = (uint8_t)(rnd() & 0xff);
  return (c & 0x7f) == 0x7f ? (uint8_t)(c ^ 1) : c; /* no NaN codes */
}

static int run(int fmt, int T, int ng, int kg, int first, int count) {
  oracle_cfg c;
  memset(&c, 0, sizeof c);
  c.hidden = fmt ? 512 : 384; c.inter = fmt ? 256 : 128; c.shared_inter = 128; c.n_experts = 16;
  c.top_k = 4; c.n_group = ng; c.topk_group = kg; c.n_shared = 1; c.routed_scale = 2.5;
  c.routed_fmt = fmt; c.bias_bf16 = fmt; c.expert_first = first; c.expert_count = count;
  const int H = c.hidden, I = c.inter, Is = c.shared_inter, E = c.n_experts, K = c.top_k;
  uint16_t* x = malloc(sizeof(uint16_t) * T * H);
  uint16_t* rw = malloc(sizeof(uint16_t) * E * H);
  float* bias = malloc(sizeof(float) * E);
  uint16_t* bias16 = malloc(sizeof(uint16_t) * E);
  for (int i = 0; i < T * H; ++i) x[i] = bf16_of(2.0 * unif());
  for (int i = 0; i < E * H; ++i) rw[i] = bf16_of(unif() / sqrt((double)H));
  for (int e = 0; e < E; ++e) { bias[e] = (float)(0.2 * unif()); bias16[e] = bf16_of(bias[e]); }
  const uint8_t* wgu[16]; const void* sgu[16]; const uint8_t* wd[16]; const void* sd[16];
  void* keep[64]; int nk = 0;
  for (int e = 0; e < E; ++e) {
    size_t ngu = fmt ? (size_t)2 * I * H / 2 : (size_t)2 * I * H, nd = fmt ? (size_t)H * I / 2 : (size_t)H * I;
    uint8_t* a = malloc(ngu); uint8_t* b = malloc(nd);
    for (size_t i = 0; i < ngu; ++i) a[i] = fmt ? (uint8_t)rnd() : fp8_code();
    for (size_t i = 0; i < nd; ++i) b[i] = fmt ? (uint8_t)rnd() : fp8_code();
    void *s1, *s2;
    if (fmt) {
      size_t n1 = (size_t)2 * I * H / 32, n2 = (size_t)H * I / 32;
      uint8_t* p1 = malloc(n1); uint8_t* p2 = malloc(n2);
      for (size_t i = 0; i < n1; ++i) p1[i] = (uint8_t)(120 + rnd() % 4);
      for (size_t i = 0; i < n2; ++i) p2[i] = (uint8_t)(120 + rnd() % 4);
      s1 = p1; s2 = p2;
    } else {
      size_t n1 = (size_t)(2 * I / 128) * (H / 128), n2 = (size_t)(H / 128) * (I / 128);
      float* p1 = malloc(4 * n1); float* p2 = malloc(4 * n2);
      for (size_t i = 0; i < n1; ++i) p1[i] = 1.0f / 1024;
      for (size_t i = 0; i < n2; ++i) p2[i] = 1.0f / 1024;
      s1 = p1; s2 = p2;
    }
    wgu[e] = a; wd[e] = b; sgu[e] = s1; sd[e] = s2;
    keep[nk++] = a; keep[nk++] = b; keep[nk++] = s1; keep[nk++] = s2;
  }
  uint8_t* shgu = malloc((size_t)2 * Is * H); uint8_t* shd = malloc((size_t)H * Is);
  float* shs1 = malloc(4 * (size_t)(2 * Is / 128) * (H / 128)); float* shs2 = malloc(4 * (size_t)(H / 128) * (Is / 128));
  for (int i = 0; i < 2 * Is * H; ++i) shgu[i] = fp8_code();
  for (int i = 0; i < H * Is; ++i) shd[i] = fp8_code();
  for (int i = 0; i < (2 * Is / 128) * (H / 128); ++i) shs1[i] = 1.0f / 1024;
  for (int i = 0; i < (H / 128) * (Is / 128); ++i) shs2[i] = 1.0f / 1024;
  const void* bp = fmt ? (const void*)bias16 : (const void*)bias;
  int32_t* ids = malloc(sizeof(int32_t) * T * K);
  double* w = malloc(sizeof(double) * T * K);
  double* ge = malloc(sizeof(double) * T); double* gg = malloc(sizeof(double) * T);
  int rc = oracle_route(&c, x, T, rw, bp, ids, w, ge, gg);
  if (rc) return 10 + rc;
  int32_t G = 0, gexp[1 + 64 * 8], gn[1 + 64 * 8], gs[1 + 64 * 8], cols[64 * 9], ug[64 * 8];
  rc = oracle_groups(&c, T, ids, &G, gexp, gn, gs, cols, ug);
  if (rc) return 20 + rc;
  double* o64 = malloc(sizeof(double) * T * H);
  uint16_t* ob = malloc(sizeof(uint16_t) * T * H);
  int32_t* rows = malloc(sizeof(int32_t) * T);
  for (int r = 0; r < T; ++r) rows[r] = T - 1 - r;
  rc = oracle_forward_rows(&c, x, T, rows, T, rw, bp, wgu, sgu, wd, sd, shgu, shs1, shd, shs2, o64, ob, 2);
  if (rc) return 30 + rc;
  for (int i = 0; i < T * H; ++i)
    if (!isfinite(o64[i])) return 40;
  for (int i = 0; i < nk; ++i) free(keep[i]);
  free(x); free(rw); free(bias); free(bias16); free(shgu); free(shd); free(shs1); free(shs2);
  free(ids); free(w); free(ge); free(gg); free(o64); free(ob); free(rows);
  return 0;
}

int main(void) {
  int rc;
  if ((rc = run(0, 5, 4, 2, 0, 0))) { fprintf(stderr, "fp8 grouped: %d\n", rc); return 1; }
  if ((rc = run(0, 3, 1, 1, 4, 8))) { fprintf(stderr, "fp8 expert range: %d\n", rc); return 1; }
  if ((rc = run(1, 4, 1, 1, 0, 0))) { fprintf(stderr, "mxfp4: %d\n", rc); return 1; }
  printf("ok\n");
  return 0;
}
