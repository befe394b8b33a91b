/*
 * moe_oracle.h -- plain fp64 CPU oracle of the small-batch decode MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this library: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP path under mixture_experts_decode_sigmoid_amd/csrc.
 *
 * What it computes is the layer's plain definition:
 *   - "Daily AI Hotspot 2026-08-21" (naphjohn LLM-blog), section "Most Worth
 *     Your Attention Today": a DeepSeek-V4-family MoE layer runs a routed
 *     expert path and a shared expert that every token goes through; the
 *     fused kernel accumulates in fp32 and writes the bf16 output once.  The
 *     same section names the MI355X-side fix: the correction bias may be
 *     bf16 and top-k may be 6 (not a power of two).
 *   - sgl-amd-mono-upstream PR #27 ("each expert once in up/gate and down"),
 *     sections Motivation and Modifications: per row, every routed pick and
 *     the shared expert is a (row, expert) use; up/gate then down per use;
 *     the grouped form must give each row what its one-row form gives.
 * The routing rule (sigmoid score, additive correction bias used only for
 * selection, node-limited group stage, normalised weights times a scale) is
 * the published DeepSeek-V3 rule; the pages name only the bias and top-k.
 * Every reading of a point the pages leave open is listed with the function
 * that makes it.
 *
 * All arithmetic is IEEE fp64.  Weight formats are decoded from their
 * published bit definitions (OCP 8-bit floating point E4M3FN; OCP MX v1.0
 * E2M1 elements with E8M0 block scales).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. */
enum { ORACLE_FMT_FP8_B128 = 0, ORACLE_FMT_MXFP4 = 1 };

typedef struct {
  int hidden;        /* H */
  int inter;         /* I, routed expert intermediate size */
  int shared_inter;  /* I_s, shared expert intermediate size */
  int n_experts;     /* E */
  int top_k;         /* K */
  int n_group;       /* n_g; 1 = ungrouped */
  int topk_group;    /* k_g groups kept */
  int n_shared;      /* 0 or 1 */
  double routed_scale;
  int routed_fmt;    /* ORACLE_FMT_*; the shared expert is always FP8_B128 */
  int bias_bf16;     /* 0: bias is fp32[E]; 1: bias is bf16[E] */
  /* Expert parallelism: the routed experts this evaluation holds are
   * expert_first .. expert_first + expert_count - 1 (count 0: all E).  Rows
   * are routed over all E experts; picks outside the range contribute
   * nothing here (another device's share of the layer). */
  int expert_first;
  int expert_count;
} oracle_cfg;

/* ---- format decode (one code -> exact fp64 value) ---- */
double oracle_dec_bf16(uint16_t bits);
double oracle_dec_e4m3(uint8_t code);
double oracle_dec_e2m1(uint8_t nibble);      /* low 4 bits used */
double oracle_dec_e8m0(uint8_t code);
uint16_t oracle_bf16_rne(double v);          /* fp64 -> bf16, round to nearest even */

/* One dequantised weight element W[n,k] of an [N,K] weight (K contiguous). */
double oracle_weight(int fmt, const uint8_t* q, const void* scale, int N, int K,
                     int n, int k);

/* ---- routing ---- */
/* Scores of one row: logits[E], s[E] = sigmoid(logit), b[E] = s + bias. */
void oracle_scores(const oracle_cfg* cfg, const uint16_t* x_row,
                   const uint16_t* router_w, const void* bias,
                   double* logits, double* s, double* b);

/* Routes T rows.  ids[T*K] in selection order, w[T*K] fp64.  Optional
 * diagnostics (may be NULL): gap_expert[T] = b of the K-th pick minus the
 * best b left out among kept groups (+inf when none is left), gap_group[T] =
 * group score of the k_g-th kept group minus the best dropped one (+inf
 * when ungrouped).  Returns 0, or -1 on a bad configuration. */
int oracle_route(const oracle_cfg* cfg, const uint16_t* x, int T,
                 const uint16_t* router_w, const void* bias,
                 int32_t* ids, double* w, double* gap_expert, double* gap_group);

/* Distinct-expert grouping of one step.  Group 0 is the shared expert
 * (expert id -1) when n_shared == 1; routed groups follow in order of first
 * use over the flat use index u = r*K + p.  Outputs:
 *   *n_groups, group_expert[G], group_ncols[G], group_col_start[G],
 *   cols[...] = r*16 + slot, slot K meaning the shared expert, listed per
 *   group in ascending u; use_group[T*K] = group of each routed use.
 * Arrays must hold 1 + T*K groups and T*(K+1) columns. */
int oracle_groups(const oracle_cfg* cfg, int T, const int32_t* ids,
                  int32_t* n_groups, int32_t* group_expert, int32_t* group_ncols,
                  int32_t* group_col_start, int32_t* cols, int32_t* use_group);

/* ---- expert FFN ---- */
/* y[H] = down( silu(gate(x)) * up(x) ) for one expert, x[H] fp64. */
void oracle_expert_ffn(int fmt, int H, int Iexp,
                       const uint8_t* w_gate_up, const void* s_gate_up,
                       const uint8_t* w_down, const void* s_down,
                       const double* x, double* y, double* mid_out);

/* ---- the layer ---- */
/* Routed weights are given per expert (arrays of E pointers; an expert no
 * row uses may be NULL).  out64[T*H] (may be NULL) and out_bf16[T*H].
 * ids/w (may be NULL) receive the routing.  nthreads <= 0: OpenMP default.
 * Returns 0, -1 on a bad configuration, -2 if a used expert is NULL. */
int oracle_forward(const oracle_cfg* cfg, const uint16_t* x, int T,
                   const uint16_t* router_w, const void* bias,
                   const uint8_t* const* w_gate_up, const void* const* s_gate_up,
                   const uint8_t* const* w_down, const void* const* s_down,
                   const uint8_t* sh_w_gate_up, const float* sh_s_gate_up,
                   const uint8_t* sh_w_down, const float* sh_s_down,
                   double* out64, uint16_t* out_bf16,
                   int32_t* ids, double* w, int nthreads);

/* Same layer for a subset of rows: only rows listed in rows[nrows] are
 * computed (routing of those rows only); out rows are written at the same
 * positions [rows[i]*H ...].  Used to check full-size runs on samples. */
int oracle_forward_rows(const oracle_cfg* cfg, const uint16_t* x, int T,
                        const int32_t* rows, int nrows,
                        const uint16_t* router_w, const void* bias,
                        const uint8_t* const* w_gate_up, const void* const* s_gate_up,
                        const uint8_t* const* w_down, const void* const* s_down,
                        const uint8_t* sh_w_gate_up, const float* sh_s_gate_up,
                        const uint8_t* sh_w_down, const float* sh_s_down,
                        double* out64, uint16_t* out_bf16, int nthreads);

int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
