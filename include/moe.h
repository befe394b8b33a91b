/*
 * moe.h -- C ABI of the fused small-batch decode MoE layer for MI355X (gfx950).
 *
 * The layer (one decode step of a DeepSeek-V3/V4-style MoE block):
 *   for each row r of x:
 *     route:  logits l = x_r . Wr^T, scores s = sigmoid(l), keys b = s + bias;
 *             optional group stage (keep the k_g groups with the largest sum of
 *             their two best keys), then the top-K keys; weights
 *             w = s / sum(s of the K picks) * routed_scale;
 *     expert: y_e(x) = W_down_e ( silu(W_gate_e x) * (W_up_e x) );
 *     out_r = y_shared(x_r) + sum_p w_p * y_{id_p}(x_r), fp32 sum, bf16 out.
 * Sources (by page and section):
 *   - "Daily AI Hotspot 2026-08-21" (naphjohn LLM-blog), "Most Worth Your
 *     Attention Today": the routed experts plus a shared expert every token
 *     passes through, fused into one persistent pass that accumulates in fp32
 *     and writes the bf16 output exactly once; on MI355X the correction bias
 *     may be bf16 and top-k may be 6.
 *   - sgl-amd-mono-upstream PR #27, Motivation and Modifications (commit 1
 *     "each expert once in up/gate and down", commit 2 "dead-batch skip"): the
 *     step's distinct experts are found from the top-k picks, each is streamed
 *     once in up/gate and in down with every using row as an MFMA column, and
 *     each row's output is summed in a fixed, row-local order.
 *
 * Conventions
 *   - Every pointer argument is device memory owned by the caller unless a
 *     comment says "host".  Nothing is allocated, freed or synchronised on the
 *     forward path; every call is asynchronous on `stream` (a hipStream_t,
 *     NULL = default stream).
 *   - The return code reports host-side validation and the launch only.
 *     Problems found on the device set bits of an error word in the workspace;
 *     read them with moe_read_error().
 *   - Tensors are row-major and contiguous; bf16 values are passed as their
 *     16-bit patterns (uint16_t).  Pointers must be 16-byte aligned.
 *   - Weight formats (weights are [N, K] with K, the reduction axis,
 *     contiguous; N = output features):
 *       MOE_FMT_FP8_B128: one byte per element, OCP FP8 E4M3FN; one fp32 scale
 *         per 128x128 block, scale grid [N/128][K/128]; element =
 *         e4m3(q[n][k]) * s[n/128][k/128].
 *       MOE_FMT_MXFP4: OCP MX FP4 (E2M1), two elements per byte, element k in
 *         the low nibble when k is even; one E8M0 scale byte per 32
 *         consecutive k, scale grid [N][K/32]; element =
 *         e2m1(q) * 2^(s - 127).
 *     W_gate_up of an expert is [2*Iexp, H]: rows 0..Iexp-1 project to the
 *     gate, rows Iexp..2*Iexp-1 to the up half.  W_down is [H, Iexp].
 *   - A workspace belongs to one stream at a time: calls that overlap on the
 *     device must use different workspaces.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
#define MOE_OK 0
#define MOE_ERR_NULL 1      /* a required pointer is NULL */
#define MOE_ERR_SHAPE 2     /* sizes outside what the kernels support */
#define MOE_ERR_FORMAT 3    /* unknown weight format or bias dtype */
#define MOE_ERR_ALIGN 4     /* a pointer is not 16-byte aligned */
#define MOE_ERR_ROWS 5      /* rows < 0, rows > max_rows, or max_rows > 64 */
#define MOE_ERR_WORKSPACE 6 /* workspace too small or not initialised */
#define MOE_ERR_ALIAS 7     /* out overlaps x, or a residual overlaps out without being it */
#define MOE_ERR_HIP 8       /* a HIP runtime call failed; see moe_last_hip_error() */

/* ---- device error bits (moe_read_error) ---- */
#define MOE_DEVERR_NONFINITE_SCORE 0x1u /* a router logit/score was not finite */
#define MOE_DEVERR_NONFINITE_MID 0x2u   /* an up/gate or down sum was not finite:
                                           a NaN weight code or E8M0 0xFF in a used
                                           expert, or a non-finite activation */
#define MOE_DEVERR_WAIT_TIMEOUT 0x4u    /* a cross-workgroup wait gave up; the
                                           output of that call is undefined and the
                                           workspace must be re-initialised */

typedef enum { MOE_FMT_FP8_B128 = 0, MOE_FMT_MXFP4 = 1 } moe_wfmt;
typedef enum { MOE_BIAS_F32 = 0, MOE_BIAS_BF16 = 1 } moe_bias_dtype;

/* Layer description (host struct). */
typedef struct {
  int hidden;        /* H: multiple of 128, 128..8192 */
  int inter;         /* I: routed expert intermediate, multiple of 128, <= 4096 */
  int shared_inter;  /* I_s: shared expert intermediate, multiple of 128, <= 4096 */
  int n_experts;     /* E: 1..256 */
  int top_k;         /* K: 1..8 and <= E (any K, not only powers of two) */
  int n_group;       /* n_g: 1 = ungrouped; must divide E with E/n_g >= 2, n_g <= 64 */
  int topk_group;    /* k_g: groups kept, 1..n_g, with k_g * E/n_g >= K */
  int n_shared;      /* 0 or 1 shared expert (weight 1, every row) */
  float routed_scale;/* multiplies the normalised routed weights (2.5 for V3) */
  int routed_fmt;    /* moe_wfmt of the routed experts */
  int shared_fmt;    /* moe_wfmt of the shared expert: MOE_FMT_FP8_B128 only */
  int bias_dtype;    /* moe_bias_dtype */
  int max_rows;      /* largest rows a call will pass; sizes the workspace; <= 64 */
} moe_config;

/* Weights (host struct of device pointers). */
typedef struct {
  const uint16_t* router_w;   /* [E, H] bf16 */
  const void* bias;           /* [E] fp32 or bf16 (bias_dtype) */
  const uint8_t* w_gate_up;   /* [E, 2I, H] FP8, or [E, 2I, H/2] MXFP4 */
  const void* s_gate_up;      /* [E, 2I/128, H/128] fp32, or [E, 2I, H/32] E8M0 bytes */
  const uint8_t* w_down;      /* [E, H, I] FP8, or [E, H, I/2] MXFP4 */
  const void* s_down;         /* [E, H/128, I/128] fp32, or [E, H, I/32] E8M0 bytes */
  const uint8_t* sh_w_gate_up;/* [2I_s, H] FP8 (n_shared == 1) */
  const float* sh_s_gate_up;  /* [2I_s/128, H/128] fp32 */
  const uint8_t* sh_w_down;   /* [H, I_s] FP8 */
  const float* sh_s_down;     /* [H/128, I_s/128] fp32 */
} moe_weights;

/* Bytes of device workspace a configuration needs (host call, no device work).
 * Returns MOE_OK, MOE_ERR_NULL or a validation code. */
int moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Initialises a workspace: clears all ws_bytes of it (the cross-workgroup
 * flags, the error word and the epoch-tagged score slots).  Call once after
 * allocating it (stream-ordered, asynchronous). */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Routing only: writes topk_ids[rows, K] (int32, in selection order: key
 * descending, lower expert index first on an exact tie) and topk_w[rows, K]
 * (fp32).  Runs the same device code as the first stage of moe_forward. */
int moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Routing and distinct-expert grouping only (the table each workgroup builds
 * in LDS), written to groups_out (int32, capacity 4 + 3*(1 + rows*K) +
 * rows*(K+1) entries):
 *   [0] = G, [1] = rows, [2] = K, [3] = n_shared,
 *   then expert[G] (-1 for the shared group), ncols[G], col_start[G],
 *   then cols[sum ncols] = row*16 + slot (slot K = the shared expert).
 * Groups: the shared expert first (if any), then routed experts in order of
 * first use over u = row*K + slot; a group's columns in ascending u. */
int moe_groups(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
               int32_t* groups_out, void* ws, size_t ws_bytes, void* stream);

/* The fused layer: out[rows, H] bf16.  One persistent launch (one workgroup
 * per CU, all resident) that routes, groups the step's distinct experts,
 * streams each used expert's weights once through up/gate and down, and
 * writes each row once.  rows == 0 is a no-op.  out must not overlap x. */
int moe_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* The fused layer with the residual add folded into its combine:
 * out[r, h] = bf16_RNE(P_shared + sum_p w[r,p] * P[r,p,h] + residual[r, h]),
 * the residual (bf16, [rows, H], row-major) added in fp32 after the same
 * fixed-order chain moe_forward forms, then rounded once.  This is the
 * fourth launch of the unfused layout (the "add" after the routed and the
 * shared expert paths) that the fused kernel absorbs, as described in
 * "Daily AI Hotspot 2026-08-21: Shared-Expert Fusion Lands on NVIDIA and AMD
 * the Same Day", section "Most Worth Your Attention Today".
 * residual is device memory the caller owns; it may be out itself (in-place
 * add: each element is read before it is written, by the same thread) but
 * may not overlap out otherwise (MOE_ERR_ALIAS); NULL with rows > 0 gives
 * MOE_ERR_NULL.  Everything else is as for moe_forward. */
int moe_forward_residual(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                         const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* Waits for `stream`, then returns the workspace's device error bits in
 * *bits (host) and clears them. */
int moe_read_error(void* ws, void* stream, uint32_t* bits);

/* Text of a return code (static string). */
const char* moe_strerror(int code);

/* The HIP error code behind the last MOE_ERR_HIP on this thread. */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif
