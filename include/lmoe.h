/*
 * lmoe.h -- C ABI of the Stable Latent MoE layer forward pass on MI355X (gfx950).
 *
 * The layer (one MoE feed-forward block of a decoder) computes, per token:
 *   1. router: scores s = sigmoid(x . W_r^T) over E routed experts; the k experts
 *      with the largest s + b are selected (b: per-expert bias, used for the
 *      selection only); their scores, renormalised to sum 1, are the combine
 *      weights;
 *   2. latent down-projection z = x . W_dn^T (hidden H -> latent L);
 *   3. tokens grouped per expert; each selected expert runs a gated FFN on z with
 *      the SiTU-GLU activation silu(cap(g)) * cap(v), cap(u) = c * tanh(u / c);
 *   4. weighted combine of the k expert outputs, then RMSNorm with gain gamma;
 *   5. up-projection back to H, plus S always-on shared experts (full width, on x).
 * The residual add is left to the caller.
 *
 * Sources -- the pages describe the layer in prose only:
 *   P1 aitrending.vip, "The 2.8-Trillion-Parameter Problem: Why Bigger Models
 *      Break the Old Playbook", TL;DR and Technical Details bullets (896 routed
 *      experts, 16 active, 2 shared; 7168 -> 3584 latent; SiTU-GLU caps gate and
 *      value to about +-100; RMSNorm before the up-projection);
 *   P2 wpnews.pro, same title (Part 1 of "Inside Kimi K3"): the MoE passage, the
 *      Stable LatentMoE passage (compress before dispatch, experts work in the
 *      latent, outputs combined then projected back; residual stays full width)
 *      and the stabilizer passage (RMSNorm right before the up-projection;
 *      SiTU-GLU bounds gate and value branches, SwiGLU-like near zero);
 *   P3 daily-ai-frontier, "苏神复盘 Kimi K3：896 个专家背后，藏着哪些关键技术取舍？",
 *      Merged summary, LatentMoE and Stable LatentMoE bullets (norm after expert
 *      aggregation and before the up-projection; shared experts always on; soft
 *      cap against BF16/FP8 range blow-up).
 * Choices the pages leave open (scoring function, combine weights, tie order,
 * SiTU-GLU formula, eps, expert width, shared width, fp8 layout) are fixed as
 * stated at each declaration below.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major [out, in] (weights) and [rows, cols] (activations).
 *   - Every tensor pointer is a device pointer owned by the caller.  The library
 *     never allocates or frees device memory; scratch comes from `ws`, a caller
 *     buffer of at least lmoe_workspace_bytes(shape) bytes, 256-byte aligned.
 *   - Weight matrices, activations and gradients move through 16-byte vector
 *     loads, DMAs and stores: their base pointers must be 16-byte aligned
 *     (LMOE_EINVAL otherwise, the message naming the pointer); scale, bias,
 *     gamma, index and routing-weight arrays need only their element size.
 *   - Inputs are read only.  Outputs must not alias inputs or each other.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream) and never synchronise with the host; no work depends on a
 *     host-side copy of device data.
 *   - The return value reports argument validation (LMOE_EINVAL, LMOE_EUNSUPPORTED
 *     for a shape/dtype combination with no kernel -- there is no fallback,
 *     LMOE_EWORKSPACE) and launch failures (LMOE_EHIP).  A fault inside a kernel
 *     surfaces at the caller's next synchronisation.  lmoe_last_error() returns a
 *     message for the calling thread's last failure.  No C++ exception crosses
 *     the ABI.  Per call the library keeps no state outside the caller's
 *     workspace: calls on different streams are independent if their
 *     workspaces differ.  Process-wide it caches, once per device, host-side
 *     facts (the compute-unit count, kernel launch attributes, the address of
 *     lmoe_forward_noalloc's scratch), each written once under a once-flag or
 *     a lock; lmoe_forward_noalloc shares one scratch array per device.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_EINVAL = 1,        /* null pointer, negative or inconsistent sizes       */
  LMOE_EUNSUPPORTED = 2,  /* valid layer, but no kernel for this shape / dtype  */
  LMOE_EWORKSPACE = 3,    /* ws_bytes below lmoe_workspace_bytes(shape)         */
  LMOE_EHIP = 4           /* a HIP launch or attribute call failed              */
} lmoe_status;

typedef enum {
  LMOE_F32 = 0,           /* IEEE binary32                                       */
  LMOE_BF16 = 1,          /* bfloat16                                           */
  LMOE_F8E4M3 = 2         /* OCP e4m3fn (bias 7, max 448, no inf), weights only  */
} lmoe_dtype;

/* Layer shape.  act: dtype of x, y, the router / down / up weights and every
 * activation the library writes (z, n, expert outputs): LMOE_F32 or LMOE_BF16.
 * w_expert: dtype of the routed and shared expert FFN weights: LMOE_F32 with an
 * F32 layer, LMOE_BF16 or LMOE_F8E4M3 with a BF16 layer.  cap: SiTU-GLU cap c
 * (> 0; +inf turns the cap off, giving SwiGLU).  rms_eps: RMSNorm epsilon (>= 0).
 * Supported sizes: H, L, I, Is multiples of 64 (of 128 with F8E4M3 weights),
 * L <= 8192, 1 <= k <= min(E, 64), E <= 1024, 0 <= S <= 8, T * k < 2^31.        */
typedef struct {
  int64_t T;              /* tokens (0 is a valid, empty call)                  */
  int32_t H;              /* hidden width                                        */
  int32_t L;              /* latent width                                        */
  int32_t E;              /* routed experts                                      */
  int32_t k;              /* experts selected per token                          */
  int32_t I;              /* routed expert intermediate width                    */
  int32_t S;              /* shared experts                                      */
  int32_t Is;             /* shared expert intermediate width                    */
  int32_t act;            /* lmoe_dtype                                          */
  int32_t w_expert;       /* lmoe_dtype                                          */
  float cap;              /* SiTU-GLU cap, 100 in the K3 layer                   */
  float rms_eps;          /* RMSNorm epsilon, 1e-6                               */
  int32_t a8;             /* 0: the routed experts multiply act-dtype activations
                             (W8A16 with F8E4M3 weights).  1: W8A8 -- z and the
                             SiTU-GLU output are quantised per token per 128
                             columns to e4m3fn (see lmoe_quantize_1x128), from
                             their fp32 values as the GEMMs accumulate them
                             (lmoe_expert_gemm: from z as given), and the
                             routed expert GEMMs multiply e4m3 by e4m3, with fp32
                             accumulation and the block scales applied once per
                             128 columns.  Needs act BF16 and w_expert F8E4M3
                             (P3 merged summary: the BF16/FP8 range problem;
                             the format is this library's reading).  Weight and
                             activation scales must be positive and finite.    */
} lmoe_shape;

/* Weights.  Expert stacks are [E, I, L] (gate, value) and [E, L, I] (out);
 * shared stacks [S, Is, H] (gate, value) and [S, H, Is] (out).  With F8E4M3
 * expert weights every expert matrix carries one fp32 scale per 128x128 block,
 * row-major over blocks: s_gate [E, I/128, L/128], s_value [E, I/128, L/128],
 * s_out [E, L/128, I/128], ss_gate/ss_value [S, Is/128, H/128], ss_out
 * [S, H/128, Is/128]; the weight value is code * scale.  Scale pointers are
 * ignored for other dtypes.  w_down = NULL and w_up = NULL select identity
 * projections (a MoE with no latent; needs L == H).                              */
typedef struct {
  const void *w_router;   /* [E, H]  act dtype                                  */
  const float *b_router;  /* [E]     selection bias                             */
  const void *w_down;     /* [L, H]  act dtype, or NULL                         */
  const void *w_gate;     /* [E, I, L] w_expert dtype                            */
  const void *w_value;    /* [E, I, L]                                          */
  const void *w_out;      /* [E, L, I]                                          */
  const float *s_gate, *s_value, *s_out;
  const float *gamma;     /* [L]     RMSNorm gain                               */
  const void *w_up;       /* [H, L]  act dtype, or NULL                         */
  const void *ws_gate;    /* [S, Is, H] w_expert dtype (NULL when S == 0)        */
  const void *ws_value;   /* [S, Is, H]                                         */
  const void *ws_out;     /* [S, H, Is]                                         */
  const float *ss_gate, *ss_value, *ss_out;
  const void *packed;     /* NULL, or the routed expert weights in the packed
                             layout of lmoe_pack_experts (BF16 layers with BF16
                             expert weights); when set, the expert GEMMs read
                             it instead of w_gate / w_value / w_out, which may
                             then be NULL                                       */
} lmoe_weights;

/* Host-only argument check (no GPU call): the checks every entry point runs
 * first, for the whole layer.  ws_bytes is compared with the requirement.     */
lmoe_status lmoe_validate(const lmoe_shape *shape, const lmoe_weights *w, size_t ws_bytes);

/* Workspace bytes that suffice for every entry point below at this shape;
 * 0 for an invalid shape.                                                      */
size_t lmoe_workspace_bytes(const lmoe_shape *shape);

/* Whole layer: y[T, H] (act dtype) = up(RMSNorm(combine(experts(z)))) + shared(x)
 * for x[T, H] (P2 Stable LatentMoE and stabilizer passages; P3 Stable LatentMoE
 * bullet).  topk_idx [T, k] int32 and topk_w [T, k] fp32 receive the selection
 * and combine weights if not NULL.  stage_events: NULL, or an array of
 * LMOE_NUM_STAGES + 1 hipEvent_t recorded on `stream` before the first stage
 * and after each stage (route GEMM, top-k, permute, expert gate/value GEMM,
 * expert down GEMM, combine + norm, up GEMM), for timing.  Part of the route
 * GEMM (its last round of shared-expert tiles) may run on a library-owned side
 * stream of the device, forked from `stream` after the route GEMM's main launch
 * and joined back before the up GEMM, so all the layer's work precedes what is
 * enqueued on `stream` after the call; the route GEMM's stage event then
 * covers its main launch only.                                                 */
#define LMOE_NUM_STAGES 7
lmoe_status lmoe_forward(const lmoe_shape *shape, const lmoe_weights *w, const void *x, void *y,
                         int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                         void *stream, void *const *stage_events);

/* The whole layer as lmoe_forward, for callers that cannot allocate device
 * memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Scratch comes from a
 * fixed array of LMOE_NOALLOC_SCRATCH_BYTES in the library's own device memory,
 * one per device, held from the first use on a device until the process ends
 * (at the K3 shape that covers up to about 350 tokens per call).  The call
 * allocates and frees nothing.  Arguments, outputs and results are those of
 * lmoe_forward (no stage events); LMOE_EWORKSPACE when
 * lmoe_workspace_bytes(shape) exceeds the array, LMOE_EUNSUPPORTED on a
 * device id of 64 or more.  Every call on one device shares that device's
 * array and leaves its contents behind (nothing in it needs to start at
 * zero): calls that overlap on one device -- on different streams, or from
 * different threads without ordering -- race on it and must not be issued.  */
#define LMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lmoe_status lmoe_forward_noalloc(const lmoe_shape *shape, const lmoe_weights *w, const void *x, void *y,
                                 int32_t *topk_idx, float *topk_w, void *stream);

/* Router and latent down-projection (P1 Technical Details; P2 MoE and Stable
 * LatentMoE passages).  One GEMM over x serves both: logits = x . W_r^T in fp32
 * (products of act-dtype operands, fp32 accumulation), z = x . W_dn^T (act
 * dtype; z = x when w_down is NULL, in which case z is not written and may be
 * NULL).  Then per token: s = sigmoid(logit) in fp32, the k largest s + b in
 * descending order, equal values ordered by ascending expert index, written to
 * topk_idx [T, k]; topk_w [T, k] = selected s / their sum.                       */
lmoe_status lmoe_route(const lmoe_shape *shape, const lmoe_weights *w, const void *x,
                       int32_t *topk_idx, float *topk_w, void *z, void *ws, size_t ws_bytes,
                       void *stream);

/* Group the T*k assignments a = t*k + j by expert with a stable counting sort:
 * offsets [E+1] (offsets[e]..offsets[e+1] is expert e's range), sorted [T*k]
 * (assignment ids, ascending token within an expert), pos [T*k] (inverse:
 * sorted[pos[a]] == a).  An id outside [0, E), or a repeat of an id already
 * listed earlier in the same token's row, is dropped: its pos is -1 and it is
 * in no expert's range.                                                        */
lmoe_status lmoe_permute(const lmoe_shape *shape, const int32_t *topk_idx, int32_t *offsets,
                         int32_t *sorted, int32_t *pos, void *ws, size_t ws_bytes, void *stream);

/* Routed experts on their latent rows (P2 stabilizer passage: gated FFN with
 * gate and value branches, SiTU-GLU).  For each expert e and each assignment in
 * its range, with t = sorted[i] / k: g = z[t] . W_g[e]^T, v = z[t] . W_v[e]^T,
 * a = silu(cap(g)) * cap(v) (fp32, rounded to act dtype), expert_out[i] =
 * a . W_o[e]^T (act dtype, [T*k, L], rows in sorted order).  z is [T, L]; pass
 * x when w_down is NULL.  Only offsets[0..E] and sorted are read; the number of
 * assignments handled is offsets[E].                                            */
lmoe_status lmoe_expert_gemm(const lmoe_shape *shape, const lmoe_weights *w, const void *z,
                             const int32_t *offsets, const int32_t *sorted, void *expert_out,
                             void *ws, size_t ws_bytes, void *stream);

/* Weighted combine and RMSNorm (P2 stabilizer passage; P3 Stable LatentMoE
 * bullet): c = sum over j ascending of topk_w[t, j] * expert_out[pos[t*k + j]]
 * (fp32; entries with pos < 0 skipped), n[t] = gamma * c / sqrt(mean(c^2) + eps)
 * in act dtype, [T, L].                                                         */
lmoe_status lmoe_combine_norm(const lmoe_shape *shape, const void *expert_out, const int32_t *pos,
                              const float *topk_w, const float *gamma, void *n, void *stream);

/* Up-projection and shared experts (P2 Stable LatentMoE passage; P1 Technical
 * Details; P3 LatentMoE bullet): y = n . W_up^T + sum_s SiTU-GLU-FFN_s(x), with
 * the shared experts at full width on x[T, H], weight 1; n is [T, L].           */
lmoe_status lmoe_up(const lmoe_shape *shape, const lmoe_weights *w, const void *n, const void *x,
                    void *y, void *ws, size_t ws_bytes, void *stream);

/* Router logits only: logits [T, E] fp32 = x . W_r^T (products of act-dtype
 * operands, fp32 accumulation), the first output of lmoe_route.  Needs
 * w_router only; no workspace.                                                */
lmoe_status lmoe_router_logits(const lmoe_shape *shape, const lmoe_weights *w, const void *x, float *logits,
                               void *stream);

/* Quantile Balancing thresholds (P3 Stable LatentMoE bullet: per-expert top-k
 * thresholds solved for directly; P2 balancing passage: read off the batch's
 * score distribution as each expert's fair share).  For each expert e, with
 * its T scores s = sigmoid(logits[:, e]) (fp32) sorted ascending and
 * h = (T - 1)(1 - k/E): tau_e = s_(floor h) + (h - floor h)(s_(floor h + 1) -
 * s_(floor h)), so about T k / E tokens score at or above tau_e; bias [E] fp32
 * receives -tau_e, the selection bias of lmoe_route / lmoe_forward that ranks
 * each expert's scores against its threshold.  logits [T, E] fp32 device
 * memory (e.g. from lmoe_router_logits); T >= 1.  The workspace (as for the
 * layer) holds T * E keys.                                                     */
lmoe_status lmoe_quantile_bias(const lmoe_shape *shape, const float *logits, float *bias, void *ws, size_t ws_bytes,
                               void *stream);

/* Packed routed-expert weights.  The expert GEMMs stream each 256-row by
 * 64-column tile of an expert matrix as one contiguous 32 KB block laid out
 * exactly as they stage it in on-chip memory, so every load is a dense 1 KB
 * run instead of 256 scattered 128-byte row pieces.  Layout (bf16, one block =
 * 256 rows x 128 bytes, row r's 16-byte chunk c stored at chunk position
 * c ^ ((r >> 1) & 7)):
 *   gate/value part: block (e, f, kt) for e < E, f < ceil(I / 128), kt < L / 64
 *     at index (e * ceil(I/128) + f) * (L/64) + kt; block row r holds k-columns
 *     64 kt .. 64 kt + 63 of gate row u (r mod 64 < 32) or value row u
 *     (r mod 64 >= 32) of expert e, u = 128 f + 32 (r / 64) + (r mod 32);
 *     rows with u >= I are zero;
 *   out part (after the gate/value part): block (e, f, kt) for f < ceil(L/256),
 *     kt < I / 64 at index (e * ceil(L/256) + f) * (I/64) + kt; block row r holds
 *     k-columns 64 kt .. 64 kt + 63 of out row 256 f + r of expert e (zero past L).
 * lmoe_packed_bytes returns the size (0 when the shape has no packed form:
 * an invalid shape, or one that is not BF16 with BF16 expert weights).
 * lmoe_pack_experts fills `packed` (device memory, 256-byte aligned, at least
 * lmoe_packed_bytes bytes) from w_gate / w_value / w_out on `stream`; it is a
 * one-time layout change of the weights, after which w->packed may point at
 * the buffer for every call of the layer.                                      */
size_t lmoe_packed_bytes(const lmoe_shape *shape);
lmoe_status lmoe_pack_experts(const lmoe_shape *shape, const lmoe_weights *w, void *packed, size_t bytes,
                              void *stream);

/* Per-token 1x128 activation quantisation of the W8A8 expert GEMMs (the
 * precision question of P3's merged summary; the format is this library's
 * reading).  x: BF16 [R, C] on the device, row-major, C a multiple of 128.
 * Outputs (device, caller-owned, not aliasing x): q [R, C] e4m3fn codes, row
 * stride C; scales [C/128, R] fp32, block-major (the scale of row r, columns
 * 128 b .. 128 b + 127 at scales[b * R + r]).  scale = amax / 448 in fp32 (1 for
 * an all-zero block); code = e4m3fn(x / scale), an fp32 division rounded to
 * nearest even.  Inputs are taken to be finite.  R = 0 is an empty call;
 * EINVAL for a negative R, C not a positive multiple of 128, or a NULL pointer.
 * Asynchronous on `stream`.                                                    */
lmoe_status lmoe_quantize_1x128(const void *x, int64_t R, int32_t C, void *q, float *scales, void *stream);

/* Backward pass of the layer (the pages motivate the cap and the norm by
 * training stability, P2 stabilizer passage): gradients of sum(y * dy) with
 * respect to x and every weight, for BF16 layers with BF16 expert weights in
 * the row-major layout (w_gate / w_value / w_out; a packed copy is not read).
 * The forward is recomputed inside, from x, with the same selection rule;
 * the selection and its bias carry no gradient, the combine weights carry the
 * router's.  Every gradient is fp32 and written whole (experts no token chose
 * get zeros).  Device pointers, caller-owned, not aliasing each other or the
 * inputs:
 *   dx [T, H] (may be NULL when T == 0); dw_router [E, H]; dw_down [L, H] (not written when w_down is
 *   NULL); dw_gate, dw_value [E, I, L]; dw_out [E, L, I]; dgamma [L];
 *   dw_up [H, L] (not written when w_up is NULL); dws_gate, dws_value
 *   [S, Is, H], dws_out [S, H, Is] (not written when S == 0).
 * dy [T, H] is BF16.  topk_idx [T, k] receives the selection if not NULL.
 * stage_events: NULL, or LMOE_NUM_BWD_STAGES + 1 hipEvent_t recorded on
 * `stream` before the first stage and after each: forward recompute, up and
 * norm/combine gradients, routed expert gradients, latent and router
 * gradients, shared expert gradients.
 * The workspace holds lmoe_backward_workspace_bytes(shape) bytes (256-byte
 * aligned).  T <= 65535.  EUNSUPPORTED for other dtypes, for a8 and for larger
 * T; EINVAL for a missing
 * pointer; EWORKSPACE for a short workspace.  Asynchronous on `stream`.      */
typedef struct {
  float *dx;
  float *dw_router;
  float *dw_down;
  float *dw_gate, *dw_value, *dw_out;
  float *dgamma;
  float *dw_up;
  float *dws_gate, *dws_value, *dws_out;
} lmoe_grads;
#define LMOE_NUM_BWD_STAGES 5
size_t lmoe_backward_workspace_bytes(const lmoe_shape *shape);
lmoe_status lmoe_backward(const lmoe_shape *shape, const lmoe_weights *w, const void *x, const void *dy,
                          int32_t *topk_idx, const lmoe_grads *grads, void *ws, size_t ws_bytes, void *stream,
                          void *const *stage_events);

/* Name of a status code; message of the calling thread's last failure.       */
const char *lmoe_status_str(lmoe_status s);
const char *lmoe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
