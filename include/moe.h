/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts expert layer.
 *
 * The layer ("Dist-MoE" blog post, section "What it is selling": caller routing
 * gives x, top-k expert ids and scores; then route on GPU -> W13 -> SwiGLU ->
 * W2 -> combine; forward is FPROP, backward splits into DGRAD and WGRAD)
 * computes, for every token t,
 *
 *     y[t] = sum_{j<k} scores[t][j] * W2_e ( silu(W1_e x[t]) * W3_e x[t] ),
 *            e = ids[t][j],  silu(z) = z / (1 + exp(-z)),
 *
 * on one GPU.  There is no expert parallelism and no collective.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous device buffers owned by the
 *     caller.  BF16 is the IEEE-754 binary32 upper half (uint16 bit pattern).
 *   - x, y, dy, dx: BF16 [T, d].  ids: int32 [T, k], distinct values in [0, E)
 *     per row (nvfp4moe README, "MoE layer").  scores, dscores: float32 [T, k].
 *   - w13: [E, 2I, d], rows [0, I) are the gate projection W1, rows [I, 2I)
 *     the up projection W3; w2: [E, d, I].  Each expert matrix is used as
 *     out = A * B^T with B stored [N, K] (nvfp4moe README, "Dense GEMM" and
 *     "Grouped GEMM").
 *   - `stream` is a hipStream_t (NULL means the null stream).  Every call that
 *     takes a stream only enqueues work on it: it never allocates device
 *     memory, never synchronises and never reads device data on the host, so
 *     it can be captured in a HIP graph (nvfp4moe README, "MoE layer": a
 *     warmed plan does not allocate and can be graph-captured).
 *   - A plan is host-side state plus a caller-allocated workspace.  It is not
 *     reentrant: use one plan per concurrently running stream (nvfp4moe README,
 *     "MoE layer"; blog post, "Caveats", item 6).
 *   - Errors found on the host are returned before anything is enqueued.
 *     Routing errors found on the device (an id outside [0, E) or repeated in
 *     a row) set a sticky flag read by moe_get_status; outputs of that call are
 *     then unspecified.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_plan_s* moe_plan_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* NULL pointer, bad size, bad enum */
    MOE_ERR_UNSUPPORTED = -2,  /* shape or mode outside the supported limits */
    MOE_ERR_WORKSPACE = -3,    /* no workspace bound, or the bound one is too small */
    MOE_ERR_STATE = -4,        /* e.g. backward without a preceding training forward */
    MOE_ERR_HIP = -5,          /* a HIP runtime call or kernel launch failed */
    MOE_ERR_ROUTING = -6,      /* device-detected invalid routing (moe_get_status) */
    MOE_ERR_TOO_LARGE = -7     /* moe_forward_static: the plan's scratch exceeds MOE_STATIC_SCRATCH_BYTES */
} moe_status_t;

typedef enum {
    MOE_BF16 = 0,              /* BF16 operands, FP32 accumulate (blog post: "BF16 Standard") */
    MOE_MXFP8_E4M3 = 1         /* OCP MXFP8: E4M3 elements, E8M0 scale per 32 along K */
} moe_precision_t;

/* path selection (moe_config_t.path) */
#define MOE_PATH_AUTO 0        /* decode kernels when T*k <= 256 and inference, else prefill */
#define MOE_PATH_PREFILL 1     /* grouped-GEMM path */
#define MOE_PATH_DECODE 2      /* weight-streaming path; requires T*k <= 256, inference, BF16 */

/* gated activation of the W13 output (moe_config_t.activation; nvfp4moe README,
 * "Supported kernel surface": SwiGLU, GeGLU and ReGLU FC1 epilogues): a = f(g) * u */
#define MOE_ACT_SWIGLU 0       /* f = silu(z) = z / (1 + e^-z) */
#define MOE_ACT_GEGLU 1        /* f = gelu(z) = z Phi(z), the exact (erf) GELU */
#define MOE_ACT_REGLU 2        /* f = max(z, 0) */

/* device status bits (moe_get_status) */
#define MOE_DEV_ID_OUT_OF_RANGE 1
#define MOE_DEV_ID_DUPLICATE 2
#define MOE_DEV_BAD_INDPTR 4   /* moe_forward_routed: m_indptr not non-decreasing from 0, or past T*k */

typedef struct {
    int32_t T;          /* physical token count, fixed per plan (blog post, "Caveats", item 2) */
    int32_t d;          /* hidden size; multiple of 64 */
    int32_t I;          /* expert intermediate size; multiple of 64 */
    int32_t E;          /* experts, 1..256 (nvfp4moe README, "Limits") */
    int32_t k;          /* experts per token, 1..min(E, 32) */
    int32_t precision;  /* moe_precision_t */
    int32_t training;   /* 1: forward saves what moe_backward needs */
    int32_t path;       /* MOE_PATH_* */
    int32_t wgrad_accumulate;  /* 1: moe_backward adds the weight gradients into dw13 / dw2
                                  (blog post, "What it is selling": in-place accumulation
                                  into the parameters' gradients); training plans only */
    int32_t recompute_h;       /* 1: the training forward does not keep h = (g, u); the
                                  backward recomputes it first, in memory the backward
                                  reuses later (blog post, "Caveats": activation-slot
                                  overflow selects recomputation); training plans only */
    int32_t activation;        /* MOE_ACT_*; every path and precision */
    int32_t mega;              /* 1: the decode path fuses W13 -> activation -> W2 into one
                                  launch chunked over I, with FP32 partial outputs that a
                                  light second launch adds up and combines (blog post, "What it
                                  is selling": Mega fuses both projections into a chunked
                                  pipeline); decode plans only (inference, BF16, T*k <= 256,
                                  path AUTO or DECODE) */
} moe_config_t;

typedef struct {
    const void* w13;          /* BF16 [E, 2I, d], or E4M3 codes (uint8) [E, 2I, d] */
    const void* w2;           /* BF16 [E, d, I],  or E4M3 codes (uint8) [E, d, I]  */
    /* MXFP8 only (NULL for BF16): E8M0 scale bytes in the block-major layout that
     * moe_prepare_weights writes, uint8 [K/128, N, 4] with the expert matrices stacked
     * as N rows: w13_scale has N = E*2I rows of K = d, w2_scale N = E*d rows of K = I.
     * Byte 4 (g N + n) + j is the scale of elements [32 (4 g + j), +32) of row n.  The
     * row-major [rows, K/32] scales of moe_quantize_mxfp8 are NOT this layout and give
     * wrong results here; prepare weights with moe_prepare_weights. */
    const uint8_t* w13_scale;
    const uint8_t* w2_scale;
    /* MXFP8 training backward only (NULL otherwise): the weights prepared along their other
     * dimension for the input-gradient products (blog post, "What it is selling": MXFP8
     * trains; each product quantizes along its own reduction dimension), as
     * moe_prepare_weights_backward writes them:
     *   w13t  E4M3 codes [E, d, 2I]: W13_e transposed, blocks of 32 along 2I;
     *         w13t_scale block-major [2I/128, E*d, 4]
     *   w2t   E4M3 codes [E, I, d]: W2_e transposed, blocks of 32 along d;
     *         w2t_scale block-major [d/128, E*I, 4] */
    const uint8_t* w13t;
    const uint8_t* w13t_scale;
    const uint8_t* w2t;
    const uint8_t* w2t_scale;
} moe_weights_t;

/* Validate cfg against the limits (K = d and I multiples of 64, at most 256
 * experts, at most 131072 routed rows T*k; nvfp4moe README, "Limits"), choose
 * the kernels and lay out the workspace.  Host only: touches no device.
 * MXFP8 plans need d % 256 == 0 and I % 128 == 0 and run the grouped-GEMM path.
 * Shapes whose activations (T*d*2 bytes), routed intermediates (T*k*2I*2) or
 * per-expert W13 (2I*d*2) reach 2^31 bytes are refused (the kernels address them
 * with 32-bit offsets).  Returns MOE_ERR_UNSUPPORTED for shapes outside the limits,
 * MOE_ERR_INVALID_ARG for NULL or non-positive sizes.  On success *out owns host
 * memory released by moe_plan_destroy. */
moe_status_t moe_plan(const moe_config_t* cfg, moe_plan_t* out);

/* Bytes of device workspace the plan needs (the analogue of planning memory
 * before creating a context; blog post, "Caveats", item 7).  0 on NULL. */
size_t moe_workspace_bytes(moe_plan_t plan);

/* The plan's memory, as text (blog post, "Caveats" and "Bottom line": plan the memory
 * and read its explanation before sizing the layer): one line per workspace region with
 * its bytes, what it holds and whether it is kept from the training forward for the
 * backward ("saved") or only used within a call ("scratch"), the totals, and the row
 * limits.  Writes at most len - 1 characters and a terminating NUL into buf (when buf
 * is not NULL and len > 0) and returns the length of the whole report, like snprintf;
 * 0 for a NULL plan.  Host only. */
size_t moe_plan_explain(moe_plan_t plan, char* buf, size_t len);

/* Give the plan a device buffer of at least moe_workspace_bytes bytes,
 * 256-byte aligned (blog post, "Caveats", item 7 and the "Dist-MoE" README intro:
 * the library owns its temporary memory, sized before the context exists; here the
 * caller allocates it, so that the calls themselves never allocate, as the nvfp4moe
 * README, "MoE layer", asks of a warmed plan); the caller keeps ownership and must
 * keep it alive while the plan is used.  Clears the device status word (synchronously, with a
 * plain memset: call it outside graph capture).  Rebinding forgets the saved
 * forward state. */
moe_status_t moe_bind_workspace(moe_plan_t plan, void* dptr, size_t bytes);

/* Release the host plan (not the caller's workspace; blog post, "Caveats": one
 * context per stream, so a plan is released by its one owner).  Returns MOE_OK;
 * NULL is accepted. */
moe_status_t moe_plan_destroy(moe_plan_t plan);

/* Deterministic dispatch (nvfp4moe README, "Grouped GEMM" and "Training"):
 *   m_indptr int32 [E+1]: exclusive scan of per-expert row counts (empty
 *            experts valid, m_indptr[E] = T*k);
 *   gather   int32 [T*k]: token of each expert-major routed row; rows of one
 *            expert are in ascending token order;
 *   slots    int32 [T, k]: routed row that holds (t, j);
 *   probs    float [T*k]: scores[t][j] moved to its routed row.
 * Bit-exact and run-to-run identical.  Uses the plan's workspace. */
moe_status_t moe_dispatch(moe_plan_t plan, const int32_t* ids, const float* scores,
                          int32_t* m_indptr, int32_t* gather, int32_t* slots, float* probs,
                          void* stream);

/* OCP MXFP8 conversion of `rows` BF16 rows of length K (a multiple of 32):
 * per block of 32 consecutive elements the scale is the smallest power of two 2^s
 * with max|v| / 2^s <= 448 (s = ceil(log2(max|v| / 448)): no element saturates), its
 * E8M0 byte clamp(s + 127, 0, 254) (0 for an all-zero block), and each element is
 * E4M3(v / 2^s), nearest-even.
 * codes uint8 [rows, K]; scales uint8 [rows, K/32].  Needs no plan.
 * Inputs are meant to be finite.  An infinite or NaN element is encoded as
 * 448 with its sign bit (E4M3's NaN codes are never written), and the scale
 * byte of its block is then not specified. */
moe_status_t moe_quantize_mxfp8(const void* v_bf16, int64_t rows, int32_t K,
                                uint8_t* codes, uint8_t* scales, void* stream);

/* Prepare BF16 weights for the MXFP8 pipeline (blog post, "What it is
 * selling": MXFP8 accepts prepared weights): quantize w13 [E,2I,d] and
 * w2 [E,d,I] along their K (last) dimension with moe_quantize_mxfp8's rule.
 * Outputs are caller-owned: codes w13_q [E,2I,d] and w2_q [E,d,I] as
 * moe_quantize_mxfp8 writes them; scales block-major: viewing w13 as
 * N = E*2I rows of length K = d (w2: N = E*d rows of length K = I), the four
 * scale bytes of blocks 4g .. 4g+3 of row n are bytes [4 (g N + n), +4), i.e.
 * uint8 [K/128, N, 4] (E*2I*d/32 and E*d*I/32 bytes).  Needs d and I multiples
 * of 128 (else MOE_ERR_UNSUPPORTED).  Meant to run outside any timed region. */
moe_status_t moe_prepare_weights(moe_plan_t plan, const void* w13_bf16, const void* w2_bf16,
                                 uint8_t* w13_q, uint8_t* w13_s, uint8_t* w2_q, uint8_t* w2_s,
                                 void* stream);

/* Prepare BF16 weights for the MXFP8 backward's input-gradient products (blog post,
 * "What it is selling": MXFP8 trains; each product quantizes its operands along its
 * own reduction dimension, so DGRAD needs the weights blocked along their other
 * dimension): w13t_q [E, d, 2I] = W13_e^T quantized in blocks of 32 along 2I,
 * w13t_s block-major [2I/128, E*d, 4]; w2t_q [E, I, d] = W2_e^T quantized along d,
 * w2t_s block-major [d/128, E*I, 4] (moe_quantize_mxfp8's rule).  Like
 * moe_prepare_weights, it is run again after every update of the BF16 weights.  Needs
 * d and I multiples of 128 (else MOE_ERR_UNSUPPORTED).  Caller-owned outputs. */
moe_status_t moe_prepare_weights_backward(moe_plan_t plan, const void* w13_bf16, const void* w2_bf16,
                                          uint8_t* w13t_q, uint8_t* w13t_s, uint8_t* w2t_q, uint8_t* w2t_s,
                                          void* stream);

/* Forward (FPROP): dispatch, [MXFP8: quantize x], grouped W13 GEMM with the
 * SwiGLU epilogue, [MXFP8: re-quantize the SwiGLU output], grouped W2 GEMM,
 * score-weighted combine in FP32 with j ascending from +0.0 and one rounding
 * to BF16 (nvfp4moe README, "MoE layer": the timed path).  y is BF16 [T, d].
 * BF16 plans take BF16 weights; MXFP8 plans take the prepared codes in w13 / w2
 * and their E8M0 scales in w13_scale / w2_scale (moe_prepare_weights layout;
 * NULL scales are MOE_ERR_INVALID_ARG).  Plans with T*k <= 256 (BF16, inference)
 * run the weight-streaming decode kernels unless cfg.path forces the prefill path.
 * With cfg.training = 1 the workspace keeps the dispatch, the W13 outputs and
 * the W2 outputs for moe_backward; a later forward overwrites them. */
moe_status_t moe_forward(moe_plan_t plan, const void* x, const int32_t* ids, const float* scores,
                         const moe_weights_t* w, void* y, void* stream);

/* Forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation, kernels
 * and result as moe_forward, bit for bit, but the scratch the plan needs lives in a
 * static array that the library holds on each GPU it runs on, of MOE_STATIC_SCRATCH_BYTES
 * (32 MiB) per device, kept until the process ends; no workspace needs to be bound.
 * The caller passes inputs and outputs as for moe_forward.  Inference plans only
 * (MOE_ERR_UNSUPPORTED for training = 1); a plan whose moe_workspace_bytes exceeds
 * MOE_STATIC_SCRATCH_BYTES returns MOE_ERR_TOO_LARGE before anything is enqueued.  It
 * calls no allocating routine (hipMalloc, hipFree or any allocating library call); the
 * first call on a device looks up that device's copy of the array.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents: calls that overlap
 * on one GPU (on different streams, or from different plans) race, so serialise them.
 * The device status word of the call lives in the array too: it is cleared at the start
 * of each call, and moe_get_status on the plan reads it until the plan's next call.
 * Leave moe_profile off (its events are created on first use). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status_t moe_forward_static(moe_plan_t plan, const void* x, const int32_t* ids, const float* scores,
                                const moe_weights_t* w, void* y, void* stream);

/* Forward of rows already in expert order (nvfp4moe README, "MoE layer": frameworks
 * that already hold expert-major rows call the layer on them directly).  For each
 * expert e and row r in [m_indptr[e], m_indptr[e+1]):
 *   out[r] = W2_e (silu(W1_e x_rows[r]) * (W3_e x_rows[r]))       (BF16, FP32 accumulate)
 * with no dispatch, no score weighting and no combine: the caller owns the routing.
 *   x_rows    BF16 [R', d] device, R' = m_indptr[E] <= T*k of the plan
 *   m_indptr  int32 [E+1] device, m_indptr[0] = 0, non-decreasing (empty experts valid)
 *   out       BF16 [R', d] device, row r written for every r < m_indptr[E]
 * The pages also pass padded_offsets, which describe their padded tile layout; these
 * kernels take ragged expert segments, so only m_indptr is needed.  An m_indptr that is
 * not non-decreasing from 0, or whose total exceeds T*k, is caught on the device: every
 * expert is then taken as empty (out is not written) and MOE_DEV_BAD_INDPTR is set
 * (moe_get_status).  Inference plans on the grouped-GEMM path (cfg.path =
 * MOE_PATH_PREFILL, or AUTO with T*k > 256) with T*k*d*2 < 2^31; others return
 * MOE_ERR_UNSUPPORTED.  MXFP8 plans take prepared weights with their scales (as
 * moe_forward does) and quantize the m_indptr[E] rows of x_rows as they stand, with
 * moe_quantize_mxfp8's rule, before W13.  It uses the plan's dispatch and intermediate workspace, which the
 * next call overwrites. */
moe_status_t moe_forward_routed(moe_plan_t plan, const void* x_rows, const int32_t* m_indptr,
                                const moe_weights_t* w, void* out, void* stream);

/* Backward (DGRAD + WGRAD + router gradient; blog post, "What it is selling";
 * nvfp4moe README, "Training") of the most recent training forward on this
 * plan, which must have used the same x, ids, scores and weights (unchanged):
 *   dx      BF16 [T, d]   = dL/dx
 *   dw13    BF16 [E,2I,d] = dL/dW13, overwritten (+0.0 for experts with no row)
 *   dw2     BF16 [E,d,I]  = dL/dW2, overwritten
 *   (with cfg.wgrad_accumulate = 1 instead dw13 = bf16(dw13 + bf16(dL/dW13)), likewise
 *    dw2: the gradient in BF16 added in FP32 to the value already there, one rounding;
 *    experts with no row keep their values)
 *   dscores f32  [T, k]   = dL/dscores[t][j] = <dy[t], expert output of (t, j)>
 * Returns MOE_ERR_STATE if no training forward ran since the workspace was
 * bound.  BF16 plans take the BF16 weights in w13 / w2.  MXFP8 plans take the
 * weights prepared by moe_prepare_weights_backward in w13t / w2t with their scales
 * (NULL: MOE_ERR_INVALID_ARG), plus, with cfg.recompute_h = 1, the forward's
 * prepared w13 and w13_scale; every expert product runs on MXFP8 operands quantized
 * along that product's reduction dimension: dO = scores * dy[token] along d, the
 * gradient (dg, du) along 2I, and, for the weight gradients, dO, a, (dg, du) and x
 * along each expert's routed rows (blocks of 32 rows in dispatch order, restarting at
 * every expert).  The forward's h and a and the gradients dA, (dg, du) are kept in
 * BF16 between kernels. */
moe_status_t moe_backward(moe_plan_t plan, const void* dy, const void* x, const moe_weights_t* w,
                          void* dx, void* dw13, void* dw2, float* dscores, void* stream);

/* Synchronise `stream`, copy the sticky device status word (MOE_DEV_* bits)
 * into *device_flags, and clear it when `clear` is non-zero.  Returns
 * MOE_ERR_ROUTING when a bit is set, MOE_OK otherwise. */
moe_status_t moe_get_status(moe_plan_t plan, int32_t* device_flags, int32_t clear, void* stream);

/* Static description of a status code (blog post, "What it is selling": unsupported
 * modes are refused when the context is created, with a reason).  Never NULL; an
 * unknown code gives "unknown status". */
const char* moe_status_string(moe_status_t status);

/* Kernel stages of moe_forward / moe_backward.  moe_backward launches SCORE_GRAD,
 * [RECOMPUTE_H,] DGRAD_W2, DGRAD_W13, DX_COMBINE, WGRAD_ROWS, WGRAD_W2, WGRAD_W13 in that order
 * (MXFP8: SCORE_GRAD, [RECOMPUTE_H,] QUANT_DO, DGRAD_W2, ACT_BWD, DGRAD_W13, DX_COMBINE,
 * QUANT_T, WGRAD_W2, QUANT_T, WGRAD_W13); the one-token decode runs W2 and the combine as
 * one kernel, recorded as DECODE_W2; a mega decode plan records its two launches (the
 * chunked products, then the sum of the chunks with the combine) as one stage, MEGA. */
#define MOE_STAGE_DISPATCH 0
#define MOE_STAGE_QUANT_X 1
#define MOE_STAGE_W13 2
#define MOE_STAGE_W2 3
#define MOE_STAGE_COMBINE 4
#define MOE_STAGE_SCORE_GRAD 5
#define MOE_STAGE_DGRAD_W2 6
#define MOE_STAGE_WGRAD_W2 7
#define MOE_STAGE_DGRAD_W13 8
#define MOE_STAGE_WGRAD_W13 9
#define MOE_STAGE_DX_COMBINE 10
#define MOE_STAGE_DECODE_W13 11
#define MOE_STAGE_DECODE_W2 12
#define MOE_STAGE_WGRAD_ROWS 13
#define MOE_STAGE_RECOMPUTE_H 14
#define MOE_STAGE_MEGA 15
#define MOE_STAGE_QUANT_DO 16     /* MXFP8 backward: dO quantized along d */
#define MOE_STAGE_ACT_BWD 17      /* MXFP8 backward: activation backward, (dg, du) quantized along 2I */
#define MOE_STAGE_QUANT_T 18      /* MXFP8 backward: weight-gradient operands quantized along rows */
#define MOE_STAGE_COUNT 19

/* Per-stage timing with HIP events, for measurement only.  While enabled,
 * moe_forward and moe_backward record a pair of HIP events around each kernel
 * stage on the caller's stream (events are created by the library on first
 * use and kept by the plan; at most 4096 pairs are held, later stages of a
 * full buffer are not recorded).  Do not enable it under graph capture.
 * moe_profile(plan, 0) disables recording and keeps what was recorded. */
moe_status_t moe_profile(moe_plan_t plan, int32_t enable);

/* Wait for the recorded events, then write for each stage s < max_stages the
 * summed duration in milliseconds (total_ms[s]) and the number of recorded
 * launches (count[s]); forget the recorded events. */
moe_status_t moe_profile_read(moe_plan_t plan, float* total_ms, int32_t* count, int32_t max_stages);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
