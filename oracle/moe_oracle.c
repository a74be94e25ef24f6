/*
 * moe_oracle.c -- plain CPU oracle for the routed Mixture-of-Experts expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Every floating-point quantity is carried in IEEE double (fp64).  Inputs
 * arrive as float32 arrays holding the exact values of the BF16 inputs.
 * The loops follow the definitions directly, token by token, with no
 * blocking or reordering.  The only threading is an OpenMP split over
 * independent outputs (tokens, or experts for the weight gradient), so the
 * result does not depend on the thread count.
 *
 * Sources (cited by page title and section):
 *   [DM]  "Dist-MoE: Meta's Blackwell SM100 MoE Kernels" blog post,
 *         section "What it is selling" (execution diagram: route on GPU ->
 *         W13 -> SwiGLU -> W2 -> combine; FPROP / DGRAD / WGRAD split).
 *   [NV]  nvfp4moe README, sections "Grouped GEMM" (expert-major rows,
 *         m_indptr of length E+1, empty experts valid), "MoE layer" (timed
 *         path; distinct expert ids per token row; probability weighting and
 *         deterministic combine), "Training" (gather / cu / probs / slots;
 *         router, input and weight gradients), "Limits".
 *   [MX]  The OCP Microscaling Formats (MX) v1.0 specification (an MX block is
 *         32 elements of one element type sharing one E8M0 power-of-two scale;
 *         elements rounded to nearest even), which the blog post's "MXFP8 E4M3"
 *         mode names.  The scale taken here is the smallest power of two that
 *         brings the block maximum within E4M3's largest normal (448):
 *         2^ceil(log2(amax / 448)), so no element saturates.  (The format
 *         fixes the encoding, not the choice of scale; the specification's
 *         reference conversion takes floor(log2(amax)) - 8 instead, which clips
 *         the elements of a block whose maximum has a significand above 1.75.)
 *
 * Readings where the pages are silent or leave a step open:
 *   - within one expert, routed rows are ordered by ascending token index
 *     (a stable counting sort of the flattened (t, j) list by expert id);
 *   - W13 is [E, 2I, d]: gate rows [0, I), up rows [I, 2I);
 *   - SwiGLU is silu(gate) * up with silu(z) = z / (1 + exp(-z)), no clamp;
 *     GeGLU uses the exact (erf) GELU, ReGLU max(z, 0);
 *   - scores weight the expert outputs in the combine, without renormalising;
 *   - dS[t][j] = <dY[t], o_(t,j)> with o the unscaled expert output.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_RANGE 1
#define ORC_ERR_DUPLICATE 2
#define ORC_ERR_ALLOC 3

/* threads the OpenMP loops below use */
int orc_num_threads(void) { return omp_get_max_threads(); }

static double silu(double z) { return z / (1.0 + exp(-z)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Gated activations of the W13 output ([NV] "Supported kernel surface": SwiGLU,
 * GeGLU and ReGLU FC1 epilogues): a = f(g) * u with
 *   act 0 (SwiGLU): f(z) = silu(z) = z / (1 + e^-z)
 *   act 1 (GeGLU):  f(z) = gelu(z) = z Phi(z) = z (1 + erf(z / sqrt 2)) / 2   (exact GELU)
 *   act 2 (ReGLU):  f(z) = relu(z) = max(z, 0)
 * and f' for the backward:
 *   silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *   gelu'(z) = Phi(z) + z phi(z), phi(z) = e^(-z^2/2) / sqrt(2 pi)
 *   relu'(z) = 1 for z > 0, else 0. */
#define ORC_ACT_SWIGLU 0
#define ORC_ACT_GEGLU 1
#define ORC_ACT_REGLU 2
static double act_f(int act, double z)
{
    if (act == ORC_ACT_GEGLU) return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
    if (act == ORC_ACT_REGLU) return z > 0.0 ? z : 0.0;
    return silu(z);
}
static double act_df(int act, double z)
{
    if (act == ORC_ACT_GEGLU)
        return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * exp(-0.5 * z * z) / sqrt(2.0 * acos(-1.0));
    if (act == ORC_ACT_REGLU) return z > 0.0 ? 1.0 : 0.0;
    const double sg = sigmoid(z);
    return sg * (1.0 + z * (1.0 - sg));
}

/* Routing precondition ([NV] "MoE layer": each token row holds distinct expert
 * indices, all in [0, E)).  Returns ORC_OK, ORC_ERR_RANGE or ORC_ERR_DUPLICATE. */
int orc_check_routing(int T, int E, int k, const int32_t* ids)
{
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t e = ids[(size_t)t * k + j];
            if (e < 0 || e >= E) return ORC_ERR_RANGE;
        }
    }
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
            for (int jj = j + 1; jj < k; ++jj)
                if (ids[(size_t)t * k + j] == ids[(size_t)t * k + jj]) return ORC_ERR_DUPLICATE;
    return ORC_OK;
}

/* Dispatch ([NV] "Grouped GEMM" and "Training"): per-expert counts, the
 * exclusive scan m_indptr[E+1], and a stable expert-major placement of every
 * (t, j): rows of one expert appear in ascending t.
 *   gather[r]     = token that routed row r comes from
 *   slots[t*k+j]  = routed row holding (t, j)
 *   probs[r]      = scores[t*k+j] moved to row r                        */
int orc_dispatch(int T, int E, int k, const int32_t* ids, const float* scores,
                 int32_t* m_indptr, int32_t* gather, int32_t* slots, float* probs)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    int64_t* cursor = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    if (!cursor) return ORC_ERR_ALLOC;
    for (size_t q = 0; q < (size_t)T * k; ++q) cursor[ids[q]] += 1;   /* counts */
    int64_t run = 0;
    for (int e = 0; e < E; ++e) {                                      /* exclusive scan */
        int64_t c = cursor[e];
        m_indptr[e] = (int32_t)run;
        cursor[e] = run;
        run += c;
    }
    m_indptr[E] = (int32_t)run;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t q = (size_t)t * k + j;
            int64_t r = cursor[ids[q]]++;
            gather[r] = t;
            slots[q] = (int32_t)r;
            probs[r] = scores[q];
        }
    }
    free(cursor);
    return ORC_OK;
}

/* One expert MLP applied to one token ([DM] "What it is selling": W13 ->
 * SwiGLU -> W2).  g[i] = W1_e[i].x, u[i] = W3_e[i].x, a = f(g)*u (act_f),
 * o[n] = W2_e[n].a.  Any of g/u/a may be used by the caller afterwards. */
static void expert_mlp(int act, int d, int I, const float* x_t, const float* w13_e, const float* w2_e,
                       double* g, double* u, double* a, double* o)
{
    for (int i = 0; i < I; ++i) {
        const float* wg = w13_e + (size_t)i * d;
        const float* wu = w13_e + (size_t)(I + i) * d;
        double sg = 0.0, su = 0.0;
        for (int c = 0; c < d; ++c) {
            sg += (double)wg[c] * (double)x_t[c];
            su += (double)wu[c] * (double)x_t[c];
        }
        g[i] = sg;
        u[i] = su;
        a[i] = act_f(act, sg) * su;
    }
    if (o) {
        for (int n = 0; n < d; ++n) {
            const float* w = w2_e + (size_t)n * I;
            double s = 0.0;
            for (int i = 0; i < I; ++i) s += (double)w[i] * a[i];
            o[n] = s;
        }
    }
}

/* Forward for a list of tokens, straight from the definition
 *   y[t] = sum_{j<k} s[t][j] * W2_e (silu(W1_e x_t) * W3_e x_t),  e = ids[t][j]
 * ([DM] "What it is selling"; [NV] "MoE layer": probability weighting and
 * combine).  y is [ntok, d]; o_out, when not NULL, receives the unscaled
 * expert outputs [ntok, k, d]; a_out, when not NULL, receives the SwiGLU
 * outputs [ntok, k, I]. */
int orc_forward_tokens(int T, int d, int I, int E, int k,
                       const float* x, const int32_t* ids, const float* scores,
                       const float* w13, const float* w2,
                       int ntok, const int32_t* toks,
                       double* y, double* o_out, double* a_out, int act)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < ntok; ++q) {
        double* buf = (double*)malloc(sizeof(double) * (3 * (size_t)I + (size_t)d));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *g = buf, *u = g + I, *a = u + I, *o = a + I;
        int t = toks[q];
        const float* x_t = x + (size_t)t * d;
        double* y_t = y + (size_t)q * d;
        for (int n = 0; n < d; ++n) y_t[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            double s = (double)scores[(size_t)t * k + j];
            expert_mlp(act, d, I, x_t, w13 + (size_t)e * 2 * I * d, w2 + (size_t)e * d * I, g, u, a, o);
            for (int n = 0; n < d; ++n) y_t[n] += s * o[n];
            if (o_out) memcpy(o_out + ((size_t)q * k + j) * d, o, sizeof(double) * (size_t)d);
            if (a_out) memcpy(a_out + ((size_t)q * k + j) * I, a, sizeof(double) * (size_t)I);
        }
        free(buf);
    }
    return failed ? ORC_ERR_ALLOC : ORC_OK;
}

/* Backward for a list of tokens (DGRAD and router gradient; [DM] "What it is
 * selling": DGRAD; [NV] "Training": input and router gradients).
 * Given dY, for every (t, j) with e = ids[t][j] and s = scores[t][j]:
 *   dS[t][j] = <dY[t], o>                       (y is linear in s)
 *   dO       = s * dY[t]
 *   dA[i]    = sum_n W2_e[n][i] dO[n]
 *   dg[i]    = dA[i] * u[i] * f'(g[i])      (SwiGLU: f' = sigmoid (1 + g (1 - sigmoid)))
 *   du[i]    = dA[i] * f(g[i])
 *   dX[t]   += W1_e^T dg + W3_e^T du
 * dx is [ntok, d], ds is [ntok, k]. */
int orc_backward_tokens(int T, int d, int I, int E, int k,
                        const float* x, const int32_t* ids, const float* scores,
                        const float* w13, const float* w2, const float* dy,
                        int ntok, const int32_t* toks, double* dx, double* ds, int act)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < ntok; ++q) {
        double* buf = (double*)malloc(sizeof(double) * (5 * (size_t)I + (size_t)d));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *g = buf, *u = g + I, *a = u + I, *dg = a + I, *du = dg + I, *o = du + I;
        int t = toks[q];
        const float* x_t = x + (size_t)t * d;
        const float* dy_t = dy + (size_t)t * d;
        double* dx_t = dx + (size_t)q * d;
        for (int c = 0; c < d; ++c) dx_t[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            double s = (double)scores[(size_t)t * k + j];
            const float* w13_e = w13 + (size_t)e * 2 * I * d;
            const float* w2_e = w2 + (size_t)e * d * I;
            expert_mlp(act, d, I, x_t, w13_e, w2_e, g, u, a, o);
            double dot = 0.0;
            for (int n = 0; n < d; ++n) dot += (double)dy_t[n] * o[n];
            ds[(size_t)q * k + j] = dot;
            for (int i = 0; i < I; ++i) {
                double dA = 0.0;
                for (int n = 0; n < d; ++n)
                    dA += (double)w2_e[(size_t)n * I + i] * (s * (double)dy_t[n]);
                dg[i] = dA * u[i] * act_df(act, g[i]);
                du[i] = dA * act_f(act, g[i]);
            }
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int i = 0; i < I; ++i)
                    acc += (double)w13_e[(size_t)i * d + c] * dg[i]
                         + (double)w13_e[(size_t)(I + i) * d + c] * du[i];
                dx_t[c] += acc;
            }
        }
        free(buf);
    }
    return failed ? ORC_ERR_ALLOC : ORC_OK;
}

/* Weight gradients (WGRAD; [DM] "What it is selling"; [NV] "Training"),
 * restricted to a list of intermediate indices icols[0..ni) so that large
 * layers can be checked on sampled columns; pass every index for the full
 * gradient.  Summing over the routed (t, j) of expert e:
 *   dW2 [e][n][q]      = sum dO[n]  * a[icols[q]]           -> dw2  [E, d, ni]
 *   dW13[e][icols[q]][c]   = sum dg[icols[q]] * x[t][c]     -> dw13 [E, 2, ni, d]
 *   dW13[e][I+icols[q]][c] = sum du[icols[q]] * x[t][c]       (index 1 of dim 2)
 * An expert that receives no row gets exactly +0.0. */
int orc_wgrad_cols(int T, int d, int I, int E, int k,
                   const float* x, const int32_t* ids, const float* scores,
                   const float* w13, const float* w2, const float* dy,
                   int ni, const int32_t* icols, double* dw2, double* dw13, int act)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
        double* buf = (double*)malloc(sizeof(double) * (3 * (size_t)ni + (size_t)d));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *aq = buf, *dgq = aq + ni, *duq = dgq + ni, *dO = duq + ni;
        double* dw2_e = dw2 + (size_t)e * d * ni;
        double* dw13_e = dw13 + (size_t)e * 2 * ni * d;
        for (size_t z = 0; z < (size_t)d * ni; ++z) dw2_e[z] = 0.0;
        for (size_t z = 0; z < (size_t)2 * ni * d; ++z) dw13_e[z] = 0.0;
        const float* w13_e = w13 + (size_t)e * 2 * I * d;
        const float* w2_e = w2 + (size_t)e * d * I;
        for (int t = 0; t < T; ++t) {
            for (int j = 0; j < k; ++j) {
                if (ids[(size_t)t * k + j] != e) continue;
                double s = (double)scores[(size_t)t * k + j];
                const float* x_t = x + (size_t)t * d;
                const float* dy_t = dy + (size_t)t * d;
                for (int n = 0; n < d; ++n) dO[n] = s * (double)dy_t[n];
                for (int q = 0; q < ni; ++q) {
                    int i = icols[q];
                    const float* wg = w13_e + (size_t)i * d;
                    const float* wu = w13_e + (size_t)(I + i) * d;
                    double sg = 0.0, su = 0.0;
                    for (int c = 0; c < d; ++c) {
                        sg += (double)wg[c] * (double)x_t[c];
                        su += (double)wu[c] * (double)x_t[c];
                    }
                    aq[q] = act_f(act, sg) * su;
                    double dA = 0.0;
                    for (int n = 0; n < d; ++n) dA += (double)w2_e[(size_t)n * I + i] * dO[n];
                    dgq[q] = dA * su * act_df(act, sg);
                    duq[q] = dA * act_f(act, sg);
                }
                for (int n = 0; n < d; ++n)
                    for (int q = 0; q < ni; ++q) dw2_e[(size_t)n * ni + q] += dO[n] * aq[q];
                for (int q = 0; q < ni; ++q)
                    for (int c = 0; c < d; ++c) {
                        dw13_e[(size_t)q * d + c] += dgq[q] * (double)x_t[c];
                        dw13_e[((size_t)ni + q) * d + c] += duq[q] * (double)x_t[c];
                    }
            }
        }
        free(buf);
    }
    return failed ? ORC_ERR_ALLOC : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * OCP MXFP8 (E4M3) reference conversion ([MX]; blog post "What it is selling":
 * MXFP8 E4M3 with prepared weights; block of 32 along K with an E8M0 scale).
 *
 * E4M3 (the OCP "E4M3FN" encoding): 1 sign, 4 exponent bits (bias 7),
 * 3 mantissa bits, no infinities, S.1111.111 is NaN, largest normal
 * 1.75 * 2^8 = 448, smallest normal 2^-6, subnormals m * 2^-9 (m = 1..7).
 * ------------------------------------------------------------------------- */

/* value of an E4M3 code (NaN codes return NAN) */
double orc_e4m3_decode(uint8_t code)
{
    int s = code >> 7, ex = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (ex == 0xF && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, ex - 7);
    return s ? -v : v;
}

/* round-to-nearest-even of a finite double onto E4M3, clamped to +-448 */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {                      /* subnormal range, step 2^-9 */
        double m = rint(ldexp(a, 9));              /* default mode: ties to even */
        return sign | (uint8_t)m;                  /* m == 8 is code 0x08 = 2^-6 */
    }
    int ex;
    double fr = frexp(a, &ex);                     /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;                                /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double m = rint((2.0 * fr - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; e += 1; }
    if (e > 8 || (e == 8 && m == 7.0)) return sign | 0x7E;
    return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Shared exponent of one block: the smallest power of two X with amax / X <= 448,
 * i.e. log2 X = ceil(log2(amax / 448)).  With amax = m * 2^e, m in [1, 2):
 * amax / 448 = (m / 1.75) * 2^(e - 8), so log2 X = e - 8 when m <= 1.75 and e - 7
 * when m > 1.75.  Stored as an E8M0 byte (biased by 127) clamped to [0, 254];
 * amax = 0 gives 0. */
uint8_t orc_mx_scale_byte(const double* v, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) { double a = fabs(v[i]); if (a > amax) amax = a; }
    if (amax == 0.0) return 0;
    int ex;
    double fr = frexp(amax, &ex);                  /* amax = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;                                /* amax = (2 fr) * 2^e */
    int shared = e - 8 + (2.0 * fr > 1.75 ? 1 : 0);
    int biased = shared + 127;
    if (biased < 0) biased = 0;
    if (biased > 254) biased = 254;
    return (uint8_t)biased;
}

/* Quantize rows of length K (K a multiple of 32) in blocks of 32:
 * codes[r][c] = E4M3(v[r][c] / 2^(scale-127)), scales[r][c/32] = E8M0 byte. */
void orc_mx_quantize(int64_t rows, int K, const float* v, uint8_t* codes, uint8_t* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double blk[32];
        for (int b = 0; b < K / 32; ++b) {
            const float* src = v + r * K + (int64_t)b * 32;
            for (int i = 0; i < 32; ++i) blk[i] = (double)src[i];
            uint8_t sb = orc_mx_scale_byte(blk, 32);
            double X = ldexp(1.0, (int)sb - 127);
            for (int i = 0; i < 32; ++i) codes[r * K + (int64_t)b * 32 + i] = orc_e4m3_encode(blk[i] / X);
            scales[r * (K / 32) + b] = sb;
        }
    }
}

/* codes * 2^(scale-127), exact in float32 for every code/scale pair used here */
void orc_mx_dequantize(int64_t rows, int K, const uint8_t* codes, const uint8_t* scales, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < K; ++c)
            out[r * K + c] = (float)(orc_e4m3_decode(codes[r * K + c])
                                     * ldexp(1.0, (int)scales[r * (K / 32) + c / 32] - 127));
}

/* Forward with MXFP8 activations: like orc_forward_tokens, but the token row
 * x_t and the SwiGLU output a are each replaced by their MX block-32
 * quantize->dequantize image before entering the W13 and W2 products (the
 * blog post's MXFP8 mode quantizes activations after routing; the weights
 * passed in are the dequantized prepared weights).  Used to separate kernel
 * error from quantization noise. */
int orc_forward_tokens_mx(int T, int d, int I, int E, int k,
                          const float* x, const int32_t* ids, const float* scores,
                          const float* w13, const float* w2,
                          int ntok, const int32_t* toks, double* y, int act)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    if (d % 32 || I % 32) return ORC_ERR_RANGE;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < ntok; ++q) {
        double* buf = (double*)malloc(sizeof(double) * 3 * (size_t)I);
        float* xq = (float*)malloc(sizeof(float) * (size_t)d);
        if (!buf || !xq) {
#pragma omp atomic write
            failed = 1;
            free(buf); free(xq);
            continue;
        }
        double *g = buf, *u = g + I, *a = u + I;
        int t = toks[q];
        const float* x_t = x + (size_t)t * d;
        for (int b = 0; b < d / 32; ++b) {
            double blk[32];
            for (int i = 0; i < 32; ++i) blk[i] = (double)x_t[b * 32 + i];
            uint8_t sb = orc_mx_scale_byte(blk, 32);
            double X = ldexp(1.0, (int)sb - 127);
            for (int i = 0; i < 32; ++i)
                xq[b * 32 + i] = (float)(orc_e4m3_decode(orc_e4m3_encode(blk[i] / X)) * X);
        }
        double* y_t = y + (size_t)q * d;
        for (int n = 0; n < d; ++n) y_t[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            double s = (double)scores[(size_t)t * k + j];
            const float* w13_e = w13 + (size_t)e * 2 * I * d;
            const float* w2_e = w2 + (size_t)e * d * I;
            expert_mlp(act, d, I, xq, w13_e, w2_e, g, u, a, NULL);
            for (int b = 0; b < I / 32; ++b) {
                uint8_t sb = orc_mx_scale_byte(a + b * 32, 32);
                double X = ldexp(1.0, (int)sb - 127);
                for (int i = 0; i < 32; ++i)
                    a[b * 32 + i] = orc_e4m3_decode(orc_e4m3_encode(a[b * 32 + i] / X)) * X;
            }
            for (int n = 0; n < d; ++n) {
                const float* w = w2_e + (size_t)n * I;
                double acc = 0.0;
                for (int i = 0; i < I; ++i) acc += (double)w[i] * a[i];
                y_t[n] += s * acc;
            }
        }
        free(buf); free(xq);
    }
    return failed ? ORC_ERR_ALLOC : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * MXFP8 training step (blog post "What it is selling": MXFP8 E4M3 trains as well
 * as infers, activations quantized after routing; FPROP, DGRAD and WGRAD).
 *
 * Every expert product takes both of its operands as MX images, blocked along that
 * product's own reduction dimension:
 *   FPROP  h = W13 x       x along d, W13 along d (its rows)
 *          o = W2 a        a along I, W2 along I (its rows)
 *   DGRAD  dA = W2^T dO    dO along d, W2 along d (its columns)
 *          dX = W13^T dh   dh = (dg, du) along 2I, W13 along 2I (its columns)
 *   WGRAD  dW2  = sum_r dO_r a_r^T     both along the routed rows of the expert
 *          dW13 = sum_r dh_r x_r^T     (blocks of 32 consecutive rows in dispatch
 *                                       order; the last block of an expert may be short)
 * with dO_r = probs[r] * dY[gather[r]].  Readings where the pages are silent:
 *   - the weights w13 / w2 passed in are the BF16 master weights; each product
 *     quantizes them along its own reduction dimension;
 *   - the activations the layer keeps for the backward (h and a) and the gradient dA
 *     are held in BF16, the precision BF16 mode keeps activations in; they are
 *     rounded to BF16 (nearest, ties to even) where they are stored, and every later
 *     quantization starts from the stored value.  dh is used unrounded by DGRAD and
 *     rounded to BF16 for WGRAD; dO and x enter unrounded.
 * Outputs (fp64), for the tokens toks[0 .. ntok) and the intermediate indices
 * icols[0 .. ni) (pass every index for the whole step):
 *   y, dx [ntok, d]; ds [ntok, k] (ds[t][j] = <dY[t], o>);
 *   dw13 [E, 2, ni, d]: gate rows icols, then up rows I + icols;  dw2 [E, d, ni].
 * An expert with no row gets zero gradients.  The weight gradients of a column need
 * that column of a and dh on every routed row; those are computed column by column,
 * apart from the token rows, which run whole. */

/* nearest BF16 value of v (ties to even); v finite and inside the normal range */
static double bf16_round(double v)
{
    if (v == 0.0) return 0.0;
    int ex;
    double m = frexp(v, &ex);                       /* |m| in [0.5, 1) */
    return ldexp(nearbyint(ldexp(m, 8)), ex - 8);   /* 8 significant bits */
}

/* MX quantize->dequantize image of n <= 32 values v[0], v[stride], ... in place;
 * missing elements of a short block count as zeros, which change nothing */
static void mx_block_image(double* v, int n, size_t stride)
{
    double blk[32] = {0};
    for (int i = 0; i < n; ++i) blk[i] = v[(size_t)i * stride];
    uint8_t sb = orc_mx_scale_byte(blk, n);
    double X = ldexp(1.0, (int)sb - 127);
    for (int i = 0; i < n; ++i) v[(size_t)i * stride] = orc_e4m3_decode(orc_e4m3_encode(blk[i] / X)) * X;
}

/* images of the `mats` matrices m + e*rows*cols (rows x cols, row-major): along
 * each row (along_rows != 0), or along each column in blocks of 32 rows */
static void mx_matrix_image(double* m, int mats, int rows, int cols, int along_rows)
{
#pragma omp parallel for schedule(static)
    for (int e = 0; e < mats; ++e) {
        double* me = m + (size_t)e * rows * cols;
        if (along_rows) {
            for (int r = 0; r < rows; ++r)
                for (int b = 0; b < cols; b += 32) mx_block_image(me + (size_t)r * cols + b, 32, 1);
        } else {
            for (int c = 0; c < cols; ++c)
                for (int b = 0; b < rows; b += 32)
                    mx_block_image(me + (size_t)b * cols + c, rows - b < 32 ? rows - b : 32, (size_t)cols);
        }
    }
}

/* the same for float matrices (the weights): each image value is an E4M3 code times
 * a power of two, exact in float32 */
static void mx_matrix_image_f(float* m, int mats, int rows, int cols, int along_rows)
{
#pragma omp parallel for schedule(static)
    for (int e = 0; e < mats; ++e) {
        float* me = m + (size_t)e * rows * cols;
        double blk[32];
        if (along_rows) {
            for (int r = 0; r < rows; ++r)
                for (int b = 0; b < cols; b += 32) {
                    for (int i = 0; i < 32; ++i) blk[i] = (double)me[(size_t)r * cols + b + i];
                    mx_block_image(blk, 32, 1);
                    for (int i = 0; i < 32; ++i) me[(size_t)r * cols + b + i] = (float)blk[i];
                }
        } else {
            for (int c = 0; c < cols; ++c)
                for (int b = 0; b < rows; b += 32) {
                    const int n = rows - b < 32 ? rows - b : 32;
                    for (int i = 0; i < n; ++i) blk[i] = (double)me[(size_t)(b + i) * cols + c];
                    mx_block_image(blk, n, 1);
                    for (int i = 0; i < n; ++i) me[(size_t)(b + i) * cols + c] = (float)blk[i];
                }
        }
    }
}

int orc_train_mx(int T, int d, int I, int E, int k,
                 const float* x, const int32_t* ids, const float* scores,
                 const float* w13, const float* w2, const float* dy, int act,
                 int ntok, const int32_t* toks, double* y, double* dx, double* ds,
                 int ni, const int32_t* icols, double* dw13, double* dw2)
{
    int rc = orc_check_routing(T, E, k, ids);
    if (rc != ORC_OK) return rc;
    if (d % 32 || I % 32) return ORC_ERR_RANGE;
    for (int q = 0; q < ntok; ++q) if (toks[q] < 0 || toks[q] >= T) return ORC_ERR_RANGE;
    for (int q = 0; q < ni; ++q) if (icols[q] < 0 || icols[q] >= I) return ORC_ERR_RANGE;
    const size_t R = (size_t)T * k, n13 = (size_t)E * 2 * I * d, n2 = (size_t)E * d * I;
    const size_t R1 = R ? R : 1;
    int32_t* m_indptr = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t* gather = (int32_t*)malloc(sizeof(int32_t) * R1);
    int32_t* slots = (int32_t*)malloc(sizeof(int32_t) * R1);
    float* probs = (float*)malloc(sizeof(float) * R1);
    float* wf13 = (float*)malloc(sizeof(float) * n13);   /* FPROP images */
    float* wf2 = (float*)malloc(sizeof(float) * n2);
    float* wb13 = (float*)malloc(sizeof(float) * n13);   /* DGRAD images */
    float* wb2 = (float*)malloc(sizeof(float) * n2);
    double* ab = (double*)malloc(sizeof(double) * R1 * (ni ? ni : 1));        /* stored a (BF16), columns icols */
    double* dhb = (double*)malloc(sizeof(double) * R1 * 2 * (ni ? ni : 1));   /* dh in BF16: dg, du of icols */
    int failed = !m_indptr || !gather || !slots || !probs || !wf13 || !wf2 || !wb13 || !wb2 || !ab || !dhb;
    if (!failed) rc = orc_dispatch(T, E, k, ids, scores, m_indptr, gather, slots, probs);
    if (!failed && rc == ORC_OK) {
        memcpy(wf13, w13, sizeof(float) * n13);
        memcpy(wb13, w13, sizeof(float) * n13);
        memcpy(wf2, w2, sizeof(float) * n2);
        memcpy(wb2, w2, sizeof(float) * n2);
        mx_matrix_image_f(wf13, E, 2 * I, d, 1);
        mx_matrix_image_f(wf2, E, d, I, 1);
        mx_matrix_image_f(wb13, E, 2 * I, d, 0);
        mx_matrix_image_f(wb2, E, d, I, 0);

        /* the token rows, whole: FPROP, DGRAD, combine and router gradient */
#pragma omp parallel for schedule(dynamic, 1)
        for (int q = 0; q < ntok; ++q) {
            double* buf = (double*)malloc(sizeof(double) * (4 * (size_t)d + 6 * (size_t)I));
            if (!buf) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *xq = buf, *dO = xq + d, *o = dO + d, *dxp = o + d, *gb = dxp + d, *ub = gb + I,
                   *a = ub + I, *dA = a + I, *dh = dA + I;
            const int t = toks[q];
            double* y_t = y + (size_t)q * d;
            double* dx_t = dx + (size_t)q * d;
            for (int n = 0; n < d; ++n) { y_t[n] = 0.0; dx_t[n] = 0.0; }
            for (int c = 0; c < d; ++c) xq[c] = (double)x[(size_t)t * d + c];
            for (int b = 0; b < d; b += 32) mx_block_image(xq + b, 32, 1);
            for (int j = 0; j < k; ++j) {
                const int e = ids[(size_t)t * k + j];
                const double s = (double)scores[(size_t)t * k + j];
                const float* f13 = wf13 + (size_t)e * 2 * I * d;
                const float* f2 = wf2 + (size_t)e * d * I;
                const float* b13 = wb13 + (size_t)e * 2 * I * d;
                const float* b2 = wb2 + (size_t)e * d * I;
                for (int i = 0; i < I; ++i) {
                    double g = 0.0, u = 0.0;
                    for (int c = 0; c < d; ++c) {
                        g += (double)f13[(size_t)i * d + c] * xq[c];
                        u += (double)f13[(size_t)(I + i) * d + c] * xq[c];
                    }
                    a[i] = act_f(act, g) * u;
                    gb[i] = bf16_round(g);
                    ub[i] = bf16_round(u);
                }
                for (int b = 0; b < I; b += 32) mx_block_image(a + b, 32, 1);
                double dot = 0.0;
                for (int n = 0; n < d; ++n) {
                    double acc = 0.0;
                    for (int i = 0; i < I; ++i) acc += (double)f2[(size_t)n * I + i] * a[i];
                    o[n] = acc;
                    y_t[n] += s * acc;
                    dot += (double)dy[(size_t)t * d + n] * acc;
                }
                ds[(size_t)q * k + j] = dot;
                /* DGRAD */
                for (int n = 0; n < d; ++n) dO[n] = s * (double)dy[(size_t)t * d + n];
                for (int b = 0; b < d; b += 32) mx_block_image(dO + b, 32, 1);
                for (int i = 0; i < I; ++i) {
                    double acc = 0.0;
                    for (int n = 0; n < d; ++n) acc += (double)b2[(size_t)n * I + i] * dO[n];
                    dA[i] = bf16_round(acc);
                }
                for (int i = 0; i < I; ++i) {
                    dh[i] = dA[i] * ub[i] * act_df(act, gb[i]);
                    dh[I + i] = dA[i] * act_f(act, gb[i]);
                }
                for (int b = 0; b < 2 * I; b += 32) mx_block_image(dh + b, 32, 1);
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int jj = 0; jj < 2 * I; ++jj) acc += (double)b13[(size_t)jj * d + c] * dh[jj];
                    dx_t[c] += acc;
                }
            }
            free(buf);
        }

        /* columns icols of a and dh on every routed row, for the weight gradients */
#pragma omp parallel for schedule(dynamic, 16)
        for (size_t r = 0; r < R; ++r) {
            double* buf = (double*)malloc(sizeof(double) * 2 * (size_t)d);
            if (!buf) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *xq = buf, *dO = xq + d;
            int e = 0;
            while (m_indptr[e + 1] <= (int32_t)r) ++e;
            const int t = gather[r];
            const double s = (double)probs[r];
            const float* f13 = wf13 + (size_t)e * 2 * I * d;
            const float* b2 = wb2 + (size_t)e * d * I;
            for (int c = 0; c < d; ++c) xq[c] = (double)x[(size_t)t * d + c];
            for (int b = 0; b < d; b += 32) mx_block_image(xq + b, 32, 1);
            for (int n = 0; n < d; ++n) dO[n] = s * (double)dy[(size_t)t * d + n];
            for (int b = 0; b < d; b += 32) mx_block_image(dO + b, 32, 1);
            for (int q = 0; q < ni; ++q) {
                const int i = icols[q];
                double g = 0.0, u = 0.0, acc = 0.0;
                for (int c = 0; c < d; ++c) {
                    g += (double)f13[(size_t)i * d + c] * xq[c];
                    u += (double)f13[(size_t)(I + i) * d + c] * xq[c];
                }
                for (int n = 0; n < d; ++n) acc += (double)b2[(size_t)n * I + i] * dO[n];
                const double gq = bf16_round(g), uq = bf16_round(u), dA = bf16_round(acc);
                ab[r * ni + q] = bf16_round(act_f(act, g) * u);
                dhb[(r * 2 + 0) * ni + q] = bf16_round(dA * uq * act_df(act, gq));
                dhb[(r * 2 + 1) * ni + q] = bf16_round(dA * act_f(act, gq));
            }
            free(buf);
        }

        /* WGRAD, one expert at a time, operands blocked along its routed rows */
#pragma omp parallel for schedule(dynamic, 1)
        for (int e = 0; e < E; ++e) {
            const int r0 = m_indptr[e], rows = m_indptr[e + 1] - r0;
            double* dw2_e = dw2 + (size_t)e * d * ni;
            double* dw13_e = dw13 + (size_t)e * 2 * ni * d;
            for (size_t z = 0; z < (size_t)d * ni; ++z) dw2_e[z] = 0.0;
            for (size_t z = 0; z < (size_t)2 * ni * d; ++z) dw13_e[z] = 0.0;
            if (rows == 0) continue;
            double* buf = (double*)malloc(sizeof(double) * (size_t)rows * (2 * (size_t)d + 3 * (size_t)ni));
            if (!buf) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double *dOt = buf, *xt = dOt + (size_t)rows * d, *at = xt + (size_t)rows * d,
                   *dht = at + (size_t)rows * ni;
            for (int q = 0; q < rows; ++q) {
                const size_t r = (size_t)(r0 + q);
                const int t = gather[r];
                for (int n = 0; n < d; ++n) {
                    dOt[(size_t)q * d + n] = (double)probs[r] * (double)dy[(size_t)t * d + n];
                    xt[(size_t)q * d + n] = (double)x[(size_t)t * d + n];
                }
                for (int c = 0; c < ni; ++c) at[(size_t)q * ni + c] = ab[r * ni + c];
                for (int c = 0; c < 2 * ni; ++c) dht[(size_t)q * 2 * ni + c] = dhb[r * 2 * ni + c];
            }
            mx_matrix_image(dOt, 1, rows, d, 0);
            mx_matrix_image(xt, 1, rows, d, 0);
            if (ni > 0) {
                mx_matrix_image(at, 1, rows, ni, 0);
                mx_matrix_image(dht, 1, rows, 2 * ni, 0);
            }
            for (int q = 0; q < rows; ++q) {
                for (int n = 0; n < d; ++n) {
                    const double gv = dOt[(size_t)q * d + n];
                    for (int c = 0; c < ni; ++c) dw2_e[(size_t)n * ni + c] += gv * at[(size_t)q * ni + c];
                }
                for (int jj = 0; jj < 2 * ni; ++jj) {
                    const double gv = dht[(size_t)q * 2 * ni + jj];
                    for (int c = 0; c < d; ++c) dw13_e[(size_t)jj * d + c] += gv * xt[(size_t)q * d + c];
                }
            }
            free(buf);
        }
    }
    free(m_indptr); free(gather); free(slots); free(probs);
    free(wf13); free(wf2); free(wb13); free(wb2);
    free(ab); free(dhb);
    if (rc != ORC_OK) return rc;
    return failed ? ORC_ERR_ALLOC : ORC_OK;
}
