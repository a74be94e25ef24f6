/* Host sanitizer run of the CPU oracle (tests/test_sanitize.py builds this file with
 * oracle/moe_oracle.c under gcc -fsanitize=address,undefined and runs it): every oracle
 * entry point on small layers, including empty experts, k = E, one token, no token and
 * invalid routing, so that an out-of-bounds access, a leak or undefined behaviour in the
 * oracle's loops stops the run.  It checks return codes and a few identities; numerical
 * parity is pinned by the Python tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_check_routing(int T, int E, int k, const int32_t* ids);
int orc_dispatch(int T, int E, int k, const int32_t* ids, const float* scores, int32_t* m_indptr,
                 int32_t* gather, int32_t* slots, float* probs);
int orc_forward_tokens(int T, int d, int I, int E, int k, const float* x, const int32_t* ids,
                       const float* scores, const float* w13, const float* w2, int ntok,
                       const int32_t* toks, double* y, double* o_out, double* a_out, int act);
int orc_backward_tokens(int T, int d, int I, int E, int k, const float* x, const int32_t* ids,
                        const float* scores, const float* w13, const float* w2, const float* dy,
                        int ntok, const int32_t* toks, double* dx, double* ds, int act);
int orc_wgrad_cols(int T, int d, int I, int E, int k, const float* x, const int32_t* ids,
                   const float* scores, const float* w13, const float* w2, const float* dy, int ni,
                   const int32_t* icols, double* dw2, double* dw13, int act);
void orc_mx_quantize(int64_t rows, int K, const float* v, uint8_t* codes, uint8_t* scales);
void orc_mx_dequantize(int64_t rows, int K, const uint8_t* codes, const uint8_t* scales, float* out);
int orc_forward_tokens_mx(int T, int d, int I, int E, int k, const float* x, const int32_t* ids,
                          const float* scores, const float* w13, const float* w2, int ntok,
                          const int32_t* toks, double* y, int act);
int orc_train_mx(int T, int d, int I, int E, int k, const float* x, const int32_t* ids,
                 const float* scores, const float* w13, const float* w2, const float* dy, int act,
                 int ntok, const int32_t* toks, double* y, double* dx, double* ds,
                 int ni, const int32_t* icols, double* dw13, double* dw2);

static uint64_t state = 88172645463325252ull;
static double uni(void)
{
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}
static float* rnd(size_t n, double scale)
{
    float* p = malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)((2.0 * uni() - 1.0) * scale);
    return p;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { if (fails++ < 10) fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); } } while (0)

static void run_layer(int T, int d, int I, int E, int k, int act, int empty_from)
{
    float* x = rnd((size_t)T * d, 1.0);
    float* w13 = rnd((size_t)E * 2 * I * d, 0.1);
    float* w2 = rnd((size_t)E * d * I, 0.1);
    float* dy = rnd((size_t)T * d, 1.0);
    float* sc = rnd((size_t)T * k, 1.0);
    int32_t* ids = malloc(sizeof(int32_t) * ((size_t)T * k + 1));
    int span = empty_from < k ? k : empty_from;       /* experts >= span get no row */
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) ids[(size_t)t * k + j] = (t + j) % span;
    int32_t* m = malloc(sizeof(int32_t) * (E + 1));
    int32_t* gather = malloc(sizeof(int32_t) * ((size_t)T * k + 1));
    int32_t* slots = malloc(sizeof(int32_t) * ((size_t)T * k + 1));
    float* probs = malloc(sizeof(float) * ((size_t)T * k + 1));
    CHECK(orc_check_routing(T, E, k, ids) == 0);
    CHECK(orc_dispatch(T, E, k, ids, sc, m, gather, slots, probs) == 0);
    CHECK(m[0] == 0 && m[E] == T * k);
    int32_t* toks = malloc(sizeof(int32_t) * (T + 1));
    for (int t = 0; t < T; ++t) toks[t] = T - 1 - t;
    double* y = calloc((size_t)T * d + 1, sizeof(double));
    double* o = calloc((size_t)T * k * d + 1, sizeof(double));
    double* a = calloc((size_t)T * k * I + 1, sizeof(double));
    double* dx = calloc((size_t)T * d + 1, sizeof(double));
    double* ds = calloc((size_t)T * k + 1, sizeof(double));
    CHECK(orc_forward_tokens(T, d, I, E, k, x, ids, sc, w13, w2, T, toks, y, o, a, act) == 0);
    CHECK(orc_backward_tokens(T, d, I, E, k, x, ids, sc, w13, w2, dy, T, toks, dx, ds, act) == 0);
    int32_t* cols = malloc(sizeof(int32_t) * I);
    for (int i = 0; i < I; ++i) cols[i] = I - 1 - i;
    double* dw2 = calloc((size_t)E * d * I, sizeof(double));
    double* dw13 = calloc((size_t)E * 2 * I * d, sizeof(double));
    CHECK(orc_wgrad_cols(T, d, I, E, k, x, ids, sc, w13, w2, dy, I, cols, dw2, dw13, act) == 0);
    for (int e = span; e < E; ++e)
        for (size_t z = 0; z < (size_t)d * I; ++z) CHECK(dw2[(size_t)e * d * I + z] == 0.0);
    if (d % 32 == 0 && I % 32 == 0) {
        double* yq = calloc((size_t)T * d + 1, sizeof(double));
        CHECK(orc_forward_tokens_mx(T, d, I, E, k, x, ids, sc, w13, w2, T, toks, yq, act) == 0);
        uint8_t* codes = malloc((size_t)T * d + 1);
        uint8_t* scales = malloc((size_t)T * d / 32 + 1);
        float* back = malloc(sizeof(float) * ((size_t)T * d + 1));
        orc_mx_quantize(T, d, x, codes, scales);
        orc_mx_dequantize(T, d, codes, scales, back);
        /* within half an E4M3 step: 1/16 of the value for a normal element; x lies in
         * (-1, 1), so a block scale is at most 2^-8 and a subnormal element is within
         * 2^-10 of the scale, 2^-18 */
        for (size_t z = 0; z < (size_t)T * d; ++z) CHECK(fabs(back[z] - x[z]) <= 0.0625 * fabs(x[z]) + 4e-6);
        /* the MXFP8 training step: every output written, unrouted experts zero */
        double* ty = calloc((size_t)T * d + 1, sizeof(double));
        double* tdx = calloc((size_t)T * d + 1, sizeof(double));
        double* tds = calloc((size_t)T * k + 1, sizeof(double));
        double* tdw13 = malloc(sizeof(double) * (size_t)E * 2 * I * d);
        double* tdw2 = malloc(sizeof(double) * (size_t)E * d * I);
        for (size_t z = 0; z < (size_t)E * d * I; ++z) tdw2[z] = NAN;
        for (size_t z = 0; z < (size_t)E * 2 * I * d; ++z) tdw13[z] = NAN;
        int32_t* all_i = malloc(sizeof(int32_t) * I);
        for (int i = 0; i < I; ++i) all_i[i] = i;
        CHECK(orc_train_mx(T, d, I, E, k, x, ids, sc, w13, w2, dy, act, T, toks, ty, tdx, tds, I, all_i,
                           tdw13, tdw2) == 0);
        /* a subset of tokens and columns writes only its own outputs */
        if (T > 1 && I > 2) {
            int32_t sub_t[1] = {T - 1}, sub_i[2] = {I - 1, 0};
            double* sy = calloc((size_t)d * 2, sizeof(double));
            double* sdw13 = calloc((size_t)E * 2 * 2 * d + 1, sizeof(double));
            double* sdw2 = calloc((size_t)E * d * 2 + 1, sizeof(double));
            CHECK(orc_train_mx(T, d, I, E, k, x, ids, sc, w13, w2, dy, act, 1, sub_t, sy, sy + d, tds, 2, sub_i,
                               sdw13, sdw2) == 0);
            free(sy); free(sdw13); free(sdw2);
        }
        free(all_i);
        for (size_t z = 0; z < (size_t)E * d * I; ++z) CHECK(!isnan(tdw2[z]));
        for (size_t z = 0; z < (size_t)E * 2 * I * d; ++z) CHECK(!isnan(tdw13[z]));
        for (int e = span; e < E; ++e)
            for (size_t z = 0; z < (size_t)d * I; ++z) CHECK(tdw2[(size_t)e * d * I + z] == 0.0);
        free(yq); free(codes); free(scales); free(back);
        free(ty); free(tdx); free(tds); free(tdw13); free(tdw2);
    }
    /* invalid routing: refused, nothing written past the arrays */
    if (T > 0) {
        int32_t keep = ids[0];
        ids[0] = E;
        CHECK(orc_dispatch(T, E, k, ids, sc, m, gather, slots, probs) == 1);
        if (k > 1) {
            ids[0] = ids[1];
            CHECK(orc_dispatch(T, E, k, ids, sc, m, gather, slots, probs) == 2);
        }
        ids[0] = keep;
    }
    free(x); free(w13); free(w2); free(dy); free(sc); free(ids); free(m); free(gather); free(slots);
    free(probs); free(toks); free(y); free(o); free(a); free(dx); free(ds); free(cols); free(dw2); free(dw13);
}

int main(void)
{
    for (int act = 0; act < 3; ++act) {
        run_layer(5, 64, 32, 4, 2, act, 4);
        run_layer(3, 64, 64, 8, 8, act, 8);      /* k = E */
        run_layer(9, 96, 32, 12, 3, act, 5);     /* experts 5..11 empty */
        run_layer(1, 32, 32, 2, 1, act, 1);      /* one token, one expert used */
        run_layer(0, 64, 32, 4, 2, act, 4);      /* no token */
    }
    if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
