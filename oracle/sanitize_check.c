/*
 * sanitize_check.c -- the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by tests/test_oracle_sanitized.py):
 * compiled together with moe_oracle.c with -fsanitize=address,undefined, it
 * calls every exported oracle function on small seeded inputs and on the
 * degenerate shapes (one token, one expert, k = E, capacity 1, every slot
 * dropped but the first, tied logits) and checks properties the pages'
 * definitions fix, so that an out-of-bounds access, a use of freed memory,
 * an integer overflow or another undefined operation anywhere in the oracle
 * stops the run, and a plainly wrong result fails it:
 *   - tied logits select experts 0..k-1 with weights 1/k;
 *   - the routing weights of a token sum to 1 and the k experts are distinct;
 *   - the dispatch keeps every expert's first cap slots in token order, its
 *     kept rows are a bijection onto [0, S), perm is -1 past S;
 *   - identity experts (W1 = [I | -I | 0], W2 = [I; -I; 0], zero biases)
 *     return every token row exactly;
 *   - the ordered co-selection counts sum to T k (k - 1) / 2;
 *   - per-token gate gradients sum to zero, so dbg sums to zero;
 *   - the balance loss is lambda (T k - drops) / (T k E).
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_threads(void);
double oracle_gelu(double u);
void oracle_gate(int64_t T, int64_t d, int64_t E, int dtype, const void* x, const float* Wg, const float* bg,
                 double* L);
void oracle_route(int64_t T, int64_t E, int64_t k, double tau, const float* L, int32_t* idx, double* w);
int64_t oracle_capacity(int64_t T, int64_t E, int64_t k, float cf);
void oracle_dispatch(int64_t T, int64_t E, int64_t k, int64_t cap, const int32_t* idx, int32_t* routed,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot);
void oracle_ffn_rows(int64_t n, const int32_t* tok, const int32_t* exp_id, int64_t d, int64_t dff, int dtype,
                     const void* x, const void* W1, const float* b1, const void* W2, const float* b2, double* out);
void oracle_layer_tokens(int64_t n, const int32_t* toks, int64_t d, int64_t dff, int64_t k, int dtype,
                         const void* x, const void* W1, const float* b1, const void* W2, const float* b2,
                         const int32_t* idx, const int32_t* slot, const double* w, double* y);
double oracle_aux(int64_t E, int64_t T, int64_t k, const int32_t* counts, double lam);
void oracle_coactivation(int64_t T, int64_t E, int64_t k, const int32_t* idx, int64_t* H, int64_t* routed);
void oracle_load_stats(int64_t E, const int64_t* load, double* mean, double* var, double* cv);
void oracle_noisy_logits(int64_t n, const float* L, const float* noise, float scale, float* out);
void oracle_route_top1_full(int64_t T, int64_t E, double tau, const float* L, int32_t* idx, double* w);
double oracle_aux_variance(int64_t E, const int64_t* load, double lam);
void oracle_window_aux(int64_t n, int64_t E, int64_t T, int64_t k, int64_t W, const int32_t* counts, double lam,
                       double* aux, double* pbar);
void oracle_ffn_backward_rows(int64_t n, const int32_t* tok, const int32_t* exp_id, const double* wt, int64_t d,
                              int64_t dff, int dtype, const void* x, const void* W1, const float* b1,
                              const void* W2, const float* b2, const float* dy, double* dw, double* dxp,
                              double* dW1, double* db1, double* dW2, double* db2);
void oracle_route_backward(int64_t T, int64_t d, int64_t E, int64_t k, double tau, int dtype, const void* x,
                           const float* Wg, const int32_t* idx, const double* w, const double* dw, double* dl,
                           double* dWg, double* dbg, double* dxg);
void oracle_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t dff, int dtype, float cf, double tau,
                          double lam, const void* x, const float* Wg, const float* bg, const void* W1,
                          const float* b1, const void* W2, const float* b2, double* Lref, float* L32, int32_t* idx,
                          double* w, int32_t* routed, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* slot, double* y, double* aux);

static int failures = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");                \
            ++failures;                           \
        }                                         \
    } while (0)

/* xorshift64*, only to fill inputs */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0;
}
static float nrand(void) { return (float)(sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307179586 * urand())); }
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* one layer shape end to end, with every function that takes it */
static void run_case(int64_t T, int64_t d, int64_t E, int64_t k, int64_t dff, float cf, double tau, int dtype,
                     int tied) {
    const size_t esz = dtype ? 2 : 4;
    void* x = malloc((size_t)(T * d) * esz);
    void* W1 = malloc((size_t)(E * d * dff) * esz);
    void* W2 = malloc((size_t)(E * dff * d) * esz);
    float* Wg = malloc(sizeof(float) * (size_t)(d * E));
    float* bg = malloc(sizeof(float) * (size_t)E);
    float* b1 = malloc(sizeof(float) * (size_t)(E * dff));
    float* b2 = malloc(sizeof(float) * (size_t)(E * d));
    for (int64_t i = 0; i < T * d; ++i) {
        const float v = nrand();
        if (dtype) ((uint16_t*)x)[i] = to_bf16(v); else ((float*)x)[i] = v;
    }
    for (int64_t i = 0; i < E * d * dff; ++i) {
        const float a = nrand() * 0.1f, b = nrand() * 0.1f;
        if (dtype) { ((uint16_t*)W1)[i] = to_bf16(a); ((uint16_t*)W2)[i] = to_bf16(b); }
        else { ((float*)W1)[i] = a; ((float*)W2)[i] = b; }
    }
    for (int64_t i = 0; i < d * E; ++i) Wg[i] = tied ? 0.0f : nrand() * 0.2f;
    for (int64_t i = 0; i < E; ++i) bg[i] = tied ? 0.0f : nrand() * 0.1f;
    for (int64_t i = 0; i < E * dff; ++i) b1[i] = nrand() * 0.1f;
    for (int64_t i = 0; i < E * d; ++i) b2[i] = nrand() * 0.1f;

    const int64_t cap = oracle_capacity(T, E, k, cf);
    const int64_t smax = T * k < E * cap ? T * k : E * cap;
    double* Lref = malloc(sizeof(double) * (size_t)(T * E));
    float* L32 = malloc(sizeof(float) * (size_t)(T * E));
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(T * k));
    double* w = malloc(sizeof(double) * (size_t)(T * k));
    int32_t* routed = malloc(sizeof(int32_t) * (size_t)E);
    int32_t* counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* perm = malloc(sizeof(int32_t) * (size_t)(smax > 0 ? smax : 1));
    int32_t* slot = malloc(sizeof(int32_t) * (size_t)(T * k));
    double* y = malloc(sizeof(double) * (size_t)(T * d));
    double aux = 0.0;
    oracle_layer_forward(T, d, E, k, dff, dtype, cf, tau, 0.01, x, Wg, bg, W1, b1, W2, b2, Lref, L32, idx, w,
                         routed, counts, offsets, perm, slot, y, &aux);

    /* routing: distinct experts, weights sum to 1; tied logits -> 0..k-1, 1/k */
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            s += w[t * k + j];
            CHECK(idx[t * k + j] >= 0 && idx[t * k + j] < E, "expert index out of range");
            for (int64_t i = 0; i < j; ++i) CHECK(idx[t * k + i] != idx[t * k + j], "repeated expert");
            if (tied) {
                CHECK(idx[t * k + j] == j, "tied logits: expert %d at position %d", idx[t * k + j], (int)j);
                CHECK(fabs(w[t * k + j] - 1.0 / (double)k) < 1e-15, "tied logits: weight");
            }
        }
        CHECK(fabs(s - 1.0) < 1e-12, "weights of token %lld sum to %g", (long long)t, s);
    }
    /* dispatch: counts, bijection, token order, drop rule */
    int64_t S = 0, drops = 0;
    for (int64_t e = 0; e < E; ++e) {
        CHECK(counts[e] <= cap && counts[e] <= routed[e], "count above capacity or routed");
        CHECK(offsets[e + 1] - offsets[e] == counts[e], "offsets");
        S += counts[e];
    }
    int32_t* seen = calloc((size_t)(smax > 0 ? smax : 1), sizeof(int32_t));
    int64_t* fill = calloc((size_t)E, sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            const int64_t r = slot[t * k + j], e = idx[t * k + j];
            if (r < 0) {
                ++drops;
                CHECK(fill[e] >= cap, "slot dropped while its expert had room");
            } else {
                CHECK(r >= offsets[e] && r < offsets[e + 1], "row outside its expert's segment");
                CHECK(r == offsets[e] + fill[e], "rows not in token order");
                CHECK(perm[r] == t, "perm/slot mismatch");
                seen[r] += 1;
            }
            ++fill[e];
        }
    for (int64_t r = 0; r < smax; ++r) CHECK(r < S ? seen[r] == 1 : perm[r] == -1, "rows not a bijection");
    CHECK(S + drops == T * k, "kept + dropped != T k");
    const double aux_cf = 0.01 * (double)(T * k - drops) / ((double)(T * k) * (double)E);
    CHECK(fabs(aux - aux_cf) <= 1e-15 + 1e-12 * aux_cf, "balance loss %g vs %g", aux, aux_cf);

    /* heat map, load statistics, router variants, losses */
    int64_t* H = malloc(sizeof(int64_t) * (size_t)(E * E));
    int64_t* rt = malloc(sizeof(int64_t) * (size_t)E);
    oracle_coactivation(T, E, k, idx, H, rt);
    int64_t hs = 0;
    for (int64_t i = 0; i < E * E; ++i) hs += H[i];
    CHECK(hs == T * k * (k - 1) / 2, "co-selection total");
    double mean, var, cv;
    oracle_load_stats(E, rt, &mean, &var, &cv);
    CHECK(fabs(mean * (double)E - (double)(T * k)) < 1e-9, "mean load");
    (void)oracle_aux_variance(E, rt, 0.01);
    float* noise = malloc(sizeof(float) * (size_t)(T * E));
    float* noisy = malloc(sizeof(float) * (size_t)(T * E));
    for (int64_t i = 0; i < T * E; ++i) noise[i] = nrand();
    oracle_noisy_logits(T * E, L32, noise, 0.1f, noisy);
    int32_t* i1 = malloc(sizeof(int32_t) * (size_t)T);
    double* w1 = malloc(sizeof(double) * (size_t)T);
    oracle_route_top1_full(T, E, tau, noisy, i1, w1);
    for (int64_t t = 0; t < T; ++t) CHECK(w1[t] > 0.0 && w1[t] <= 1.0 && i1[t] >= 0 && i1[t] < E, "top-1");
    double wa[3], pb[3 * 1024];
    if (E <= 1024) {
        int32_t* seq = malloc(sizeof(int32_t) * (size_t)(3 * E));
        for (int64_t b = 0; b < 3; ++b)
            for (int64_t e = 0; e < E; ++e) seq[b * E + e] = counts[e];
        oracle_window_aux(3, E, T, k, 2, seq, 0.01, wa, pb);
        CHECK(fabs(wa[2] - aux) <= 1e-12 * (aux + 1e-30), "window loss of constant batches");
        free(seq);
    }

    /* expert FFN on every kept row, and the backward of the layer */
    int32_t* tok = malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    int32_t* eid = malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    double* wt = malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j)
            if (slot[t * k + j] >= 0) { tok[n] = (int32_t)t; eid[n] = idx[t * k + j]; wt[n] = w[t * k + j]; ++n; }
    double* o = malloc(sizeof(double) * (size_t)((n > 0 ? n : 1) * d));
    oracle_ffn_rows(n, tok, eid, d, dff, dtype, x, W1, b1, W2, b2, o);
    float* dy = malloc(sizeof(float) * (size_t)(T * d));
    for (int64_t i = 0; i < T * d; ++i) dy[i] = nrand();
    double* dwr = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* dxp = malloc(sizeof(double) * (size_t)((n > 0 ? n : 1) * d));
    double* dW1 = calloc((size_t)(E * d * dff), sizeof(double));
    double* db1 = calloc((size_t)(E * dff), sizeof(double));
    double* dW2 = calloc((size_t)(E * dff * d), sizeof(double));
    double* db2 = calloc((size_t)(E * d), sizeof(double));
    oracle_ffn_backward_rows(n, tok, eid, wt, d, dff, dtype, x, W1, b1, W2, b2, dy, dwr, dxp, dW1, db1, dW2, db2);
    double* dw = calloc((size_t)(T * k), sizeof(double));
    for (int64_t i = 0, m = 0; i < T * k; ++i)
        if (slot[i] >= 0) dw[i] = dwr[m++];
    double* dl = malloc(sizeof(double) * (size_t)(T * E));
    double* dWg = malloc(sizeof(double) * (size_t)(d * E));
    double* dbg = malloc(sizeof(double) * (size_t)E);
    double* dxg = malloc(sizeof(double) * (size_t)(T * d));
    oracle_route_backward(T, d, E, k, tau, dtype, x, Wg, idx, w, dw, dl, dWg, dbg, dxg);
    double sb = 0.0, mb = 0.0;
    for (int64_t e = 0; e < E; ++e) { sb += dbg[e]; mb = fmax(mb, fabs(dbg[e])); }
    CHECK(fabs(sb) <= 1e-9 * (mb + 1e-30) * (double)E + 1e-300, "gate bias gradients sum to %g", sb);

    free(x); free(W1); free(W2); free(Wg); free(bg); free(b1); free(b2); free(Lref); free(L32); free(idx); free(w);
    free(routed); free(counts); free(offsets); free(perm); free(slot); free(y); free(seen); free(fill); free(H);
    free(rt); free(noise); free(noisy); free(i1); free(w1); free(tok); free(eid); free(wt); free(o); free(dy);
    free(dwr); free(dxp); free(dW1); free(db1); free(dW2); free(db2); free(dw); free(dl); free(dWg); free(dbg);
    free(dxg);
}

/* identity experts return every token row exactly (no capacity limit, k = 1) */
static void identity_experts(void) {
    const int64_t T = 9, d = 5, E = 3, dff = 4 * d;
    float* x = malloc(sizeof(float) * T * d);
    float* W1 = calloc((size_t)(E * d * dff), sizeof(float));
    float* W2 = calloc((size_t)(E * dff * d), sizeof(float));
    float* b1 = calloc((size_t)(E * dff), sizeof(float));
    float* b2 = calloc((size_t)(E * d), sizeof(float));
    for (int64_t i = 0; i < T * d; ++i) x[i] = nrand();
    for (int64_t e = 0; e < E; ++e)
        for (int64_t c = 0; c < d; ++c) {
            W1[(e * d + c) * dff + c] = 1.0f;
            W1[(e * d + c) * dff + d + c] = -1.0f;
            W2[(e * dff + c) * d + c] = 1.0f;
            W2[(e * dff + d + c) * d + c] = -1.0f;
        }
    int32_t tok[9], eid[9];
    for (int64_t t = 0; t < T; ++t) { tok[t] = (int32_t)t; eid[t] = (int32_t)(t % E); }
    double* o = malloc(sizeof(double) * T * d);
    oracle_ffn_rows(T, tok, eid, d, dff, 0, x, W1, b1, W2, b2, o);
    for (int64_t i = 0; i < T * d; ++i)
        CHECK(fabs(o[i] - (double)x[i]) <= 1e-15 * fabs((double)x[i]) + 1e-300, "identity expert");
    CHECK(oracle_gelu(0.0) == 0.0, "GELU(0)");
    free(x); free(W1); free(W2); free(b1); free(b2); free(o);
}

int main(void) {
    identity_experts();
    /* T, d, E, k, d_ff, capacity factor, tau, dtype, tied logits */
    run_case(37, 16, 6, 2, 24, 1.0f, 1.0, 0, 0);
    run_case(50, 24, 8, 3, 40, 0.75f, 0.7, 1, 0);
    run_case(1, 8, 4, 2, 8, 1.0f, 1.0, 1, 0);      /* one token */
    run_case(20, 8, 1, 1, 16, 0.0f, 1.0, 0, 0);    /* one expert */
    run_case(15, 8, 4, 4, 16, 0.0f, 0.2, 0, 0);    /* k = E, soft */
    run_case(30, 8, 5, 2, 8, 0.02f, 1.0, 1, 0);    /* capacity 1 */
    run_case(12, 8, 7, 3, 8, 1.0f, 1.0, 0, 1);     /* tied logits */
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle under ASan/UBSan: every check passed (%d threads)\n", oracle_threads());
    return 0;
}
