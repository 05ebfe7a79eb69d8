/*
 * moe_oracle.c -- plain, slow CPU oracle of the MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
 * the benchmark's cpu_baseline leg may load or call this library.  It shares
 * no code, header, table or helper with the HIP library: it is written
 * directly from the definitions on the pages, in double precision, with plain
 * loops (no blocking, no fusion, no BLAS, no intrinsics).
 *
 * Pages cited (by title and section):
 *   [PithTrain]  "Native MoE training system PithTrain: core optimisations from
 *                sparse communication to dynamic memory management"
 *   [PyTorchMoE] "PyTorch distributed MoE training: principles, implementation
 *                and optimisation"
 *   [EP]         "Expert Parallelism: Scaling Mixture-of-Experts Models"
 *
 * Readings where the pages are silent or ambiguous (each one is also checked
 * by a pin in the test suite):
 *   - top-k order: descending logit, ties to the LOWER expert index, -0 == +0;
 *   - softmax over the k selected logits, divided by a temperature tau;
 *   - capacity cap = min(T, ceil(cf*T*k/E)), no limit (cap = T) when cf <= 0;
 *     slots over capacity are dropped in token order (t, then j) and the
 *     surviving weights are not renormalised;
 *   - expert-contiguous packed layout: expert e owns rows
 *     [offsets[e], offsets[e+1]) in increasing token order;
 *   - GELU is the exact erf form;
 *   - balance loss lambda * sum_e p_e q_e with p_e the kept fraction of the
 *     T*k slots and q_e = 1/E.
 *
 * Storage formats: dtype 0 = float32, dtype 1 = bfloat16 given as raw uint16
 * bit patterns.  Every element is converted exactly to double before use.
 * Inputs must be finite.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void* p, int dtype, int64_t i) {
    if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exact-erf GELU: u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)).
 * [PithTrain] section 4.1 (nn.GELU in the expert) and [PyTorchMoE] section
 * 3.2 (F.gelu in Expert.forward); both default to the erf form. */
double oracle_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }

/* Gate logits L[t,e] = sum_i x[t,i] Wg[i,e] (+ bg[e]) in double.
 * [PithTrain] section 4.1: a linear gate over the token vector; the optional
 * bias follows the gate of [PyTorchMoE] section 3.2.  Routing in fp32 or
 * wider: [EP] section 5.5. */
void oracle_gate(int64_t T, int64_t d, int64_t E, int dtype, const void* x,
                 const float* Wg, const float* bg, double* L) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* row = L + t * E;
        for (int64_t e = 0; e < E; ++e) row[e] = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double xi = elem(x, dtype, t * d + i);
            const float* w = Wg + i * E;
            for (int64_t e = 0; e < E; ++e) row[e] += xi * (double)w[e];
        }
        if (bg)
            for (int64_t e = 0; e < E; ++e) row[e] += (double)bg[e];
    }
}

typedef struct {
    float v;
    int32_t e;
} orc_key;

/* descending value; equal values (including -0 vs +0) -> lower index first */
static int orc_key_cmp(const void* a, const void* b) {
    const orc_key* p = (const orc_key*)a;
    const orc_key* q = (const orc_key*)b;
    if (p->v > q->v) return -1;
    if (p->v < q->v) return 1;
    return (p->e < q->e) ? -1 : (p->e > q->e ? 1 : 0);
}

/* Top-k selection and softmax over the selected logits.
 * [PithTrain] section 4.1: topk(logits, k) then softmax over the k values.
 * [EP] section 2.2: weights softmax(logit / temperature); the hybrid form
 * screens a coarse top-8 and soft-weights only those 8.
 * L are the fp32 logits under test; w is computed in double. */
void oracle_route(int64_t T, int64_t E, int64_t k, double tau, const float* L,
                  int32_t* idx, double* w) {
#pragma omp parallel
    {
        orc_key* keys = (orc_key*)malloc((size_t)E * sizeof(orc_key));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t e = 0; e < E; ++e) {
                keys[e].v = L[t * E + e];
                keys[e].e = (int32_t)e;
            }
            qsort(keys, (size_t)E, sizeof(orc_key), orc_key_cmp);
            double top = (double)keys[0].v, z = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                idx[t * k + j] = keys[j].e;
                double p = exp(((double)keys[j].v - top) / tau);
                w[t * k + j] = p;
                z += p;
            }
            for (int64_t j = 0; j < k; ++j) w[t * k + j] /= z;
        }
        free(keys);
    }
}

void oracle_load_stats(int64_t E, const int64_t* load, double* mean, double* var, double* cv);

/* Exploration noise of the stable layer in [PyTorchMoE] section 4.3: during
 * training the gate logits get scale * (standard normal draw) added before
 * routing (scale 0.1 on the page).  The draws are an input.  The page does
 * this in fp32, product first, then the sum, each rounded to fp32; the
 * routing decision is taken on that fp32 value.  Here each step is exact in
 * double (a product of two floats has 48 significant bits; a sum of two
 * floats that does not fit 53 bits is dominated by its larger term) and is
 * then rounded once to float. */
void oracle_noisy_logits(int64_t n, const float* L, const float* noise, float scale, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        float p = (float)((double)scale * (double)noise[i]);
        out[i] = (float)((double)L[i] + (double)p);
    }
}

/* Top-1 router of [PyTorchMoE] sections 2.3 and 4.3: a softmax over all E
 * logits (divided by tau), the expert of the largest probability (ties to the
 * lower index, as for top-k), and that probability as its weight.
 * L are the fp32 logits under test; w in double. */
void oracle_route_top1_full(int64_t T, int64_t E, double tau, const float* L, int32_t* idx, double* w) {
    for (int64_t t = 0; t < T; ++t) {
        const float* row = L + t * E;
        int64_t best = 0;
        for (int64_t e = 1; e < E; ++e)
            if (row[e] > row[best]) best = e;   /* strict: equal values keep the lower index */
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) z += exp(((double)row[e] - (double)row[best]) / tau);
        idx[t] = (int32_t)best;
        w[t] = 1.0 / z;
    }
}

/* Load-variance balance loss of [PyTorchMoE] section 3.3 item 1 (used with
 * weight 0.01 by the stable layer of section 4.3): lambda times the mean
 * squared deviation of the per-expert loads from their mean. */
double oracle_aux_variance(int64_t E, const int64_t* load, double lam) {
    double m, v, c;
    oracle_load_stats(E, load, &m, &v, &c);
    return lam * v;
}

/* Per-expert capacity.  [PithTrain] section 4.3 item 1 defines the capacity
 * as a factor times the per-expert share of the batch; with k slots per token
 * the share is T*k/E.  cap = min(T, ceil(cf*T*k/E)); cf <= 0 means no limit.
 * cf is the float32 value the caller passes; cf*T*k is exact in double while
 * T*k < 2^29, and the ceiling is found with exact integer-valued products. */
int64_t oracle_capacity(int64_t T, int64_t E, int64_t k, float cf) {
    if (!(cf > 0.0f)) return T;
    double q = (double)cf * (double)T * (double)k;
    int64_t c = (int64_t)ceil(q / (double)E);
    while (c > 0 && (double)(c - 1) * (double)E >= q) --c;
    while ((double)c * (double)E < q) ++c;
    return c < T ? c : T;
}

/* Capacity-limited dispatch into expert-contiguous buffers.
 * [PithTrain] section 4.3 item 1: tokens beyond an expert's capacity are
 * dropped.  [EP] section 4.2: an expert bucket pool sized by the per-expert
 * maximum, tokens written straight to their expert's bucket.
 * Slots are visited in token order (t, then j); an expert keeps its first
 * cap slots.  routed[e] counts all slots, counts[e] the kept ones.
 * perm has min(T*k, E*cap) entries: perm[row] = token for row < S, -1 after.
 * slot[t,j] = row, or -1 when dropped. */
void oracle_dispatch(int64_t T, int64_t E, int64_t k, int64_t cap,
                     const int32_t* idx, int32_t* routed, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* slot) {
    int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* local = (int64_t*)malloc((size_t)(T * k) * sizeof(int64_t));
    for (int64_t e = 0; e < E; ++e) routed[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            routed[e] += 1;
            if (fill[e] < cap)
                local[t * k + j] = fill[e]++;
            else
                local[t * k + j] = -1;
        }
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) {
        counts[e] = (int32_t)fill[e];
        offsets[e + 1] = offsets[e] + counts[e];
    }
    int64_t smax = T * k < E * cap ? T * k : E * cap;
    for (int64_t r = 0; r < smax; ++r) perm[r] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            if (local[s] >= 0) {
                int64_t row = offsets[idx[s]] + local[s];
                perm[row] = (int32_t)t;
                slot[s] = (int32_t)row;
            } else {
                slot[s] = -1;
            }
        }
    }
    free(local);
    free(fill);
}

/* Expert FFN on listed (token, expert) pairs:
 *   out[i] = W2[e]^T GELU(W1[e]^T x[t] + b1[e]) + b2[e],  (t, e) = (tok[i], exp[i])
 * with W1[e] stored [d, d_ff] and W2[e] stored [d_ff, d], row-major.
 * [PithTrain] section 4.1 (Linear(dim, 4 dim), GELU, Linear(4 dim, dim));
 * [PyTorchMoE] section 3.2 (Expert: linear2(gelu(linear1(x))), with biases).
 * Everything in double; h is not rounded. */
void oracle_ffn_rows(int64_t n, const int32_t* tok, const int32_t* exp_id,
                     int64_t d, int64_t dff, int dtype, const void* x,
                     const void* W1, const float* b1, const void* W2,
                     const float* b2, double* out) {
#pragma omp parallel
    {
        double* a = (double*)malloc((size_t)dff * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            int64_t t = tok[i], e = exp_id[i];
            for (int64_t f = 0; f < dff; ++f) a[f] = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                double xv = elem(x, dtype, t * d + c);
                int64_t base = (e * d + c) * dff;
                if (dtype == ORC_BF16) {
                    const uint16_t* w = (const uint16_t*)W1 + base;
                    for (int64_t f = 0; f < dff; ++f) a[f] += xv * bf16_to_double(w[f]);
                } else {
                    const float* w = (const float*)W1 + base;
                    for (int64_t f = 0; f < dff; ++f) a[f] += xv * (double)w[f];
                }
            }
            for (int64_t f = 0; f < dff; ++f) a[f] = oracle_gelu(a[f] + (double)b1[e * dff + f]);
            double* o = out + i * d;
            for (int64_t m = 0; m < d; ++m) o[m] = 0.0;
            for (int64_t f = 0; f < dff; ++f) {
                double hv = a[f];
                int64_t base = (e * dff + f) * d;
                if (dtype == ORC_BF16) {
                    const uint16_t* w = (const uint16_t*)W2 + base;
                    for (int64_t m = 0; m < d; ++m) o[m] += hv * bf16_to_double(w[m]);
                } else {
                    const float* w = (const float*)W2 + base;
                    for (int64_t m = 0; m < d; ++m) o[m] += hv * (double)w[m];
                }
            }
            for (int64_t m = 0; m < d; ++m) o[m] += (double)b2[e * d + m];
        }
        free(a);
    }
}

/* Layer output for listed tokens:
 *   y[t] = sum over j with slot[t,j] >= 0 of w[t,j] * FFN_{idx[t,j]}(x[t]),
 * summed in j order; a token whose slots were all dropped gets 0.
 * [PithTrain] section 4.1: each expert's output, scaled by the token's
 * routing weight for that expert, is added into the token's output row. */
void oracle_layer_tokens(int64_t n, const int32_t* toks, int64_t d, int64_t dff,
                         int64_t k, int dtype, const void* x, const void* W1,
                         const float* b1, const void* W2, const float* b2,
                         const int32_t* idx, const int32_t* slot, const double* w,
                         double* y) {
    int64_t nk = 0;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j)
            if (slot[(int64_t)toks[i] * k + j] >= 0) ++nk;
    int32_t* rt = (int32_t*)calloc((size_t)(nk ? nk : 1), sizeof(int32_t));
    int32_t* re = (int32_t*)calloc((size_t)(nk ? nk : 1), sizeof(int32_t));
    double* o = (double*)malloc((size_t)(nk ? nk : 1) * (size_t)d * sizeof(double));
    int64_t r = 0;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j) {
            int64_t s = (int64_t)toks[i] * k + j;
            if (slot[s] >= 0) {
                rt[r] = toks[i];
                re[r] = idx[s];
                ++r;
            }
        }
    oracle_ffn_rows(nk, rt, re, d, dff, dtype, x, W1, b1, W2, b2, o);
    r = 0;
    for (int64_t i = 0; i < n; ++i) {
        double* yr = y + i * d;
        for (int64_t m = 0; m < d; ++m) yr[m] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t s = (int64_t)toks[i] * k + j;
            if (slot[s] >= 0) {
                for (int64_t m = 0; m < d; ++m) yr[m] += w[s] * o[r * d + m];
                ++r;
            }
        }
    }
    free(o);
    free(re);
    free(rt);
}

/* Derivative of the exact GELU: d/du [u Phi(u)] = Phi(u) + u phi(u). */
static double orc_gelu_grad(double u) {
    return 0.5 * (1.0 + erf(u / sqrt(2.0))) + u * exp(-0.5 * u * u) / sqrt(2.0 * M_PI);
}

/* Backward of the expert FFN for listed kept rows.  Row i is token tok[i]
 * routed to expert exp_id[i] with routing weight wt[i]; with
 *   a = W1[e]^T x + b1[e],  h = GELU(a),  o = W2[e]^T h + b2[e]
 * and the row's upstream gradient g = wt[i] * dy[tok[i]] (the combine adds
 * w * o into y, [PithTrain] section 4.1):
 *   dw[i]   = dy[tok] . o                  (gradient w.r.t. the routing weight)
 *   dW2[e] += h g^T,  db2[e] += g,  dh = W2[e] g,  da = dh * GELU'(a),
 *   dW1[e] += x da^T, db1[e] += da,  dxp[i] = W1[e] da   (gradient w.r.t. x)
 * dW1 [E,d,dff], db1 [E,dff], dW2 [E,dff,d], db2 [E,d] are accumulated (the
 * caller zeroes them); experts without rows keep their zeros, which is the
 * expert-grained gradient of [EP] section 4.3 (inactive experts get none).
 * Rows are taken in order; the loops inside a row run in parallel over
 * disjoint outputs. */
void oracle_ffn_backward_rows(int64_t n, const int32_t* tok, const int32_t* exp_id, const double* wt,
                              int64_t d, int64_t dff, int dtype, const void* x, const void* W1,
                              const float* b1, const void* W2, const float* b2, const float* dy,
                              double* dw, double* dxp, double* dW1, double* db1, double* dW2, double* db2) {
    double* a = (double*)malloc((size_t)dff * sizeof(double));
    double* h = (double*)malloc((size_t)dff * sizeof(double));
    double* da = (double*)malloc((size_t)dff * sizeof(double));
    double* xr = (double*)malloc((size_t)d * sizeof(double));
    double* g = (double*)malloc((size_t)d * sizeof(double));
    for (int64_t i = 0; i < n; ++i) {
        const int64_t t = tok[i], e = exp_id[i];
        const int64_t w1 = e * d * dff, w2 = e * dff * d;
        for (int64_t c = 0; c < d; ++c) {
            xr[c] = elem(x, dtype, t * d + c);
            g[c] = wt[i] * (double)dy[t * d + c];
        }
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < dff; ++f) {
            double acc = (double)b1[e * dff + f];
            for (int64_t c = 0; c < d; ++c) acc += xr[c] * elem(W1, dtype, w1 + c * dff + f);
            a[f] = acc;
            h[f] = oracle_gelu(acc);
        }
        double dot = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : dot)
        for (int64_t c = 0; c < d; ++c) {
            double o = (double)b2[e * d + c];
            for (int64_t f = 0; f < dff; ++f) o += h[f] * elem(W2, dtype, w2 + f * d + c);
            dot += (double)dy[t * d + c] * o;
        }
        dw[i] = dot;
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < dff; ++f) {
            double dh = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                dh += elem(W2, dtype, w2 + f * d + c) * g[c];
                dW2[w2 + f * d + c] += h[f] * g[c];
            }
            da[f] = dh * orc_gelu_grad(a[f]);
            db1[e * dff + f] += da[f];
        }
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < d; ++c) {
            db2[e * d + c] += g[c];
            double acc = 0.0;
            for (int64_t f = 0; f < dff; ++f) {
                acc += elem(W1, dtype, w1 + c * dff + f) * da[f];
                dW1[w1 + c * dff + f] += xr[c] * da[f];
            }
            dxp[i * d + c] = acc;
        }
    }
    free(g);
    free(xr);
    free(da);
    free(h);
    free(a);
}

/* Backward of the gate ([PithTrain] section 4.1: w = softmax over the k
 * selected logits, [EP] section 2.2: divided by tau).  The selection itself
 * is piecewise constant, so only the selected logits get gradient:
 *   dl[t, idx_j] = w_j (dw_j - sum_i w_i dw_i) / tau,  0 for the others;
 * then through the linear gate: dWg[i][e] = sum_t x[t][i] dl[t][e],
 * dbg[e] = sum_t dl[t][e], dxg[t][i] = sum_e Wg[i][e] dl[t][e].
 * w and dw are [T,k] in double (dw of a dropped slot is 0). */
void oracle_route_backward(int64_t T, int64_t d, int64_t E, int64_t k, double tau, int dtype, const void* x,
                           const float* Wg, const int32_t* idx, const double* w, const double* dw, double* dl,
                           double* dWg, double* dbg, double* dxg) {
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t j = 0; j < k; ++j) s += w[t * k + j] * dw[t * k + j];
        for (int64_t e = 0; e < E; ++e) dl[t * E + e] = 0.0;
        for (int64_t j = 0; j < k; ++j) dl[t * E + idx[t * k + j]] = w[t * k + j] * (dw[t * k + j] - s) / tau;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d; ++i) {
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t) acc += elem(x, dtype, t * d + i) * dl[t * E + e];
            dWg[i * E + e] = acc;
        }
    }
    for (int64_t e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) acc += dl[t * E + e];
        dbg[e] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int64_t e = 0; e < E; ++e) acc += (double)Wg[i * E + e] * dl[t * E + e];
            dxg[t * d + i] = acc;
        }
    }
}

/* Balance loss lambda * sum_e p_e q_e, p_e = counts[e] / (T k), q_e = 1/E.
 * [EP] section 2.3 (taken as printed; with q_e constant the value only
 * depends on the kept total). */
double oracle_aux(int64_t E, int64_t T, int64_t k, const int32_t* counts, double lam) {
    double s = 0.0;
    for (int64_t e = 0; e < E; ++e) s += ((double)counts[e] / (double)(T * k)) * (1.0 / (double)E);
    return lam * s;
}

/* Routing heat map, [EP] section 3.2 step 1: for every token, every pair of
 * its chosen experts adds one to H[i][j], where i is the expert at the
 * earlier position of the token's top-k list and j the one at the later
 * position.  The page notes the matrix is not symmetric; reading it as these
 * ordered pairs, H + H^T counts the tokens that chose both experts.
 * routed[e] counts every slot (t, j) that chose e ([EP] section 2.1, the
 * per-expert load). */
void oracle_coactivation(int64_t T, int64_t E, int64_t k, const int32_t* idx, int64_t* H,
                         int64_t* routed) {
    for (int64_t i = 0; i < E * E; ++i) H[i] = 0;
    for (int64_t e = 0; e < E; ++e) routed[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        const int32_t* row = idx + t * k;
        for (int64_t a = 0; a < k; ++a) {
            routed[row[a]] += 1;
            for (int64_t b = a + 1; b < k; ++b) H[(int64_t)row[a] * E + row[b]] += 1;
        }
    }
}

/* Load statistics of the per-expert loads: mean, population variance (the
 * balance loss of [PyTorchMoE] section 3.3 item 1: the mean squared
 * deviation of the loads from their mean) and coefficient of variation
 * std / mean ([EP] section 2.1). */
void oracle_load_stats(int64_t E, const int64_t* load, double* mean, double* var, double* cv) {
    double s = 0.0;
    for (int64_t e = 0; e < E; ++e) s += (double)load[e];
    double m = s / (double)E;
    double q = 0.0;
    for (int64_t e = 0; e < E; ++e) q += ((double)load[e] - m) * ((double)load[e] - m);
    *mean = m;
    *var = q / (double)E;
    *cv = m > 0.0 ? sqrt(*var) / m : 0.0;
}

/* Balance loss over a sliding window of batches, [EP] section 2.3: the share
 * p_e of each expert is averaged over the last W batches (W = 100 on the
 * page) before lambda * sum_e p_e q_e, q_e = 1/E, is taken.  counts holds the
 * per-expert counts of n successive batches, [n][E]; after batch b the
 * window is batches max(0, b-W+1) .. b.  Writes aux[b] and pbar[b][E]. */
void oracle_window_aux(int64_t n, int64_t E, int64_t T, int64_t k, int64_t W, const int32_t* counts,
                       double lam, double* aux, double* pbar) {
    for (int64_t b = 0; b < n; ++b) {
        int64_t first = b - W + 1 < 0 ? 0 : b - W + 1;
        double m = (double)(b - first + 1);
        double s = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t c = first; c <= b; ++c) acc += (double)counts[c * E + e] / ((double)T * (double)k);
            pbar[b * E + e] = acc / m;
            s += pbar[b * E + e] * (1.0 / (double)E);
        }
        aux[b] = lam * s;
    }
}

/* Whole layer, oracle-only mode: the routing uses the oracle's own logits
 * rounded to float32 (the precision the routing decision is taken in). */
void oracle_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t dff,
                          int dtype, float cf, double tau, double lam,
                          const void* x, const float* Wg, const float* bg,
                          const void* W1, const float* b1, const void* W2,
                          const float* b2, double* Lref, float* L32, int32_t* idx,
                          double* w, int32_t* routed, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* slot,
                          double* y, double* aux) {
    oracle_gate(T, d, E, dtype, x, Wg, bg, Lref);
    for (int64_t i = 0; i < T * E; ++i) L32[i] = (float)Lref[i];
    oracle_route(T, E, k, tau, L32, idx, w);
    int64_t cap = oracle_capacity(T, E, k, cf);
    oracle_dispatch(T, E, k, cap, idx, routed, counts, offsets, perm, slot);
    int32_t* toks = (int32_t*)malloc((size_t)T * sizeof(int32_t));
    for (int64_t t = 0; t < T; ++t) toks[t] = (int32_t)t;
    oracle_layer_tokens(T, toks, d, dff, k, dtype, x, W1, b1, W2, b2, idx, slot, w, y);
    free(toks);
    *aux = oracle_aux(E, T, k, counts, lam);
}
