/*
 * CPU oracle for the forward pass of one top-k Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the GPU library.
 *
 * Plain, slow, fp64.  Every stored input (fp32 or bf16) is widened exactly
 * to double, and every sum is taken in double in a fixed order.  No blocking,
 * fusion or reordering beyond what the definitions below state.
 *
 * What it computes, and where the pages define it:
 *   - router logits  h(x) = W_r x, W_r in R^{E x d}, no bias
 *       ("Mixture-of-Experts Internals", sec. 2.1 Router Architecture;
 *        "Mixture of Experts: What Actually Happens...", Step 1)
 *   - scores: softmax over all E (sec. 2.1 above), or a per-expert sigmoid
 *       ("Mixture-of-Experts, from the router to the all-to-all", The router)
 *   - top-k set I: the k largest, taken on the logits (softmax and sigmoid are
 *       strictly increasing, so the set is the same); equal logits go to the
 *       lower expert index; ids are listed by descending logit
 *   - gates: g_i = s_i / sum_{j in I} s_j for i in I when renormalising
 *       (sec. 2.1 above), else g_i = s_i (Switch's top-1 form, "from the
 *       router to the all-to-all", The router)
 *   - experts: f_e(x) = W_down (silu(W_gate x) * (W_up x)), silu(z) = z/(1+e^-z)
 *       ("What Actually Happens...", DenseFFN and Step 4; "8.6 Mixture of
 *        Experts", sec. 2)
 *   - output: y = sum_{i in I} g_i f_i(x) (+ f_shared(x) with weight 1)
 *       ("8.6 Mixture of Experts", sec. 2 boxed equation and sec. 4.1)
 *   - dispatch: tokens grouped by expert, experts in index order, tokens in
 *       ascending order inside each group ("What Actually Happens...", Step 3)
 *
 * Layouts (row-major): x [T,d]; w_router [E,d]; w_gate, w_up [E,d_ff,d];
 * w_down [E,d,d_ff]; ws_gate, ws_up [d_ff_s,d]; ws_down [d,d_ff_s].
 * dtype 0 = fp32, 1 = bf16 (uint16 bit patterns).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2   /* fp64 inputs: only for finite-difference checks of the gradients */
#define OR_SOFTMAX 0
#define OR_SIGMOID 1

static double widen(const void* base, int dtype, int64_t i) {
    if (dtype == OR_F64) return ((const double*)base)[i];
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* logits[t,e] = sum_i x[t,i] * w_r[e,i], for t in [t0, t0+n). */
void oracle_logits(int64_t n, int64_t t0, int d, int E, const void* x, const void* w_r, int dtype,
                   double* logits, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t tt = 0; tt < n; ++tt) {
        int64_t t = t0 + tt;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += widen(x, dtype, t * (int64_t)d + i) * widen(w_r, dtype, (int64_t)e * d + i);
            logits[tt * E + e] = acc;
        }
    }
}

/* Scores of one token from its logits. */
static void scores_of(const double* l, int E, int score_fn, double* s) {
    if (score_fn == OR_SOFTMAX) {
        double m = l[0];
        for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) { s[e] = exp(l[e] - m); z += s[e]; }
        for (int e = 0; e < E; ++e) s[e] /= z;
    } else {
        for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + exp(-l[e]));
    }
}

/* Does expert a come before expert b in the selection order?
 * Larger logit first; equal logits: lower index first. */
static int before(const double* l, int a, int b) {
    if (l[a] != l[b]) return l[a] > l[b];
    return a < b;
}

/*
 * Routing of n tokens from their logits [n,E].
 *   ids   [n,k]  chosen experts, in selection order
 *   gates [n,k]  gate of each chosen expert
 *   scores [n,E] (nullable) all scores
 *   gap_score, gap_key [n] (nullable): s_(k)-s_(k+1) and key_(k)-key_(k+1)
 *       in selection order (key = the selection value below); +inf when
 *       k == E.
 *   bias [E] (nullable): a per-expert bias for choosing only; the gates use
 *       the unbiased scores.  bias_on_scores = 0: key = logit + bias
 *       ("Mixture-of-Experts Internals", sec. 3.3: top-k over the modified
 *       routing logits); 1: key = score + bias ("Mixture-of-Experts, from the
 *       router to the all-to-all", Load balancing: the bias is added to the
 *       scores for choosing).  Without a bias, key = logit.
 *   forced_ids [n,k] (nullable): skip selection and use these ids.
 */
static int route_one(int E, int k, int score_fn, int renorm, const double* l, const double* bias,
                     int bias_on_scores, const int32_t* forced, int32_t* id, double* gates,
                     double* scores, double* gap_score, double* gap_key, double* s, double* key,
                     int* order) {
    scores_of(l, E, score_fn, s);
    if (scores) memcpy(scores, s, sizeof(double) * E);
    for (int e = 0; e < E; ++e)
        key[e] = bias ? (bias_on_scores ? s[e] : l[e]) + bias[e] : l[e];
    /* full selection order by insertion: plain and obviously correct */
    for (int e = 0; e < E; ++e) {
        int p = e;
        while (p > 0 && before(key, e, order[p - 1])) { order[p] = order[p - 1]; --p; }
        order[p] = e;
    }
    if (forced) {
        for (int j = 0; j < k; ++j) {
            if (forced[j] < 0 || forced[j] >= E) return -2;
            id[j] = forced[j];
        }
    } else {
        for (int j = 0; j < k; ++j) id[j] = order[j];
    }
    if (gap_score) *gap_score = (k < E) ? s[order[k - 1]] - s[order[k]] : INFINITY;
    if (gap_key) *gap_key = (k < E) ? key[order[k - 1]] - key[order[k]] : INFINITY;
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += s[id[j]];
    for (int j = 0; j < k; ++j) gates[j] = renorm ? s[id[j]] / denom : s[id[j]];
    return 0;
}

int oracle_route(int64_t n, int E, int k, int score_fn, int renorm, const double* logits,
                 const double* bias, int bias_on_scores, const int32_t* forced_ids, int32_t* ids,
                 double* gates, double* scores, double* gap_score, double* gap_key, int nthreads) {
    if (k < 1 || k > E) return -2;
    int err = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc(sizeof(double) * E);
        double* key = (double*)malloc(sizeof(double) * E);
        int* order = (int*)malloc(sizeof(int) * E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            int rc = route_one(E, k, score_fn, renorm, logits + t * E, bias, bias_on_scores,
                               forced_ids ? forced_ids + t * k : NULL, ids + t * k, gates + t * k,
                               scores ? scores + t * E : NULL, gap_score ? gap_score + t : NULL,
                               gap_key ? gap_key + t : NULL, s, key, order);
            if (rc) {
#pragma omp atomic write
                err = rc;
            }
        }
        free(s); free(key); free(order);
    }
    return err;
}

/*
 * Group the T*k (token, slot) pairs by expert: expert 0's pairs first, then
 * expert 1's, ...; inside a group, pairs in ascending pair index p = t*k + j
 * ("What Actually Happens...", Step 3).
 *   cap: each expert keeps at most cap pairs, the first ones in that order;
 *       the others are dropped ("8.6 Mixture of Experts", sec. 3.2; "from the
 *       router to the all-to-all", Capacity and token dropping).  cap < 0:
 *       no limit.
 *   counts [E] (pairs kept), offsets [E+1], sorted_pairs [T*k] (pair index at
 *   each grouped position; -1 past the kept pairs), pair_pos [T*k] (grouped
 *   position of each pair, -1 if dropped).
 */
int oracle_dispatch(int64_t T, int k, int E, int64_t cap, const int32_t* ids, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos) {
    int64_t P = T * k;
    int64_t pos = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return -2;
        pair_pos[p] = -1;
        sorted_pairs[p] = -1;
    }
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
        int32_t c = 0;
        for (int64_t p = 0; p < P; ++p) {
            if (ids[p] == e && (cap < 0 || c < cap)) {
                sorted_pairs[pos] = (int32_t)p;
                pair_pos[p] = (int32_t)pos;
                ++pos; ++c;
            }
        }
        counts[e] = c;
    }
    offsets[E] = (int32_t)pos;
    return 0;
}

/*
 * One SwiGLU expert on one token vector (fp64):
 *   a = W_gate x, b = W_up x, h = silu(a) * b, o = W_down h.
 * wg, wu: [f, d]; wd: [d, f], all at element offset `woff_in` / `woff_dn` of
 * their arrays.  h_out (nullable) gets h [f].
 */
static void swiglu_one(int d, int f, const void* x, int64_t xoff, int dtype, const void* wg,
                       const void* wu, int64_t woff_in, const void* wd, int64_t woff_dn,
                       double* h, double* o) {
    for (int r = 0; r < f; ++r) {
        double a = 0.0, b = 0.0;
        for (int i = 0; i < d; ++i) {
            double xi = widen(x, dtype, xoff + i);
            a += widen(wg, dtype, woff_in + (int64_t)r * d + i) * xi;
            b += widen(wu, dtype, woff_in + (int64_t)r * d + i) * xi;
        }
        h[r] = silu(a) * b;
    }
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int r = 0; r < f; ++r) acc += widen(wd, dtype, woff_dn + (int64_t)c * f + r) * h[r];
        o[c] = acc;
    }
}

/*
 * Expert e applied to rows `rows[0..n)` of x: h_out [n,f] (nullable),
 * o_out [n,d].
 */
void oracle_expert_rows(int d, int f, int e, const void* x, int dtype, const int32_t* rows,
                        int64_t n, const void* wg, const void* wu, const void* wd,
                        double* h_out, double* o_out, int nthreads) {
#pragma omp parallel num_threads(nthreads)
    {
        double* h = (double*)malloc(sizeof(double) * f);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            swiglu_one(d, f, x, (int64_t)rows[i] * d, dtype, wg, wu, (int64_t)e * f * d, wd,
                       (int64_t)e * d * f, h, o_out + i * d);
            if (h_out) memcpy(h_out + i * f, h, sizeof(double) * f);
        }
        free(h);
    }
}

/*
 * Layer output for the tokens listed in `tokens[0..n)`, token by token, in
 * the per-token form y = sum_j g_j f_{ids_j}(x) + f_shared(x).
 *   forced_ids [n,k] (nullable): use these ids instead of selecting.
 *   bias [E] (nullable), bias_on_scores: selection-only bias (route_one).
 *   keep [n,k] (nullable): 0 marks a pair dropped for capacity; a dropped
 *       pair contributes nothing ("8.6 Mixture of Experts", sec. 3.2).
 *   y [n,d]; ids_out [n,k], gates_out [n,k] (both nullable).
 */
int oracle_forward_tokens(int d, int E, int k, int f, int num_shared, int f_s, int score_fn,
                          int renorm, int dtype, const void* x, const void* w_r, const void* wg,
                          const void* wu, const void* wd, const void* sg, const void* su,
                          const void* sd, const double* bias, int bias_on_scores,
                          const int32_t* tokens, int64_t n, const int32_t* forced_ids,
                          const int32_t* keep, double* y, int32_t* ids_out, double* gates_out,
                          int nthreads) {
    if (k < 1 || k > E || num_shared < 0 || num_shared > 1) return -2;
    int err = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* l = (double*)malloc(sizeof(double) * E);
        double* s = (double*)malloc(sizeof(double) * E);
        double* key = (double*)malloc(sizeof(double) * E);
        int* order = (int*)malloc(sizeof(int) * E);
        int32_t* id = (int32_t*)malloc(sizeof(int32_t) * k);
        double* g = (double*)malloc(sizeof(double) * k);
        int fmax = f > f_s ? f : f_s;
        double* h = (double*)malloc(sizeof(double) * fmax);
        double* o = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            int64_t t = tokens[i];
            for (int e = 0; e < E; ++e) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += widen(x, dtype, t * d + c) * widen(w_r, dtype, (int64_t)e * d + c);
                l[e] = acc;
            }
            int rc = route_one(E, k, score_fn, renorm, l, bias, bias_on_scores,
                               forced_ids ? forced_ids + i * k : NULL, id, g, NULL, NULL, NULL,
                               s, key, order);
            if (rc) {
#pragma omp atomic write
                err = rc;
                continue;
            }
            double* yt = y + i * d;
            for (int c = 0; c < d; ++c) yt[c] = 0.0;
            for (int j = 0; j < k; ++j) {
                if (keep && !keep[i * k + j]) continue;
                swiglu_one(d, f, x, t * d, dtype, wg, wu, (int64_t)id[j] * f * d, wd,
                           (int64_t)id[j] * d * f, h, o);
                for (int c = 0; c < d; ++c) yt[c] += g[j] * o[c];
            }
            if (num_shared) {
                swiglu_one(d, f_s, x, t * d, dtype, sg, su, 0, sd, 0, h, o);
                for (int c = 0; c < d; ++c) yt[c] += o[c];
            }
            if (ids_out) memcpy(ids_out + i * k, id, sizeof(int32_t) * k);
            if (gates_out) memcpy(gates_out + i * k, g, sizeof(double) * k);
        }
        free(l); free(s); free(key); free(order); free(id); free(g); free(h); free(o);
    }
    return err;
}

/*
 * Whole layer in the expert-loop form ("What Actually Happens...", Step 3):
 * for each expert in index order, the tokens that chose it (ascending), each
 * token's output accumulating g * f_e(x) in expert order; then the shared
 * expert.  Routing (ids, gates) is an input here, from oracle_route.
 *   y [T,d].
 */
int oracle_forward_expert_loop(int64_t T, int d, int E, int k, int f, int num_shared, int f_s,
                               int dtype, const void* x, const void* wg, const void* wu,
                               const void* wd, const void* sg, const void* su, const void* sd,
                               const int32_t* ids, const double* gates, double* y, int nthreads) {
    for (int64_t i = 0; i < T * d; ++i) y[i] = 0.0;
    for (int e = 0; e < E; ++e) {
#pragma omp parallel num_threads(nthreads)
        {
            double* h = (double*)malloc(sizeof(double) * f);
            double* o = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                for (int j = 0; j < k; ++j) {
                    if (ids[t * k + j] != e) continue;
                    swiglu_one(d, f, x, t * d, dtype, wg, wu, (int64_t)e * f * d, wd,
                               (int64_t)e * d * f, h, o);
                    for (int c = 0; c < d; ++c) y[t * d + c] += gates[t * k + j] * o[c];
                }
            }
            free(h); free(o);
        }
    }
    if (num_shared) {
#pragma omp parallel num_threads(nthreads)
        {
            double* h = (double*)malloc(sizeof(double) * f_s);
            double* o = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                swiglu_one(d, f_s, x, t * d, dtype, sg, su, 0, sd, 0, h, o);
                for (int c = 0; c < d; ++c) y[t * d + c] += o[c];
            }
            free(h); free(o);
        }
    }
    return 0;
}

/*
 * Backward pass of the layer for a fixed routing (the selection is piecewise
 * constant, so its ids are an input), by the chain rule on the forward above.
 * With L = sum_t <dy_t, y_t>:
 *   pair (t, j), expert e = ids[t,j], gate g_j:
 *     a = W_gate,e x, u = W_up,e x, h = silu(a) * u, o = W_down,e h
 *     dL/dg_j = <dy, o>,  dL/do = g_j dy
 *     dh = W_down,e^T (g_j dy); da = dh * u * silu'(a); du = dh * silu(a)
 *     dW_down,e += (g_j dy) h^T; dW_gate,e += da x^T; dW_up,e += du x^T
 *     dx += W_gate,e^T da + W_up,e^T du
 *   gates -> logits: dL/dl_m = sum_j dL/dg_j * dg_j/dl_m, with g_j the
 *     renormalised (or raw) score of the chosen expert j, the scores a
 *     softmax over all E or per-expert sigmoids; the Jacobian entries are
 *     written out term by term below.
 *   router: dW_r += dl x^T; dx += W_r^T dl
 *   shared expert (weight 1): as a pair with g = 1 and its own weights.
 * ("8.6 Mixture of Experts", sec. 2: the gate and expert paths; the router
 * receives gradient only through the gates of the chosen experts,
 * "Mixture-of-Experts Internals", sec. 2.2.)
 * Outputs (fp64, overwritten): dx [T,d], dwr [E,d], dwg, dwu [E,f,d],
 * dwd [E,d,f], dsg, dsu [f_s,d], dsd [d,f_s] (the last three when
 * num_shared).  keep [T*k] (nullable): 0 marks a pair an expert capacity
 * dropped, as in oracle_forward_tokens.  Serial over tokens (the weight
 * gradients are sums over them).
 */
int oracle_backward(int64_t T, int d, int E, int k, int f, int num_shared, int f_s, int score_fn,
                    int renorm, int dtype, const void* x, const void* w_r, const void* wg,
                    const void* wu, const void* wd, const void* sg, const void* su, const void* sd,
                    const int32_t* ids, const double* dy, double* dx, double* dwr, double* dwg,
                    double* dwu, double* dwd, double* dsg, double* dsu, double* dsd, const int32_t* keep) {
    if (k < 1 || k > E) return -2;
    /* dwr == NULL: dx only (every weight gradient pointer ignored, nothing summed into them) */
    const int wgrads = dwr != NULL;
    memset(dx, 0, sizeof(double) * T * d);
    if (wgrads) {
        memset(dwr, 0, sizeof(double) * E * d);
        memset(dwg, 0, sizeof(double) * E * f * d);
        memset(dwu, 0, sizeof(double) * E * f * d);
        memset(dwd, 0, sizeof(double) * E * d * f);
    }
    if (num_shared && wgrads) {
        memset(dsg, 0, sizeof(double) * f_s * d);
        memset(dsu, 0, sizeof(double) * f_s * d);
        memset(dsd, 0, sizeof(double) * d * f_s);
    }
    int fm = f > f_s ? f : f_s;
    double* l = (double*)malloc(sizeof(double) * E);
    double* s = (double*)malloc(sizeof(double) * E);
    double* dl = (double*)malloc(sizeof(double) * E);
    double* g = (double*)malloc(sizeof(double) * k);
    double* dg = (double*)malloc(sizeof(double) * k);
    double* a = (double*)malloc(sizeof(double) * fm);
    double* u = (double*)malloc(sizeof(double) * fm);
    double* h = (double*)malloc(sizeof(double) * fm);
    double* dh = (double*)malloc(sizeof(double) * fm);
    double* o = (double*)malloc(sizeof(double) * d);
    int err = 0;
    for (int64_t t = 0; t < T && !err; ++t) {
        const double* dyt = dy + t * d;
        double* dxt = dx + t * d;
        /* logits, scores, gates of the given ids */
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += widen(x, dtype, t * d + c) * widen(w_r, dtype, (int64_t)e * d + c);
            l[e] = acc;
        }
        scores_of(l, E, score_fn, s);
        double S = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[t * k + j];
            if (e < 0 || e >= E) { err = -2; break; }
            S += s[e];
        }
        if (err) break;
        for (int j = 0; j < k; ++j) g[j] = renorm ? s[ids[t * k + j]] / S : s[ids[t * k + j]];
        /* experts; a pair the capacity dropped adds nothing to y, so its gate
           gets no gradient and its expert none from it */
        for (int j = 0; j < k; ++j) {
            int e = ids[t * k + j];
            int64_t win = (int64_t)e * f * d, wdn = (int64_t)e * d * f;
            if (keep && !keep[t * k + j]) {
                dg[j] = 0.0;
                continue;
            }
            for (int r = 0; r < f; ++r) {
                double aa = 0.0, bb = 0.0;
                for (int c = 0; c < d; ++c) {
                    double xc = widen(x, dtype, t * d + c);
                    aa += widen(wg, dtype, win + (int64_t)r * d + c) * xc;
                    bb += widen(wu, dtype, win + (int64_t)r * d + c) * xc;
                }
                a[r] = aa; u[r] = bb; h[r] = silu(aa) * bb;
            }
            double dgj = 0.0;
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int r = 0; r < f; ++r) acc += widen(wd, dtype, wdn + (int64_t)c * f + r) * h[r];
                o[c] = acc;
                dgj += dyt[c] * acc;
            }
            dg[j] = dgj;
            for (int r = 0; r < f; ++r) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += widen(wd, dtype, wdn + (int64_t)c * f + r) * g[j] * dyt[c];
                dh[r] = acc;
            }
            if (wgrads)
                for (int c = 0; c < d; ++c)
                    for (int r = 0; r < f; ++r) dwd[wdn + (int64_t)c * f + r] += g[j] * dyt[c] * h[r];
            for (int r = 0; r < f; ++r) {
                double sig = 1.0 / (1.0 + exp(-a[r]));
                double dsilu = sig * (1.0 + a[r] * (1.0 - sig));        /* d/da of a * sigmoid(a) */
                double da = dh[r] * u[r] * dsilu;
                double du = dh[r] * a[r] * sig;
                for (int c = 0; c < d; ++c) {
                    double xc = widen(x, dtype, t * d + c);
                    if (wgrads) {
                        dwg[win + (int64_t)r * d + c] += da * xc;
                        dwu[win + (int64_t)r * d + c] += du * xc;
                    }
                    dxt[c] += widen(wg, dtype, win + (int64_t)r * d + c) * da +
                              widen(wu, dtype, win + (int64_t)r * d + c) * du;
                }
            }
        }
        /* gates -> logits */
        for (int m = 0; m < E; ++m) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int e = ids[t * k + j];
                /* ds_e / dl_m */
                double dse_dlm;
                if (score_fn == OR_SOFTMAX) dse_dlm = s[e] * ((e == m ? 1.0 : 0.0) - s[m]);
                else dse_dlm = (e == m) ? s[e] * (1.0 - s[e]) : 0.0;
                double dgj_dlm;
                if (renorm) {
                    /* g_j = s_e / S, S = sum over the chosen of s */
                    double dS_dlm = 0.0;
                    for (int i = 0; i < k; ++i) {
                        int ei = ids[t * k + i];
                        if (score_fn == OR_SOFTMAX) dS_dlm += s[ei] * ((ei == m ? 1.0 : 0.0) - s[m]);
                        else dS_dlm += (ei == m) ? s[ei] * (1.0 - s[ei]) : 0.0;
                    }
                    dgj_dlm = dse_dlm / S - s[e] * dS_dlm / (S * S);
                } else {
                    dgj_dlm = dse_dlm;
                }
                acc += dg[j] * dgj_dlm;
            }
            dl[m] = acc;
        }
        for (int m = 0; m < E; ++m)
            for (int c = 0; c < d; ++c) {
                if (wgrads) dwr[(int64_t)m * d + c] += dl[m] * widen(x, dtype, t * d + c);
                dxt[c] += widen(w_r, dtype, (int64_t)m * d + c) * dl[m];
            }
        /* shared expert */
        if (num_shared) {
            for (int r = 0; r < f_s; ++r) {
                double aa = 0.0, bb = 0.0;
                for (int c = 0; c < d; ++c) {
                    double xc = widen(x, dtype, t * d + c);
                    aa += widen(sg, dtype, (int64_t)r * d + c) * xc;
                    bb += widen(su, dtype, (int64_t)r * d + c) * xc;
                }
                a[r] = aa; u[r] = bb; h[r] = silu(aa) * bb;
            }
            for (int r = 0; r < f_s; ++r) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += widen(sd, dtype, (int64_t)c * f_s + r) * dyt[c];
                dh[r] = acc;
            }
            if (wgrads)
                for (int c = 0; c < d; ++c)
                    for (int r = 0; r < f_s; ++r) dsd[(int64_t)c * f_s + r] += dyt[c] * h[r];
            for (int r = 0; r < f_s; ++r) {
                double sig = 1.0 / (1.0 + exp(-a[r]));
                double dsilu = sig * (1.0 + a[r] * (1.0 - sig));
                double da = dh[r] * u[r] * dsilu;
                double du = dh[r] * a[r] * sig;
                for (int c = 0; c < d; ++c) {
                    double xc = widen(x, dtype, t * d + c);
                    if (wgrads) {
                        dsg[(int64_t)r * d + c] += da * xc;
                        dsu[(int64_t)r * d + c] += du * xc;
                    }
                    dxt[c] += widen(sg, dtype, (int64_t)r * d + c) * da + widen(su, dtype, (int64_t)r * d + c) * du;
                }
            }
        }
    }
    free(l); free(s); free(dl); free(g); free(dg); free(a); free(u); free(h); free(dh); free(o);
    return err;
}

/*
 * Single elements of the expert weight gradients of oracle_backward, each a
 * sum over the pairs routed to its expert (or over all tokens for the shared
 * expert, gate 1), so that full-size layers can be checked on a sample:
 *   kind 0: dW_gate[e][r][c] = sum_p da_p[r] x_t[c]
 *   kind 1: dW_up[e][r][c]   = sum_p du_p[r] x_t[c]
 *   kind 2: dW_down[e][c][r] = sum_p g_p dy_t[c] h_p[r]
 *   kind 3, 4, 5: the same for the shared expert (e ignored, g = 1)
 * with, for pair p = (t, j) of expert e and row r of its inner width:
 *   a = <W_gate,e[r], x_t>, u = <W_up,e[r], x_t>, h = silu(a) u,
 *   dh = g <W_down,e[:, r], dy_t>, da = dh u silu'(a), du = dh silu(a),
 * the gates g of the given ids as in oracle_backward ("8.6 Mixture of
 * Experts", sec. 2).  Pairs are visited in token order.  Returns 0, or -2 for
 * an invalid id or kind.
 */
int oracle_backward_weight_samples(int64_t T, int d, int E, int k, int f, int f_s, int score_fn, int renorm,
                                   int dtype, const void* x, const void* w_r, const void* wg, const void* wu,
                                   const void* wd, const void* sg, const void* su, const void* sd,
                                   const int32_t* ids, const double* dy, int n, const int32_t* kind,
                                   const int32_t* eidx, const int32_t* ridx, const int32_t* cidx, double* out) {
    if (k < 1 || k > E) return -2;
    for (int64_t i = 0; i < T * k; ++i)
        if (ids[i] < 0 || ids[i] >= E) return -2;
    for (int q = 0; q < n; ++q)
        if (kind[q] < 0 || kind[q] > 5 || (kind[q] < 3 && (eidx[q] < 0 || eidx[q] >= E))) return -2;
    /* the gates of every pair, from the recomputed logits */
    double* gates = (double*)malloc(sizeof(double) * T * k);
#pragma omp parallel
    {
        double* l = (double*)malloc(sizeof(double) * E);
        double* s = (double*)malloc(sizeof(double) * E);
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < T; ++t) {
            for (int e = 0; e < E; ++e) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += widen(x, dtype, t * d + c) * widen(w_r, dtype, (int64_t)e * d + c);
                l[e] = acc;
            }
            scores_of(l, E, score_fn, s);
            double S = 0.0;
            for (int j = 0; j < k; ++j) S += s[ids[t * k + j]];
            for (int j = 0; j < k; ++j) gates[t * k + j] = renorm ? s[ids[t * k + j]] / S : s[ids[t * k + j]];
        }
        free(l); free(s);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < n; ++q) {
        const int shared = kind[q] >= 3, kd = kind[q] % 3, e = eidx[q], r = ridx[q], c = cidx[q];
        const int fw = shared ? f_s : f;
        const void* G = shared ? sg : wg;
        const void* U = shared ? su : wu;
        const void* D = shared ? sd : wd;
        const int64_t win = shared ? 0 : (int64_t)e * f * d, wdn = shared ? 0 : (int64_t)e * d * f;
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            for (int j = 0; j < (shared ? 1 : k); ++j) {
                if (!shared && ids[t * k + j] != e) continue;
                const double g = shared ? 1.0 : gates[t * k + j];
                const double* dyt = dy + t * d;
                double aa = 0.0, bb = 0.0;
                for (int i = 0; i < d; ++i) {
                    const double xi = widen(x, dtype, t * d + i);
                    aa += widen(G, dtype, win + (int64_t)r * d + i) * xi;
                    bb += widen(U, dtype, win + (int64_t)r * d + i) * xi;
                }
                if (kd == 2) {
                    acc += g * dyt[c] * silu(aa) * bb;
                    continue;
                }
                double dh = 0.0;
                for (int i = 0; i < d; ++i) dh += widen(D, dtype, wdn + (int64_t)i * fw + r) * dyt[i];
                dh *= g;
                const double sig = 1.0 / (1.0 + exp(-aa));
                const double xc = widen(x, dtype, t * d + c);
                if (kd == 0) acc += dh * bb * (sig * (1.0 + aa * (1.0 - sig))) * xc;
                else acc += dh * aa * sig * xc;
            }
        }
        out[q] = acc;
    }
    free(gates);
    return 0;
}
