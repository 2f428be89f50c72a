/*
 * Plain, slow CPU oracle of the sparse Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every floating-point step is carried out in double precision on the exact
 * input values (bf16 and fp32 inputs widen to double without error). Loops
 * follow the definitions on the pages one to one; there is no blocking, no
 * fusion and no reordering beyond the definitions. OpenMP only splits the
 * independent per-token and per-row loops; the slot pass is serial.
 * Limits: E <= 1024 (fixed per-token arrays); the Python wrapper checks it.
 *
 * Sources (page title, then the step, slide or panel used):
 *   [P1] "Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"
 *        (12-step single-token MoE walk-through):
 *        STEP 2 (router scores), STEP 3-4 (noise), STEP 5 (KeepTopK with a
 *        -inf mask), STEP 6 (softmax), STEP 7 (dispatch), STEP 8-10 (expert
 *        FFN: up-projection, ReLU, down-projection), STEP 11-12 (gate scaling
 *        and weighted sum).
 *   [P2] "nanoMoEの深層解剖：Mixture of Expertsにおける条件分岐を排除した並列演算実装"
 *        (nanoMoE slides): slide 11 (router in full precision),
 *        slides 12-13 (top-k then masked softmax), slide 14 and slides 15-23
 *        (capacity: rank of each assignment in top-1-first, token order;
 *        ranks at or past capacity dropped), slides 24-29 and 33-40 (combine
 *        weights are the raw gates; a dropped assignment contributes 0).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - The pages' router runs in full precision (fp32). The ranking decision is
 *     therefore taken on the float32 rounding of the double-precision score.
 *   - Equal scores rank the lower expert index first.
 *   - Capacity C = ceil(cf * k * N / E) over the call's N tokens (the slide's
 *     get_capacity body is elided), evaluated in double.
 *   - No renormalisation of gates after drops; all-dropped tokens output 0.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------- */
/* [P1 STEP 2, STEP 4]  s = W_g x + eps; the caller passes eps (= sigma*N(0,1)
 * plus any constant score offset) as a dense [N,E] tensor or NULL.          */
/* [P2 slide 11] the router runs in full precision: the decision value is the
 * float32 rounding of the exact score.                                      */
/* [P1 STEP 5] KeepTopK: the k largest scores, in descending order.          */
/* [P1 STEP 6] softmax over the -inf-masked vector = softmax over the k kept
 * scores, since exp(-inf) = 0.                                              */
void oracle_router(int64_t N, int64_t d, int64_t E, int32_t k,
                   const double *x, const double *Wg, const double *noise,
                   float *scores, int32_t *idx, double *gate)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < N; ++t) {
        float s[1024];
        unsigned char taken[1024];
        const double *xt = x + t * d;
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            const double *w = Wg + e * d;
            for (int64_t i = 0; i < d; ++i)
                acc += w[i] * xt[i];
            if (noise)
                acc += noise[t * E + e];
            s[e] = (float)acc;
            taken[e] = 0;
            if (scores)
                scores[t * E + e] = s[e];
        }
        /* top-k by repeated selection; strict '>' keeps the lower index on ties */
        for (int32_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || s[e] > s[best])
                    best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = (int32_t)best;
        }
        /* softmax over the k survivors (shifted by the largest; same value) */
        double m = (double)s[idx[t * k]];
        double den = 0.0;
        for (int32_t j = 0; j < k; ++j)
            den += exp((double)s[idx[t * k + j]] - m);
        for (int32_t j = 0; j < k; ++j)
            gate[t * k + j] = exp((double)s[idx[t * k + j]] - m) / den;
    }
}

/* [P2 slide 14] per-expert capacity for a call of N tokens.                 */
int64_t oracle_capacity(int64_t N, int64_t E, int32_t k, double cf)
{
    if (N <= 0)
        return 0;
    return (int64_t)ceil(cf * (double)((int64_t)k * N) / (double)E);
}

/* [P2 slides 14-23] slot of each assignment: its rank among the assignments
 * to the same expert, counted over all top-1 choices in token order, then all
 * top-2 choices in token order, and so on. Ranks >= C are dropped (-1).
 * used[e] = number of kept assignments of expert e.                         */
void oracle_assign(int64_t N, int64_t E, int32_t k, int64_t C,
                   const int32_t *idx, int32_t *slot, int32_t *used)
{
    for (int64_t e = 0; e < E; ++e)
        used[e] = 0;
    int64_t count[1024];
    for (int64_t e = 0; e < E; ++e)
        count[e] = 0;
    for (int32_t j = 0; j < k; ++j) {
        for (int64_t t = 0; t < N; ++t) {
            int32_t e = idx[t * k + j];
            int64_t r = count[e]++;
            slot[t * k + j] = (r < C) ? (int32_t)r : -1;
        }
    }
    for (int64_t e = 0; e < E; ++e)
        used[e] = (int32_t)(count[e] < C ? count[e] : C);
}

/* Router statistics of one call. The pages name a router's load imbalance
 * and its capacity drops as what must be watched ("MoE（Mixture of Experts）
 * とは？", section on MoE's weak points: the work of experts is easily
 * skewed; "게이팅 위기(Gating Crisis)", the load-balancing challenge and the
 * capacity-drop panel), and give no loss formula, so these are the counts
 * that define them: for expert e, demand[e] = the number of assignments
 * (t, j) routed to e before the capacity clip (the running count of
 * [P2 slide 14] at its end), drops[e] = how many of them reach rank C or
 * more, i.e. demand[e] - min(demand[e], C), and gate_sum[e] = the sum of the
 * gates g_{t,j} of those assignments (kept or dropped), in token order. */
void oracle_router_stats(int64_t N, int64_t E, int32_t k, int64_t C, const int32_t *idx,
                         const double *gate, int32_t *demand, int32_t *drops,
                         double *gate_sum)
{
    for (int64_t e = 0; e < E; ++e) {
        demand[e] = 0;
        gate_sum[e] = 0.0;
    }
    for (int64_t t = 0; t < N; ++t)
        for (int32_t j = 0; j < k; ++j) {
            const int32_t e = idx[t * k + j];
            demand[e] += 1;
            gate_sum[e] += gate[t * k + j];
        }
    for (int64_t e = 0; e < E; ++e)
        drops[e] = demand[e] > C ? (int32_t)(demand[e] - C) : 0;
}

/* [P2 slide 32] the nanoMoE expert's activation, torch's default GELU:
 * x * Phi(x) with Phi the standard normal distribution function,
 * Phi(x) = (1 + erf(x / sqrt(2))) / 2 (C library erf, double).            */
static double oracle_gelu(double z)
{
    return 0.5 * z * (1.0 + erf(z * 0.70710678118654752440));
}

/* Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds
 * on a 4 x 64-bit counter under a 2 x 64-bit key. A round multiplies
 * counter words 0 and 2 by the two round multipliers into 128-bit products,
 * and the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); between
 * rounds each key word grows by its Weyl constant (the golden ratio and
 * sqrt(3) - 1 in 64-bit fixed point). out = the counter after round ten. */
void oracle_philox4x64(const uint64_t *ctr, const uint64_t *key, uint64_t *out)
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* [P2 slide 32] training-mode dropout on an expert's output row (after
 * the down product and its bias). Element i of the row of assignment a
 * (a = t k + j) is kept when its 32-bit word w(a, i) >= floor(p 2^32), and
 * a kept element is scaled by 1 / (1 - p), so its mean is unchanged;
 * dropped elements become 0. w(a, i) is half (i mod 2; 0 = the low half)
 * of output word (i mod 8) / 2 of Philox4x64-10 at counter
 * (i / 8, a, offset, 0) under key (seed, 0). */
uint32_t oracle_dropout_threshold(double p)
{
    return (uint32_t)floor(p * 4294967296.0);
}

static int dropout_keep(int64_t a, int64_t i, uint32_t thresh, uint64_t seed, uint64_t offset)
{
    const uint64_t ctr[4] = {(uint64_t)(i / 8), (uint64_t)a, offset, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t r[4];
    oracle_philox4x64(ctr, key, r);
    const uint64_t wd = r[(i % 8) / 2];
    const uint32_t w = (uint32_t)(i % 2 ? wd >> 32 : wd);
    return w >= thresh;
}

/* Dropout of n rows y [n, d], row r being assignment arows[r]'s output. */
void oracle_dropout_rows(int64_t n, int64_t d, const int64_t *arows, double p, uint64_t seed,
                         uint64_t offset, double *y)
{
    const uint32_t thresh = oracle_dropout_threshold(p);
    const double scale = 1.0 / (1.0 - p);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < d; ++i)
            y[r * d + i] = dropout_keep(arows[r], i, thresh, seed, offset) ? y[r * d + i] * scale
                                                                           : 0.0;
}

/* [P1 STEP 8-10] one expert on a list of its tokens: for each listed token
 * row x_t, z = W_up x_t, h = ReLU(z), y = W_down h. W_up is [d_ff, d] and
 * W_down is [d, d_ff], row-major. y is [n, d]. hbuf must hold
 * (OpenMP team size) * d_ff doubles.
 * [P2 slide 32] the slides' expert variant: z gets the bias bup[f] before
 * the activation, which is GELU when act == 1, and y gets bdown[o] (either
 * bias may be NULL: none).                                                  */
void oracle_expert_rows(int64_t d, int64_t d_ff, int64_t n, const int64_t *tokens,
                        const double *x, const double *Wup, const double *Wdown,
                        int32_t act, const double *bup, const double *bdown,
                        double *y, double *hbuf)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        int tid = 0;
#ifdef _OPENMP
        extern int omp_get_thread_num(void);
        tid = omp_get_thread_num();
#endif
        double *h = hbuf + (int64_t)tid * d_ff;
        const double *xt = x + tokens[r] * d;
        for (int64_t f = 0; f < d_ff; ++f) {
            double z = 0.0;
            const double *w = Wup + f * d;
            for (int64_t i = 0; i < d; ++i)
                z += w[i] * xt[i];
            if (bup)
                z += bup[f];
            h[f] = act == 1 ? oracle_gelu(z) : (z > 0.0 ? z : 0.0);
        }
        double *yr = y + r * d;
        for (int64_t o = 0; o < d; ++o) {
            double acc = 0.0;
            const double *w = Wdown + o * d_ff;
            for (int64_t f = 0; f < d_ff; ++f)
                acc += w[f] * h[f];
            if (bdown)
                acc += bdown[o];
            yr[o] = acc;
        }
    }
}

/* Derivative of the exact GELU z Phi(z): Phi(z) + z phi(z), with Phi the
 * standard normal distribution function and phi its density. */
static double oracle_gelu_grad(double z)
{
    const double Phi = 0.5 * (1.0 + erf(z * 0.70710678118654752440));
    const double phi = 0.39894228040143267794 * exp(-0.5 * z * z);
    return Phi + z * phi;
}

/* The expert variant the backward differentiates: activation (0 ReLU,
 * 1 GELU), optional biases bup [E, d_ff] and bdown [E, d], where their
 * gradients go (dbup, dbdown; NULL: not accumulated), and the dropout on the
 * expert outputs (p, seed, offset). */
typedef struct {
    int32_t act;
    const double *bup, *bdown;
    double *dbup, *dbdown;
    double p;                  /* dropout probability (0: none) */
    uint64_t seed, offset;     /* its generator's key and counter word */
} expert_variant;

static double act_of(int32_t act, double z)
{
    return act == 1 ? oracle_gelu(z) : (z > 0.0 ? z : 0.0);
}

static double act_grad(int32_t act, double z)
{
    return act == 1 ? oracle_gelu_grad(z) : (z > 0.0 ? 1.0 : 0.0);
}

/* The backward of one token t: adds its terms to dx_t and, when the
 * pointers are not NULL, to dWg, dWup, dWdown and the bias gradients.
 * gate, slot, idx are the routing of all tokens; z, h, y, dz, mk [d_ff or d]
 * and dg [k] are scratch. */
static void backward_token(int64_t t, int64_t d, int32_t k, int64_t d_ff,
                           const double *x, const double *Wg, const double *Wup,
                           const double *Wdown, const expert_variant *v,
                           const double *dout, const int32_t *idx, const double *gate,
                           const int32_t *slot, double *dxt, double *dWg, double *dWup,
                           double *dWdown, double *z, double *h, double *y, double *dz,
                           double *dg, double *mk)
{
    const double *xt = x + t * d;
    const double *go = dout + t * d;
    const uint32_t thresh = oracle_dropout_threshold(v->p);
    for (int32_t j = 0; j < k; ++j) {
        dg[j] = 0.0;
        if (slot[t * k + j] < 0)
            continue;                      /* dropped: contributes nothing */
        const int64_t e = idx[t * k + j];
        const double g = gate[t * k + j];
        const double *wu = Wup + e * d_ff * d;
        const double *wd = Wdown + e * d * d_ff;
        for (int64_t f = 0; f < d_ff; ++f) {
            double acc = 0.0;
            for (int64_t i = 0; i < d; ++i)
                acc += wu[f * d + i] * xt[i];
            if (v->bup)
                acc += v->bup[e * d_ff + f];
            z[f] = acc;
            h[f] = act_of(v->act, acc);
        }
        /* dropout factor m_o of each output element: 1 / (1 - p) or 0 */
        for (int64_t o = 0; o < d; ++o)
            mk[o] = v->p > 0.0 ? (dropout_keep(t * k + j, o, thresh, v->seed, v->offset)
                                      ? 1.0 / (1.0 - v->p) : 0.0)
                               : 1.0;
        for (int64_t o = 0; o < d; ++o) {
            double acc = 0.0;
            for (int64_t f = 0; f < d_ff; ++f)
                acc += wd[o * d_ff + f] * h[f];
            if (v->bdown)
                acc += v->bdown[e * d + o];
            y[o] = acc * mk[o];
        }
        /* combine: dg = <dout_t, y>; through the dropout, dy = g dout_t m */
        double a = 0.0;
        for (int64_t o = 0; o < d; ++o)
            a += go[o] * y[o];
        dg[j] = a;
        /* down: dW_down += dy h^T, db_down += dy; dh = W_down^T dy */
        if (dWdown) {
            double *gwd = dWdown + e * d * d_ff;
            for (int64_t o = 0; o < d; ++o) {
                const double dyo = g * go[o] * mk[o];
                for (int64_t f = 0; f < d_ff; ++f)
                    gwd[o * d_ff + f] += dyo * h[f];
            }
        }
        if (v->dbdown)
            for (int64_t o = 0; o < d; ++o)
                v->dbdown[e * d + o] += g * go[o] * mk[o];
        /* activation: dz = dh act'(z) */
        for (int64_t f = 0; f < d_ff; ++f) {
            double acc = 0.0;
            for (int64_t o = 0; o < d; ++o)
                acc += wd[o * d_ff + f] * (g * go[o] * mk[o]);
            dz[f] = acc * act_grad(v->act, z[f]);
        }
        /* up: dW_up += dz x_t^T, db_up += dz; dx_t += W_up^T dz */
        if (dWup) {
            double *gwu = dWup + e * d_ff * d;
            for (int64_t f = 0; f < d_ff; ++f)
                for (int64_t i = 0; i < d; ++i)
                    gwu[f * d + i] += dz[f] * xt[i];
        }
        if (v->dbup)
            for (int64_t f = 0; f < d_ff; ++f)
                v->dbup[e * d_ff + f] += dz[f];
        for (int64_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int64_t f = 0; f < d_ff; ++f)
                acc += wu[f * d + i] * dz[f];
            dxt[i] += acc;
        }
    }
    /* softmax over the kept scores, then the score product */
    double gdg = 0.0;
    for (int32_t j = 0; j < k; ++j)
        gdg += gate[t * k + j] * dg[j];
    for (int32_t j = 0; j < k; ++j) {
        const int64_t e = idx[t * k + j];
        const double ds = gate[t * k + j] * (dg[j] - gdg);
        for (int64_t i = 0; i < d; ++i) {
            if (dWg)
                dWg[e * d + i] += ds * xt[i];
            dxt[i] += ds * Wg[e * d + i];
        }
    }
}

/* Routing of all tokens followed by the backward of the tokens listed in
 * rows (all N when rows is NULL). Weight gradients are accumulated when
 * their pointers are not NULL; dx holds one row per listed token. */
static int backward_impl(int64_t N, int64_t d, int64_t E, int32_t k, int64_t d_ff, int64_t C,
                         const double *x, const double *Wg, const double *noise,
                         const double *Wup, const double *Wdown, const expert_variant *v,
                         const double *dout, int64_t nrows, const int64_t *rows, double *dx,
                         double *dWg, double *dWup, double *dWdown)
{
    float *scores = (float *)malloc(sizeof(float) * (size_t)(N * E + 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * k + 1));
    double *gate = (double *)malloc(sizeof(double) * (size_t)(N * k + 1));
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * k + 1));
    int32_t *used = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    double *z = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    double *dz = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *dg = (double *)malloc(sizeof(double) * (size_t)k);
    double *mk = (double *)malloc(sizeof(double) * (size_t)d);
    int rc = 0;
    if (!scores || !idx || !gate || !slot || !used || !z || !h || !y || !dz || !dg || !mk) {
        rc = -1;
        goto done;
    }
    oracle_router(N, d, E, k, x, Wg, noise, scores, idx, gate);
    oracle_assign(N, E, k, C, idx, slot, used);
    for (int64_t i = 0; i < nrows * d; ++i)
        dx[i] = 0.0;
    if (dWg)
        for (int64_t i = 0; i < E * d; ++i)
            dWg[i] = 0.0;
    if (dWup)
        for (int64_t i = 0; i < E * d_ff * d; ++i)
            dWup[i] = 0.0;
    if (dWdown)
        for (int64_t i = 0; i < E * d * d_ff; ++i)
            dWdown[i] = 0.0;
    if (v->dbup)
        for (int64_t i = 0; i < E * d_ff; ++i)
            v->dbup[i] = 0.0;
    if (v->dbdown)
        for (int64_t i = 0; i < E * d; ++i)
            v->dbdown[i] = 0.0;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t t = rows ? rows[r] : r;
        backward_token(t, d, k, d_ff, x, Wg, Wup, Wdown, v, dout, idx, gate, slot, dx + r * d,
                       dWg, dWup, dWdown, z, h, y, dz, dg, mk);
    }
done:
    free(scores); free(idx); free(gate); free(slot); free(used);
    free(z); free(h); free(y); free(dz); free(dg); free(mk);
    return rc;
}

/* The layer's backward pass (the next row after the forward: gradients
 * through the gates to the router and through the experts; dropout off).
 * Derived by the chain rule from the forward above, for a loss whose
 * gradient with respect to out is dout [N, d]:
 *   combine  out_t = sum_j g_tj y_tj (kept j)      -> dy_tj = g_tj dout_t,
 *                                                     dg_tj = <dout_t, y_tj>
 *            (dropped j: dy = 0 and dg = 0)
 *   softmax  g_tj = exp(s_j) / sum_l exp(s_l) over the k kept scores
 *                                                  -> ds_j = g_j (dg_j - sum_l g_l dg_l);
 *            scores outside the top-k get no gradient (the -inf mask; the
 *            choice of the top k is piecewise constant)
 *   scores   s_te = W_g[e] x_t + noise_te           -> dW_g[e] += ds_te x_t,
 *                                                     dx_t += ds_te W_g[e]
 *   expert   z = W_up x_t + b_up, h = act(z),       -> dW_down += dy h^T, db_down += dy,
 *            y = W_down h + b_down                     dh = W_down^T dy, dz = dh act'(z),
 *                                                     dW_up += dz x_t^T, db_up += dz,
 *                                                     dx_t += W_up^T dz
 * with act ReLU (act == 0; act'(z) = [z > 0]) or the exact GELU (act == 1;
 * [P2 slide 32]); bup [E, d_ff] and bdown [E, d] may be NULL (no biases),
 * and dbup, dbdown are written when not NULL. With dropout p > 0 the expert
 * output is y m (m the dropout factor of each element, see
 * oracle_dropout_rows), so dg = <dout_t, y m> and dy = g dout_t m. The gate derivative treats
 * the float32 rounding of the scores as the identity. Sums over tokens run
 * in token order, then choice order. dx [N, d], dWg [E, d], dWup
 * [E, d_ff, d], dWdown [E, d, d_ff]; C = capacity. Scratch is allocated here
 * (test infrastructure; not a hot path). Returns 0, or -1 if an allocation
 * fails. Serial on purpose: the sums into the weight gradients have one
 * fixed order. */
int oracle_backward(int64_t N, int64_t d, int64_t E, int32_t k, int64_t d_ff, int64_t C,
                    const double *x, const double *Wg, const double *noise,
                    const double *Wup, const double *Wdown, int32_t act, const double *bup,
                    const double *bdown, double p, uint64_t seed, uint64_t offset,
                    const double *dout, double *dx, double *dWg, double *dWup, double *dWdown,
                    double *dbup, double *dbdown)
{
    const expert_variant v = {act, bup, bdown, dbup, dbdown, p, seed, offset};
    return backward_impl(N, d, E, k, d_ff, C, x, Wg, noise, Wup, Wdown, &v, dout, N, NULL, dx,
                         dWg, dWup, dWdown);
}

/* dx of the listed tokens only (rows[r] in [0, N)), as oracle_backward
 * computes it: the routing covers all N tokens, since capacity decides a
 * token's kept choices from every earlier assignment, but the expert terms
 * are evaluated for the listed tokens alone. dx_rows is [nrows, d]. */
int oracle_backward_rows(int64_t N, int64_t d, int64_t E, int32_t k, int64_t d_ff, int64_t C,
                         const double *x, const double *Wg, const double *noise,
                         const double *Wup, const double *Wdown, int32_t act,
                         const double *bup, const double *bdown, double p, uint64_t seed,
                         uint64_t offset, const double *dout, int64_t nrows,
                         const int64_t *rows, double *dx_rows)
{
    const expert_variant v = {act, bup, bdown, NULL, NULL, p, seed, offset};
    return backward_impl(N, d, E, k, d_ff, C, x, Wg, noise, Wup, Wdown, &v, dout, nrows, rows,
                         dx_rows, NULL, NULL, NULL);
}

/* Sampled weight gradients of one expert e: for each listed hidden unit f,
 * row f of dW_up[e] (dWup_rows [nf, d]) and column f of dW_down[e]
 * (dWdown_cols [nf, d], entry o = dW_down[e][o][f]), with the same terms and
 * token order as oracle_backward. Wup_e [d_ff, d] and Wdown_e [d, d_ff] are
 * expert e's matrices, bup_e [d_ff] its up bias or NULL; the routing covers
 * all N tokens; p, seed, offset: the dropout, as in oracle_backward. Per
 * token routed to e and kept: g = its gate, dy = g dout_t m,
 * z_f = W_up[e][f] x_t + b_up[e][f], dW_down[e][:, f] += dy act(z_f),
 * dz_f = act'(z_f) <W_down[e][:, f], dy>, dW_up[e][f] += dz_f x_t. Returns
 * 0, or -1 if an allocation fails. */
int oracle_backward_expert_units(int64_t N, int64_t d, int64_t E, int32_t k, int64_t d_ff,
                                 int64_t C, const double *x, const double *Wg,
                                 const double *noise, int64_t e, const double *Wup_e,
                                 const double *Wdown_e, int32_t act, const double *bup_e,
                                 double p, uint64_t seed, uint64_t offset,
                                 const double *dout, int64_t nf, const int64_t *fs,
                                 double *dWup_rows, double *dWdown_cols)
{
    const uint32_t thresh = oracle_dropout_threshold(p);
    float *scores = (float *)malloc(sizeof(float) * (size_t)(N * E + 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * k + 1));
    double *gate = (double *)malloc(sizeof(double) * (size_t)(N * k + 1));
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * k + 1));
    int32_t *used = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int rc = 0;
    if (!scores || !idx || !gate || !slot || !used) {
        rc = -1;
        goto done;
    }
    oracle_router(N, d, E, k, x, Wg, noise, scores, idx, gate);
    oracle_assign(N, E, k, C, idx, slot, used);
    for (int64_t i = 0; i < nf * d; ++i) {
        dWup_rows[i] = 0.0;
        dWdown_cols[i] = 0.0;
    }
    for (int64_t t = 0; t < N; ++t) {
        const double *xt = x + t * d;
        const double *go = dout + t * d;
        for (int32_t j = 0; j < k; ++j) {
            if (idx[t * k + j] != e || slot[t * k + j] < 0)
                continue;
            const double g = gate[t * k + j];
            for (int64_t q = 0; q < nf; ++q) {
                const int64_t f = fs[q];
                double z = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    z += Wup_e[f * d + i] * xt[i];
                if (bup_e)
                    z += bup_e[f];
                const double h = act_of(act, z);
                double dh = 0.0;
                for (int64_t o = 0; o < d; ++o) {
                    const double m = p > 0.0 ? (dropout_keep(t * k + j, o, thresh, seed, offset)
                                                    ? 1.0 / (1.0 - p) : 0.0)
                                             : 1.0;
                    const double dyo = g * go[o] * m;
                    dWdown_cols[q * d + o] += dyo * h;
                    dh += Wdown_e[o * d_ff + f] * dyo;
                }
                const double dz = dh * act_grad(act, z);
                for (int64_t i = 0; i < d; ++i)
                    dWup_rows[q * d + i] += dz * xt[i];
            }
        }
    }
done:
    free(scores); free(idx); free(gate); free(slot); free(used);
    return rc;
}

/* [P1 STEP 11-12, P2 slides 38-40] output rows: each kept assignment's
 * expert output scaled by its gate, summed in choice order j = 0..k-1.
 * Dropped assignments (slot -1) contribute nothing, so a token with every
 * choice dropped gets 0. gate, slot are [n, k]; y is [n, k, d]; out [n, d]. */
void oracle_combine(int64_t n, int64_t d, int32_t k, const double *gate,
                    const int32_t *slot, const double *y, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double *o = out + r * d;
        for (int64_t i = 0; i < d; ++i)
            o[i] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            if (slot[r * k + j] < 0)
                continue;
            double g = gate[r * k + j];
            const double *yj = y + (r * k + j) * d;
            for (int64_t i = 0; i < d; ++i)
                o[i] += g * yj[i];
        }
    }
}

int oracle_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
