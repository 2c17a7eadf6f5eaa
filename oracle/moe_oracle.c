/*
 * moe_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, obviously-correct CPU implementation of the forward pass of
 * a GShard mixture-of-experts feed-forward layer, accumulating in fp64.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the HIP library;
 * neither side includes or links the other.
 *
 * Sources (pages about GShard; section names as they appear on each page):
 *  [card]  "GShard: Scaling Giant Models with Conditional Computation and
 *          Automatic Sharding" (inference-research paper card), method
 *          paragraph: top-2 gating with softmax-normalised top-2 weights,
 *          auxiliary loss N*sum_j f_j*P_j plus a z-loss, tokens over an
 *          expert's capacity dropped, capacity set by capacity_factor.
 *  [blog]  "GShard: Scaling Giant Neural Networks with Conditional
 *          Computation", section "Mixture-of-Experts Implementation"
 *          (equation G(x) = Softmax(x . W_g), top-k of the gate), paragraph
 *          "Expert Capacity", section "Core Components" ("Expert Networks":
 *          each expert is a feed-forward network).
 *  [atlas] "GShard (Expert Parallelism)", "In plain words": tokens are sent
 *          to the experts by an all-to-all and returned.
 *  [claim] research-vault atomic claim IX2-0404, section "WideEP",
 *          "Evidence": expert results come back by a second all-to-all.
 *
 * Readings where the pages leave a step open (each one is a choice made here):
 *  - capacity C = ceil(capacity_factor * k * S / E), one group = all S tokens;
 *  - top-k is taken on the fp32 logits, larger first, equal logits ordered by
 *    lower expert index (-0 and +0 compare equal);
 *  - slots are handed out rank by rank (all first choices, then all second
 *    choices, ...), tokens in order inside a rank; an assignment whose slot
 *    would be >= C is dropped;
 *  - the top-k weights are renormalised over the k selected experts before
 *    capacity and are not renormalised again after drops;
 *  - N in the auxiliary loss is E; f_j is the fraction of tokens whose first
 *    choice is j before capacity; P_j is the mean full softmax probability;
 *  - the z-loss is the mean over tokens of the squared natural-log
 *    logsumexp of the logits;
 *  - the two all-to-alls become a local permute into [E,C,d] buffers and a
 *    gate-weighted combine back to token order (one device, no collectives);
 *  - each expert is ReLU(x W1^T + b1) W2^T + b2 with W1 [h,d], W2 [d,h].
 *
 * Activation arrays (x, W1, b1, W2, b2) are fp32 or bf16; bf16 values are
 * passed as their raw 16-bit patterns and widened exactly.  Everything the
 * oracle computes is carried in fp64; only the logits are rounded to fp32,
 * since that is the precision the router is defined in here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one activation element to fp64.  A bf16 value is the top
 * half of the fp32 with the same sign, exponent and leading mantissa bits. */
static double act_at(const void *base, int dtype, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t act_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* Expert capacity: C = ceil(cf * k * S / E).  [card] method paragraph
 * (capacity governed by capacity_factor); [blog] "Expert Capacity". */
int oracle_capacity(int S, int E, int k, double capacity_factor)
{
    if (S < 0 || E < 1 || k < 1 || !(capacity_factor > 0.0))
        return -1;
    double v = capacity_factor * (double)k * (double)S / (double)E;
    return (int)ceil(v);
}

/* Router logits l[s,j] = sum_i x[s,i] * Wg[j,i] + bg[j], fp64 accumulation,
 * one rounding to fp32.  [blog] "Mixture-of-Experts Implementation",
 * G(x) = Softmax(x . W_g); Wg is stored [E,d] (the transpose of W_g). */
void oracle_logits(int S, int d, int E, const void *x, int x_dtype,
                   const float *wg, const float *bg, float *logits)
{
    #pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        for (int j = 0; j < E; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += act_at(x, x_dtype, (size_t)s * d + i) * (double)wg[(size_t)j * d + i];
            if (bg)
                acc += (double)bg[j];
            logits[(size_t)s * E + j] = (float)acc;
        }
    }
}

/* Routing of S tokens over E experts with top-k and capacity C.
 *
 * Per token ([blog] gating equation; [card] top-2 with softmax-normalised
 * weights):
 *   m = max_j l_j,  lse = m + ln sum_j exp(l_j - m),  p_j = exp(l_j - lse);
 *   idx[s,0..k-1] = experts ordered by (l descending, index ascending);
 *   w[s,r] = p[idx[s,r]] / sum_r' p[idx[s,r']].
 * Capacity ([card] drops over capacity):
 *   one counter per expert; for r = 0..k-1, for s = 0..S-1: the assignment
 *   (s,r) to e = idx[s,r] takes slot cnt[e] if cnt[e] < C, else slot -1;
 *   cnt[e] += 1.  counts[r,e] is the number of rank-r assignments to e.
 * Losses ([card] auxiliary loss and z-loss):
 *   aux = E * sum_j f_j P_j, f_j = counts[0,j] / S, P_j = sum_s p[s,j] / S;
 *   z   = sum_s lse_s^2 / S.
 *
 * Outputs: idx [S,k] int32, w [S,k] fp64, slot [S,k] int32, counts [k,E]
 * int32, lse [S] fp64, psum [E] fp64 (sum_s p[s,j]), losses [2] fp64. */
void oracle_route(int S, int E, int k, int C, const float *logits,
                  int32_t *idx, double *w, int32_t *slot, int32_t *counts,
                  double *lse, double *psum, double *losses)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)S * (size_t)E);

    #pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        const float *l = logits + (size_t)s * E;
        double m = (double)l[0];
        for (int j = 1; j < E; ++j)
            if ((double)l[j] > m)
                m = (double)l[j];
        double sum = 0.0;
        for (int j = 0; j < E; ++j)
            sum += exp((double)l[j] - m);
        double lse_s = m + log(sum);
        lse[s] = lse_s;
        for (int j = 0; j < E; ++j)
            p[(size_t)s * E + j] = exp((double)l[j] - lse_s);

        /* Top-k by repeated selection: each round takes the largest logit
         * among experts not yet taken; scanning j upward with a strict '>'
         * keeps the lower index among equal logits. */
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int j = 0; j < E; ++j) {
                int taken = 0;
                for (int q = 0; q < r; ++q)
                    if (idx[(size_t)s * k + q] == j)
                        taken = 1;
                if (taken)
                    continue;
                if (best < 0 || l[j] > l[best])
                    best = j;
            }
            idx[(size_t)s * k + r] = best;
        }

        double den = 0.0;
        for (int r = 0; r < k; ++r)
            den += p[(size_t)s * E + idx[(size_t)s * k + r]];
        for (int r = 0; r < k; ++r)
            w[(size_t)s * k + r] = p[(size_t)s * E + idx[(size_t)s * k + r]] / den;
    }

    /* Capacity-limited slots, rank-major then token order. */
    int32_t *cnt = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    memset(counts, 0, sizeof(int32_t) * (size_t)k * (size_t)E);
    for (int r = 0; r < k; ++r) {
        for (int s = 0; s < S; ++s) {
            int e = idx[(size_t)s * k + r];
            slot[(size_t)s * k + r] = cnt[e] < C ? cnt[e] : -1;
            cnt[e] += 1;
            counts[(size_t)r * E + e] += 1;
        }
    }
    free(cnt);

    for (int j = 0; j < E; ++j) {
        double acc = 0.0;
        for (int s = 0; s < S; ++s)
            acc += p[(size_t)s * E + j];
        psum[j] = acc;
    }
    double aux = 0.0;
    for (int j = 0; j < E; ++j) {
        double f = (double)counts[j] / (double)S; /* rank-0 row of counts */
        double P = psum[j] / (double)S;
        aux += f * P;
    }
    aux *= (double)E;
    double z = 0.0;
    for (int s = 0; s < S; ++s)
        z += lse[s] * lse[s];
    z /= (double)S;
    losses[0] = S > 0 ? aux : 0.0;
    losses[1] = S > 0 ? z : 0.0;
    free(p);
}

/* Overflow re-routing, a reading of [blog] "Expert Capacity" (tokens over an
 * expert's capacity are dropped "or routed to alternative experts"; the pages
 * give no rule).  After the capacity pass (oracle_route), the j-th dropped
 * assignment of token s (dropped ranks in rank order, j = 0, 1, ...) is
 * offered to the token's (k+j)-th ranked expert: all E experts ordered by
 * (logit descending, index ascending), ranks counted from 0, so the offer
 * goes to the best expert outside the token's top-k, then the next, and so
 * on.  Offers are taken virtual rank by virtual rank (j = 0 for every token,
 * then j = 1, ...), tokens in order; an offer is accepted while its expert
 * holds fewer than C rows (rows kept by the capacity pass plus offers
 * accepted before it), and is otherwise dropped for good.  No offer exists
 * when k + j >= E.  The assignment keeps its weight w[s,r].
 * In:  idx [S,k] (the top-k), slot [S,k] from the capacity pass.
 * Out: serve [S,k] (the expert serving (s,r): idx unless re-routed),
 *      slot updated in place, accepted [E] (offers each expert took). */
void oracle_reroute(int S, int E, int k, int C, const float *logits, const int32_t *idx,
                    int32_t *serve, int32_t *slot, int32_t *accepted)
{
    int32_t *cnt = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (size_t q = 0; q < (size_t)S * k; ++q) {
        serve[q] = idx[q];
        if (slot[q] >= 0)
            cnt[idx[q]] += 1;                  /* rows kept by the capacity pass */
    }
    memset(accepted, 0, sizeof(int32_t) * (size_t)E);
    /* offers[s*k + j]: rank r of the token's j-th dropped assignment, or -1 */
    int32_t *offer_r = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *offer_e = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *taken = (int32_t *)malloc(sizeof(int32_t) * (size_t)(2 * k + 1));
    for (int s = 0; s < S; ++s) {
        const float *l = logits + (size_t)s * E;
        int nt = 0;
        for (int r = 0; r < k; ++r)
            taken[nt++] = idx[(size_t)s * k + r];
        int j = 0;
        for (int r = 0; r < k; ++r) {
            offer_r[(size_t)s * k + r] = -1;
            offer_e[(size_t)s * k + r] = -1;
        }
        for (int r = 0; r < k; ++r) {
            if (slot[(size_t)s * k + r] >= 0)
                continue;
            /* the next expert in the token's ranking after those taken */
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int used = 0;
                for (int t = 0; t < nt; ++t)
                    if (taken[t] == e)
                        used = 1;
                if (used)
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            offer_r[(size_t)s * k + j] = r;
            offer_e[(size_t)s * k + j] = best;   /* -1 when k + j >= E */
            if (best >= 0)
                taken[nt++] = best;
            ++j;
        }
    }
    for (int j = 0; j < k; ++j) {
        for (int s = 0; s < S; ++s) {
            int r = offer_r[(size_t)s * k + j], e = offer_e[(size_t)s * k + j];
            if (r < 0 || e < 0)
                continue;
            if (cnt[e] < C) {
                serve[(size_t)s * k + r] = e;
                slot[(size_t)s * k + r] = cnt[e];
                cnt[e] += 1;
                accepted[e] += 1;
            }
        }
    }
    free(cnt);
    free(offer_r);
    free(offer_e);
    free(taken);
}

/* Dispatch, the local stand-in for the first all-to-all ([atlas] "In plain
 * words"): xd[e,c,:] = x[s,:] for every kept assignment (s,r) with
 * e = idx[s,r], c = slot[s,r].  Slots nobody was assigned stay zero.  The
 * copy is of the stored elements, so xd has x's dtype. */
void oracle_dispatch(int S, int d, int E, int C, int k, const void *x, int dtype,
                     const int32_t *idx, const int32_t *slot, void *xd)
{
    size_t es = act_size(dtype);
    memset(xd, 0, es * (size_t)E * (size_t)C * (size_t)d);
    for (int s = 0; s < S; ++s) {
        for (int r = 0; r < k; ++r) {
            int c = slot[(size_t)s * k + r];
            if (c < 0)
                continue;
            int e = idx[(size_t)s * k + r];
            memcpy((char *)xd + es * (((size_t)e * C + c) * d),
                   (const char *)x + es * ((size_t)s * d), es * (size_t)d);
        }
    }
}

/* Expert FFNs ([blog] "Core Components", Expert Networks): for each expert e
 * and each filled slot c < occ[e]:
 *   hid = max(W1_e xd[e,c] + b1_e, 0);   out[e,c] = W2_e hid + b2_e,
 * in fp64 with no intermediate rounding.  W1 [E,h,d], W2 [E,d,h], b1 [E,h],
 * b2 [E,d] (biases may be NULL = 0).  Rows c >= occ[e] of out are zero. */
void oracle_expert_ffn(int E, int C, int d, int h, const int32_t *occ,
                       const void *xd, int dtype, const void *w1, const void *b1,
                       const void *w2, const void *b2, double *out)
{
    memset(out, 0, sizeof(double) * (size_t)E * (size_t)C * (size_t)d);
    #pragma omp parallel
    {
        double *hid = (double *)malloc(sizeof(double) * (size_t)h);
        #pragma omp for collapse(2) schedule(dynamic, 4)
        for (int e = 0; e < E; ++e) {
            for (int c = 0; c < C; ++c) {
                if (c >= occ[e])
                    continue;
                size_t row = (size_t)e * C + c;
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) *
                               act_at(xd, dtype, row * d + i);
                    if (b1)
                        acc += act_at(b1, dtype, (size_t)e * h + j);
                    hid[j] = acc > 0.0 ? acc : 0.0;
                }
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) * hid[j];
                    if (b2)
                        acc += act_at(b2, dtype, (size_t)e * d + i);
                    out[row * d + i] = acc;
                }
            }
        }
        free(hid);
    }
}

/* Combine, the local stand-in for the second all-to-all ([claim] "Evidence"):
 * y[s] = sum over kept r of w[s,r] * out[idx[s,r], slot[s,r]]; a token whose
 * assignments were all dropped gets y[s] = 0. */
void oracle_combine(int S, int d, int E, int C, int k, const double *out,
                    const int32_t *idx, const int32_t *slot, const double *w,
                    double *y)
{
    (void)E;
    #pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        for (int i = 0; i < d; ++i)
            y[(size_t)s * d + i] = 0.0;
        for (int r = 0; r < k; ++r) {
            int c = slot[(size_t)s * k + r];
            if (c < 0)
                continue;
            int e = idx[(size_t)s * k + r];
            const double *o = out + ((size_t)e * C + c) * d;
            for (int i = 0; i < d; ++i)
                y[(size_t)s * d + i] += w[(size_t)s * k + r] * o[i];
        }
    }
}

/* The layer output of selected tokens computed without any buffer:
 * y[s] = sum over kept r of w[s,r] * FFN_{idx[s,r]}(x[s]).  This is the same
 * definition as dispatch -> expert FFN -> combine, written per token, so that
 * single rows of a full-size layer can be checked. */
void oracle_token_output(int ns, const int64_t *tokens, int d, int h, int k,
                         const void *x, int dtype, const void *w1, const void *b1,
                         const void *w2, const void *b2, const int32_t *idx,
                         const int32_t *slot, const double *w, double *y)
{
    #pragma omp parallel
    {
        double *hid = (double *)malloc(sizeof(double) * (size_t)h);
        #pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < ns; ++t) {
            int64_t s = tokens[t];
            for (int i = 0; i < d; ++i)
                y[(size_t)t * d + i] = 0.0;
            for (int r = 0; r < k; ++r) {
                if (slot[(size_t)s * k + r] < 0)
                    continue;
                int e = idx[(size_t)s * k + r];
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) *
                               act_at(x, dtype, (size_t)s * d + i);
                    if (b1)
                        acc += act_at(b1, dtype, (size_t)e * h + j);
                    hid[j] = acc > 0.0 ? acc : 0.0;
                }
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) * hid[j];
                    if (b2)
                        acc += act_at(b2, dtype, (size_t)e * d + i);
                    y[(size_t)t * d + i] += w[(size_t)s * k + r] * acc;
                }
            }
        }
        free(hid);
    }
}

/* ------------------------------------------------------------------------
 * Backward pass of the layer (training is the pages' setting: [card] method
 * paragraph trains with the auxiliary loss and the z-loss; [blog] "Core
 * Components" and "Performance Analysis" describe training the sparse layer).
 *
 * The routing (top-k set, ranks, slots, drops) and f_j are piecewise
 * constant in the inputs; the gradient is that of the smooth function they
 * select, for the loss
 *     L = sum_s dy[s] . y[s] + g_aux * aux + g_z * z.
 * Per kept assignment (s,r) with e = idx[s,r], row u = pre-activation:
 *     u = W1_e x_s + b1_e,  a = max(u, 0),  o = W2_e a + b2_e,
 *     y_s += w[s,r] o.
 * Chain rule, written out:
 *     dO = w[s,r] dy_s;              dw[s,r] = dy_s . o  (0 when dropped)
 *     dW2_e += dO a^T;  db2_e += dO;  da = W2_e^T dO;  du = da * [u > 0]
 *     dW1_e += du x_s^T; db1_e += du;  dx_s += W1_e^T du.
 * Router: w[s,.] is the softmax of the k selected logits (the renormalised
 * probabilities p_j / sum_sel p), so
 *     dl[s, idx[s,r]] += w[s,r] (dw[s,r] - sum_r' w[s,r'] dw[s,r']);
 * aux = E sum_j f_j P_j with f_j fixed and P_j = (1/S) sum_s p[s,j], so with
 * a_j = E f_j / S:  dl[s,j] += g_aux p[s,j] (a_j - sum_j' p[s,j'] a_j');
 * z = (1/S) sum_s lse_s^2:  dl[s,j] += g_z (2/S) lse_s p[s,j].
 * Then dWg = sum_s dl_s x_s^T, dbg = sum_s dl_s, dx_s += Wg^T dl_s.
 * The logits' fp32 rounding is treated as the identity.
 *
 * Inputs as in the forward; logits [S,E] fp32 fix the routing; dy [S,d] in
 * the activation dtype.  Outputs (fp64, all required): dx [S,d], dwg [E,d],
 * dbg [E], dw1 [E,h,d], db1 [E,h], dw2 [E,d,h], db2 [E,d], dl [S,E],
 * dw [S,k]. */
/* Gradient of the logits dl [S,E] (fp64) from the gradient dw [S,k] of the
 * renormalised top-k weights, the aux loss (weight g_aux; counts [k,E] give
 * f_j from their rank-0 row) and the z-loss (weight g_z):
 *   dl[s, idx_r] += w_r (dw_r - sum_r' w_r' dw_r')      (softmax of the
 *                                                       selected logits)
 *   dl[s, j] += g_aux p_sj (a_j - sum_j' p_sj' a_j'),   a_j = E f_j / S
 *   dl[s, j] += g_z (2/S) lse_s p_sj
 * with p and lse from the fp32 logits.  [card] method paragraph (aux loss
 * and z-loss); [blog] "Mixture-of-Experts Implementation" (softmax gate). */
void oracle_router_backward(int S, int E, int k, const float *logits, const int32_t *idx,
                            const double *w, const double *dw, const int32_t *counts,
                            double g_aux, double g_z, double *dl)
{
    #pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        const float *l = logits + (size_t)s * E;
        double *g = dl + (size_t)s * E;
        double m = (double)l[0];
        for (int j = 1; j < E; ++j)
            if ((double)l[j] > m)
                m = (double)l[j];
        double sum = 0.0;
        for (int j = 0; j < E; ++j)
            sum += exp((double)l[j] - m);
        double lse = m + log(sum);
        double pa = 0.0;
        for (int j = 0; j < E; ++j) {
            double p = exp((double)l[j] - lse);
            double a_j = (double)E * (double)counts[j] / (double)S / (double)S;
            pa += p * a_j;
        }
        for (int j = 0; j < E; ++j) {
            double p = exp((double)l[j] - lse);
            double a_j = (double)E * (double)counts[j] / (double)S / (double)S;
            g[j] = g_aux * p * (a_j - pa) + g_z * 2.0 / (double)S * lse * p;
        }
        double wdw = 0.0;
        for (int r = 0; r < k; ++r)
            wdw += w[(size_t)s * k + r] * dw[(size_t)s * k + r];
        for (int r = 0; r < k; ++r) {
            size_t q = (size_t)s * k + r;
            g[idx[q]] += w[q] * (dw[q] - wdw);
        }
    }
}

void oracle_layer_backward(int S, int d, int h, int E, int k, int C, int reroute,
                           const void *x, int dtype, const float *wg, const float *logits,
                           const void *w1, const void *b1, const void *w2, const void *b2,
                           const void *dy, double g_aux, double g_z,
                           double *dx, double *dwg, double *dbg, double *dw1, double *db1,
                           double *dw2, double *db2, double *dl, double *dw)
{
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)k * E);
    double *w = (double *)malloc(sizeof(double) * ((size_t)S * k + 1));
    double *lse = (double *)malloc(sizeof(double) * ((size_t)S + 1));
    double *psum = (double *)malloc(sizeof(double) * (size_t)E);
    double losses[2];
    oracle_route(S, E, k, C, logits, idx, w, slot, counts, lse, psum, losses);
    /* the expert that serves each assignment (re-routing moves some); the
     * router's selected-softmax term keeps the top-k idx */
    int32_t *serve = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *acc_e = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (reroute)
        oracle_reroute(S, E, k, C, logits, idx, serve, slot, acc_e);
    else
        memcpy(serve, idx, sizeof(int32_t) * (size_t)S * k);

    /* per-assignment hidden activations a and pre-activation gradients du */
    size_t nas = (size_t)S * k;
    double *a_all = (double *)calloc(nas * (size_t)h + 1, sizeof(double));
    double *du_all = (double *)calloc(nas * (size_t)h + 1, sizeof(double));
    memset(dx, 0, sizeof(double) * (size_t)S * d);

    #pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)h);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double *da = (double *)malloc(sizeof(double) * (size_t)h);
        #pragma omp for schedule(dynamic, 1)
        for (int s = 0; s < S; ++s) {
            for (int r = 0; r < k; ++r) {
                size_t q = (size_t)s * k + r;
                dw[q] = 0.0;
                if (slot[q] < 0)
                    continue;
                int e = serve[q];
                double *a = a_all + q * h;
                double *du = du_all + q * h;
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) *
                               act_at(x, dtype, (size_t)s * d + i);
                    if (b1)
                        acc += act_at(b1, dtype, (size_t)e * h + j);
                    u[j] = acc;
                    a[j] = acc > 0.0 ? acc : 0.0;
                }
                double dwq = 0.0;
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) * a[j];
                    if (b2)
                        acc += act_at(b2, dtype, (size_t)e * d + i);
                    o[i] = acc;
                    dwq += act_at(dy, dtype, (size_t)s * d + i) * acc;
                }
                dw[q] = dwq;
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) *
                               (w[q] * act_at(dy, dtype, (size_t)s * d + i));
                    da[j] = acc;
                    du[j] = u[j] > 0.0 ? acc : 0.0;
                }
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) * du[j];
                    dx[(size_t)s * d + i] += acc;
                }
            }
        }
        free(u);
        free(o);
        free(da);
    }

    /* expert weight gradients, one expert per task */
    #pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
        for (size_t t = 0; t < (size_t)d * h; ++t)
            dw2[(size_t)e * d * h + t] = 0.0;
        for (size_t t = 0; t < (size_t)h * d; ++t)
            dw1[(size_t)e * h * d + t] = 0.0;
        for (int i = 0; i < d; ++i)
            db2[(size_t)e * d + i] = 0.0;
        for (int j = 0; j < h; ++j)
            db1[(size_t)e * h + j] = 0.0;
        for (int s = 0; s < S; ++s) {
            for (int r = 0; r < k; ++r) {
                size_t q = (size_t)s * k + r;
                if (slot[q] < 0 || serve[q] != e)
                    continue;
                const double *a = a_all + q * h;
                const double *du = du_all + q * h;
                for (int i = 0; i < d; ++i) {
                    double dO = w[q] * act_at(dy, dtype, (size_t)s * d + i);
                    db2[(size_t)e * d + i] += dO;
                    for (int j = 0; j < h; ++j)
                        dw2[((size_t)e * d + i) * h + j] += dO * a[j];
                }
                for (int j = 0; j < h; ++j) {
                    db1[(size_t)e * h + j] += du[j];
                    for (int i = 0; i < d; ++i)
                        dw1[((size_t)e * h + j) * d + i] += du[j] * act_at(x, dtype, (size_t)s * d + i);
                }
            }
        }
    }

    /* router: gradient of the logits, then of Wg, bg and x */
    oracle_router_backward(S, E, k, logits, idx, w, dw, counts, g_aux, g_z, dl);
    #pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        const double *g = dl + (size_t)s * E;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < E; ++j)
                acc += g[j] * (double)wg[(size_t)j * d + i];
            dx[(size_t)s * d + i] += acc;
        }
    }
    #pragma omp parallel for schedule(static)
    for (int j = 0; j < E; ++j) {
        double bacc = 0.0;
        for (int s = 0; s < S; ++s)
            bacc += dl[(size_t)s * E + j];
        dbg[j] = bacc;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int s = 0; s < S; ++s)
                acc += dl[(size_t)s * E + j] * act_at(x, dtype, (size_t)s * d + i);
            dwg[(size_t)j * d + i] = acc;
        }
    }
    free(idx);
    free(slot);
    free(counts);
    free(w);
    free(lse);
    free(psum);
    free(a_all);
    free(du_all);
    free(serve);
    free(acc_e);
}

/* Backward entries computed one by one, for full-size checks (same chain
 * rule as oracle_layer_backward, evaluated only where asked).  Routing comes
 * from the fp32 logits with capacity C.
 *   dx rows of the given tokens: expert part sum_r W1_e^T du plus the router
 *   part Wg^T dl_s, with dw from the token's own expert outputs;
 *   weight-gradient entries: kind 1 = dW1[e,a,b] (a < h, b < d), 2 = dW2[e,a,b]
 *   (a < d, b < h), 3 = db1[e,a], 4 = db2[e,a], each a sum over the kept
 *   assignments of expert e. */
void oracle_backward_entries(int S, int d, int h, int E, int k, int C, int reroute,
                             const void *x, int dtype, const float *wg, const float *logits,
                             const void *w1, const void *b1, const void *w2, const void *b2,
                             const void *dy, double g_aux, double g_z,
                             int ntok, const int64_t *tokens, double *dx_rows,
                             int nent, const int32_t *kind, const int32_t *ent_e,
                             const int32_t *ent_a, const int32_t *ent_b, double *ent_val)
{
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)k * E);
    double *w = (double *)malloc(sizeof(double) * ((size_t)S * k + 1));
    double *lse = (double *)malloc(sizeof(double) * ((size_t)S + 1));
    double *psum = (double *)malloc(sizeof(double) * (size_t)E);
    double losses[2];
    oracle_route(S, E, k, C, logits, idx, w, slot, counts, lse, psum, losses);
    int32_t *serve = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * k + 1));
    int32_t *acc_e = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (reroute)
        oracle_reroute(S, E, k, C, logits, idx, serve, slot, acc_e);
    else
        memcpy(serve, idx, sizeof(int32_t) * (size_t)S * k);

    /* dx rows */
    #pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)h);
        double *a = (double *)malloc(sizeof(double) * (size_t)h);
        double *du = (double *)malloc(sizeof(double) * (size_t)h);
        double dwr[64]; /* k <= 64 */
        double *dl = (double *)malloc(sizeof(double) * (size_t)E);
        #pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < ntok; ++t) {
            int64_t s = tokens[t];
            double *out = dx_rows + (size_t)t * d;
            for (int i = 0; i < d; ++i)
                out[i] = 0.0;
            for (int r = 0; r < k; ++r) {
                size_t q = (size_t)s * k + r;
                dwr[r] = 0.0;
                if (slot[q] < 0)
                    continue;
                int e = serve[q];
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) *
                               act_at(x, dtype, (size_t)s * d + i);
                    if (b1)
                        acc += act_at(b1, dtype, (size_t)e * h + j);
                    u[j] = acc;
                    a[j] = acc > 0.0 ? acc : 0.0;
                }
                double dwq = 0.0;
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) * a[j];
                    if (b2)
                        acc += act_at(b2, dtype, (size_t)e * d + i);
                    dwq += act_at(dy, dtype, (size_t)s * d + i) * acc;
                }
                dwr[r] = dwq;
                for (int j = 0; j < h; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += act_at(w2, dtype, ((size_t)e * d + i) * h + j) *
                               (w[q] * act_at(dy, dtype, (size_t)s * d + i));
                    du[j] = u[j] > 0.0 ? acc : 0.0;
                }
                for (int i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < h; ++j)
                        acc += act_at(w1, dtype, ((size_t)e * h + j) * d + i) * du[j];
                    out[i] += acc;
                }
            }
            /* the router part needs this token's dl row only: the selected
             * term from a one-token call (loss weights 0), then the aux and z
             * terms, which depend on the whole batch through S */
            oracle_router_backward(1, E, k, logits + (size_t)s * E, idx + (size_t)s * k,
                                   w + (size_t)s * k, dwr, counts, 0.0, 0.0, dl);
            {
                const float *l = logits + (size_t)s * E;
                double pa = 0.0;
                for (int j = 0; j < E; ++j)
                    pa += exp((double)l[j] - lse[s]) * (double)E * (double)counts[j] / (double)S / (double)S;
                for (int j = 0; j < E; ++j) {
                    double p = exp((double)l[j] - lse[s]);
                    double a_j = (double)E * (double)counts[j] / (double)S / (double)S;
                    dl[j] += g_aux * p * (a_j - pa) + g_z * 2.0 / (double)S * lse[s] * p;
                }
            }
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < E; ++j)
                    acc += dl[j] * (double)wg[(size_t)j * d + i];
                out[i] += acc;
            }
        }
        free(u);
        free(a);
        free(du);
        free(dl);
    }

    /* weight-gradient entries */
    #pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < nent; ++t) {
        int e = ent_e[t], ka = ent_a[t], kb = ent_b[t];
        double acc = 0.0;
        for (int s = 0; s < S; ++s) {
            for (int r = 0; r < k; ++r) {
                size_t q = (size_t)s * k + r;
                if (slot[q] < 0 || serve[q] != e)
                    continue;
                if (kind[t] == 2 || kind[t] == 4) {
                    double dO = w[q] * act_at(dy, dtype, (size_t)s * d + ka);
                    if (kind[t] == 4) {
                        acc += dO;
                        continue;
                    }
                    double uu = 0.0;
                    for (int i = 0; i < d; ++i)
                        uu += act_at(w1, dtype, ((size_t)e * h + kb) * d + i) *
                              act_at(x, dtype, (size_t)s * d + i);
                    if (b1)
                        uu += act_at(b1, dtype, (size_t)e * h + kb);
                    acc += dO * (uu > 0.0 ? uu : 0.0);
                } else {
                    /* du[ka] for this assignment */
                    double uu = 0.0;
                    for (int i = 0; i < d; ++i)
                        uu += act_at(w1, dtype, ((size_t)e * h + ka) * d + i) *
                              act_at(x, dtype, (size_t)s * d + i);
                    if (b1)
                        uu += act_at(b1, dtype, (size_t)e * h + ka);
                    if (!(uu > 0.0))
                        continue;
                    double da = 0.0;
                    for (int i = 0; i < d; ++i)
                        da += act_at(w2, dtype, ((size_t)e * d + i) * h + ka) *
                              (w[q] * act_at(dy, dtype, (size_t)s * d + i));
                    acc += kind[t] == 3 ? da : da * act_at(x, dtype, (size_t)s * d + kb);
                }
            }
        }
        ent_val[t] = acc;
    }
    free(idx);
    free(slot);
    free(counts);
    free(w);
    free(lse);
    free(psum);
    free(serve);
    free(acc_e);
}
