/*
 * moe.h -- C ABI of the MI355X (gfx950) GShard mixture-of-experts layer.
 *
 * The library computes the forward pass of one GShard MoE feed-forward layer
 * on one GPU's share of tokens and experts:
 *
 *   logits   l = x . Wg^T + bg                         (router, fp32)
 *   p        = softmax(l),  lse = logsumexp(l)
 *   top-k    idx[s,0..k-1]: largest logits first, equal logits -> lower index
 *   weights  w[s,r] = p[idx[s,r]] / sum_r' p[idx[s,r']]
 *   slots    rank by rank, tokens in order; slot >= C -> dropped (-1)
 *   dispatch xd[e,c,:] = x[s,:]                 (local stand-in, all-to-all)
 *   experts  out[e,c] = ReLU(xd[e,c] W1_e^T + b1_e) W2_e^T + b2_e
 *   combine  y[s] = sum over kept r of w[s,r] out[idx[s,r], slot[s,r]]
 *   losses   aux = E * sum_j f_j P_j,  z = mean_s lse_s^2
 *
 * Sources: "GShard: Scaling Giant Models with Conditional Computation and
 * Automatic Sharding" (inference-research paper card), method paragraph (top-2
 * with softmax-normalised weights, aux loss N*sum f_j*P_j plus a z-loss, drops
 * over a capacity set by capacity_factor); "GShard: Scaling Giant Neural
 * Networks with Conditional Computation" (blog), section "Mixture-of-Experts
 * Implementation" (G(x) = Softmax(x . W_g), top-k), paragraph "Expert
 * Capacity", section "Core Components" (experts are feed-forward networks);
 * "GShard (Expert Parallelism)" (atlas), "In plain words" (tokens go to the
 * experts by an all-to-all and return); research-vault claim IX2-0404,
 * section "WideEP", "Evidence" (results come back by a second all-to-all).
 *
 * Readings fixed by this library where the pages leave a step open:
 *   C = ceil(capacity_factor * k * S / E) unless moe_config.capacity > 0;
 *   f_j = (first choices of expert j before capacity) / S, N = E;
 *   P_j = mean over tokens of the full softmax probability;
 *   z = mean over tokens of the squared natural-log logsumexp;
 *   weights are renormalised over the k selected experts before capacity and
 *   not again after drops; a token with every assignment dropped gets y = 0.
 *
 * Conventions shared by every entry point
 *   Pointers.  Every array argument is a DEVICE pointer to memory the caller
 *     owns (for example a torch tensor's data_ptr()).  The config is host
 *     memory.  The library allocates and frees nothing and keeps no pointer
 *     after a call returns.  Its only process-wide state is a per-device
 *     cache of the compute-unit count and, for moe_gate_noalloc, the
 *     per-device address of its static scratch (both filled on first use,
 *     never changed).
 *   Execution.  Work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous: outputs are valid once the stream has been synchronised.
 *     The library performs no host<->device copies and no synchronisation.
 *   Layouts.  Row-major, no padding:  x, y [S,d];  Wg [E,d] fp32;  bg [E]
 *     fp32;  W1 [E,h,d];  b1 [E,h];  W2 [E,d,h];  b2 [E,d];  xd, out [E,C,d]
 *     ([S*k,d] with MOE_CFG_DROPLESS);
 *     logits [S,E] fp32;  topk_idx, slot [S,k] int32;  topk_w [S,k] fp32;
 *     counts [k,E] int32 (assignments of rank r to expert e before capacity;
 *     one more row with MOE_CFG_REROUTE);
 *     losses [2] fp32 = {aux, z}.
 *   Dtypes.  x, W1, b1, W2, b2, xd, out and y share act_dtype (fp32 or
 *     bf16, with fp32 accumulation).  Wg, bg, logits, topk_w and losses are
 *     always fp32.  Biases b1/b2/bg may be NULL (= zero).
 *   Errors.  Arguments are validated on the host before anything is
 *     enqueued; a failed check returns MOE_ERR_INVALID_ARG (bad value or NULL
 *     required pointer), MOE_ERR_UNSUPPORTED (valid but outside what the
 *     kernels handle: see moe_config) or MOE_ERR_WORKSPACE (ws too small) and
 *     has no side effect.  A failed kernel launch returns MOE_ERR_HIP.  The
 *     library never aborts and throws nothing across the ABI.
 *   Buffers.  Slots of xd/out past an expert's occupancy are left as they
 *     were (never read by later steps).  NaN/Inf inputs are not supported.
 *   Alignment.  Activation-typed arrays (x, xd, out, y, W1, b1, W2, b2,
 *     hidden, dy, dx and the expert weight gradients), w_gate and dw_gate
 *     start on 16-byte boundaries; a misaligned one is MOE_ERR_INVALID_ARG.
 *   Workspace.  `ws` is device scratch of at least moe_workspace_bytes()
 *     bytes, 256-byte aligned; its contents do not persist between calls.
 *     Calls that share a workspace must be ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4,
    MOE_ERR_SCRATCH_LIMIT = 5  /* moe_gate_noalloc: the shape needs more scratch
                                  than MOE_STATIC_SCRATCH_BYTES */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape.  Valid: S >= 0; d_model, d_ff >= 1; 1 <= E; 1 <= k <= E;
 * capacity_factor > 0 when capacity == 0; capacity >= 0.
 * Supported by the kernels (else MOE_ERR_UNSUPPORTED): E <= 2048, k <= 8,
 * k * E <= 16384, d_model and d_ff multiples of 64 for bf16 and of 4 for
 * fp32, R * max(d_model, d_ff) < 2^31 with R = moe_dispatch_rows,
 * S * max(d_model, E) < 2^31, and one expert matrix under 4 GiB
 * (d_model * d_ff * element size < 2^32 bytes).
 * Source of the shape: "GShard: Scaling Giant Models with Conditional
 * Computation and Automatic Sharding" (paper card), method paragraph (top-2
 * of E experts, capacity from capacity_factor); k > 2 generalises the top-2
 * rule ("GShard: Scaling Giant Neural Networks with Conditional Computation"
 * (blog), "Mixture-of-Experts Implementation": top-k). */
typedef struct moe_config {
    int32_t S;               /* tokens on this GPU                         */
    int32_t d_model;         /* d: model width                             */
    int32_t d_ff;            /* h: expert hidden width                     */
    int32_t E;               /* experts on this GPU                        */
    int32_t k;               /* experts per token                          */
    int32_t capacity;        /* C per expert; 0 = ceil(cf * k * S / E)     */
    double capacity_factor;  /* cf                                         */
    int32_t act_dtype;       /* moe_dtype                                  */
    uint32_t flags;          /* MOE_CFG_* bits; all others must be 0       */
} moe_config;

/* moe_config.flags: dropless routing.  No assignment is dropped and no
 * capacity padding exists: the dispatch buffer xd and the expert output out
 * hold S*k rows [S*k,d], one per (token, rank) assignment, in variable-length
 * expert segments.  Segment e starts at row seg_e = sum_{e'<e} n_e' (n_e =
 * sum_r counts[r,e]), experts in index order; inside a segment rows follow
 * the capacity mode's slot order (rank by rank, tokens in order).  slot[s,r]
 * is then the assignment's global row seg_e + position (never -1), and the
 * expert step reads and writes row seg_e + c for c < n_e.  capacity must be 0
 * and capacity_factor is ignored.  Same arithmetic as the capacity mode with
 * a capacity no expert can reach, without its E*C-row buffers.  Source:
 * "GShard: Scaling Giant Models with Conditional Computation and Automatic
 * Sharding" (inference-research paper card), method paragraph: the token
 * dropping of capacity-limited routing is what the later MegaBlocks work
 * removes. */
#define MOE_CFG_DROPLESS 1u

/* moe_config.flags: overflow re-routing (not with MOE_CFG_DROPLESS).  The
 * blog ("GShard: Scaling Giant Neural Networks with Conditional Computation",
 * paragraph "Expert Capacity") lets tokens over capacity go to other experts
 * instead of being dropped, and gives no rule for it; this library's rule:
 * after the capacity pass, the j-th dropped assignment of token s (dropped
 * ranks in rank order) is offered to the token's (k+j)-th ranked expert (all
 * E experts ordered by logit descending, index ascending; none when
 * k + j >= E).  Offers take capacity after every real assignment, virtual
 * rank by virtual rank (j = 0 for all tokens, then j = 1, ...), tokens in
 * order; an offer is accepted while its expert holds fewer than C rows and is
 * otherwise dropped for good.  An accepted assignment keeps its weight
 * topk_w[s,r]; topk_idx[s,r] then names the expert that serves it and
 * slot[s,r] its row there.  counts gains a row: counts [k+1,E], row k = the
 * offers each expert accepted (rows 0..k-1 and the losses are unchanged).
 * The backward differentiates the weights through the top-k logits, which it
 * ranks again from `logits`. */
#define MOE_CFG_REROUTE 2u

/* moe_gate flag: read `logits` as an input instead of computing them from x,
 * Wg and bg (x, w_gate and gate_bias may then be NULL). */
#define MOE_GATE_LOGITS_IN 1u

/* Number of events moe_layer_forward records when stage_events != NULL:
 * [0] start, [1] after router logits, [2] after softmax/top-k, [3] after
 * the slot scan, [4] after slot positions and losses, [5] after dispatch,
 * [6] after expert GEMM 1, [7] after expert GEMM 2, [8] after combine. */
#define MOE_NUM_STAGE_EVENTS 9

/* Capacity C of the config (capacity if > 0, else ceil(cf*k*S/E); S with
 * MOE_CFG_DROPLESS, which no expert can exceed), or -1 if the config is
 * invalid.  Source: blog, paragraph "Expert Capacity" (a per-expert token
 * limit set by the capacity factor); paper card, method paragraph. */
int32_t moe_capacity(const moe_config *cfg);

/* Rows of the dispatch buffer xd and the expert output out: E*C in capacity
 * mode, S*k with MOE_CFG_DROPLESS; -1 if the config is invalid.  Source: the
 * per-expert buffers of the dispatch step (atlas, "In plain words"). */
int64_t moe_dispatch_rows(const moe_config *cfg);

/* Device workspace bytes that moe_layer_forward needs (enough for every
 * other entry point too) when all of its optional outputs are NULL.  (No
 * passage: the workspace is this library's own scratch.) */
moe_status moe_workspace_bytes(const moe_config *cfg, size_t *bytes);

/* Static text for a status code. */
const char *moe_status_string(int32_t status);

/* Router, top-k and capacity slots.  Source: blog, "Mixture-of-Experts
 * Implementation" (G(x) = Softmax(x . W_g), the top-k experts of it); paper
 * card, method paragraph (top-2 gating, softmax-normalised top-2 weights,
 * auxiliary loss and z-loss, tokens over capacity dropped); blog, paragraph
 * "Expert Capacity".
 * In:  x [S,d] act, w_gate [E,d] fp32, gate_bias [E] fp32 or NULL
 *      (all unused with MOE_GATE_LOGITS_IN).
 * Out: logits [S,E] fp32 (input with MOE_GATE_LOGITS_IN; may be NULL
 *      otherwise, then kept in ws), topk_idx [S,k], topk_w [S,k],
 *      slot [S,k] (-1 = dropped; with MOE_CFG_DROPLESS the global row in
 *      xd/out), counts [k,E] ([k+1,E] with MOE_CFG_REROUTE), losses [2].
 * A top-k decision of token s between logits closer than the margin
 * tau_s = 32 * 2^-24 * (|x_s| max_j |Wg_j| + max_j |bg_j| / 8) (Euclidean
 * row norms) is re-evaluated: the tied logits are recomputed with fp64
 * accumulation and rounded once to fp32, and the stored logits hold those
 * values.  The margin scales with the inputs as the logit GEMM's rounding
 * error does, so it stays well above that error at any scale of x, Wg and
 * bg, and the decisions are those of an exactly rounded fp32 router. */
moe_status moe_gate(const moe_config *cfg, const void *x, const float *w_gate,
                    const float *gate_bias, float *logits, int32_t *topk_idx,
                    float *topk_w, int32_t *slot, int32_t *counts, float *losses,
                    uint32_t flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the library's static device scratch (per GPU), the most that
 * moe_gate_noalloc may use. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)

/* moe_gate without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (minus ws, ws_bytes), same kernels and
 * same results as moe_gate.  Its scratch is a static device array of
 * MOE_STATIC_SCRATCH_BYTES bytes inside the library: each GPU the library
 * runs on holds its own copy from the first call on that GPU until the
 * process ends.  The call allocates and frees nothing.  Its first call on a
 * device looks the array's address up once (hipGetSymbolAddress) and keeps
 * it; later calls reuse it.  A shape whose router scratch would exceed the
 * array (the router part of moe_workspace_bytes: room for the logits, the
 * per-tile histograms and probability partials, the m-tile table and the
 * re-routing offers) is refused with MOE_ERR_SCRATCH_LIMIT before anything
 * is enqueued; the five benchmark shapes fit (the largest, S = 65536 tokens
 * over E = 64 experts, needs about 19 MiB).  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (nothing in it needs to start at zero): calls that
 * overlap on one GPU race, so order them on one stream or serialise them. */
moe_status moe_gate_noalloc(const moe_config *cfg, const void *x, const float *w_gate,
                            const float *gate_bias, float *logits, int32_t *topk_idx,
                            float *topk_w, int32_t *slot, int32_t *counts, float *losses,
                            uint32_t flags, hipStream_t stream);

/* Permute token rows into per-expert capacity buffers (the local stand-in
 * for the dispatch all-to-all; source: atlas "GShard (Expert Parallelism)",
 * "In plain words": tokens are sent to their experts by an all-to-all): xd[idx[s,r], slot[s,r], :] = x[s, :] for
 * every slot[s,r] >= 0 (with MOE_CFG_DROPLESS: xd[slot[s,r], :] = x[s, :]).
 * Bit-exact copy.  Needs no workspace. */
moe_status moe_dispatch(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                        const int32_t *slot, void *xd, hipStream_t stream);

/* Expert FFNs over the filled slots (source: blog, section "Core
 * Components", "Expert Networks": each expert is a feed-forward network; the
 * ReLU two-layer form is the workload's): for e < E and c < occ_e =
 * min(sum_r counts[r,e], C): out[e,c] = ReLU(xd[e,c] W1_e^T + b1_e) W2_e^T
 * + b2_e, fp32 accumulation; the hidden activations are rounded to act_dtype
 * (they live in ws).  Rows c >= occ_e of out are not written.  With
 * MOE_CFG_DROPLESS, occ_e = n_e and row (e,c) is row seg_e + c of the
 * [S*k,d] buffers (seg_e as defined at MOE_CFG_DROPLESS); counts are those
 * moe_gate wrote (they total S*k): a segment that would reach past row S*k
 * is cut there, so no access leaves the buffers. */
moe_status moe_expert_ffn(const moe_config *cfg, const void *xd, const int32_t *counts,
                          const void *w1, const void *b1, const void *w2, const void *b2,
                          void *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine back to token order (the local stand-in for the
 * second all-to-all; source: research-vault claim IX2-0404, "WideEP",
 * "Evidence": results return by a second all-to-all; the weights are the
 * paper card's softmax-normalised top-2 weights): y[s] = sum over slot[s,r] >= 0 of
 * topk_w[s,r] * out[topk_idx[s,r], slot[s,r]], fp32 accumulation, rounded
 * to act_dtype; y[s] = 0 when every assignment of s was dropped.  With
 * MOE_CFG_DROPLESS the row read is out[slot[s,r]].  Needs no workspace. */
moe_status moe_combine(const moe_config *cfg, const void *out, const int32_t *topk_idx,
                       const int32_t *slot, const float *topk_w, void *y,
                       hipStream_t stream);

/* The whole forward pass: gate, slots, dispatch, expert FFNs, combine and
 * losses, enqueued back to back with no host synchronisation (the passages
 * cited at moe_gate, moe_dispatch, moe_expert_ffn and moe_combine).
 * Required: x, w_gate, w1, w2, y, ws.  Optional (NULL = not wanted, kept in
 * ws): gate_bias, b1, b2, logits, topk_idx, topk_w, slot, counts, losses,
 * xd, out, hidden.  When xd and out are both NULL one workspace buffer serves
 * as both.  hidden [E,C,h] ([S*k,h] with MOE_CFG_DROPLESS), act dtype:
 * receives the expert hidden activations ReLU(xd W1^T + b1) of the filled
 * rows, which moe_layer_backward can then reuse instead of recomputing.  With bf16 activations, xd NULL and S*d*2 < 2^32 bytes, no dispatch
 * buffer is written at all: the first expert GEMM reads each slot's row
 * straight from x through an inverse slot map (same results bit for bit;
 * the dispatch stage then takes no time).  stage_events: NULL, or an array
 * of MOE_NUM_STAGE_EVENTS events created by the caller, recorded on `stream`
 * between the steps (for timing); NULL entries are skipped (each recorded
 * event costs a few microseconds of queue time between two kernels). */
moe_status moe_layer_forward(const moe_config *cfg, const void *x, const float *w_gate,
                             const float *gate_bias, const void *w1, const void *b1,
                             const void *w2, const void *b2, void *y, float *logits,
                             int32_t *topk_idx, float *topk_w, int32_t *slot,
                             int32_t *counts, float *losses, void *xd, void *out,
                             void *hidden, void *ws, size_t ws_bytes,
                             hipEvent_t *stage_events, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 * The pages' setting is training: the layer is trained with its auxiliary
 * loss and z-loss ("GShard: Scaling Giant Models with Conditional Computation
 * and Automatic Sharding" (inference-research paper card), method
 * paragraph).  moe_layer_backward returns the gradients of
 *     L = sum_s dy[s] . y[s] + g_aux * aux + g_z * z
 * for the routing a forward call chose (top-k set, slots and drops, and the
 * first-choice fractions f_j, which are piecewise constant, are held fixed):
 *   per kept assignment (s,r) of expert e at row u, with a = ReLU(W1_e x_s +
 *   b1_e) and o = out[u]:  dO = w[s,r] dy_s;  dw[s,r] = dy_s . o;
 *   dW2_e += dO a^T;  db2_e += dO;  du = (W2_e^T dO) * [a > 0];
 *   dW1_e += du x_s^T;  db1_e += du;  dx_s += W1_e^T du;
 *   the renormalised top-k weights are the softmax of the k selected logits:
 *   dl[s, idx_r] += w_r (dw_r - sum_r' w_r' dw_r');
 *   aux: dl[s,j] += g_aux p_sj (a_j - sum_j' p_sj' a_j'), a_j = E f_j / S;
 *   z:   dl[s,j] += g_z (2/S) lse_s p_sj;
 *   dWg = sum_s dl_s x_s^T;  dbg = sum_s dl_s;  dx_s += Wg^T dl_s.
 * Supported for bf16 activations with S*d*2 < 2^32 bytes (else
 * MOE_ERR_UNSUPPORTED), in capacity, dropless and re-routing modes (with
 * MOE_CFG_REROUTE, topk_idx names the serving experts: the expert side
 * follows them, and the weights' logit gradient goes to the router's own
 * top-k, ranked again from `logits`).
 * In:  x, w_gate, w1, b1 (NULL = 0), w2 as given to the forward; the
 *      forward's outputs logits, topk_idx, topk_w, slot, counts and out
 *      (the expert outputs, [E,C,d] or [S*k,d]); hidden: NULL (the hidden
 *      activations are recomputed, one more expert GEMM) or the forward's
 *      `hidden` output (read only); dy [S,d] act; the loss weights g_aux and
 *      g_z (finite).
 * Out: dx [S,d] act, dw_gate [E,d] fp32, db_gate [E] fp32 (NULL = not
 *      wanted), dw1 [E,h,d] act, db1 [E,h] act (NULL = not wanted),
 *      dw2 [E,d,h] act, db2 [E,d] act (NULL = not wanted).
 * Precision: fp32 accumulation everywhere; the hidden activations are the
 * forward's (bf16, saved or recomputed bit-identically), dO, du and the
 * expert-side input gradient are rounded to bf16 once.  dl is fp32; its
 * products (dl Wg for dx, dl^T x for dWg) run on the bf16 MFMAs with dl, and
 * for dx also Wg, split into hi + lo bf16 parts (relative error about 2^-16);
 * dWg and dbg are fp32 sums over fixed token chunks (deterministic).
 * ws: at least moe_backward_workspace_bytes() bytes, 256-byte aligned.
 * stage_events: NULL, or MOE_NUM_BWD_EVENTS caller-created events recorded
 * on `stream` between the steps (NULL entries skipped). */
#define MOE_NUM_BWD_EVENTS 9 /* [0] start, [1] after occupancy / m-tile lists /
    inverse map / dispatched rows, [2] after the hidden-activation recompute, [3] after the combine
    and router backward, [4] after dW2 and db2, [5] after dU, [6] after dW1
    and db1, [7] after the expert-side input gradient, [8] after dx, dWg, dbg */
moe_status moe_backward_workspace_bytes(const moe_config *cfg, size_t *bytes);
moe_status moe_layer_backward(const moe_config *cfg, const void *x, const float *w_gate,
                              const void *w1, const void *b1, const void *w2,
                              const float *logits, const int32_t *topk_idx,
                              const float *topk_w, const int32_t *slot,
                              const int32_t *counts, const void *out, const void *hidden,
                              const void *dy, float g_aux, float g_z, void *dx, float *dw_gate,
                              float *db_gate, void *dw1, void *db1, void *dw2, void *db2,
                              void *ws, size_t ws_bytes, hipEvent_t *stage_events,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
