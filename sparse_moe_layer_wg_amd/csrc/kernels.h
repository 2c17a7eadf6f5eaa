// Internal launchers of the MoE-layer kernels.  Each returns the HIP status of
// its launch; the C ABI in moe_api.hip maps failures to MOE_ERR_HIP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ gate
// logits[s,j] = sum_i x[s,i] * wg[j,i] + bg[j]   (fp32 accumulation); also
// the squared row norms xn2[s] = |x[s,:]|^2 and wn2[j] = |wg[j,:]|^2, the
// scale of the router's refinement margin.
hipError_t launch_gate_logits(const void* x, bool x_bf16, const float* wg, const float* bg,
                              float* logits, float* xn2, float* wn2, int S, int d, int E,
                              hipStream_t st);

struct RouteParams {
    float* logits;          // [S,E]; refined entries are written back
    const void* x;          // for refinement (NULL when refinement is off)
    bool x_bf16;
    const float* wg;
    const float* bg;
    int S, d, E, k, nb;     // nb = ceil(S / kTokBlock)
    float tau;              // margin per unit of logit scale; 0 disables refinement
    const float* xn2;       // [S] squared norms of the token rows (with tau > 0)
    const float* wn2;       // [E] squared norms of the router rows (with tau > 0)
    int32_t* topk_idx;      // [S,k]
    float* topk_w;          // [S,k]
    int32_t* hist;          // [E][k*nb] per-(rank, token block) expert counts
    float* ppart;           // [nb][E]  per-block sums of softmax probabilities
    float* zpart;           // [nb]     per-block sums of lse^2
};
hipError_t launch_route(const RouteParams& p, hipStream_t st);

// ------------------------------------------------------------------ slots
// In-place exclusive scan of hist rows (per expert, over (rank, block)
// tiles); writes counts [k,E], occupancy occ[e] = min(n_e, C) and
// psum[e] = sum over blocks of ppart[b][e].
hipError_t launch_slot_scan(int32_t* hist, int E, int k, int nb, int C, int32_t* counts,
                            int32_t* occ, const float* ppart, double* psum, hipStream_t st);
// losses = {aux, z}; mt_start[e] = sum_{e'<e} ceil(occ[e']/bm) (E+1 entries);
// zeroes the n_ctr GEMM tile counters.
// slot[s,r] from the scanned tile bases and stable in-tile ranks (with inv
// non-null also the inverse map inv[row] = s of every kept assignment); in
// the same launch, aux = E * sum_j f_j P_j and z = mean lse^2 into losses,
// the GEMM m-tile prefix (m-tile height bm) into mt_start, and n_ctr tile
// counters zeroed.  Padded rows (compact false): slot = position in the
// expert, row = e*C + slot.  Compact rows: slot = row = seg[e] + position
// with seg the exclusive prefix of occ over experts, also written to seg
// (the expert GEMMs' row0).
hipError_t launch_positions_finalize(const int32_t* topk_idx, const int32_t* hist_base, int S,
                                     int E, int k, int nb, int C, bool compact, int32_t* slot,
                                     int32_t* inv, const double* psum, const float* zpart,
                                     const int32_t* counts, const int32_t* occ, int bm,
                                     float* losses, int32_t* mt_start, int32_t* seg,
                                     int32_t* ctr, int n_ctr, hipStream_t st);
// Occupancy (and m-tile prefix) straight from counts [k,E] (standalone FFN,
// backward); zeroes the n_ctr GEMM tile counters; with seg non-null also the
// exclusive prefix of occ over experts (compact rows), every segment cut to
// end by row `rows` (the compact buffers' length).  m-tiles are bm rows high
// and an expert's last one may take `extra` more rows (expert_mtiles).
// With reroute, counts has a row k of accepted re-routed assignments, added
// to the occupancy.
hipError_t launch_occupancy(const int32_t* counts, int E, int k, int C, int bm, int extra,
                            int32_t* occ, int32_t* mt_start, int32_t* seg, int rows,
                            int32_t* ctr, int n_ctr, hipStream_t st, bool reroute = false);
// Overflow re-routing after the capacity pass (padded rows only): offers of
// dropped assignments to the tokens' next-ranked experts, taken in slot order
// within the remaining capacity.  Moves accepted assignments in topk_idx /
// slot (and inv when non-null), writes counts row k (accepted per expert),
// raises occ, rebuilds the m-tile prefix (height bm) and zeroes n_ctr tile
// counters.  Scratch: offer_e, offer_r [S,k], hist [E][k*nb] int32 (fully
// written, no clearing needed).
hipError_t launch_reroute(const float* logits, int32_t* topk_idx, int32_t* slot, int32_t* inv,
                          int32_t* counts, int32_t* occ, int32_t* mt_start, int32_t* ctr,
                          int n_ctr, int S, int E, int k, int nb, int C, int bm,
                          int32_t* offer_e, int32_t* offer_r, int32_t* hist, hipStream_t st);
// Zero losses and counts (empty input).
hipError_t launch_zero_outputs(int32_t* counts, int n_counts, float* losses, hipStream_t st);

// ------------------------------------------------------------------ permute
// Assignment (s,r) with expert e = topk_idx[s,r] and c = slot[s,r] is row
// e*stride + c of xd / out, kept when 0 <= e < E and 0 <= c < limit
// (padded rows: stride = limit = C; compact rows: stride 0, limit S*k).
hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, const int32_t* slot,
                           void* xd, int S, int d, int k, int E, int stride, int limit,
                           int elem_bytes, hipStream_t st);
hipError_t launch_combine(const void* out, const int32_t* topk_idx, const int32_t* slot,
                          const float* topk_w, void* y, int S, int d, int k, int E, int stride,
                          int limit, bool bf16, hipStream_t st);

// ------------------------------------------------------------------ expert GEMMs
// Per expert e, rows m < occ[e]:
//   Cout[e,m,n] = act(sum_k A[e,m,k] * B[e,n,k] + bias[e,n]),  act = ReLU or id.
// A [E,C,K], B [E,N,K], bias [E,N] or NULL, Cout [E,C,N]; all act dtype.
// With row0 non-null, expert e's rows start at row row0[e] of A, a_rows and
// Cout instead of e*C (compact expert segments).  With a_rows non-null, row m
// of expert e is instead row a_rows[e*C + m] (a_rows[row0[e] + m]) of A [*,K]
// (a gather straight from the token rows: the dispatch permute fused into the
// loads).
struct GemmParams {
    const void* A;
    const void* B;
    const void* bias;
    void* Cout;
    const int32_t* occ;
    const int32_t* mt_start;
    const int32_t* mt_expert;  // expert of each m-tile (mt_start[E] entries)
    const int32_t* a_rows;  // NULL, or the token row of each filled row
    const int32_t* row0;    // NULL (row e*C), or [E] first row of each expert
    int32_t* tile_ctr;      // 8 counters (one per XCD chunk), zero at launch
    int E, C, N, K;
    bool relu;
};
// m-tiles of an expert with occ filled rows.  Tiles are bm rows high, and an
// expert's last m-tile may reach `extra` rows further.  The forward GEMM uses
// extra = kStripRows with bm = 256 (strip_rows): it runs those rows as an
// extra strip against the weight fragments it already holds instead of as a
// nearly empty m-tile of their own.  The backward GEMMs use extra = 0.
constexpr int kStripRows = 32;
__host__ __device__ inline int expert_mtiles(int occ, int bm, int extra) {
    if (occ <= 0) return 0;
    return occ <= bm + extra ? 1 : (occ - extra + bm - 1) / bm;
}
inline int strip_rows(int bm) { return bm == 256 ? kStripRows : 0; }
// The m-tile prefix mt_start [E+1] is followed in memory by the expert of
// every m-tile; room for both: (E + 1) + mtile_table_len(E, C, rows) int32,
// where rows bounds the filled rows of all experts together (m-tiles are at
// least 64 rows high).
inline size_t mtile_table_len(int E, int C, size_t rows) {
    const size_t per_expert = (size_t)E * ((C + 63) / 64), total = (rows + 63) / 64 + E;
    return per_expert < total ? per_expert : total;
}
// m-tile height the expert GEMMs use for a layer shape (the m-tile prefix
// mt_start must be built with the same value).
int gemm_block_m(bool bf16, int S, int E, int k);
hipError_t launch_expert_gemm(const GemmParams& p, bool bf16, int bm, hipStream_t st);
// Compute units of the current device (cached per device).
int device_cus();

// ------------------------------------------------------------------ backward
// Expert GEMMs of the backward pass (bf16, fp32 accumulation), per expert e
// with rows r = row0[e] + m (row0 NULL: e*C + m), m < occ[e]:
//   dgrad:  Cout[r, n] = sum_k A[r, k] * B[e, k, n]     (B is W [E,K,N])
//           with mask: Cout[r, n] = 0 where mask[r, n] <= 0 (mask may be
//           Cout itself); m-tiles of 256 rows from mt_start/mt_expert built
//           with bm = 256, extra = 0.
//   wgrad:  Cout[e, m, n] = sum over rows r of A[r, m] * B[b(r), n]
//           (A [*,M], B [*,N] row-major; b(r) = b_rows[r] or r), every
//           (m, n) < (M, N) written, zero for an empty expert.
struct BwdGemmParams {
    const void* A;
    const void* B;
    void* Cout;
    const void* mask;          // dgrad: NULL or [rows, N]
    const int32_t* occ;
    const int32_t* mt_start;   // dgrad: m-tile prefix [E+1] ...
    const int32_t* mt_expert;  // ... and the expert of each m-tile
    const int32_t* row0;       // NULL (row e*C) or [E]
    const int32_t* b_rows;     // wgrad: NULL or [rows] token row of each row
    void* bias_grad;           // wgrad: NULL, or [E, M] column sums of A over
                               // the expert's rows (the bias gradient)
    int32_t* tile_ctr;         // 8 counters, zero at launch
    int E, C, M, N, K;
    size_t rows;               // rows of the expert buffers (E*C or S*k)
    int lda;                   // wgrad: row stride of A in elements (0: M)
    bool out_f32;              // wgrad: Cout and bias_grad fp32 (else bf16)
};
hipError_t launch_bwd_gemm(const BwdGemmParams& p, bool wgrad, bool mask, hipStream_t st);

// inv[e*stride + slot[s,r]] = s for every kept assignment (stride 0: the
// slot is the row).
hipError_t launch_inverse_rows(const int32_t* topk_idx, const int32_t* slot, int S, int k,
                               int E, int stride, int limit, int32_t* inv, hipStream_t st);
// Combine backward: for kept (s,r) at row u, dO[u] = bf16(w[s,r] * dy[s]) and
// dw[s,r] = dy[s] . out[u] (fp32); dw = 0 for dropped assignments.
hipError_t launch_combine_bwd(const void* dy, const void* out, const int32_t* topk_idx,
                              const int32_t* slot, const float* topk_w, void* dO, float* dw,
                              int S, int d, int k, int E, int stride, int limit,
                              hipStream_t st);
// Router backward: gradient of the logits dl [S,E] (fp32) from the top-k
// weight gradient dw, the aux loss (weight g_aux, first-choice counts) and
// the z-loss (weight g_z).  topk_from_logits: the weights' top-k is ranked
// again from the logits (topk_idx holds serving experts after re-routing).
hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                             const float* dw, const int32_t* counts, float g_aux, float g_z,
                             float* dl, int S, int E, int k, bool topk_from_logits,
                             hipStream_t st);
// Router side of the gradients, on the bf16 MFMAs with two-term splits
// (v = hi + lo, hi = bf16(v), lo = bf16(v - hi); relative error about 2^-16):
//   dx[s, i] = bf16(sum_j dl[s, j] wg[j, i] + sum over kept r of dX[u(s,r), i])
//   dwg[j, i] = sum_s dl[s, j] x[s, i];   dbg[j] = sum_s dl[s, j]  (fp32;
//   dbg may be NULL)
// dwg runs as a weight-gradient GEMM over token chunks with fp32 partials,
// summed in chunk order.  `work` holds router_grads_workspace bytes.
size_t router_grads_workspace(int S, int d, int E);
hipError_t launch_router_grads(const float* dl, const float* wg, const void* x, const void* dX,
                               const int32_t* topk_idx, const int32_t* slot, void* dx,
                               float* dwg, float* dbg, int S, int d, int E, int k, int stride,
                               int limit, void* work, hipStream_t st);
// Fill n bytes with zero (a kernel, so that it can sit in a captured graph).
hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t st);

}  // namespace moe
