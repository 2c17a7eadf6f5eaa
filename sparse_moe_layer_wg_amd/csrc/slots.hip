// Capacity-limited slot assignment and the load-balance / z losses.
//
// Method: "GShard: Scaling Giant Models with Conditional Computation and
// Automatic Sharding" (paper card), method paragraph: assignments beyond an
// expert's capacity (set by capacity_factor) are dropped; aux loss
// N*sum_j f_j*P_j plus a z-loss.  "GShard: Scaling Giant Neural Networks with
// Conditional Computation" (blog), paragraph "Expert Capacity".
//
// Slot order (a reading the pages leave open): all first choices, then all
// second choices, ..., each in token order.  The assignment stream is cut
// into tiles t = (rank r, token block b) in that order.  The router kernel
// counts each tile's assignments per expert; a per-expert exclusive scan over
// tiles gives every tile its base position; inside a tile the stable rank of
// a token among earlier tokens with the same expert comes from wavefront
// ballots.  Positions never depend on atomic ordering, so slots are
// deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Exclusive scan of the 256-thread block; returns the prefix of `v` and
// writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int t = s_wave[w];
        before += w < wave ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// m-tile prefix mt_start [E+1] of the experts' filled rows occ, then the
// expert of every m-tile; with seg non-null also seg[e] = sum_{e'<e} occ[e']
// (compact rows).  All 256 threads of the block call it.
__device__ void tile_prefix(const int32_t* __restrict__ occ, int E, int bm, int extra,
                            int* s_wave, int32_t* __restrict__ mt_start,
                            int32_t* __restrict__ seg) {
    const int tid = threadIdx.x;
    int carry = 0, rcarry = 0;
    for (int base = 0; base < E; base += 256) {
        const int e = base + tid;
        const int o = e < E ? occ[e] : 0;
        const int v = expert_mtiles(o, bm, extra);
        int total;
        const int ex = block_exclusive_scan(v, s_wave, &total);
        if (e < E) {
            mt_start[e] = carry + ex;
            for (int i = 0; i < v; ++i) mt_start[E + 1 + carry + ex + i] = e;
        }
        carry += total;
        if (seg) {
            int rtotal;
            const int rex = block_exclusive_scan(o, s_wave, &rtotal);
            if (e < E) seg[e] = rcarry + rex;
            rcarry += rtotal;
        }
    }
    if (tid == 0) mt_start[E] = carry;
}

// One block per expert: hist[e][0..T) becomes the exclusive positions;
// counts[r,e] and occ[e] follow.  The block also sums the router's per-block
// probability partials of expert e into psum[e] (fixed assignment of blocks to
// threads and a fixed tree, so the sum is deterministic).
__global__ __launch_bounds__(256) void slot_scan_kernel(int32_t* __restrict__ hist, int E, int k,
                                                        int nb, int C,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ occ,
                                                        const float* __restrict__ ppart,
                                                        double* __restrict__ psum) {
    __shared__ int s_wave[4];
    __shared__ int s_rank_start[kMaxK + 1];
    __shared__ double s_red[256];
    const int e = blockIdx.x, tid = threadIdx.x;
    double pa = 0.0;
#pragma unroll 4
    for (int b = tid; b < nb; b += 256) pa += (double)ppart[(size_t)b * E + e];
    s_red[tid] = pa;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) s_red[tid] += s_red[tid + off];
        __syncthreads();
    }
    if (tid == 0) psum[e] = s_red[0];
    // Each thread takes CH consecutive entries of a 256*CH-entry chunk: all
    // of its loads go out at once and one block scan of the per-thread sums
    // covers the chunk (a row of k*nb entries is one chunk up to 2048).
    constexpr int CH = 8;
    const int T = k * nb;
    int32_t* row = hist + (size_t)e * T;
    int carry = 0;
    for (int base = 0; base < T; base += 256 * CH) {
        const int i0 = base + tid * CH;
        int v[CH], sum = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = i0 + j < T ? row[i0 + j] : 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) sum += v[j];
        int total;
        int run = carry + block_exclusive_scan(sum, s_wave, &total);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int i = i0 + j;
            if (i < T) {
                row[i] = run;
                if (i % nb == 0) s_rank_start[i / nb] = run;
            }
            run += v[j];
        }
        carry += total;
    }
    __syncthreads();
    if (tid < k) {
        const int start = s_rank_start[tid];
        const int end = tid + 1 < k ? s_rank_start[tid + 1] : carry;
        counts[(size_t)tid * E + e] = end - start;
    }
    if (tid == 0) occ[e] = carry < C ? carry : C;
}

// aux = E * sum_j f_j P_j with f_j = counts[0,j] / S and P_j = psum[j] / S;
// z = (sum of the block partials of lse^2) / S.  Sums run in a fixed order
// in fp64, so the result is deterministic.  Also the per-expert m-tile
// prefix for the expert GEMMs.
__device__ void finalize_block(const double* __restrict__ psum, const float* __restrict__ zpart,
                               const int32_t* __restrict__ counts,
                               const int32_t* __restrict__ occ, int S, int E, int nb, int bm,
                               float* __restrict__ losses, int32_t* __restrict__ mt_start,
                               int32_t* __restrict__ seg, int32_t* __restrict__ ctr,
                               int n_ctr) {
    __shared__ double s_red[256];
    __shared__ int s_wave[4];
    const int tid = threadIdx.x;
    for (int i = tid; i < n_ctr; i += 256) ctr[i] = 0;
    double term = 0.0;
    for (int j = tid; j < E; j += 256) term += (double)counts[j] * psum[j];
    s_red[tid] = term;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) s_red[tid] += s_red[tid + off];
        __syncthreads();
    }
    const double aux_sum = s_red[0];
    __syncthreads();
    double z = 0.0;
    for (int b = tid; b < nb; b += 256) z += (double)zpart[b];
    s_red[tid] = z;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) s_red[tid] += s_red[tid + off];
        __syncthreads();
    }
    if (tid == 0) {
        const double Sd = (double)S;
        losses[0] = (float)((double)E * aux_sum / (Sd * Sd));
        losses[1] = (float)(s_red[0] / Sd);
    }
    tile_prefix(occ, E, bm, bm == 256 ? kStripRows : 0, s_wave, mt_start, seg);
}

// One block (4 waves) per token block; wave w takes ranks w, w+4, ...
// Compact rows: the block first scans occ into its own copy of the segment
// starts (E <= kMaxE), so it needs nothing from the finalize block.
__device__ void positions_block(int b, const int32_t* __restrict__ topk_idx,
                                const int32_t* __restrict__ hist_base, int S, int E, int k,
                                int nb, int C, int nbits, const int32_t* __restrict__ occ,
                                bool compact, int32_t* __restrict__ slot,
                                int32_t* __restrict__ inv) {
    __shared__ int s_seg[kMaxE];
    __shared__ int s_wave[4];
    if (compact) {
        int carry = 0;
        for (int base = 0; base < E; base += 256) {
            const int e = base + threadIdx.x;
            int total;
            const int ex = block_exclusive_scan(e < E ? occ[e] : 0, s_wave, &total);
            if (e < E) s_seg[e] = carry + ex;
            carry += total;
        }
        __syncthreads();
    }
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = b * kTokBlock + lane;
    const bool valid = s < S;
    const int T = k * nb;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int r = wave; r < k; r += 4) {
        const int e = valid ? topk_idx[(size_t)s * k + r] : 0;
        uint64_t same = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool one = (e >> bit) & 1;
            const uint64_t ones = __ballot(one);
            same &= one ? ones : ~ones;
        }
        const int before = __popcll(same & lt_mask);
        if (valid) {
            const int pos = hist_base[(size_t)e * T + (size_t)r * nb + b] + before;
            const bool kept = pos < C;
            const int row = compact ? s_seg[e] + pos : e * C + pos;
            slot[(size_t)s * k + r] = kept ? (compact ? row : pos) : -1;
            if (inv && kept) inv[row] = s;
        }
    }
}

// occ[e] = min(sum_r counts[r,e], C), the m-tile prefix and the expert of
// every m-tile (one block); with seg non-null also the compact segment
// starts, the segments held within `rows` rows.
__global__ __launch_bounds__(256) void occupancy_kernel(const int32_t* __restrict__ counts, int E,
                                                        int k, int C, int bm, int extra,
                                                        int32_t* __restrict__ occ,
                                                        int32_t* __restrict__ mt_start,
                                                        int32_t* __restrict__ seg, int rows,
                                                        int32_t* __restrict__ ctr, int n_ctr,
                                                        bool reroute) {
    __shared__ int s_wave[4];
    const int tid = threadIdx.x;
    for (int i = tid; i < n_ctr; i += 256) ctr[i] = 0;
    for (int e = tid; e < E; e += 256) {
        long long n = 0;
        for (int r = 0; r < k; ++r) n += counts[(size_t)r * E + e];
        int o = n < 0 ? 0 : n < C ? (int)n : C;
        if (reroute) {
            // row k: re-routed assignments the expert accepted (within C)
            const int a = counts[(size_t)k * E + e];
            o += a < 0 ? 0 : a < C - o ? a : C - o;
        }
        occ[e] = o;
    }
    __syncthreads();  // each thread reads other threads' occ below
    if (seg) {
        // Compact segments end to end; counts totalling more than `rows` are
        // invalid, and a segment that would pass row `rows` is cut there.
        int carry = 0;
        for (int base = 0; base < E; base += 256) {
            const int e = base + tid;
            const int o = e < E ? occ[e] : 0;
            int total;
            const int ex = block_exclusive_scan(o, s_wave, &total);
            if (e < E) {
                const long long start = (long long)carry + ex;
                seg[e] = start < rows ? (int)start : rows;
                const long long room = start < rows ? rows - start : 0;
                occ[e] = o < room ? o : (int)room;
            }
            carry = carry + total < rows ? carry + total : rows;
        }
        __syncthreads();
    }
    tile_prefix(occ, E, bm, extra, s_wave, mt_start, nullptr);
}

// ------------------------------------------------------------ re-routing
// Overflow re-routing (the capacity paragraph of the GShard blog allows
// overflowing tokens to go to alternative experts; the rule here is a
// reading): the j-th dropped assignment of a token (dropped ranks in rank
// order) is offered to the token's (k+j)-th ranked expert, by (logit
// descending, index ascending).  Offers form virtual ranks j = 0..k-1 after
// the k real ones and take capacity in the same order as real assignments
// (virtual rank by virtual rank, tokens in order), so the tile histogram,
// scan and in-tile ballot ranks of the capacity pass serve again.

// One block per 64-token routing tile.  A token's offers (expert, original
// rank) for virtual ranks j < its dropped count (-1 elsewhere) are found by
// L lanes, each holding V of its logits (experts li + L*q): per offer, every
// lane takes its largest order key (logit descending, index ascending) among
// experts not yet taken and the L lanes reduce it with shuffles; 64/L tokens
// share a wave.  The tile's offer histogram is then written whole into
// hist[e][j*nb + b] (every entry, zeros included, so nothing is cleared
// beforehand).  Dynamic LDS: k*E ints.
constexpr int kOfferThreads = 256;

template <int L, int V>
__global__ __launch_bounds__(kOfferThreads) void reroute_offers_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ slot, int S, int E, int k, int nb, int32_t* __restrict__ offer_e,
    int32_t* __restrict__ offer_r, int32_t* __restrict__ hist) {
    static_assert(V <= 32, "taken bits per lane");
    extern __shared__ int s_h[];                  // [k][E] offers of this tile
    __shared__ int s_off[kMaxK][kTokBlock];       // offered expert per (j, token)
    constexpr int TPW = kWave / L;                // tokens per wave and round
    constexpr int TPR = TPW * (kOfferThreads / kWave);   // tokens per block and round
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int g = lane / L, li = lane % L;
    const int b = blockIdx.x;
    for (int i = tid; i < k * E; i += kOfferThreads) s_h[i] = 0;
    for (int t0 = 0; t0 < kTokBlock; t0 += TPR) {
        const int t = t0 + wave * TPW + g;         // this group's token in the tile
        const int s = b * kTokBlock + t;
        const bool live = s < S;
        float v[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int j = li + L * q;
            v[q] = live && j < E ? logits[(size_t)s * E + j] : 0.f;
        }
        uint32_t taken = 0;   // the top-k are not alternatives
        uint32_t drop = 0;    // dropped ranks of the token
        for (int r = 0; r < k; ++r) {
            const int e = live ? topk_idx[(size_t)s * k + r] : -1;
            if (e >= 0 && e % L == li) taken |= 1u << (e / L);
            if (live && slot[(size_t)s * k + r] < 0) drop |= 1u << r;
        }
        int j = 0;
        for (int r = 0; r < k; ++r) {   // every group takes part in every step
            const bool want = ((drop >> r) & 1u) && k + j < E;
            uint64_t best = 0;
            if (want) {
#pragma unroll
                for (int q = 0; q < V; ++q) {
                    const int e = li + L * q;
                    if (e < E && !((taken >> q) & 1u)) {
                        const uint64_t key = (static_cast<uint64_t>(float_order_key(v[q])) << 32) |
                                             (0xffffffffu - static_cast<uint32_t>(e));
                        best = key > best ? key : best;
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < L; off <<= 1) {
                const uint64_t o = __shfl_xor(best, off, kWave);
                best = o > best ? o : best;
            }
            if ((drop >> r) & 1u) {
                const int e = want ? (int)(0xffffffffu - static_cast<uint32_t>(best)) : -1;
                if (e >= 0 && e % L == li) taken |= 1u << (e / L);
                if (li == 0) {
                    offer_e[(size_t)s * k + j] = e;
                    offer_r[(size_t)s * k + j] = r;
                    s_off[j][t] = e;
                }
                ++j;
            }
        }
        if (li == 0) {
            for (; j < k; ++j) {
                if (live) {
                    offer_e[(size_t)s * k + j] = -1;
                    offer_r[(size_t)s * k + j] = -1;
                }
                s_off[j][t] = -1;
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < k * kTokBlock; i += kOfferThreads) {
        const int e = s_off[i / kTokBlock][i % kTokBlock];
        if (e >= 0) atomicAdd(&s_h[(i / kTokBlock) * E + e], 1);
    }
    __syncthreads();
    const size_t T = (size_t)k * nb;
    for (int i = tid; i < k * E; i += kOfferThreads) {
        const int jj = i / E, e = i - jj * E;
        hist[(size_t)e * T + (size_t)jj * nb + b] = s_h[i];
    }
}

// One block per expert: the expert's offers, in slot order (virtual rank,
// then tile), get the rows after its o = occ[e] filled ones: hist becomes
// o + exclusive position.  counts[k, e] = accepted = min(offers, C - o) and
// occ[e] grows by it.
__global__ __launch_bounds__(256) void reroute_scan_kernel(int32_t* __restrict__ hist, int E,
                                                           int k, int nb, int C,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ occ) {
    __shared__ int s_wave[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    const int T = k * nb;
    int32_t* row = hist + (size_t)e * T;
    const int o = occ[e];
    // CH consecutive entries per thread, one block scan per 256*CH entries
    // (as in slot_scan_kernel)
    constexpr int CH = 8;
    int carry = 0;
    for (int base = 0; base < T; base += 256 * CH) {
        const int i0 = base + tid * CH;
        int v[CH], sum = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = i0 + j < T ? row[i0 + j] : 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) sum += v[j];
        int total;
        int run = o + carry + block_exclusive_scan(sum, s_wave, &total);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (i0 + j < T) row[i0 + j] = run;
            run += v[j];
        }
        carry += total;
    }
    __syncthreads();   // every thread has read occ[e]
    if (tid == 0) {
        const int room = C - o;
        const int a = carry < room ? carry : room;
        counts[(size_t)k * E + e] = a;
        occ[e] = o + a;
    }
}

// Blocks 0..nb-1, one per routing tile, wave w taking virtual ranks w, w+4,
// ...: an offer's row is its expert's scanned base plus its stable rank among
// the tile's offers to that expert (ballots over the expert bits); it is
// accepted when the row is below C, and the assignment moves there.  Block
// nb rebuilds the m-tile prefix from the grown occupancies and zeroes the
// n_ctr GEMM tile counters.
__global__ __launch_bounds__(256) void reroute_positions_kernel(
    const int32_t* __restrict__ offer_e, const int32_t* __restrict__ offer_r,
    const int32_t* __restrict__ hist_row, const int32_t* __restrict__ occ, int S, int E, int k,
    int nb, int C, int nbits, int bm, int extra, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ slot, int32_t* __restrict__ inv, int32_t* __restrict__ mt_start,
    int32_t* __restrict__ ctr, int n_ctr) {
    const int b = blockIdx.x;
    if (b == nb) {
        __shared__ int s_wave[4];
        for (int i = threadIdx.x; i < n_ctr; i += 256) ctr[i] = 0;
        tile_prefix(occ, E, bm, extra, s_wave, mt_start, nullptr);
        return;
    }
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = b * kTokBlock + lane;
    const int T = k * nb;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int j = wave; j < k; j += 4) {
        const int e = s < S ? offer_e[(size_t)s * k + j] : -1;
        const bool has = e >= 0;
        uint64_t same = __ballot(has);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool one = (e >> bit) & 1;
            const uint64_t ones = __ballot(one);
            same &= one ? ones : ~ones;
        }
        const int before = __popcll(same & lt_mask);
        if (has) {
            const int row = hist_row[(size_t)e * T + (size_t)j * nb + b] + before;
            if (row < C) {
                const int r = offer_r[(size_t)s * k + j];
                topk_idx[(size_t)s * k + r] = e;
                slot[(size_t)s * k + r] = row;
                if (inv) inv[(size_t)e * C + row] = s;
            }
        }
    }
}

__global__ void zero_outputs_kernel(int32_t* counts, int n, float* losses) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (counts && i < n) counts[i] = 0;
    if (losses && i < 2) losses[i] = 0.f;
}

}  // namespace

hipError_t launch_slot_scan(int32_t* hist, int E, int k, int nb, int C, int32_t* counts,
                            int32_t* occ, const float* ppart, double* psum, hipStream_t st) {
    slot_scan_kernel<<<E, 256, 0, st>>>(hist, E, k, nb, C, counts, occ, ppart, psum);
    return hipGetLastError();
}

// Slot positions (blocks 0..nb-1) and, in one extra block, the losses, the
// GEMM m-tile prefix and the tile counters: the latter need only the slot
// scan's results, so both run in one launch.
__global__ __launch_bounds__(256) void positions_finalize_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ hist_base, int S, int E,
    int k, int nb, int C, int nbits, bool compact, int32_t* __restrict__ slot,
    int32_t* __restrict__ inv, const double* __restrict__ psum, const float* __restrict__ zpart,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ occ, int bm,
    float* __restrict__ losses, int32_t* __restrict__ mt_start, int32_t* __restrict__ seg,
    int32_t* __restrict__ ctr, int n_ctr) {
    if ((int)blockIdx.x < nb)
        positions_block(blockIdx.x, topk_idx, hist_base, S, E, k, nb, C, nbits, occ, compact,
                        slot, inv);
    else
        finalize_block(psum, zpart, counts, occ, S, E, nb, bm, losses, mt_start,
                       compact ? seg : nullptr, ctr, n_ctr);
}

hipError_t launch_positions_finalize(const int32_t* topk_idx, const int32_t* hist_base, int S,
                                     int E, int k, int nb, int C, bool compact, int32_t* slot,
                                     int32_t* inv, const double* psum, const float* zpart,
                                     const int32_t* counts, const int32_t* occ, int bm,
                                     float* losses, int32_t* mt_start, int32_t* seg,
                                     int32_t* ctr, int n_ctr, hipStream_t st) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    positions_finalize_kernel<<<nb + 1, 256, 0, st>>>(
        topk_idx, hist_base, S, E, k, nb, C, nbits, compact, slot, inv, psum, zpart, counts, occ,
        bm, losses, mt_start, seg, ctr, n_ctr);
    return hipGetLastError();
}

hipError_t launch_occupancy(const int32_t* counts, int E, int k, int C, int bm, int extra,
                            int32_t* occ, int32_t* mt_start, int32_t* seg, int rows,
                            int32_t* ctr, int n_ctr, hipStream_t st, bool reroute) {
    occupancy_kernel<<<1, 256, 0, st>>>(counts, E, k, C, bm, extra, occ, mt_start, seg, rows,
                                        ctr, n_ctr, reroute);
    return hipGetLastError();
}

hipError_t launch_zero_outputs(int32_t* counts, int n_counts, float* losses, hipStream_t st) {
    const int n = n_counts > 2 ? n_counts : 2;
    zero_outputs_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(counts, n_counts, losses);
    return hipGetLastError();
}

hipError_t launch_reroute(const float* logits, int32_t* topk_idx, int32_t* slot, int32_t* inv,
                          int32_t* counts, int32_t* occ, int32_t* mt_start, int32_t* ctr,
                          int n_ctr, int S, int E, int k, int nb, int C, int bm,
                          int32_t* offer_e, int32_t* offer_r, int32_t* hist, hipStream_t st) {
    if (S == 0) return hipSuccess;
    const size_t lds = (size_t)k * E * sizeof(int);
    auto offers = [&](auto kern) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        kern<<<nb, kOfferThreads, lds, st>>>(logits, topk_idx, slot, S, E, k, nb, offer_e,
                                             offer_r, hist);
    };
    // L lanes per token: the smallest power of two giving at most 16 logits
    // per lane (32 for E > 1024)
    if (E <= 64) offers(&reroute_offers_kernel<4, 16>);
    else if (E <= 128) offers(&reroute_offers_kernel<8, 16>);
    else if (E <= 256) offers(&reroute_offers_kernel<16, 16>);
    else if (E <= 512) offers(&reroute_offers_kernel<32, 16>);
    else if (E <= 1024) offers(&reroute_offers_kernel<64, 16>);
    else offers(&reroute_offers_kernel<64, 32>);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    reroute_scan_kernel<<<E, 256, 0, st>>>(hist, E, k, nb, C, counts, occ);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    reroute_positions_kernel<<<nb + 1, 256, 0, st>>>(offer_e, offer_r, hist, occ, S, E, k, nb, C,
                                                     nbits, bm, strip_rows(bm), topk_idx, slot,
                                                     inv, mt_start, ctr, n_ctr);
    return hipGetLastError();
}

}  // namespace moe
