// Backward pass of the layer: everything except the expert GEMMs.
//
// Method: the layer is trained with its auxiliary loss and z-loss ("GShard:
// Scaling Giant Models with Conditional Computation and Automatic Sharding"
// (paper card), method paragraph).  The routing (top-k set, slots, drops)
// and the first-choice fractions f_j are piecewise constant; the gradient is
// that of L = sum dy.y + g_aux * aux + g_z * z with them held fixed:
//   combine:  dO[u] = w[s,r] dy[s],  dw[s,r] = dy[s] . O[u]   (u = row of (s,r))
//   router:   the renormalised top-k weights are the softmax of the k
//             selected logits, so dl[s, idx_r] += w_r (dw_r - sum_r' w_r' dw_r');
//             aux = E sum_j f_j P_j adds g_aux p_j (a_j - sum_j' p_j' a_j') with
//             a_j = E f_j / S;  z = mean lse^2 adds g_z (2/S) lse p_j;
//   gate:     dWg = dl^T x,  dbg = colsum dl,  dx += dl Wg;
//   dispatch: dx[s] += sum over kept r of dX[u(s,r)].
// Kernels here are HBM- or latency-bound; one wave per token where a token's
// rows are touched, fp32 arithmetic, fixed reduction orders (deterministic).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;  // one token per wave

__global__ void inverse_rows_kernel(const int32_t* __restrict__ topk_idx,
                                    const int32_t* __restrict__ slot, int S, int k, int E,
                                    int stride, int limit, int32_t* __restrict__ inv) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)S * k) return;
    const int c = slot[i], e = topk_idx[i];
    if (c >= 0 && c < limit && e >= 0 && e < E) inv[(int64_t)e * stride + c] = (int32_t)(i / k);
}

// Row u of assignment (s,r) in the expert buffers, or -1 when dropped.
__device__ __forceinline__ int64_t assignment_row(const int32_t* __restrict__ topk_idx,
                                                  const int32_t* __restrict__ slot, int64_t q,
                                                  int E, int stride, int limit) {
    const int c = slot[q], e = topk_idx[q];
    return (c >= 0 && c < limit && e >= 0 && e < E) ? (int64_t)e * stride + c : -1;
}

__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const u32x4_t* __restrict__ dy, const u32x4_t* __restrict__ out,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot,
    const float* __restrict__ topk_w, u32x4_t* __restrict__ dO, float* __restrict__ dw, int S,
    int nvec, int k, int E, int stride, int limit) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(blockIdx.x * kTokPerBlock + wave);
    if (s >= S) return;
    // all ranks in one pass over the columns: dy is read once and the k
    // expert-output rows are loaded together (u[r] < 0: absent or dropped)
    int64_t u[kMaxK];
    float w[kMaxK], dot[kMaxK];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        u[r] = r < k ? assignment_row(topk_idx, slot, (int64_t)s * k + r, E, stride, limit) : -1;
        w[r] = u[r] >= 0 ? topk_w[(int64_t)s * k + r] : 0.f;
        dot[r] = 0.f;
    }
    const u32x4_t* y = dy + (int64_t)s * nvec;
    for (int i = lane; i < nvec; i += kWave) {
        const u32x4_t yv = y[i];
        u32x4_t ov[kMaxK];
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)
            if (u[r] >= 0) ov[r] = out[u[r] * nvec + i];
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (u[r] < 0) continue;
            u32x4_t gv;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float y0 = __uint_as_float(yv[c] << 16);
                const float y1 = __uint_as_float(yv[c] & 0xffff0000u);
                dot[r] = fmaf(y0, __uint_as_float(ov[r][c] << 16), dot[r]);
                dot[r] = fmaf(y1, __uint_as_float(ov[r][c] & 0xffff0000u), dot[r]);
                gv[c] = pack_bf16x2(w[r] * y0, w[r] * y1);
            }
            dO[u[r] * nvec + i] = gv;
        }
    }
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        if (r >= k) break;
        const float t = u[r] >= 0 ? wave_sum_f32(dot[r]) : 0.f;
        if (lane == 0) dw[(int64_t)s * k + r] = t;
    }
}

// One wave per token; lanes stride over the E logits.
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ dw,
    const int32_t* __restrict__ counts, float g_aux, float g_z, float* __restrict__ dl, int S,
    int E, int k, bool topk_from_logits) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(blockIdx.x * kTokPerBlock + wave);
    if (s >= S) return;
    const float* l = logits + (int64_t)s * E;
    // the top-k the weights belong to: topk_idx, or (re-routing moved some
    // assignments there) the top-k again from the logits, ranked by (logit
    // descending, index ascending) as the router ranks them
    int sel[kMaxK];
    for (int r = 0; r < k; ++r) {
        if (!topk_from_logits) {
            sel[r] = topk_idx[(int64_t)s * k + r];
            continue;
        }
        uint64_t best = 0;
        for (int j = lane; j < E; j += kWave) {
            bool used = false;
            for (int q = 0; q < r; ++q) used |= sel[q] == j;
            if (used) continue;
            const uint64_t key = (static_cast<uint64_t>(float_order_key(l[j])) << 32) |
                                 (0xffffffffu - static_cast<uint32_t>(j));
            best = key > best ? key : best;
        }
        best = wave_max_u64(best);
        sel[r] = (int)(0xffffffffu - __builtin_amdgcn_readfirstlane((uint32_t)best));
    }
    float m = -INFINITY;
    for (int j = lane; j < E; j += kWave) m = fmaxf(m, l[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    float se = 0.f;
    for (int j = lane; j < E; j += kWave) se += expf(l[j] - m);
    se = wave_sum_f32(se);
    const float lse = m + logf(se);
    // a_j = E f_j / S with f_j = counts[0,j] / S
    const float a_scale = (float)E / ((float)S * (float)S);
    float pa = 0.f;
    for (int j = lane; j < E; j += kWave) pa += expf(l[j] - lse) * (a_scale * (float)counts[j]);
    pa = wave_sum_f32(pa);
    const float zc = g_z * 2.f / (float)S * lse;
    float* g = dl + (int64_t)s * E;
    for (int j = lane; j < E; j += kWave) {
        const float p = expf(l[j] - lse);
        g[j] = g_aux * p * (a_scale * (float)counts[j] - pa) + zc * p;
    }
    // selected experts: w_r (dw_r - sum_r' w_r' dw_r'), added after the dense
    // terms by the lane that wrote them (same lane: j % 64)
    float wdw = 0.f;
    for (int r = 0; r < k; ++r) wdw += topk_w[(int64_t)s * k + r] * dw[(int64_t)s * k + r];
    for (int r = 0; r < k; ++r) {
        const int j = sel[r];
        if ((j & (kWave - 1)) == lane)
            g[j] += topk_w[(int64_t)s * k + r] * (dw[(int64_t)s * k + r] - wdw);
    }
}

// dWg and dbg from the chunked weight-gradient GEMM over [dl_hi | dl_lo]:
// part [nchunk][2E'][d] and bpart [nchunk][2E'] hold each token chunk's
// products with the hi and the lo plane; both planes of every chunk are
// added in chunk order (fixed, so the sums are deterministic).
__global__ __launch_bounds__(256) void router_dw_sum_kernel(const float* __restrict__ part,
                                                            const float* __restrict__ bpart,
                                                            int nchunk, int E, int Ep, int d,
                                                            float* __restrict__ dwg,
                                                            float* __restrict__ dbg) {
    // 64 four-column outputs per block (d is a multiple of 16); thread group
    // g of 4 adds chunks [g*nchunk/4, (g+1)*nchunk/4) in order, then group
    // 0 adds the four group sums in order
    __shared__ f32x4_t s_sum[4][64];
    const int g = threadIdx.x >> 6, o = threadIdx.x & 63;
    const int64_t i4 = (int64_t)blockIdx.x * 64 + o;
    const int64_t n4 = (int64_t)E * d / 4, slab = (int64_t)2 * Ep * d, lo = (int64_t)Ep * d;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (i4 < n4) {
        const int64_t i = 4 * i4;
        const int c_beg = g * nchunk / 4, c_end = (g + 1) * nchunk / 4;
        for (int c0 = c_beg; c0 < c_end; c0 += 4) {
            // the loads of four chunks first, then the additions in order
            f32x4_t v[8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u < c_end ? c0 + u : c_end - 1;
                v[2 * u] = *reinterpret_cast<const f32x4_t*>(part + c * slab + i);
                v[2 * u + 1] = *reinterpret_cast<const f32x4_t*>(part + c * slab + lo + i);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (c0 + u < c_end) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[q] += v[2 * u][q];
                        acc[q] += v[2 * u + 1][q];
                    }
                }
        }
    }
    s_sum[g][o] = acc;
    __syncthreads();
    if (g == 0 && i4 < n4) {
        f32x4_t t = s_sum[0][o];
#pragma unroll
        for (int u = 1; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] += s_sum[u][o][q];
        *reinterpret_cast<f32x4_t*>(dwg + 4 * i4) = t;
    }
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (dbg && j < E) {
        float a = 0.f;
        for (int c = 0; c < nchunk; ++c) {
            a += bpart[(int64_t)c * 2 * Ep + j];
            a += bpart[(int64_t)c * 2 * Ep + Ep + j];
        }
        dbg[j] = a;
    }
}

// n bytes, n even (every array here holds 2- or 4-byte elements).
__global__ void zero_bytes_kernel(uint32_t* __restrict__ p, size_t n) {
    const size_t words = n / 4;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
    if ((n & 2) && blockIdx.x == 0 && threadIdx.x == 0)
        reinterpret_cast<uint16_t*>(p)[2 * words] = 0u;
}

// Router gradients on the bf16 MFMAs: dl [S,E] and Wg [E,d] are fp32; with
// v = hi + lo (hi = bf16(v), lo = bf16(v - hi)) for both, dl Wg is taken as
// dl_hi W_hi + dl_lo W_hi + dl_hi W_lo (the dropped lo*lo term is 2^-16 of the
// product, far below the bf16 rounding of dx).  The three products become one
// GEMM over K = 3E' (E' = E rounded up to 64, zero padded):
//   A [S, 3E'] = [dl_hi | dl_lo | dl_hi],  B [3E', d] = [W_hi ; W_hi ; W_lo].
// The first 2E' columns of A also serve dWg = dl^T x = dl_hi^T x + dl_lo^T x
// (x is bf16, so that split is the only approximation).  count1 receives S
// (the one "expert" of the dx GEMM); occc the token count of each of the
// nchunk chunks of kc tokens that the dWg GEMM takes as its "experts"; ctr
// its 8 tile counters are zeroed.
__global__ void router_dx_split_kernel(const float* __restrict__ dl, const float* __restrict__ wg,
                                       int S, int E, int Ep, int d, bf16_t* __restrict__ a,
                                       bf16_t* __restrict__ b, int32_t* __restrict__ count1,
                                       int32_t* __restrict__ occc, int nchunk, int kc,
                                       int32_t* __restrict__ ctr) {
    const int64_t na = (int64_t)S * Ep, nb = (int64_t)Ep * d;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na + nb;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < na) {
            const int64_t s = i / Ep;
            const int j = (int)(i - s * Ep);
            const float v = j < E ? dl[s * E + j] : 0.f;
            const bf16_t hi = f32_to_bf16(v);
            const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
            bf16_t* row = a + s * 3 * Ep;
            row[j] = hi;
            row[Ep + j] = lo;
            row[2 * Ep + j] = hi;
        } else {
            const int64_t q = i - na;
            const int j = (int)(q / d), c = (int)(q - (int64_t)j * d);
            const float v = j < E ? wg[(int64_t)j * d + c] : 0.f;
            const bf16_t hi = f32_to_bf16(v);
            const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
            b[(int64_t)j * d + c] = hi;
            b[((int64_t)Ep + j) * d + c] = hi;
            b[((int64_t)2 * Ep + j) * d + c] = lo;
        }
    }
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) count1[0] = S;
        if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
        for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
            const int64_t left = (int64_t)S - (int64_t)c * kc;
            occc[c] = (int32_t)(left < kc ? left : kc);
        }
    }
}

// dx[s] = bf16(dxr[s] + sum over kept r of dX[u(s,r)]): one wave per token,
// fp32 sums in rank order.
__global__ __launch_bounds__(256) void dx_assemble_kernel(
    const u32x4_t* __restrict__ dxr, const u32x4_t* __restrict__ dX,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot,
    u32x4_t* __restrict__ dx, int S, int nvec, int k, int E, int stride, int limit) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(blockIdx.x * kTokPerBlock + wave);
    if (s >= S) return;
    int64_t u[kMaxK];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r)
        u[r] = r < k ? assignment_row(topk_idx, slot, (int64_t)s * k + r, E, stride, limit) : -1;
    for (int i = lane; i < nvec; i += kWave) {
        float acc[8];
        const u32x4_t v0 = dxr[(int64_t)s * nvec + i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __uint_as_float(v0[q] << 16);
            acc[2 * q + 1] = __uint_as_float(v0[q] & 0xffff0000u);
        }
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (u[r] >= 0) {
                const u32x4_t v = dX[u[r] * nvec + i];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += __uint_as_float(v[q] << 16);
                    acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
                }
            }
        }
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        dx[(int64_t)s * nvec + i] = o;
    }
}

}  // namespace

hipError_t launch_inverse_rows(const int32_t* topk_idx, const int32_t* slot, int S, int k,
                               int E, int stride, int limit, int32_t* inv, hipStream_t st) {
    const int64_t n = (int64_t)S * k;
    if (n == 0) return hipSuccess;
    inverse_rows_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(topk_idx, slot, S, k, E,
                                                                    stride, limit, inv);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* out, const int32_t* topk_idx,
                              const int32_t* slot, const float* topk_w, void* dO, float* dw,
                              int S, int d, int k, int E, int stride, int limit,
                              hipStream_t st) {
    if (S == 0) return hipSuccess;
    combine_bwd_kernel<<<(unsigned)ceil_div(S, kTokPerBlock), 256, 0, st>>>(
        static_cast<const u32x4_t*>(dy), static_cast<const u32x4_t*>(out), topk_idx, slot,
        topk_w, static_cast<u32x4_t*>(dO), dw, S, d / 8, k, E, stride, limit);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                             const float* dw, const int32_t* counts, float g_aux, float g_z,
                             float* dl, int S, int E, int k, bool topk_from_logits,
                             hipStream_t st) {
    if (S == 0) return hipSuccess;
    router_bwd_kernel<<<(unsigned)ceil_div(S, kTokPerBlock), 256, 0, st>>>(
        logits, topk_idx, topk_w, dw, counts, g_aux, g_z, dl, S, E, k, topk_from_logits);
    return hipGetLastError();
}

namespace {
// Token chunks of the dWg GEMM: about one output tile per compute unit, each
// chunk a multiple of 64 tokens and at least 256.
int router_dw_chunks(int S, int d, int E, int* kc) {
    const int Ep = (E + 63) / 64 * 64;
    const long long per = ceil_div(2 * Ep, 256) * ceil_div(d, 256);   // tiles per chunk
    long long n = ceil_div((long long)device_cus(), per);
    const long long most = ceil_div(S, 256);
    if (n > most) n = most;
    if (n < 1) n = 1;
    long long c = ceil_div(ceil_div(S, n), 64) * 64;
    if (c < 1) c = 64;
    *kc = (int)c;
    return (int)ceil_div(S, c);
}

// Workspace layout of the router gradients (byte offsets).
struct RouterWork {
    size_t A, B, dxr, tab, ctr, occc, ctr2, part, bpart, end;
};
RouterWork router_work(int S, int d, int E) {
    const size_t Ep = (size_t)(E + 63) / 64 * 64;
    int kc = 0;
    const size_t nchunk = S > 0 ? (size_t)router_dw_chunks(S, d, E, &kc) : 0;
    RouterWork w{};
    size_t o = 0;
    auto take = [&](size_t n) {
        const size_t at = o;
        o += (n + 255) & ~(size_t)255;
        return at;
    };
    w.A = take((size_t)S * 3 * Ep * 2);
    w.B = take(3 * Ep * (size_t)d * 2);
    w.dxr = take((size_t)S * d * 2);
    w.tab = take((2 + 1 + 2 + mtile_table_len(1, S, (size_t)S)) * 4);
    w.ctr = take(8 * 4);
    w.occc = take(nchunk * 4);
    w.ctr2 = take(8 * 4);
    w.part = take(nchunk * 2 * Ep * (size_t)d * 4);
    w.bpart = take(nchunk * 2 * Ep * 4);
    w.end = o;
    return w;
}
}  // namespace

size_t router_grads_workspace(int S, int d, int E) { return router_work(S, d, E).end; }

hipError_t launch_router_grads(const float* dl, const float* wg, const void* x, const void* dX,
                               const int32_t* topk_idx, const int32_t* slot, void* dx,
                               float* dwg, float* dbg, int S, int d, int E, int k, int stride,
                               int limit, void* work, hipStream_t st) {
    if (S == 0) return hipSuccess;
    const int Ep = (E + 63) / 64 * 64;
    int kc = 0;
    const int nchunk = router_dw_chunks(S, d, E, &kc);
    const RouterWork w = router_work(S, d, E);
    char* base = static_cast<char*>(work);
    bf16_t* A = reinterpret_cast<bf16_t*>(base + w.A);
    bf16_t* B = reinterpret_cast<bf16_t*>(base + w.B);
    void* dxr = base + w.dxr;
    int32_t* tab = reinterpret_cast<int32_t*>(base + w.tab);
    int32_t* ctr = reinterpret_cast<int32_t*>(base + w.ctr);
    int32_t* occc = reinterpret_cast<int32_t*>(base + w.occc);
    int32_t* ctr2 = reinterpret_cast<int32_t*>(base + w.ctr2);
    float* part = reinterpret_cast<float*>(base + w.part);
    float* bpart = reinterpret_cast<float*>(base + w.bpart);
    int32_t* count1 = tab;   // [1]
    int32_t* occ1 = tab + 1; // [1]
    int32_t* mt1 = tab + 2;  // [2] prefix, then the m-tile experts
    const int64_t n = (int64_t)S * Ep + (int64_t)Ep * d;
    const unsigned g = (unsigned)(ceil_div(n, 256) < 8192 ? ceil_div(n, 256) : 8192);
    router_dx_split_kernel<<<g, 256, 0, st>>>(dl, wg, S, E, Ep, d, A, B, count1, occc, nchunk, kc,
                                              ctr2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // dx: one "expert" of S rows, K = 3E'
    err = launch_occupancy(count1, 1, 1, S, 256, 0, occ1, mt1, nullptr, S, ctr, 8, st);
    if (err != hipSuccess) return err;
    BwdGemmParams b{};
    b.A = A;
    b.B = B;
    b.Cout = dxr;
    b.occ = occ1;
    b.mt_start = mt1;
    b.mt_expert = mt1 + 2;
    b.tile_ctr = ctr;
    b.E = 1;
    b.C = S;
    b.N = d;
    b.K = 3 * Ep;
    b.rows = (size_t)S;
    err = launch_bwd_gemm(b, false, false, st);
    if (err != hipSuccess) return err;
    dx_assemble_kernel<<<(unsigned)ceil_div(S, kTokPerBlock), 256, 0, st>>>(
        static_cast<const u32x4_t*>(dxr), static_cast<const u32x4_t*>(dX), topk_idx, slot,
        static_cast<u32x4_t*>(dx), S, d / 8, k, E, stride, limit);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // dWg: a weight gradient over token chunks ("experts" of kc rows), M = 2E'
    // ([dl_hi | dl_lo], rows 3E' apart), N = d, fp32 partials and column sums
    BwdGemmParams r{};
    r.A = A;
    r.lda = 3 * Ep;
    r.B = x;
    r.Cout = part;
    r.bias_grad = bpart;
    r.out_f32 = true;
    r.occ = occc;
    r.tile_ctr = ctr2;
    r.E = nchunk;
    r.C = kc;
    r.M = 2 * Ep;
    r.N = d;
    r.rows = (size_t)S;
    err = launch_bwd_gemm(r, true, false, st);
    if (err != hipSuccess) return err;
    const int64_t nblk = ceil_div((int64_t)E * d / 4, 64);
    router_dw_sum_kernel<<<(unsigned)(nblk * 256 >= E ? nblk : ceil_div(E, 256)), 256, 0, st>>>(
        part, bpart, nchunk, E, Ep, d, dwg, dbg);
    return hipGetLastError();
}

hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t st) {
    if (!p || n == 0) return hipSuccess;
    const size_t words = n / 4;
    const unsigned grid = (unsigned)(words / 256 + 1 < 4096 ? words / 256 + 1 : 4096);
    zero_bytes_kernel<<<grid, 256, 0, st>>>(static_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

}  // namespace moe
