// Router of the GShard MoE layer on gfx950: logits, softmax, top-k with
// renormalised weights, and the per-tile statistics that slot assignment and
// the losses are built from.
//
// Method: "GShard: Scaling Giant Neural Networks with Conditional Computation"
// (blog), section "Mixture-of-Experts Implementation": G(x) = Softmax(x . W_g)
// and the top-k experts of each token; "GShard: Scaling Giant Models with
// Conditional Computation and Automatic Sharding" (paper card), method
// paragraph: top-2 with softmax-normalised top-2 weights, aux loss
// N*sum_j f_j*P_j and a z-loss.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------
// Router logits, fp32 FMA.  Block tile 64 tokens x 64 experts, k-step 32;
// 256 threads, each owns a 4x4 grid of outputs strided by 16 so that LDS
// reads are conflict-free broadcasts.  Every output accumulates its d
// products in index order.
// ---------------------------------------------------------------------------
namespace {
constexpr int GL_BM = 64, GL_BN = 64, GL_BK = 32;

template <bool XBF16>
__global__ __launch_bounds__(256) void gate_logits_kernel(const void* __restrict__ xv,
                                                          const float* __restrict__ wg,
                                                          const float* __restrict__ bg,
                                                          float* __restrict__ logits, int S,
                                                          int d, int E) {
    __shared__ float As[GL_BK][GL_BM + 1];
    __shared__ float Bs[GL_BK][GL_BN + 1];
    const int tid = threadIdx.x;
    const int s0 = blockIdx.y * GL_BM;
    const int j0 = blockIdx.x * GL_BN;
    const int ty = tid / 16, tx = tid % 16;
    // loader mapping: 64 rows x 32 k per tile, 8 consecutive k per thread
    const int lrow = tid / 4, lk = (tid % 4) * 8;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < d; k0 += GL_BK) {
        float av[8], bv[8];
        const int gs = s0 + lrow, gj = j0 + lrow;
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = 0.f, bv[q] = 0.f;
        if (gs < S) {
            if (XBF16) {
                const bf16_t* xr = static_cast<const bf16_t*>(xv) + (size_t)gs * d;
                if (k0 + lk + 8 <= d) {
                    u32x4_t raw = *reinterpret_cast<const u32x4_t*>(xr + k0 + lk);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        av[2 * q] = __uint_as_float(raw[q] << 16);
                        av[2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
                    }
                } else {
                    for (int q = 0; q < 8; ++q)
                        if (k0 + lk + q < d) av[q] = bf16_to_f32(xr[k0 + lk + q]);
                }
            } else {
                const float* xr = static_cast<const float*>(xv) + (size_t)gs * d;
                for (int q = 0; q < 8; ++q)
                    if (k0 + lk + q < d) av[q] = xr[k0 + lk + q];
            }
        }
        if (gj < E) {
            const float* wr = wg + (size_t)gj * d;
            for (int q = 0; q < 8; ++q)
                if (k0 + lk + q < d) bv[q] = wr[k0 + lk + q];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            As[lk + q][lrow] = av[q];
            Bs[lk + q][lrow] = bv[q];
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < GL_BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = s0 + ty + 16 * i;
        if (s >= S) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = j0 + tx + 16 * j;
            if (e < E) logits[(size_t)s * E + e] = acc[i][j] + (bg ? bg[e] : 0.f);
        }
    }
}
}  // namespace

hipError_t launch_gate_logits(const void* x, bool x_bf16, const float* wg, const float* bg,
                              float* logits, int S, int d, int E, hipStream_t st) {
    dim3 grid((unsigned)ceil_div(E, GL_BN), (unsigned)ceil_div(S, GL_BM));
    if (x_bf16)
        gate_logits_kernel<true><<<grid, 256, 0, st>>>(x, wg, bg, logits, S, d, E);
    else
        gate_logits_kernel<false><<<grid, 256, 0, st>>>(x, wg, bg, logits, S, d, E);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route: one wavefront per token, 16 tokens per wave, 64 tokens per block
// (one routing tile).  Lane l holds the logits of experts l, l+64, ...
//
// Top-k uses a 64-bit key per logit: the order-preserving uint32 image of
// the fp32 value (with -0 folded onto +0) above the bitwise complement of
// the expert index, so one wave max-reduction yields the largest logit and,
// among equal logits, the lowest index.
//
// Refinement: the fp32 logit GEMM accumulates differently from an exactly
// rounded dot product.  When two consecutive values among the top k+1 lie
// within `tau` of each other, every logit within `tau` of the (k+1)-th is
// recomputed with fp64 accumulation, rounded once to fp32 and written back,
// and the selection is redone; no decision is then taken on a difference
// smaller than the GEMM's rounding error.
// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ float key_value(uint64_t key) {
    uint32_t u = static_cast<uint32_t>(key >> 32);
    uint32_t bits = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(bits);
}
__device__ __forceinline__ int key_index(uint64_t key) {
    return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key & 0xffffffffu));
}

template <int EQ>
__device__ __forceinline__ void select_topn(const float (&v)[EQ], int E, int lane, int n,
                                            uint64_t (&top)[kMaxK + 1]) {
    uint32_t taken = 0;
#pragma unroll
    for (int r = 0; r < kMaxK + 1; ++r) {
        if (r >= n) break;
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            if (j < E && !((taken >> q) & 1u)) {
                uint64_t key = (static_cast<uint64_t>(float_order_key(v[q])) << 32) |
                               (0xffffffffu - static_cast<uint32_t>(j));
                best = key > best ? key : best;
            }
        }
        best = wave_max_u64(best);
        top[r] = best;
        const int j = key_index(best);
        if ((j & (kWave - 1)) == lane) taken |= 1u << (j / kWave);
    }
}

template <int EQ>
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
    extern __shared__ unsigned char smem[];
    const int E = p.E, k = p.k, nb = p.nb;
    int* s_hist = reinterpret_cast<int*>(smem);                 // [k][E]
    float* s_p = reinterpret_cast<float*>(s_hist + k * E);      // [4][E]
    __shared__ float s_z[4];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int b = blockIdx.x;
    for (int i = tid; i < k * E; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();

    float pacc[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) pacc[q] = 0.f;
    float zacc = 0.f;
    const int nsel = k + 1 <= E ? k + 1 : E;

    for (int t = 0; t < kTokBlock / 4; ++t) {
        const int s = b * kTokBlock + wave * (kTokBlock / 4) + t;
        if (s >= p.S) break;
        float* lrow = p.logits + (size_t)s * E;
        float v[EQ];
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            v[q] = j < E ? lrow[j] : 0.f;
        }
        uint64_t top[kMaxK + 1];
        select_topn<EQ>(v, E, lane, nsel, top);

        if (p.tau > 0.f) {
            bool close = false;
            float last = key_value(top[0]);
#pragma unroll
            for (int r = 0; r < kMaxK; ++r) {
                if (r + 1 < nsel) {
                    close |= (key_value(top[r]) - key_value(top[r + 1])) < p.tau;
                    last = key_value(top[r + 1]);
                }
            }
            if (close) {
                const float thr = last - p.tau;
#pragma unroll
                for (int q = 0; q < EQ; ++q) {
                    const int jl = lane + kWave * q;
                    uint64_t cand = __ballot(jl < E && v[q] >= thr);
                    while (cand) {
                        const int cl = __ffsll(static_cast<long long>(cand)) - 1;
                        cand &= cand - 1;
                        const int j = cl + kWave * q;
                        const float* wr = p.wg + (size_t)j * p.d;
                        double acc = 0.0;
                        if (p.x_bf16) {
                            const bf16_t* xr = static_cast<const bf16_t*>(p.x) + (size_t)s * p.d;
                            for (int i = lane; i < p.d; i += kWave)
                                acc += (double)bf16_to_f32(xr[i]) * (double)wr[i];
                        } else {
                            const float* xr = static_cast<const float*>(p.x) + (size_t)s * p.d;
                            for (int i = lane; i < p.d; i += kWave)
                                acc += (double)xr[i] * (double)wr[i];
                        }
                        acc = wave_sum_f64(acc);
                        if (p.bg) acc += (double)p.bg[j];
                        const float nv = (float)acc;
                        if (lane == cl) {
                            v[q] = nv;
                            lrow[j] = nv;
                        }
                    }
                }
                select_topn<EQ>(v, E, lane, k, top);
            }
        }

        // softmax over all E logits, stabilised by the largest
        const float m = key_value(top[0]);
        float ev[EQ], part = 0.f;
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            ev[q] = j < E ? expf(v[q] - m) : 0.f;
            part += ev[q];
        }
        const float sum = wave_sum_f32(part);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int q = 0; q < EQ; ++q) pacc[q] += ev[q] * inv;
        const float lse = m + logf(sum);
        zacc += lse * lse;

        // renormalised top-k weights: p_r / sum_r' p_r' = e_r / sum_r' e_r'
        float den = 0.f;
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)
            if (r < k) den += expf(key_value(top[r]) - m);
        if (lane < k) {
            uint64_t mine = top[0];
#pragma unroll
            for (int r = 1; r < kMaxK; ++r)
                if (r == lane) mine = top[r];
            const int j = key_index(mine);
            p.topk_idx[(size_t)s * k + lane] = j;
            p.topk_w[(size_t)s * k + lane] = expf(key_value(mine) - m) / den;
            atomicAdd(&s_hist[lane * E + j], 1);
        }
    }

    // deterministic block reduction of the probability and lse^2 partials
#pragma unroll
    for (int q = 0; q < EQ; ++q) {
        const int j = lane + kWave * q;
        if (j < E) s_p[wave * E + j] = pacc[q];
    }
    if (lane == 0) s_z[wave] = zacc;
    __syncthreads();
    for (int j = tid; j < E; j += blockDim.x)
        p.ppart[(size_t)b * E + j] = ((s_p[j] + s_p[E + j]) + s_p[2 * E + j]) + s_p[3 * E + j];
    if (tid == 0) p.zpart[b] = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
    const int T = k * nb;
    for (int i = tid; i < k * E; i += blockDim.x) {
        const int r = i / E, e = i - r * E;
        p.hist[(size_t)e * T + (size_t)r * nb + b] = s_hist[i];
    }
}

template <int EQ>
hipError_t launch_route_t(const RouteParams& p, hipStream_t st) {
    const size_t lds = sizeof(int) * (size_t)p.k * p.E + sizeof(float) * 4 * (size_t)p.E;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<EQ>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    route_kernel<EQ><<<p.nb, 256, lds, st>>>(p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
    const int eq = (int)ceil_div(p.E, kWave);
    if (eq <= 1) return launch_route_t<1>(p, st);
    if (eq <= 2) return launch_route_t<2>(p, st);
    if (eq <= 4) return launch_route_t<4>(p, st);
    if (eq <= 8) return launch_route_t<8>(p, st);
    if (eq <= 16) return launch_route_t<16>(p, st);
    return launch_route_t<32>(p, st);
}

}  // namespace moe
