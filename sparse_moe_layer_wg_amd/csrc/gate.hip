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
// Router logits, fp32 FMA (fp32 activations).  Block tile 64 tokens x 64 experts, k-step 32;
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

// ---------------------------------------------------------------------------
// Router logits for bf16 activations on the MFMA units.  Each fp32 router
// weight is split exactly into three bf16 terms, w = hi + lo1 + lo2 (hi is w
// rounded to bf16, lo1 the rounded remainder, lo2 what is left; 3 x 8
// significand bits cover fp32's 24).  A bf16 x bf16 product is exact in fp32,
// so x . w = x . hi + x . (lo1 + lo2) with fp32 accumulation throughout:
// v_mfma_f32_32x32x16_bf16 accumulates x . hi in one accumulator and the two
// small terms in another, which are added (with the bias) at the end.
// Block tile 64 tokens x 64 experts x 64 k, 4 waves of 32 x 32; operands are
// staged through registers into two LDS buffers (x as is, the weight as three
// bf16 planes, XOR-swizzled by row like the expert GEMMs).  Rows past S or E
// load a clamped valid row and are never stored.
namespace {
constexpr int GM_BM = 64, GM_BN = 64, GM_BK = 64, GM_CH = GM_BK / 8;

__device__ __forceinline__ int gm_swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

// Exact three-way bf16 split of 8 fp32 values into three 16-byte chunks.
__device__ __forceinline__ void split3(const f32x4_t& a, const f32x4_t& b, u32x4_t& hi,
                                       u32x4_t& l1, u32x4_t& l2) {
    float w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    bf16_t h[8], m[8], t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16(w[i]);
        const float r1 = w[i] - bf16_to_f32(h[i]);
        m[i] = f32_to_bf16(r1);
        t[i] = f32_to_bf16(r1 - bf16_to_f32(m[i]));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        hi[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
        l1[q] = (uint32_t)m[2 * q] | ((uint32_t)m[2 * q + 1] << 16);
        l2[q] = (uint32_t)t[2 * q] | ((uint32_t)t[2 * q + 1] << 16);
    }
}

__global__ __launch_bounds__(256, 2) void gate_logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                                  const float* __restrict__ wg,
                                                                  const float* __restrict__ bg,
                                                                  float* __restrict__ logits,
                                                                  int S, int d, int E) {
    // stage: A [64][8 chunks], then three weight planes [64][8 chunks]
    constexpr int A_SZ = GM_BM * GM_CH, B_SZ = GM_BN * GM_CH, STAGE = A_SZ + 3 * B_SZ;
    __shared__ u32x4_t smem[2 * STAGE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int s0 = blockIdx.x * GM_BM, j0 = blockIdx.y * GM_BN;

    // loader: x chunks c = tid + 256*i (i < 2): row c/8, chunk c%8;
    // weight chunk-pairs c = tid + 256*i (i < 2): row c/8, k chunk c%8
    // (two float4 = 8 consecutive k, split into three bf16 chunks)
    const bf16_t* xa[2];
    const float* wb[2];
    int ald[2], bld[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
        xa[i] = x + (size_t)min(s0 + row, S - 1) * d + ch * 8;
        wb[i] = wg + (size_t)min(j0 + row, E - 1) * d + ch * 8;
        ald[i] = row * GM_CH + gm_swz(row, ch);
        bld[i] = A_SZ + row * GM_CH + gm_swz(row, ch);
    }
    u32x4_t rx[2];
    f32x4_t rw[2][2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            rx[i] = *reinterpret_cast<const u32x4_t*>(xa[i] + k0);
            rw[i][0] = *reinterpret_cast<const f32x4_t*>(wb[i] + k0);
            rw[i][1] = *reinterpret_cast<const f32x4_t*>(wb[i] + k0 + 4);
        }
    };
    auto sstore = [&](int buf) {
        u32x4_t* st = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            st[ald[i]] = rx[i];
            u32x4_t h, l1, l2;
            split3(rw[i][0], rw[i][1], h, l1, l2);
            st[bld[i]] = h;
            st[bld[i] + B_SZ] = l1;
            st[bld[i] + 2 * B_SZ] = l2;
        }
    };

    f32x16_t acc_hi, acc_lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_hi[r] = 0.f, acc_lo[r] = 0.f;
    const int frow = lane & 31, fhalf = lane >> 5;
    const int KT = d / GM_BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * GM_BK);
        const u32x4_t* st = smem + buf * STAGE;
#pragma unroll
        for (int ks = 0; ks < GM_BK / 16; ++ks) {
            const int c = 2 * ks + fhalf;
            const int ra = wm * 32 + frow, rb = wn * 32 + frow;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, st[ra * GM_CH + gm_swz(ra, c)]);
            const int bo = A_SZ + rb * GM_CH + gm_swz(rb, c);
            const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, st[bo]);
            const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, st[bo + B_SZ]);
            const bf16x8_t b2 = __builtin_bit_cast(bf16x8_t, st[bo + 2 * B_SZ]);
            acc_hi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc_hi, 0, 0, 0);
            acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc_lo, 0, 0, 0);
            acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b2, acc_lo, 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }
    // 32x32 accumulator layout: lane l holds column l%32, register r row
    // 8*(r/4) + 4*(l/32) + r%4.
    const int j = j0 + wn * 32 + frow;
    if (j < E) {
        const float bj = bg ? bg[j] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int s = s0 + wm * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
            if (s < S) logits[(size_t)s * E + j] = (acc_hi[r] + acc_lo[r]) + bj;
        }
    }
}
}  // namespace

hipError_t launch_gate_logits(const void* x, bool x_bf16, const float* wg, const float* bg,
                              float* logits, int S, int d, int E, hipStream_t st) {
    if (x_bf16 && d % GM_BK == 0) {
        dim3 grid((unsigned)ceil_div(S, GM_BM), (unsigned)ceil_div(E, GM_BN));
        gate_logits_mfma_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), wg, bg,
                                                      logits, S, d, E);
    } else {
        dim3 grid((unsigned)ceil_div(E, GL_BN), (unsigned)ceil_div(S, GL_BM));
        if (x_bf16)
            gate_logits_kernel<true><<<grid, 256, 0, st>>>(x, wg, bg, logits, S, d, E);
        else
            gate_logits_kernel<false><<<grid, 256, 0, st>>>(x, wg, bg, logits, S, d, E);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route: one wavefront per token at a time; a block of 16 waves (4 when
// E > 512) owns one 64-token routing tile.  Lane l holds the logits of
// experts l, l+64, ...
//
// Top-k uses a 64-bit key per logit: the order-preserving uint32 image of
// the fp32 value (with -0 folded onto +0) above the bitwise complement of
// the expert index, so one wave max-reduction yields the largest logit and,
// among equal logits, the lowest index.
//
// Refinement: the logit GEMM accumulates in fp32, so its values can differ
// by a few ulps from exactly rounded dot products.  The ordered top-k depends
// only on the comparisons between sorted neighbours r, r+1 for r < k.  When
// such a pair differs by less than `tau` (well above the GEMM's error), the
// chain of sorted neighbours linked by differences below tau is recomputed
// with fp64 accumulation, rounded once to fp32 (the stored logits are
// overwritten) and the selection is redone.  Experts outside the chain differ
// from it by at least tau, so their order against it is already certain.
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

constexpr int kMaxSel = 16;  // sorted positions examined for near-tie clusters

// Next-largest key among the experts not yet taken (wave-uniform result);
// marks it taken in the owner lane's bitmask.
template <int EQ>
__device__ __forceinline__ uint64_t select_next(const float (&v)[EQ], int E, int lane,
                                                uint32_t& taken) {
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
    // every lane holds the same key: keep it in scalar registers
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(best >> 32));
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(best));
    best = (static_cast<uint64_t>(hi) << 32) | lo;
    const int j = key_index(best);
    if ((j & (kWave - 1)) == lane) taken |= 1u << (j / kWave);
    return best;
}

// fp64 dot products x[s,:] . wg[j_u,:] (+ bg) for up to four experts, rounded
// once to fp32.  Lanes take 8-element (bf16) or 4-element (fp32) chunks.
__device__ __forceinline__ void refine_group(const RouteParams& p, int s, const int (&js)[4],
                                             float (&nv)[4]) {
    const int lane = threadIdx.x & (kWave - 1);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (p.x_bf16) {
        const bf16_t* xr = static_cast<const bf16_t*>(p.x) + (size_t)s * p.d;
#pragma unroll 1
        for (int i = lane * 8; i < p.d; i += kWave * 8) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(xr + i);
            float xv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[2 * q] = __uint_as_float(raw[q] << 16);
                xv[2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (js[u] < 0) continue;
                const f32x4_t* wr = reinterpret_cast<const f32x4_t*>(p.wg + (size_t)js[u] * p.d + i);
                const f32x4_t w0 = wr[0], w1 = wr[1];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[u] += (double)xv[q] * (double)w0[q];
                    acc[u] += (double)xv[4 + q] * (double)w1[q];
                }
            }
        }
    } else {
        const float* xr = static_cast<const float*>(p.x) + (size_t)s * p.d;
#pragma unroll 1
        for (int i = lane * 4; i < p.d; i += kWave * 4) {
            const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xr + i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (js[u] < 0) continue;
                const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(p.wg + (size_t)js[u] * p.d + i);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u] += (double)xv[q] * (double)w0[q];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        double t = wave_sum_f64(acc[u]);
        if (js[u] >= 0 && p.bg) t += (double)p.bg[js[u]];
        nv[u] = (float)t;
    }
}

// Replaces the logits of experts js[u] by nv[u]: in the owner lane's
// registers and in the stored logits row.
template <int EQ>
__device__ __forceinline__ void apply_refined(float (&v)[EQ], float* lrow, const int (&js)[4],
                                              const float (&nv)[4], int lane) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = js[u];
        if (j < 0 || (j & (kWave - 1)) != lane) continue;
#pragma unroll
        for (int q = 0; q < EQ; ++q)
            if (q == (j >> 6)) v[q] = nv[u];
        lrow[j] = nv[u];
    }
}

// NW waves per block share one 64-token routing tile, 64/NW tokens each.
template <int EQ, int NW>
__global__ __launch_bounds__(NW * 64) void route_kernel(RouteParams p) {
    extern __shared__ unsigned char smem[];
    const int E = p.E, k = p.k, nb = p.nb;
    int* s_hist = reinterpret_cast<int*>(smem);                 // [k][E]
    float* s_p = reinterpret_cast<float*>(s_hist + k * E);      // [NW][E]
    __shared__ float s_z[NW];
    __shared__ int s_cand[NW][kMaxSel];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int b = blockIdx.x;
    for (int i = tid; i < k * E; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();

    float pacc[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) pacc[q] = 0.f;
    float zacc = 0.f;
    const int nsel = k + 1 <= E ? k + 1 : E;

    for (int t = 0; t < kTokBlock / NW; ++t) {
        const int s = b * kTokBlock + wave * (kTokBlock / NW) + t;
        if (s >= p.S) break;
        float* lrow = p.logits + (size_t)s * E;
        float v[EQ];
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            v[q] = j < E ? lrow[j] : 0.f;
        }
        // top[r]: key of the r-th largest logit (wave-uniform)
        uint64_t top[kMaxSel];
        uint32_t taken = 0;
#pragma unroll
        for (int r = 0; r < kMaxK + 1; ++r)
            if (r < nsel) top[r] = select_next<EQ>(v, E, lane, taken);

        if (p.tau > 0.f && nsel > 1) {
            // Pair r joins sorted positions r and r+1 and is "close" when their
            // difference is below tau.  Pairs r < k decide the ordered top-k.
            bool need = false;
#pragma unroll
            for (int r = 0; r < kMaxK; ++r)
                if (r < k && r + 1 < nsel)
                    need |= key_value(top[r]) - key_value(top[r + 1]) < p.tau;
            if (need) {
                // follow a chain of close pairs past position k
                int n = nsel;
#pragma unroll
                for (int r = 2; r < kMaxSel; ++r) {
                    if (r == n && n < E && key_value(top[r - 2]) - key_value(top[r - 1]) < p.tau) {
                        top[r] = select_next<EQ>(v, E, lane, taken);
                        ++n;
                    }
                }
                const bool overflow =
                    n == kMaxSel && n < E &&
                    key_value(top[kMaxSel - 2]) - key_value(top[kMaxSel - 1]) < p.tau;
                int ncand = 0;
                if (!overflow) {
                    // members of the close chains that contain a pair r < k
                    uint32_t closebits = 0;
#pragma unroll
                    for (int r = 0; r + 1 < kMaxSel; ++r)
                        if (r + 1 < n && key_value(top[r]) - key_value(top[r + 1]) < p.tau)
                            closebits |= 1u << r;
                    uint32_t members = 0;
                    int r = 0;
                    while (r + 1 < n) {
                        if (!((closebits >> r) & 1u)) {
                            ++r;
                            continue;
                        }
                        const int a = r;
                        while (r + 1 < n && ((closebits >> r) & 1u)) ++r;
                        if (a < k) members |= ((2u << r) - 1u) & ~((1u << a) - 1u);
                    }
#pragma unroll
                    for (int q = 0; q < kMaxSel; ++q) {
                        if ((members >> q) & 1u) {
                            s_cand[wave][ncand] = key_index(top[q]);
                            ++ncand;
                        }
                    }
                }
                // a chain longer than kMaxSel: refine every logit of the token
                const int total = overflow ? E : ncand;
                for (int g = 0; g < total; g += 4) {
                    int js[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        js[u] = g + u < total ? (overflow ? g + u : s_cand[wave][g + u]) : -1;
                    float nv[4];
                    refine_group(p, s, js, nv);
                    apply_refined<EQ>(v, lrow, js, nv, lane);
                }
                taken = 0;
#pragma unroll
                for (int r = 0; r < kMaxK; ++r)
                    if (r < k) top[r] = select_next<EQ>(v, E, lane, taken);
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
    for (int j = tid; j < E; j += blockDim.x) {
        float a = s_p[j];
#pragma unroll
        for (int w = 1; w < NW; ++w) a += s_p[w * E + j];
        p.ppart[(size_t)b * E + j] = a;
    }
    if (tid == 0) {
        float a = s_z[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) a += s_z[w];
        p.zpart[b] = a;
    }
    const int T = k * nb;
    for (int i = tid; i < k * E; i += blockDim.x) {
        const int r = i / E, e = i - r * E;
        p.hist[(size_t)e * T + (size_t)r * nb + b] = s_hist[i];
    }
}

template <int EQ, int NW>
hipError_t launch_route_t(const RouteParams& p, hipStream_t st) {
    const size_t lds = sizeof(int) * (size_t)p.k * p.E + sizeof(float) * NW * (size_t)p.E;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<EQ, NW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    route_kernel<EQ, NW><<<p.nb, NW * 64, lds, st>>>(p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
    const int eq = (int)ceil_div(p.E, kWave);
    if (eq <= 1) return launch_route_t<1, 16>(p, st);
    if (eq <= 2) return launch_route_t<2, 16>(p, st);
    if (eq <= 4) return launch_route_t<4, 16>(p, st);
    if (eq <= 8) return launch_route_t<8, 16>(p, st);
    if (eq <= 16) return launch_route_t<16, 4>(p, st);
    return launch_route_t<32, 4>(p, st);
}

}  // namespace moe
