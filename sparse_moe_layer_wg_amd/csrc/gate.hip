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

__global__ __launch_bounds__(256) void gate_logits_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          const float* __restrict__ bg,
                                                          float* __restrict__ logits,
                                                          float* __restrict__ xn2,
                                                          float* __restrict__ wn2, int S,
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
    float xsq = 0.f, wsq = 0.f;   // this thread's share of the row norms

    for (int k0 = 0; k0 < d; k0 += GL_BK) {
        float av[8], bv[8];
        const int gs = s0 + lrow, gj = j0 + lrow;
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = 0.f, bv[q] = 0.f;
        if (gs < S) {
            const float* xr = x + (size_t)gs * d;
            for (int q = 0; q < 8; ++q)
                if (k0 + lk + q < d) av[q] = xr[k0 + lk + q];
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
            xsq = fmaf(av[q], av[q], xsq);
            wsq = fmaf(bv[q], bv[q], wsq);
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
    // row norms: the 4 loader threads of a row (consecutive lanes) add their
    // shares; x from the first expert tile's blocks, wg from the first token
    // tile's
    xsq += __shfl_xor(xsq, 1);
    xsq += __shfl_xor(xsq, 2);
    wsq += __shfl_xor(wsq, 1);
    wsq += __shfl_xor(wsq, 2);
    if ((tid & 3) == 0) {
        if (xn2 && blockIdx.x == 0 && s0 + lrow < S) xn2[s0 + lrow] = xsq;
        if (wn2 && blockIdx.y == 0 && j0 + lrow < E) wn2[j0 + lrow] = wsq;
    }
}
}  // namespace

// ---------------------------------------------------------------------------
// Router logits for bf16 activations on the MFMA units.  Each fp32 router
// weight is split exactly into three bf16 terms, w = hi + lo1 + lo2 (hi is w
// rounded to bf16, lo1 the rounded remainder, lo2 what is left; 3 x 8
// significand bits cover fp32's 24), in registers as the weight tile is
// staged into LDS (three planes).  A bf16 x bf16 product is exact in fp32,
// so x . w = x . hi + x . (lo1 + lo2) with fp32 accumulation throughout:
// v_mfma_f32_32x32x16_bf16 accumulates x . hi in one accumulator and the two
// small terms in another, which are added (with the bias) at the end.
// Block tile 128 tokens x 64 experts x 64 k, 8 waves (4 x 2) of 32 x 32; the
// taller tile reads each weight tile once for 128 tokens, half the weight
// traffic from L2 per MFMA of a 64-token tile (measured faster at every
// shape; no single unit is saturated: matrix pipes busy a quarter to a third
// of the time, the texture path a quarter, L2 hit rate 70-80%).
// Operands are staged through registers into two LDS buffers (x and the
// three weight planes, XOR-swizzled by row), with the global loads two
// k-tiles ahead; the fp32 weights are read once per block, 32 bytes per
// thread per k-tile.  Rows past S or E load a clamped valid row and are
// never stored.
namespace {
constexpr int GM_BM = 128, GM_BN = 64, GM_BK = 64, GM_CH = GM_BK / 8, GM_NT = 512;
// k-tiles of global loads in flight (register slots).  Two: 114 VGPRs, so two
// 512-thread blocks still share a CU; three need 137 and leave one.
constexpr int GM_PF = 2;

__device__ __forceinline__ int gm_swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

// Exact three-way bf16 split of 8 fp32 weights into three chunks of 8 bf16:
// hi = bf16(w), lo1 = bf16(w - hi), lo2 = w - hi - lo1 (exact in bf16).
__device__ __forceinline__ void split3(const f32x4_t& w0, const f32x4_t& w1, u32x4_t& hi,
                                       u32x4_t& lo1, u32x4_t& lo2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // weights 2q, 2q+1, two at a time through the packed conversion
        const float a = q < 2 ? w0[2 * q] : w1[2 * q - 4];
        const float b = q < 2 ? w0[2 * q + 1] : w1[2 * q - 3];
        const uint32_t h = pack_bf16x2(a, b);
        const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xffff0000u);
        const uint32_t m = pack_bf16x2(ra, rb);
        hi[q] = h;
        lo1[q] = m;
        lo2[q] = pack_bf16x2(ra - __uint_as_float(m << 16), rb - __uint_as_float(m & 0xffff0000u));
    }
}

__global__ __launch_bounds__(GM_NT, 1) void gate_logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                                  const float* __restrict__ wg,
                                                                  const float* __restrict__ bg,
                                                                  float* __restrict__ logits,
                                                                  float* __restrict__ xn2,
                                                                  float* __restrict__ wn2,
                                                                  int S, int d, int E) {
    // stage: A [128][8 chunks], then three weight planes [64][8 chunks]
    constexpr int A_SZ = GM_BM * GM_CH, B_SZ = GM_BN * GM_CH, STAGE = A_SZ + 3 * B_SZ;
    __shared__ u32x4_t smem[2 * STAGE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int s0 = blockIdx.x * GM_BM, j0 = blockIdx.y * GM_BN;

    // loader: x chunks c = tid + GM_NT*i (i < 2) and 8 consecutive fp32
    // weights, c = tid: row c/8, k 8*(c%8) .. +7, one chunk of each plane
    constexpr int XI = GM_BM * GM_CH / GM_NT;
    static_assert(GM_BN * GM_CH == GM_NT, "one weight-plane chunk per thread");
    const bf16_t* xa[XI];
    int ald[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int c = tid + GM_NT * i, row = c >> 3, ch = c & 7;
        xa[i] = x + (size_t)min(s0 + row, S - 1) * d + ch * 8;
        ald[i] = row * GM_CH + gm_swz(row, ch);
    }
    const float* wb;
    int bld;
    {
        const int row = tid >> 3, ch = tid & 7;
        wb = wg + (size_t)min(j0 + row, E - 1) * d + ch * 8;
        bld = A_SZ + row * GM_CH + gm_swz(row, ch);
    }
    // the loads of k-tile t sit in register slot t % GM_PF until staged
    u32x4_t rx[GM_PF][XI];
    f32x4_t rw[GM_PF][2];
    // this thread's shares of the squared row norms (x rows tid/8 + 64 i,
    // router row tid/8), added as the chunks are staged by the blocks that
    // store them: x by the first expert tile, wg by the first token tile
    const bool xnorm = xn2 && blockIdx.y == 0, wnorm = wn2 && blockIdx.x == 0;
    float xsq[XI], wsq = 0.f;
#pragma unroll
    for (int i = 0; i < XI; ++i) xsq[i] = 0.f;
    auto gload = [&](int k0, int sl) {
#pragma unroll
        for (int i = 0; i < XI; ++i) rx[sl][i] = *reinterpret_cast<const u32x4_t*>(xa[i] + k0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            rw[sl][q] = *reinterpret_cast<const f32x4_t*>(wb + k0 + 4 * q);
    };
    auto sstore = [&](int buf, int sl) {
        u32x4_t* st = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            st[ald[i]] = rx[sl][i];
            if (xnorm) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __uint_as_float(rx[sl][i][q] << 16);
                    const float hi = __uint_as_float(rx[sl][i][q] & 0xffff0000u);
                    xsq[i] = fmaf(lo, lo, fmaf(hi, hi, xsq[i]));
                }
            }
        }
        if (wnorm) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) wsq = fmaf(rw[sl][q][u], rw[sl][q][u], wsq);
        }
        u32x4_t hi, lo1, lo2;
        split3(rw[sl][0], rw[sl][1], hi, lo1, lo2);
        st[bld] = hi;
        st[bld + B_SZ] = lo1;
        st[bld + 2 * B_SZ] = lo2;
    };

    f32x16_t acc_hi, acc_lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_hi[r] = 0.f, acc_lo[r] = 0.f;
    const int frow = lane & 31, fhalf = lane >> 5;
    const int KT = d / GM_BK;
#pragma unroll
    for (int t = 0; t < GM_PF; ++t) gload(min(t, KT - 1) * GM_BK, t);
    sstore(0, 0);
    __syncthreads();
    // k-tile kt: the loads of k-tile kt+GM_PF go into the slot k-tile kt has
    // left (staged to LDS at the end of the previous k-tile), and k-tile kt+1
    // is staged at the end, its loads having had a whole k-tile more to
    // land.  The loads are issued on every k-tile (past the end: the last
    // k-tile again, never used), so that the compiler's wait before a slot is
    // read leaves the same number of later loads in flight on every path; a
    // conditional issue made it wait for all of them (a full vmcnt(0)).  The
    // loop is unrolled by GM_PF so that the slots are static registers.
    // (Two-deep against one: 4-11% faster, logits bit-identical.)
    for (int kb = 0; kb < KT; kb += GM_PF)
#pragma unroll
    for (int u = 0; u < GM_PF; ++u) {
        const int kt = kb + u;
        if (kt >= KT) break;
        const int buf = kt & 1;
        gload(min(kt + GM_PF, KT - 1) * GM_BK, u);
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
        if (kt + 1 < KT) sstore(buf ^ 1, (u + 1) % GM_PF);
        __syncthreads();
    }
    // row norms: the 8 loader threads of a row (consecutive lanes) add their
    // shares; x from the first expert tile's blocks, wg from the first token
    // tile's
#pragma unroll
    for (int m = 1; m < GM_CH; m <<= 1) {
#pragma unroll
        for (int i = 0; i < XI; ++i) xsq[i] += __shfl_xor(xsq[i], m);
        wsq += __shfl_xor(wsq, m);
    }
    if ((tid & (GM_CH - 1)) == 0) {
        if (xnorm) {
#pragma unroll
            for (int i = 0; i < XI; ++i) {
                const int row = (tid + GM_NT * i) / GM_CH;
                if (s0 + row < S) xn2[s0 + row] = xsq[i];
            }
        }
        if (wnorm && j0 + tid / GM_CH < E) wn2[j0 + tid / GM_CH] = wsq;
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
                              float* logits, float* xn2, float* wn2, int S, int d, int E,
                              hipStream_t st) {
    if (x_bf16) {
        // bf16 layers have d a multiple of 64 (checked when the layer is planned)
        if (d % GM_BK != 0) return hipErrorInvalidValue;
        dim3 grid((unsigned)ceil_div(S, GM_BM), (unsigned)ceil_div(E, GM_BN));
        gate_logits_mfma_kernel<<<grid, GM_NT, 0, st>>>(static_cast<const bf16_t*>(x), wg, bg,
                                                        logits, xn2, wn2, S, d, E);
    } else {
        dim3 grid((unsigned)ceil_div(E, GL_BN), (unsigned)ceil_div(S, GL_BM));
        gate_logits_kernel<<<grid, 256, 0, st>>>(static_cast<const float*>(x), wg, bg, logits,
                                                 xn2, wn2, S, d, E);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route.  For E <= 256, route_fast_kernel gives each token 1 to 8 lanes and
// hands only near-tie tokens to the wave router below.  Otherwise (and
// for those tokens) one wavefront routes one token at a time; a block of 16
// waves (4 when E > 512) owns one 64-token routing tile.  Lane l holds the
// logits of experts l, l+64, ...
//
// Top-k uses a 64-bit key per logit: the order-preserving uint32 image of
// the fp32 value (with -0 folded onto +0) above the bitwise complement of
// the expert index, so one wave max-reduction yields the largest logit and,
// among equal logits, the lowest index.
//
// Refinement: the logit GEMM accumulates in fp32, so its values can differ
// by a few ulps from exactly rounded dot products.  The ordered top-k depends
// only on the comparisons between sorted neighbours r, r+1 for r < k.  When
// such a pair differs by less than the token's margin tau (well above the
// GEMM's error, and scaled with the token's magnitudes: margin_scale), the
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
// once to fp32.  Lanes take 8-element (bf16) or 4-element (fp32) chunks.  A
// slot without an expert (js[u] < 0) reads the first expert's row and its
// sum is dropped, so every load of a chunk is issued before the chunk's
// products (and four chunks' loads are in flight): the loop is bound by
// memory latency, not by the arithmetic.
__device__ __forceinline__ void refine_group(const RouteParams& p, int s, const int (&js)[4],
                                             float (&nv)[4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const float* wr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        wr[u] = p.wg + (size_t)__builtin_amdgcn_readfirstlane(js[u] >= 0 ? js[u] : js[0]) * p.d;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (p.x_bf16) {
        const bf16_t* xr = static_cast<const bf16_t*>(p.x) + (size_t)s * p.d;
#pragma unroll 4
        for (int i = lane * 8; i < p.d; i += kWave * 8) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(xr + i);
            f32x4_t w0[4], w1[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                w0[u] = *reinterpret_cast<const f32x4_t*>(wr[u] + i);
                w1[u] = *reinterpret_cast<const f32x4_t*>(wr[u] + i + 4);
            }
            float xv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[2 * q] = __uint_as_float(raw[q] << 16);
                xv[2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[u] += (double)xv[q] * (double)w0[u][q];
                    acc[u] += (double)xv[4 + q] * (double)w1[u][q];
                }
        }
    } else {
        const float* xr = static_cast<const float*>(p.x) + (size_t)s * p.d;
#pragma unroll 4
        for (int i = lane * 4; i < p.d; i += kWave * 4) {
            const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xr + i);
            f32x4_t w0[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w0[u] = *reinterpret_cast<const f32x4_t*>(wr[u] + i);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u] += (double)xv[q] * (double)w0[u][q];
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
        // a select per register (a guarded store lets the compiler index v
        // dynamically, which moves it to scratch memory)
#pragma unroll
        for (int q = 0; q < EQ; ++q) v[q] = q == (j >> 6) ? nv[u] : v[q];
        lrow[j] = nv[u];
    }
}

// Scale of the refinement margin, computed by every wave for itself (all 64
// lanes active): wmax = max_j |wg[j,:]| and bmax = max_j |bg[j]|.  Token s
// then refines a top-k decision closer than p.tau * (|x[s,:]| wmax + bmax/8).
// By Cauchy-Schwarz |x_s . w_j| <= |x_s| |w_j|: the first term follows the
// magnitude of the partial sums whose fp32 roundings make the logit GEMM's
// error, whatever the scale of x and Wg; the second covers the single
// rounding of the bias addition (a quarter ulp of the bias at p.tau = 32 ulp
// of 1.0).
struct MarginScale {
    float wmax, bmax;
};
__device__ __forceinline__ MarginScale margin_scale(const RouteParams& p, int lane) {
    MarginScale m{0.f, 0.f};
    if (p.tau > 0.f) {
        float w = 0.f, b = 0.f;
        for (int j = lane; j < p.E; j += kWave) {
            w = fmaxf(w, p.wn2[j]);
            if (p.bg) b = fmaxf(b, fabsf(p.bg[j]));
        }
        m.wmax = sqrtf(wave_max_nonneg_f32(w));
        m.bmax = wave_max_nonneg_f32(b);
    }
    return m;
}
__device__ __forceinline__ float token_margin(const RouteParams& p, const MarginScale& m, int s) {
    return p.tau > 0.f ? p.tau * (sqrtf(p.xn2[s]) * m.wmax + 0.125f * m.bmax) : 0.f;
}

// Routes token s with the whole wave (lane l holds experts l, l+64, ...):
// top-k with near-tie refinement, softmax, renormalised weights, outputs and
// the histogram; adds the token's probabilities to pacc and lse^2 to zacc.
// s_cand: kMaxSel ints of LDS private to this wave.
template <int EQ>
// lds_row: NULL (the logits are read from p.logits), or the token's raw
// logits in LDS, which are read and then zeroed; tau_in: the token's margin
// when already known (>= 0), else computed here; seed: NULL, or the token's
// k+1 largest keys already sorted (LDS), which then replace the first k+1
// selections.
__device__ void route_token_wave(const RouteParams& p, const MarginScale& ms, int s, int lane,
                                 int* s_hist, int* s_cand, float (&pacc)[EQ], float& zacc,
                                 float* lds_row, float tau_in, const uint64_t* seed) {
    const int E = p.E, k = p.k;
    const int nsel = k + 1 <= E ? k + 1 : E;
    float* lrow = p.logits + (size_t)s * E;
    float v[EQ];
    // two loops, not one pointer chosen between LDS and global memory (that
    // makes generic flat loads, which wait on both counters)
    if (lds_row) {
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            v[q] = j < E ? lds_row[j] : 0.f;
            if (j < E) lds_row[j] = 0.f;
        }
    } else {
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
            const int j = lane + kWave * q;
            v[q] = j < E ? lrow[j] : 0.f;
        }
    }
    // The sorted keys live one per lane: lane r holds the key of the r-th
    // largest logit (r < n), so the close pairs come from one ballot and no
    // array of keys sits in scalar registers.
    uint64_t kl = 0;
    uint32_t taken = 0;
    uint64_t top0 = 0;
    float v_prev = 0.f, v_last = 0.f;   // values of the last two keys taken
    if (seed) {
        // the same keys in the same order as the selections below would take
        // them: lane r keeps key r, and each listed expert's owner lane marks
        // it taken
#pragma unroll 1
        for (int r = 0; r < nsel; ++r) {
            const uint64_t key = seed[r];
            if (lane == r) kl = key;
            const int j = key_index(key);
            if ((j & (kWave - 1)) == lane) taken |= 1u << (j / kWave);
        }
        top0 = seed[0];
        v_last = key_value(seed[nsel - 1]);
        v_prev = nsel >= 2 ? key_value(seed[nsel - 2]) : 0.f;
    } else {
#pragma unroll 1
        for (int r = 0; r < nsel; ++r) {
            const uint64_t key = select_next<EQ>(v, E, lane, taken);
            if (lane == r) kl = key;
            if (r == 0) top0 = key;
            v_prev = v_last;
            v_last = key_value(key);
        }
    }

    const float tau = tau_in >= 0.f ? tau_in : token_margin(p, ms, s);
    if (tau > 0.f && nsel > 1) {
        // Pair r joins sorted positions r and r+1 and is "close" when their
        // difference is below tau.  Pairs r < k decide the ordered top-k.
        auto close_pairs = [&](int n) {
            const float vl = key_value(kl);
            const float vn = __shfl_down(vl, 1);
            return static_cast<uint32_t>(__ballot(lane + 1 < n && vl - vn < tau));
        };
        uint32_t closebits = close_pairs(nsel);
        if (closebits & ((1u << k) - 1u)) {
            // follow a chain of close pairs past position k
            int n = nsel;
#pragma unroll 1
            while (n < kMaxSel && n < E && v_prev - v_last < tau) {
                const uint64_t key = select_next<EQ>(v, E, lane, taken);
                if (lane == n) kl = key;
                v_prev = v_last;
                v_last = key_value(key);
                ++n;
            }
            const bool overflow = n == kMaxSel && n < E && v_prev - v_last < tau;
            int ncand = 0;
            if (!overflow) {
                // members of the close chains that contain a pair r < k
                closebits = close_pairs(n);
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
                // their experts, in sorted order
                if (lane < kMaxSel && ((members >> lane) & 1u))
                    s_cand[__popc(members & ((1u << lane) - 1u))] = key_index(kl);
                ncand = __popc(members);
            }
            // a chain longer than kMaxSel: refine every logit of the token
            const int total = overflow ? E : ncand;
            for (int g = 0; g < total; g += 4) {
                int js[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    js[u] = g + u < total ? (overflow ? g + u : s_cand[g + u]) : -1;
                float nv[4];
                refine_group(p, s, js, nv);
                apply_refined<EQ>(v, lrow, js, nv, lane);
            }
            taken = 0;
            kl = 0;
#pragma unroll 1
            for (int r = 0; r < k; ++r) {
                const uint64_t key = select_next<EQ>(v, E, lane, taken);
                if (lane == r) kl = key;
                if (r == 0) top0 = key;
            }
        }
    }

    // softmax over all E logits, stabilised by the largest
    const float m = key_value(top0);
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
    // (summed in rank order; lane r holds the r-th key)
    float den = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r)
        if (r < k) den += expf(key_value(readlane_u64(kl, r)) - m);
    if (lane < k) {
        const int j = key_index(kl);
        p.topk_idx[(size_t)s * k + lane] = j;
        p.topk_w[(size_t)s * k + lane] = expf(key_value(kl) - m) / den;
        atomicAdd(&s_hist[lane * E + j], 1);
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
    const MarginScale ms = margin_scale(p, lane);
    for (int i = tid; i < k * E; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();

    float pacc[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) pacc[q] = 0.f;
    float zacc = 0.f;

    for (int t = 0; t < kTokBlock / NW; ++t) {
        const int s = b * kTokBlock + wave * (kTokBlock / NW) + t;
        if (s >= p.S) break;
        route_token_wave<EQ>(p, ms, s, lane, s_hist, s_cand[wave], pacc, zacc, nullptr, -1.f,
                             nullptr);
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

// Fast route for E <= 32*L (L = 1, 2, 4 or 8): one block per 64-token tile
// with L lanes per token (64*L threads).  Lane l of a token holds the
// logits of experts 4*(l + L*i) + u (i < 8, u < 4), keeps its own top-K1
// (K1 >= k+1) in registers sorted by (logit descending, index ascending),
// and the token's lanes merge their lists with shuffles.  A token whose
// top-k has a near tie (a sorted pair r < k closer than tau) is routed
// afterwards by route_token_wave, which refines and decides it exactly as
// route_kernel does; it contributes nothing to the fast pass.  Per-expert
// probability sums run through LDS in token order, so the partials stay
// deterministic.
template <int L, int K1>
__global__ __launch_bounds__(64 * L) void route_fast_kernel(RouteParams p) {
    constexpr int NT = 64 * L, EQ = (L + 1) / 2;   // threads; wave-router experts per lane
    extern __shared__ unsigned char smem[];
    const int E = p.E, k = p.k, nb = p.nb;
    const int EP = E + 4;                                        // padded row of s_pt
    int* s_hist = reinterpret_cast<int*>(smem);                  // [k][E]
    float* s_pt = reinterpret_cast<float*>(s_hist + k * E);      // [64][EP] probabilities
    float* s_slow = s_pt + kTokBlock * EP;                       // [L][E] slow-path sums
    __shared__ float s_lse2[kTokBlock], s_z[L], s_tau[kTokBlock];
    __shared__ int s_flag[kTokBlock], s_list[kTokBlock], s_nlist;
    __shared__ int s_cand[L][kMaxSel];
    __shared__ uint64_t s_seed[kTokBlock][K1];                  // flagged tokens' top keys

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = tid / L, l = tid % L;                          // token of the tile, part
    const int b = blockIdx.x;
    const int s = b * kTokBlock + t;
    const bool live = s < p.S;
    // this lane's logits (16-byte loads when every row is 16-byte aligned),
    // issued first so that their latency covers the set-up below
    float v[32];
    const float* lrow = p.logits + (size_t)(live ? s : 0) * E;
    const bool vec = (E & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j0 = 4 * (l + L * i);
        if (vec && live && j0 + 3 < E) {
            const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(lrow + j0);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[4 * i + u] = q4[u];
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[4 * i + u] = live && j0 + u < E ? lrow[j0 + u] : 0.f;
        }
    }
    const MarginScale ms = margin_scale(p, lane);
    for (int i = tid; i < k * E; i += NT) s_hist[i] = 0;
    // Local top-K1.  Experts are visited in decreasing index order, so a new
    // entry has a lower index than every listed one and an entry carried down
    // sorted above its neighbours: ">=" on the key alone orders by (key
    // descending, index ascending).  Padding experts (key 0) fill the list
    // first and are displaced by any real logit.
    const int nsel = k + 1 <= E ? k + 1 : E;
    uint32_t tk[K1];
    int ti[K1];
#pragma unroll
    for (int r = 0; r < K1; ++r) {
        tk[r] = 0u;
        ti[r] = 0x7fffffff;
    }
#pragma unroll
    for (int i = 7; i >= 0; --i)
#pragma unroll
        for (int u = 3; u >= 0; --u) {
            const int j = 4 * (l + L * i) + u;
            uint32_t key = j < E ? float_order_key(v[4 * i + u]) : 0u;
            int idx = j;
#pragma unroll
            for (int r = 0; r < K1; ++r) {
                const bool gt = key >= tk[r];
                const uint32_t kk = gt ? tk[r] : key;
                const int ii = gt ? ti[r] : idx;
                tk[r] = gt ? key : tk[r];
                ti[r] = gt ? idx : ti[r];
                key = kk;
                idx = ii;
            }
        }
    // merge the token's L lists: nsel rounds of a group maximum
    uint32_t gk[K1];
    int gi[K1];
#pragma unroll
    for (int r = 0; r < K1; ++r) {
        gk[r] = 0u;
        gi[r] = 0x7fffffff;
        if (r < nsel) {
            uint32_t bk = tk[0];
            int bi = ti[0];
#pragma unroll
            for (int m = 1; m < L; m <<= 1) {
                const uint32_t ok = __shfl_xor(bk, m);
                const int oi = __shfl_xor(bi, m);
                const bool take = ok > bk || (ok == bk && oi < bi);
                bk = take ? ok : bk;
                bi = take ? oi : bi;
            }
            gk[r] = bk;
            gi[r] = bi;
            if (ti[0] == bi) {   // this lane owned it: pop its head
#pragma unroll
                for (int q = 0; q + 1 < K1; ++q) {
                    tk[q] = tk[q + 1];
                    ti[q] = ti[q + 1];
                }
                tk[K1 - 1] = 0u;
                ti[K1 - 1] = 0x7fffffff;
            }
        }
    }
    auto kval = [](uint32_t u) {
        return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
    };
    bool flag = false;
    const float tau = live ? token_margin(p, ms, s) : 0.f;
    if (tau > 0.f && nsel > 1) {
#pragma unroll
        for (int r = 0; r + 1 < K1; ++r)
            if (r < k && r + 1 < nsel) flag |= kval(gk[r]) - kval(gk[r + 1]) < tau;
    }
    const bool fast = live && !flag;
    // a flagged token's raw logits, margin and sorted top k+1 keys go to LDS
    // for the wave router (its probability row is written there only by
    // that router, as zeros)
    if (live && flag && l == 0) {
#pragma unroll
        for (int r = 0; r < K1; ++r)
            if (r < nsel)
                s_seed[t][r] = (static_cast<uint64_t>(gk[r]) << 32) |
                               (0xffffffffu - static_cast<uint32_t>(gi[r]));
    }
    if (live && flag) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = 4 * (l + L * i) + u;
                if (j < E) s_pt[t * EP + j] = v[4 * i + u];
            }
    }
    if (l == 0) s_tau[t] = tau;

    // softmax over the token's E logits, stabilised by the largest
    // (__expf: the hardware exp2 of x*log2(e), within ~2e-6 relative here)
    const float m = kval(gk[0]);
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * (l + L * i) + u;
            v[4 * i + u] = j < E ? __expf(v[4 * i + u] - m) : 0.f;
            part += v[4 * i + u];
        }
#pragma unroll
    for (int msk = 1; msk < L; msk <<= 1) part += __shfl_xor(part, msk);
    const float inv = 1.0f / part;
    // probabilities of this token to its LDS row (zeros unless fast)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * (l + L * i) + u;
            if (j < E && !(live && flag)) s_pt[t * EP + j] = fast ? v[4 * i + u] * inv : 0.f;
        }
    if (l == 0) {
        const float lse = m + logf(part);
        s_lse2[t] = fast ? lse * lse : 0.f;
        s_flag[t] = live && flag;
    }
    __syncthreads();   // s_hist cleared; rows and flags written
    if (fast) {
        // renormalised top-k weights: p_r / sum_r' p_r' = e_r / sum_r' e_r'
        float den = 0.f;
#pragma unroll
        for (int r = 0; r + 1 < K1; ++r)
            if (r < k) den += __expf(kval(gk[r]) - m);
#pragma unroll
        for (int r = 0; r + 1 < K1; ++r) {
            if (r < k && r % L == l) {
                p.topk_idx[(size_t)s * k + r] = gi[r];
                p.topk_w[(size_t)s * k + r] = __expf(kval(gk[r]) - m) / den;
                atomicAdd(&s_hist[r * E + gi[r]], 1);
            }
        }
    }
    // flagged tokens, in token order, go to the wave router
    if (wave == 0) {
        const bool f = s_flag[lane] != 0;
        const uint64_t bal = __ballot(f);
        if (f) s_list[__popcll(bal & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) s_nlist = __popcll(bal);
    }
    __syncthreads();
    float pacc[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) pacc[q] = 0.f;
    float zacc = 0.f;
    const int nl = s_nlist;
    for (int f = wave; f < nl; f += L)
        route_token_wave<EQ>(p, ms, b * kTokBlock + s_list[f], lane, s_hist, s_cand[wave], pacc,
                             zacc, s_pt + s_list[f] * EP, s_tau[s_list[f]], s_seed[s_list[f]]);
#pragma unroll
    for (int q = 0; q < EQ; ++q) {
        const int j = lane + 64 * q;
        if (j < E) s_slow[wave * E + j] = pacc[q];
    }
    if (lane == 0) s_z[wave] = zacc;
    __syncthreads();

    // deterministic partials: fast tokens in a fixed order, then the waves'
    for (int j = tid; j < E; j += NT) {
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int q = 0; q < kTokBlock; q += 4)
#pragma unroll
            for (int u = 0; u < 4; ++u) a4[u] += s_pt[(q + u) * EP + j];
        float a = (a4[0] + a4[1]) + (a4[2] + a4[3]);
#pragma unroll
        for (int w = 0; w < L; ++w) a += s_slow[w * E + j];
        p.ppart[(size_t)b * E + j] = a;
    }
    if (wave == 0) {
        float a = wave_sum_f32(s_lse2[lane]);
        if (lane == 0) {
#pragma unroll
            for (int w = 0; w < L; ++w) a += s_z[w];
            p.zpart[b] = a;
        }
    }
    const int T = k * nb;
    for (int i = tid; i < k * E; i += NT) {
        const int r = i / E, e = i - r * E;
        p.hist[(size_t)e * T + (size_t)r * nb + b] = s_hist[i];
    }
}

template <int L, int K1>
hipError_t launch_route_fast_t(const RouteParams& p, hipStream_t st) {
    const size_t lds = sizeof(int) * (size_t)p.k * p.E +
                       sizeof(float) * ((size_t)kTokBlock * (p.E + 4) + (size_t)L * p.E);
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_fast_kernel<L, K1>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    route_fast_kernel<L, K1><<<p.nb, 64 * L, lds, st>>>(p);
    return hipGetLastError();
}
template <int L>
hipError_t launch_route_fast_k(const RouteParams& p, hipStream_t st) {
    if (p.k <= 2) return launch_route_fast_t<L, 3>(p, st);
    if (p.k <= 4) return launch_route_fast_t<L, 5>(p, st);
    return launch_route_fast_t<L, kMaxK + 1>(p, st);
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
    const int lanes = (int)ceil_div(p.E, 32);   // fast route: 32 logits per lane
    if (lanes <= 1) return launch_route_fast_k<1>(p, st);
    if (lanes <= 2) return launch_route_fast_k<2>(p, st);
    if (lanes <= 4) return launch_route_fast_k<4>(p, st);
    if (lanes <= 8) return launch_route_fast_k<8>(p, st);
    if (eq <= 1) return launch_route_t<1, 16>(p, st);
    if (eq <= 2) return launch_route_t<2, 16>(p, st);
    if (eq <= 4) return launch_route_t<4, 16>(p, st);
    if (eq <= 8) return launch_route_t<8, 16>(p, st);
    if (eq <= 16) return launch_route_t<16, 4>(p, st);
    return launch_route_t<32, 4>(p, st);
}

}  // namespace moe
