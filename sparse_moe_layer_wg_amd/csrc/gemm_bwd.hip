// Expert GEMMs of the backward pass: data gradients (dgrad) and weight
// gradients (wgrad) over the same variable-occupancy expert rows as the
// forward.
//
// Method: the layer's expert networks are feed-forward networks ("GShard:
// Scaling Giant Neural Networks with Conditional Computation" (blog), section
// "Core Components", "Expert Networks"), trained with the layer ("GShard:
// Scaling Giant Models with Conditional Computation and Automatic Sharding"
// (paper card), method paragraph).  With O = ReLU(X W1^T + b1) W2^T + b2 per
// expert, the chain rule gives, per expert e over its filled rows:
//   dgrad 2:  dU = (dO . W2_e) * [H > 0]      [rows,d] x [d,h]   (K = d)
//   dgrad 1:  dX = dU . W1_e                  [rows,h] x [h,d]   (K = h)
//   wgrad 2:  dW2_e = dO^T . H                [d,rows] x [rows,h] (K = rows)
//   wgrad 1:  dW1_e = dU^T . X                [h,rows] x [rows,d] (K = rows)
// In the forward both MFMA operands are stored with K contiguous.  Here the
// weights of a dgrad and both operands of a wgrad are stored with K as the
// slow index ("K-major": W2_e is [d,h] and dgrad 2 contracts over d).  Such an
// operand is loaded as 8 K-rows x 4 columns per thread (8-byte loads, a
// wave covering 256 contiguous columns of each K-row), transposed in
// registers and written to LDS as K-contiguous rows, the layout the MFMA
// fragments read.  The rest follows the forward kernel: 256x256x64 tiles,
// 8 waves of 128x64, v_mfma_f32_32x32x16_bf16 with fp32 accumulation, two LDS
// stages, the epilogue staged through LDS into 16-byte row stores, and a
// persistent grid that takes tiles from per-XCD atomic counters.
//   dgrad tiles follow the forward's m-tile list (ragged rows, weights fixed);
//   rows past an expert's occupancy load a clamped valid row and are never
//   stored.  dgrad 2 applies the ReLU mask in its row stores (reading H at
//   the same place; dU may overwrite H in place).
//   wgrad tiles cover each expert's full [M,N] weight gradient; the
//   contraction runs over the expert's filled rows (K = occ[e], any length,
//   zero included: the tile then stores zeros); rows past the occupancy
//   load as zero.  X rows may be gathered from the token rows through the
//   inverse slot map.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTH = 512;                     // 8 waves: 2 (m) x 4 (n)
constexpr int WM = 128, WNT = 64;            // wave tile
constexpr int TM = WM / 32, TN = WNT / 32;   // 32x32 MFMA blocks per wave
constexpr int RS = BK * 2 + 16;              // LDS row stride (bytes, padded)
constexpr int BOFF = BM * RS;                // B rows after the A rows
constexpr int STAGE = (BM + BN) * RS;
constexpr int EPS = WNT * 2 + 8;             // epilogue staging row (bytes)
static_assert(NTH / 64 * WM * EPS <= 2 * STAGE, "epilogue staging fits LDS");

// One column of 8 K-rows x 4 bf16 columns as 8 K values (a 16-byte LDS row
// chunk): column col of v[r] is half (col & 1) of word (col >> 1).
__device__ __forceinline__ u32x4_t column8(const uint2 (&v)[8], bool hi_word, uint32_t sel) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t a = hi_word ? v[2 * q].y : v[2 * q].x;
        const uint32_t b = hi_word ? v[2 * q + 1].y : v[2 * q + 1].x;
        o[q] = __builtin_amdgcn_perm(b, a, sel);  // low half: K-row 2q, high: 2q+1
    }
    return o;
}

// K-major operand store: lane l holds columns 4l..4l+3 of 8 K-rows and writes
// each column as a 16-byte chunk of LDS row 4l + col.  Rows 4 apart are 576
// bytes apart, a multiple of the bank width, so writing column c in every
// lane at once would put 16 lanes on the same banks.  Store c instead writes
// column (c + l/2) % 4: each group of 8 lanes (128 bytes, written together)
// then covers every bank once; with (c + l/4) % 4 two lanes of a group still
// shared banks (SQ_LDS_BANK_CONFLICT 1.2-1.9e7 cycles per launch, now 0).
struct KMajorStore {
    int off[4];        // LDS byte offset of store c (row and K chunk)
    uint32_t sel[4];   // byte selector of the column's half
    bool hi[4];        // column in the upper word
    __device__ KMajorStore(int lane, int wave, int rs) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int col = (c + (lane >> 1)) & 3;
            off[c] = (4 * lane + col) * rs + wave * 16;
            sel[c] = (col & 1) ? 0x07060302u : 0x05040100u;
            hi[c] = (col >> 1) != 0;
        }
    }
    __device__ __forceinline__ void store(char* base, const uint2 (&v)[8]) const {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4_t*>(base + off[c]) = column8(v, hi[c], sel[c]);
    }
};

// One output tile: expert, origin, rows (M), k-tiles and the expert's
// first row; ca/cb: this lane's first column of the K-major pieces (clamped
// into range; clamped columns are never stored).
struct BwdTile {
    int e, m0, n0, M, KT, Keff, ca, cb;
    size_t row_e;
    uint32_t aoff[4];  // dgrad: byte offsets of this thread's A chunks from
                       // the expert's first row (rows clamped to the filled ones)
};

template <bool WGRAD>
__device__ __forceinline__ BwdTile decode_tile(const BwdGemmParams& p, int t, int MT, int NT,
                                               int lane) {
    BwdTile u;
    if constexpr (WGRAD) {
        u.e = t / (MT * NT);
        const int r = t - u.e * MT * NT;
        u.m0 = (r / NT) * BM;
        u.n0 = (r % NT) * BN;
        u.M = p.M;
        u.Keff = __builtin_amdgcn_readfirstlane(p.occ[u.e]);
        u.KT = (u.Keff + BK - 1) / BK;
    } else {
        const int q = t / NT;
        u.e = __builtin_amdgcn_readfirstlane(p.mt_expert[q]);
        const int mt0 = __builtin_amdgcn_readfirstlane(p.mt_start[u.e]);
        u.m0 = (q - mt0) * BM;
        u.n0 = (t - q * NT) * BN;
        u.M = __builtin_amdgcn_readfirstlane(p.occ[u.e]);
        u.Keff = p.K;
        u.KT = p.K / BK;
    }
    u.row_e = p.row0 ? (size_t)__builtin_amdgcn_readfirstlane(p.row0[u.e]) : (size_t)u.e * p.C;
    u.ca = WGRAD ? min(u.m0 + 4 * lane, u.M - 4) : 0;
    u.cb = min(u.n0 + 4 * lane, p.N - 4);
    if constexpr (!WGRAD) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rg = min(u.m0 + (tid >> 3) + 64 * i, u.M - 1);
            u.aoff[i] = (uint32_t)rg * (uint32_t)p.K * 2u + (uint32_t)(tid & 7) * 16u;
        }
    }
    return u;
}

// OUTF32 (weight gradients only): Cout and bias_grad in fp32, stored
// straight from the accumulators (four consecutive columns per lane and
// register quad), and A rows p.lda elements apart.
template <bool WGRAD, bool MASK, bool OUTF32>
__global__ __launch_bounds__(NTH, 1) void gemm_bwd_kernel(BwdGemmParams p) {
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
    __shared__ float s_bias[WGRAD ? NTH / 64 : 1][WGRAD ? BM : 1];
    __shared__ int s_next;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4;
    const int frow = lane & 31, fhalf = lane >> 5;
    const int N = p.N;
    const int NT = (N + BN - 1) / BN;
    const int MT = WGRAD ? (p.M + BM - 1) / BM : 0;
    const int T = WGRAD ? p.E * MT * NT : p.mt_start[p.E] * NT;
    const int per = (T + 7) >> 3;
    const int xcd = blockIdx.x & 7;
    const int t_end = min(T, (xcd + 1) * per);

    const int fa_off = (wm * WM + frow) * RS + fhalf * 16;
    const int fb_off = BOFF + (wn * WNT + frow) * RS + fhalf * 16;
    // K-contiguous loader (dgrad A): row tid/8 + 64*i, 16-byte chunk tid%8
    const int r_off = (tid >> 3) * RS + (tid & 7) * 16;
    // K-major loader: K-rows 8*wave .. 8*wave+7, columns 4*lane .. 4*lane+3
    const KMajorStore kst(lane, wave, RS);
    u32x4_t ra[4];       // dgrad A: 4 K-contiguous 16-byte chunks
    uint2 va[8], vb[8];  // K-major operands: 8 K-rows x 4 columns
    // Loads address a wave-uniform row base (scalar registers) plus a 32-bit
    // per-lane byte offset, so that each K-row costs no vector registers.
    const char* __restrict__ Ac = reinterpret_cast<const char*>(p.A);
    const char* __restrict__ Bc = reinterpret_cast<const char*>(p.B);
    auto gload = [&](const BwdTile& u, int kt) {
        const int kb = kt * BK;
        if constexpr (WGRAD) {
            // rows past the occupancy load as zero
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int k = kb + 8 * wave + r;
                va[r] = make_uint2(0u, 0u);
                vb[r] = make_uint2(0u, 0u);
                if (k < u.Keff) {   // wave-uniform
                    const size_t ar = u.row_e + k;
                    const size_t br =
                        p.b_rows ? (size_t)__builtin_amdgcn_readfirstlane(p.b_rows[ar]) : ar;
                    const size_t lda = OUTF32 && p.lda > 0 ? (size_t)p.lda : (size_t)u.M;
                    va[r] = *reinterpret_cast<const uint2*>(Ac + ar * lda * 2 +
                                                            (uint32_t)u.ca * 2u);
                    vb[r] = *reinterpret_cast<const uint2*>(Bc + br * N * 2 +
                                                            (uint32_t)u.cb * 2u);
                }
            }
        } else {
            const char* Ak = Ac + (u.row_e * p.K + kb) * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ra[i] = *reinterpret_cast<const u32x4_t*>(Ak + u.aoff[i]);
            const char* Wk = Bc + ((size_t)u.e * p.K + kb + 8 * wave) * N * 2;
            const uint32_t ob = (uint32_t)u.cb * 2u;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                vb[r] = *reinterpret_cast<const uint2*>(Wk + (size_t)r * N * 2 + ob);
        }
    };
    auto sstore = [&](int buf) {
        char* st = smem + buf * STAGE;
        if constexpr (WGRAD) {
            kst.store(st, va);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4_t*>(st + r_off + i * 64 * RS) = ra[i];
        }
        kst.store(st + BOFF, vb);
    };

    // Tiles of this XCD's chunk come from an atomic counter.  The tile after
    // the current one is claimed when the current one starts, so that the
    // loads of its first k-tile can be issued before the current epilogue
    // (a weight-gradient tile has only occ/64 k-tiles: its first load and its
    // epilogue would otherwise both sit exposed).
    if (tid == 0) s_next = xcd * per + atomicAdd(&p.tile_ctr[xcd], 1);
    __syncthreads();
    int t = __builtin_amdgcn_readfirstlane(s_next);
    BwdTile cur{};
    if (t < t_end) {
        cur = decode_tile<WGRAD>(p, t, MT, NT, lane);
        if (cur.KT > 0) gload(cur, 0);
    }
    while (t < t_end) {
        __syncthreads();   // the previous epilogue's LDS reads are done
        if (tid == 0) s_next = xcd * per + atomicAdd(&p.tile_ctr[xcd], 1);
        // bias gradient (weight gradients, first n-tile): column sums of A
        const bool bias = WGRAD && p.bias_grad && cur.n0 == 0;
        float csum[4] = {0.f, 0.f, 0.f, 0.f};
        auto add_bias = [&]() {
            if (bias) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    csum[0] += __uint_as_float(va[r].x << 16);
                    csum[1] += __uint_as_float(va[r].x & 0xffff0000u);
                    csum[2] += __uint_as_float(va[r].y << 16);
                    csum[3] += __uint_as_float(va[r].y & 0xffff0000u);
                }
            }
        };

        // ---------------------------------------------------------- k-loop
        f32x16_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        if (cur.KT > 0) {
            add_bias();
            sstore(0);
        }
        __syncthreads();   // stage 0 filled; s_next visible to every wave

        // One k-tile from LDS buffer kt&1, as in the forward kernel: with
        // REFILL, k-tile kt+1 is loaded into registers during the first
        // 16-wide step and transposed into the other buffer during the last;
        // the fragments of step ks+1 are read while the MFMAs of step ks run.
        // Instruction groups keep memory and VALU work spread over the MFMAs
        // (a wave issues in order).
        bf16x8_t fa[2][TM], fb[2][TN];
        auto load_frags = [&](const char* st, int ks, int slot) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[slot][i] = *reinterpret_cast<const bf16x8_t*>(st + fa_off + i * 32 * RS + ks * 32);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[slot][j] = *reinterpret_cast<const bf16x8_t*>(st + fb_off + j * 32 * RS + ks * 32);
        };
        auto ktile = [&](auto refill_tag, int kt) {
            constexpr bool REFILL = decltype(refill_tag)::value;
            constexpr int KS = BK / 16;
            constexpr int NL = WGRAD ? 16 : 12;    // global loads per thread
            constexpr int NW = WGRAD ? 8 : 8;      // LDS stores per thread
            constexpr int NF = TM + TN;            // fragment reads per step
            constexpr int NM = TM * TN;            // MFMAs per step
            const char* st = smem + (kt & 1) * STAGE;
            load_frags(st, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (REFILL) {
                    if (ks == 0) gload(cur, kt + 1);
                    if (ks == KS - 1) {
                        add_bias();
                        sstore((kt + 1) & 1);
                    }
                }
                if (ks + 1 < KS) load_frags(st, ks + 1, (ks + 1) & 1);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
                if (REFILL && ks == 0) {
#pragma unroll
                    for (int g = 0; g < NM; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x020, NL / NM, 0);  // VMEM read
                        if (g < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
                    }
                } else if (REFILL && ks == KS - 1) {
#pragma unroll
                    for (int g = 0; g < NM; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);      // VALU
                        __builtin_amdgcn_sched_group_barrier(0x200, NW / NM, 0); // LDS write
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
                    }
                } else if (ks + 1 < KS) {
#pragma unroll
                    for (int g = 0; g < NF; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
                        __builtin_amdgcn_sched_group_barrier(0x008, NM / NF, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
        };
        if constexpr (WGRAD) {
            // A weight-gradient tile runs only occ/64 k-tiles; there the plain
            // loop (loads first, transposes and stores after the MFMAs) measured
            // faster than the interleaved one.
            for (int kt = 0; kt < cur.KT; ++kt) {
                const bool more = kt + 1 < cur.KT;
                if (more) gload(cur, kt + 1);
                const char* st = smem + (kt & 1) * STAGE;
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    load_frags(st, ks, 0);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
                }
                if (more) {
                    add_bias();
                    sstore((kt + 1) & 1);
                }
                __syncthreads();
            }
        } else {
            int kt = 0;
            for (; kt + 1 < cur.KT; ++kt) ktile(std::true_type{}, kt);
            if (kt < cur.KT) ktile(std::false_type{}, kt);
        }

        // next tile: decode it and start loading its first k-tile
        const int tn = __builtin_amdgcn_readfirstlane(s_next);
        BwdTile nxt{};
        if (tn < t_end) {
            nxt = decode_tile<WGRAD>(p, tn, MT, NT, lane);
            if (nxt.KT > 0) gload(nxt, 0);
        }

        // ---------------------------------------------------------- epilogue
        // Accumulator block (n x m): lane l holds row m = l%32, register r
        // column n = 8*(r/4) + 4*(l/32) + r%4.  Rounded to bf16, staged per
        // wave in LDS, stored as 16-byte row chunks.
        if (bias) {
            // column sums: each wave covered its 8 of every 64 K-rows
#pragma unroll
            for (int c = 0; c < 4; ++c) s_bias[wave][4 * lane + c] = csum[c];
        }
        if constexpr (OUTF32) {
            float* __restrict__ Cf = static_cast<float*>(p.Cout) + (size_t)cur.e * p.M * N;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = cur.m0 + wm * WM + i * 32 + frow;
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = cur.n0 + wn * WNT + j * 32 + 8 * q + 4 * fhalf;
                        if (m < cur.M && n < N) {
                            f32x4_t v;
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
                            *reinterpret_cast<f32x4_t*>(Cf + (size_t)m * N + n) = v;
                        }
                    }
            }
        } else {
            char* ep = smem + wave * (WM * EPS);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = j * 32 + 8 * q + 4 * fhalf;
                        const f32x16_t& a = acc[i][j];
                        *reinterpret_cast<uint2*>(ep + (i * 32 + frow) * EPS + nl * 2) =
                            make_uint2(pack_bf16x2(a[4 * q], a[4 * q + 1]),
                                       pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
                    }
            __builtin_amdgcn_wave_barrier();
            constexpr int CPR = WNT * 2 / 16;   // 16-byte chunks per staged row
            constexpr int NIT = WM * CPR / 64;  // chunks per lane
            const int nw = cur.n0 + wn * WNT;
            bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.Cout) +
                                        (WGRAD ? (size_t)cur.e * p.M * N : cur.row_e * N);
            const bf16_t* __restrict__ mk =
                MASK ? static_cast<const bf16_t*>(p.mask) + cur.row_e * N : nullptr;
            // the mask chunks of all of this lane's rows are loaded together
            // (rows and columns clamped into range; unused ones are never
            // applied), so their latency is paid once per tile, not per row;
            // each chunk is read before this lane overwrites it (dU may
            // replace H in place)
            u32x4_t hvs[MASK ? NIT : 1];
            if constexpr (MASK) {
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int row = it * (64 / CPR) + lane / CPR, ch = lane % CPR;
                    const int m = min(cur.m0 + wm * WM + row, cur.M - 1);
                    const int n = min(nw + ch * 8, N - 8);
                    hvs[it] = *reinterpret_cast<const u32x4_t*>(mk + (size_t)m * N + n);
                }
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int row = it * (64 / CPR) + lane / CPR, ch = lane % CPR;
                const int m = cur.m0 + wm * WM + row, n = nw + ch * 8;
                u32x4_t ov = *reinterpret_cast<const u32x4_t*>(ep + row * EPS + ch * 16);
                if (m < cur.M && n < N) {
                    if constexpr (MASK) {
                        // dReLU: keep the gradient where the forward's hidden
                        // value is positive (bf16 > 0: sign clear, not zero)
                        const u32x4_t hv = hvs[it];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint32_t hlo = hv[c] & 0xffffu, hhi = hv[c] >> 16;
                            const uint32_t keep = ((hlo != 0u && hlo < 0x8000u) ? 0xffffu : 0u) |
                                                  ((hhi != 0u && hhi < 0x8000u) ? 0xffff0000u : 0u);
                            ov[c] &= keep;
                        }
                    }
                    *reinterpret_cast<u32x4_t*>(Cout + (size_t)m * N + n) = ov;
                }
            }
        }
        if (bias) {
            __syncthreads();
            if (tid < BM && cur.m0 + tid < cur.M) {
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < NTH / 64; ++w) v += s_bias[w][tid];
                if constexpr (OUTF32)
                    static_cast<float*>(p.bias_grad)[(size_t)cur.e * cur.M + cur.m0 + tid] = v;
                else
                    static_cast<bf16_t*>(p.bias_grad)[(size_t)cur.e * cur.M + cur.m0 + tid] =
                        f32_to_bf16(v);
            }
        }
        t = tn;
        cur = nxt;
    }  // tile loop
}

}  // namespace

hipError_t launch_bwd_gemm(const BwdGemmParams& p, bool wgrad, bool mask, hipStream_t st) {
    if (p.E == 0 || p.N == 0) return hipSuccess;
    long long tiles;
    if (wgrad) {
        if (p.M == 0) return hipSuccess;
        tiles = (long long)p.E * ceil_div(p.M, BM) * ceil_div(p.N, BN);
    } else {
        if (p.C == 0 && !p.row0) return hipSuccess;
        tiles = (long long)mtile_table_len(p.E, p.C, p.rows) * ceil_div(p.N, BN);
    }
    const long long slots = (long long)(device_cus() / 8) * 8;
    const unsigned grid = (unsigned)(tiles < slots ? ceil_div(tiles, 8) * 8 : slots);
    if (grid == 0) return hipSuccess;
    if (wgrad && p.out_f32)
        gemm_bwd_kernel<true, false, true><<<grid, NTH, 0, st>>>(p);
    else if (wgrad)
        gemm_bwd_kernel<true, false, false><<<grid, NTH, 0, st>>>(p);
    else if (mask)
        gemm_bwd_kernel<false, true, false><<<grid, NTH, 0, st>>>(p);
    else
        gemm_bwd_kernel<false, false, false><<<grid, NTH, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace moe
