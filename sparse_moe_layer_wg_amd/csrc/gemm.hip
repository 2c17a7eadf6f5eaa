// Expert FFN GEMMs over variable-occupancy capacity buffers.
//
// Method: "GShard: Scaling Giant Neural Networks with Conditional Computation"
// (blog), section "Core Components", "Expert Networks": every expert is a
// feed-forward network; section "Performance Analysis", "FLOPs Analysis": a
// token costs k expert FFNs.  Here expert e computes, for its filled slots
// m < occ[e] only,
//   GEMM 1:  H[e,m,:] = ReLU(xd[e,m,:] . W1[e]^T + b1[e])     (N = h, K = d)
//   GEMM 2:  O[e,m,:] = H[e,m,:] . W2[e]^T + b2[e]            (N = d, K = h)
// Both are "A . B^T" with A [E,C,K] and B [E,N,K] row-major, K contiguous in
// both operands, which is the operand order the MFMA fragments want.
//
// bf16 path: gfx950 v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//   Block tile BM x 256 x 64.  BM = 256: 512 threads = 8 waves in a 2 x 4
//   grid, 128 x 64 per wave (two waves per SIMD, 128 fp32 accumulators per
//   lane); BM = 128 (experts with few rows): 4 waves of 64 x 128.
//   Operands go from global memory straight into two LDS buffers
//   (global_load_lds_dwordx4, 1 KB = 8 rows per wave instruction), so no
//   registers stage them and no LDS stores are issued.  The fragments of the
//   next step are read from LDS while the current MFMAs run (spread with
//   sched_group_barrier), across k-tile boundaries too: a k-tile's one
//   barrier comes before its last step, after which the copies of k-tile
//   t+2 go into the buffer every wave has just finished reading and the
//   last step's MFMAs run while k-tile t+1's first fragments are read, so no
//   wave starts a k-tile waiting for LDS (1-2% faster than a closing barrier
//   per k-tile, same results bit for bit).  Measured from L2,
//   the copies move as many bytes per clock as loads into registers, and
//   against that register-staged loop (padded LDS rows) this runs the
//   expert GEMMs 2-4% faster on average with the same results bit for bit
//   (the stores and the waits for them were a tenth of the waves' cycles).
//   LDS rows are 128 bytes with their 16-byte chunks XOR-swizzled by row,
//   so the 16 rows a fragment read touches at one chunk fall on distinct
//   bank groups.
//   Rows past an expert's occupancy (and columns past N) load a clamped
//   valid row; their results are never stored.
//   An expert's last 256-row m-tile may hold up to 32 more rows (a strip):
//   each wave multiplies them against B fragments it already holds, so an
//   expert with 257..288 rows costs one m-tile, not a second, nearly empty
//   one that reloads all of W.
//   The MFMAs take the weight fragment as their first operand, so each lane
//   ends with four consecutive output columns per register quad; bias, ReLU
//   and bf16 rounding are applied there, and lane pairs (l, l+32) exchange
//   halves with v_permlane32_swap so that each lane stores 8 consecutive
//   columns as one 16-byte chunk straight from registers.
//   With a_rows set, A rows are gathered from the token rows through the
//   inverse slot map (the dispatch permute fused into the loads).  With row0
//   set, expert e's rows start at row0[e] instead of e*C: the compact expert
//   segments of dropless routing, laid end to end with no padding.
//   Tiles come from a compact list: expert e owns m-tiles
//   [mt_start[e], mt_start[e+1]) (built on the device from the occupancies),
//   ordered by expert, then in groups of 4 n-tiles (m-tile-major inside a
//   group, n-tile fastest).  The grid is persistent, one block per
//   CU; block b runs on XCD b % 8, XCD x owns the x-th eighth of the list and
//   its blocks take that chunk's tiles in order from an atomic counter, so
//   the blocks of one XCD work on neighbouring tiles (sharing A and B tiles
//   through L2) at the same time and tiles of unequal cost balance out.
//   The shader clock falls with the matrix work: about 1.7 GHz while the
//   large (MFMA-bound) shapes run, 2.2 GHz at the weight-streaming ones.
#include "common.h"
#include "kernels.h"

#include <atomic>

#include <type_traits>

namespace moe {
namespace {

// Block tile BM x BN; WNC waves along N (2 or 4), 2 along M: 4 or 8 waves.
template <int BM, int BN, int WNC, bool RELU>
__global__ __launch_bounds__(128 * WNC, 1) void gemm_bf16_kernel(GemmParams p) {
    constexpr int NTH = 128 * WNC;             // threads per block
    constexpr int NW = NTH / 64;               // waves
    constexpr int BK = 64;                     // k-tile
    constexpr int RB = BK * 2;                 // LDS row: 128 bytes, 8 swizzled chunks
    constexpr int WM = BM / 2, WNT = BN / WNC; // wave tile
    constexpr int TM = WM / 32, TN = WNT / 32; // 32x32 MFMA tiles per wave
    constexpr int KS = BK / 16;                // MFMA k steps per k-tile
    // An expert's last m-tile may carry SR more rows (the strip): each wave
    // multiplies them into SB extra 32x32 blocks, with B fragments it holds.
    constexpr int SR = BM == 256 ? kStripRows : 0;
    constexpr int SB = BN / 32 / NW;           // strip blocks per wave
    constexpr int AG = BM / 8 / NW;            // 1 KB copies (8 rows) per wave: A
    constexpr int BG = BN / 8 / NW;            //   and B
    constexpr int SOFF = BM * RB;              // byte offset of the strip rows
    constexpr int BOFF = (BM + SR) * RB;       // byte offset of B in a stage
    constexpr int STAGE = BOFF + BN * RB;      // bytes per LDS buffer
    static_assert(SR == 0 || (SR / 8 <= NW && SB * 2 == TN),
                  "strip: one copy per wave of the first SR/8; a wave row's share of the B fragments");
    static_assert(AG * NW * 8 == BM && BG * NW * 8 == BN, "whole 8-row copies per wave");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int N = p.N, K = p.K;
    const int NT = (N + BN - 1) / BN;
    const int T = p.mt_start[p.E] * NT;
    const int per = (T + 7) >> 3;
    const int xcd = blockIdx.x & 7;
    const int t_end = min(T, (xcd + 1) * per);
    __shared__ int s_next;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / WNC, wn = wave % WNC;
    const int frow = lane & 31, fhalf = lane >> 5;
    const int KT = K / BK;
    // LDS rows are unpadded; chunk c of row r sits in slot c ^ swz(r), with
    // swz(r) = (r >> 1) & 7, so the 16 rows a fragment read touches at one
    // chunk fall on distinct bank groups.  A fragment row of this lane is
    // frow + 32*i (+ a multiple of 32), whose swizzle is swz(frow): step ks
    // reads chunk 2*ks + fhalf at the same slot offset co[ks] in every row.
    auto swz = [](int r) { return (r >> 1) & 7; };
    const int fa_off = (wm * WM + frow) * RB;
    const int fb_off = BOFF + (wn * WNT + frow) * RB;
    const int fs_off = SOFF + frow * RB;
    int co[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) co[ks] = ((2 * ks + fhalf) ^ swz(frow)) * 16;
    // Copy g of a wave fills LDS rows 8*(wave + NW*g) .. +7: lane l writes
    // row 8*(wave + NW*g) + l/8, slot l%8, i.e. chunk (l%8) ^ swz(row).
    const int crow = lane >> 3;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

    // Tiles of this XCD's chunk are handed out on demand (tiles differ in
    // cost: partly filled m-tiles skip MFMAs).  The next tile is claimed at
    // the start of each epilogue and published at its end, so the atomic's
    // latency overlaps the epilogue and does not wait for its stores.
    if (tid == 0) s_next = xcd * per + atomicAdd(&p.tile_ctr[xcd], 1);
    for (;;) {
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(s_next);
        if (t >= t_end) break;
        // expert and m-/n-tile of tile t (uniform values, kept in scalar
        // registers; the loads themselves go through the vector path)
        const int q = t / NT;
        const int e = __builtin_amdgcn_readfirstlane(p.mt_expert[q]);
        const int mt0 = __builtin_amdgcn_readfirstlane(p.mt_start[e]);
        const int mtiles = __builtin_amdgcn_readfirstlane(p.mt_start[e + 1]) - mt0;
        // Within an expert, tiles run in groups of GN n-tiles: n-tile fastest
        // inside a group, then m-tile, then the next group, so each A panel
        // serves GN neighbouring tiles and each B panel all m-tiles of a group
        // while they are in L2.
        constexpr int GN = 4;
        const int local = t - mt0 * NT;
        const int ng = local / (mtiles * GN);
        const int gsize = min(GN, NT - ng * GN);
        const int r = local - ng * mtiles * GN;
        const int mi = r / gsize;
        const int m0 = mi * BM, n0 = (ng * GN + r % gsize) * BN;
        const int M = __builtin_amdgcn_readfirstlane(p.occ[e]);
        const bool strip = SR > 0 && mi == mtiles - 1 && M - m0 > BM;
        // first row of expert e: e*C in padded buffers, row0[e] in compact ones
        const size_t row_e = p.row0 ? (size_t)__builtin_amdgcn_readfirstlane(p.row0[e])
                                    : (size_t)e * p.C;
        const char* __restrict__ Ab = reinterpret_cast<const char*>(
            static_cast<const bf16_t*>(p.A) + (p.a_rows ? (size_t)0 : row_e * K));
        const int32_t* __restrict__ arow = p.a_rows ? p.a_rows + row_e : nullptr;
        const char* __restrict__ Bb =
            reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.B) + (size_t)e * N * K);

        // Global byte offsets of this lane's chunks (rows past the occupancy
        // or past N load a clamped valid row).
        uint32_t aoff[AG], boff[BG], soff = 0;
#pragma unroll
        for (int g = 0; g < AG; ++g) {
            const int lr = 8 * (wave + NW * g) + crow;
            const int rg = min(m0 + lr, M - 1);
            aoff[g] = (uint32_t)(arow ? arow[rg] : rg) * (uint32_t)K * 2u +
                      (uint32_t)(((lane & 7) ^ swz(lr)) * 16);
        }
#pragma unroll
        for (int g = 0; g < BG; ++g) {
            const int lr = 8 * (wave + NW * g) + crow;
            boff[g] = (uint32_t)min(n0 + lr, N - 1) * (uint32_t)K * 2u +
                      (uint32_t)(((lane & 7) ^ swz(lr)) * 16);
        }
        if (SR > 0 && wave < SR / 8) {
            const int lr = 8 * wave + crow;                 // strip row
            const int rg = min(m0 + BM + lr, M - 1);
            soff = (uint32_t)(arow ? arow[rg] : rg) * (uint32_t)K * 2u +
                   (uint32_t)(((lane & 7) ^ swz(lr)) * 16);
        }
        // k-tile kt into LDS buffer buf by global->LDS copies
        // (global_load_lds_dwordx4: the wave-uniform base + k offset in
        // scalar registers, the lane's 32-bit offset in a vector register,
        // the 1 KB destination in M0, written one wait state ahead; M0 is
        // saved and restored around it).  They are asm so that the compiler
        // does not make the fragment reads of the other buffer wait for
        // them; the k-tile waits for its copies itself before its closing
        // barrier.
        auto copy = [](const char* base, uint32_t voff, uint32_t lds) {
            uint32_t saved;
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %1\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %2, %3\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(saved)
                : "s"(lds), "v"(voff), "s"(base)
                : "memory");
        };
        auto gcopy = [&](auto strip_tag, int kt, int buf) {
            const uint32_t kb = (uint32_t)kt * BK * 2u;
            const char* Ak = Ab + kb;
            const char* Bk = Bb + kb;
            const uint32_t st = lds0 + (uint32_t)(buf * STAGE);
#pragma unroll
            for (int g = 0; g < AG; ++g) copy(Ak, aoff[g], st + (uint32_t)((wv + NW * g) * 1024));
#pragma unroll
            for (int g = 0; g < BG; ++g)
                copy(Bk, boff[g], st + (uint32_t)(BOFF + (wv + NW * g) * 1024));
            if constexpr (decltype(strip_tag)::value) {
                if (wv < SR / 8) copy(Ak, soff, st + (uint32_t)(SOFF + wv * 1024));
            }
        };

        // Fragment (32x32x16): lane l supplies row l%32 and the 8 consecutive
        // k at (l/32)*8 of the 16-wide step, i.e. chunk 2*ks + l/32 of the
        // row.  Only the first VI of the wave's TM row sub-tiles are read.
        bf16x8_t fa[2][TM], fb[2][TN], fs[2];
        auto load_frags = [&](auto vi_tag, auto strip_tag, const char* st, int ks, int slot) {
            constexpr int VI = decltype(vi_tag)::value;
            if constexpr (decltype(strip_tag)::value)
                fs[slot] = *reinterpret_cast<const bf16x8_t*>(st + fs_off + co[ks]);
#pragma unroll
            for (int i = 0; i < VI; ++i)
                fa[slot][i] = *reinterpret_cast<const bf16x8_t*>(st + fa_off + co[ks] + i * 32 * RB);
            if constexpr (VI > 0) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb[slot][j] =
                        *reinterpret_cast<const bf16x8_t*>(st + fb_off + co[ks] + j * 32 * RB);
            }
        };

        f32x16_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        f32x16_t acc_s[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_s[b][r] = 0.f;

        // One k-tile from LDS buffer kt&1.  The fragments of step 0 were read
        // during the previous k-tile; each step multiplies the fragments read
        // one step earlier while reading the next step's.  With NEXT (a k-tile
        // kt+1 follows), the barrier comes before the last step: once every
        // wave's copies of k-tile kt+1 have landed and every wave has read its
        // last fragments of k-tile kt, the copies of k-tile kt+2 go into this
        // buffer, and the last step's MFMAs (whose fragments are already in
        // registers) run while the first fragments of k-tile kt+1 are read.
        // So no wave starts a k-tile waiting for LDS, and each copy has a
        // whole k-tile to land.
        // VI: how many of this wave's TM row sub-tiles hold filled rows; the
        // MFMAs of the others are skipped (an expert's last m-tile is
        // usually partly empty).  Every wave still takes part in the copies
        // and barriers.
        auto ktile = [&](auto next_tag, auto vi_tag, auto strip_tag, int kt) {
            constexpr bool NEXT = decltype(next_tag)::value;
            constexpr int VI = decltype(vi_tag)::value;
            constexpr int SI = decltype(strip_tag)::value ? 1 : 0;
            constexpr int NF = TM + TN + SI;       // fragment reads per step
            constexpr int NM = TM * TN + SI * SB;  // MFMAs per step (full tile)
            const char* st = smem + (kt & 1) * STAGE;
            const char* sn = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (NEXT) {
                    if (ks == KS - 1) {
                        __builtin_amdgcn_s_waitcnt(0);   // this wave's copies landed
                        __syncthreads();
                        if (kt + 2 < KT) gcopy(strip_tag, kt + 2, kt & 1);
                    }
                }
                if (ks + 1 < KS) load_frags(vi_tag, strip_tag, st, ks + 1, (ks + 1) & 1);
                else if constexpr (NEXT) load_frags(vi_tag, strip_tag, sn, 0, 0);
#pragma unroll
                for (int i = 0; i < VI; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
                if constexpr (SI) {
                    // strip columns of this wave: its B fragments wm*SB + b
#pragma unroll
                    for (int b = 0; b < SB; ++b) {
                        const bf16x8_t bs = wm ? fb[ks & 1][SB + b] : fb[ks & 1][b];
                        acc_s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bs, fs[ks & 1], acc_s[b],
                                                                           0, 0, 0);
                    }
                }
                // the next step's fragment reads spread over the MFMAs (a
                // wave issues in order, so a burst would stall its MFMAs)
                if (ks + 1 < KS || NEXT) {
#pragma unroll
                    for (int g = 0; g < NF; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
                        __builtin_amdgcn_sched_group_barrier(0x008, NM / NF, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto kloop = [&](auto vi_tag, auto strip_tag) {
            gcopy(strip_tag, 0, 0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (KT > 1) gcopy(strip_tag, 1, 1);
            load_frags(vi_tag, strip_tag, smem, 0, 0);
            int kt = 0;
            for (; kt + 1 < KT; ++kt) ktile(std::true_type{}, vi_tag, strip_tag, kt);
            ktile(std::false_type{}, vi_tag, strip_tag, kt);
        };
        // filled 32-row sub-tiles of this wave (wave-uniform); 3 runs as TM
        const int rows_left = M - m0 - wm * WM;
        const int vi = rows_left <= 0 ? 0 : min(TM, (rows_left + 31) / 32);
        constexpr std::false_type no_strip{};
        if (strip) kloop(std::integral_constant<int, TM>{}, std::bool_constant<(SR > 0)>{});
        else if (vi == 0) kloop(std::integral_constant<int, 0>{}, no_strip);
        else if (vi == 1) kloop(std::integral_constant<int, 1>{}, no_strip);
        else if (TM > 2 && vi == 2) kloop(std::integral_constant<int, (TM > 2 ? 2 : TM)>{}, no_strip);
        else kloop(std::integral_constant<int, TM>{}, no_strip);

        int nx = 0;
        if (tid == 0) nx = xcd * per + atomicAdd(&p.tile_ctr[xcd], 1);
        // Epilogue.  The MFMAs take the weight fragment as their first
        // operand, so a 32x32 accumulator block is (n x m): lane l holds row
        // m = l%32 and register r column n = 8*(r/4) + 4*(l/32) + r%4, i.e.
        // four consecutive columns per register quad.  Bias and ReLU are
        // applied there.
        bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.Cout) + row_e * N;
        const bf16_t* bias = p.bias ? static_cast<const bf16_t*>(p.bias) + (size_t)e * N : nullptr;
        auto finish4 = [&](const f32x16_t& a, int q, int n) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = a[4 * q + r];
            if (bias && n < N) {
                const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
                v[0] += __uint_as_float(bb.x << 16);
                v[1] += __uint_as_float(bb.x & 0xffff0000u);
                v[2] += __uint_as_float(bb.y << 16);
                v[3] += __uint_as_float(bb.y & 0xffff0000u);
            }
            if (RELU) {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = v[r] > 0.f ? v[r] : 0.f;
            }
            return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        };
        // Lanes l and l+32 hold columns 4 apart: one swap of the upper half's
        // even quads with the lower half's odd quads (v_permlane32_swap) gives
        // every lane 8 consecutive columns, stored as one 16-byte chunk
        // straight from registers (32 bytes of a row per lane pair).
        const int nw = n0 + wn * WNT;               // first column of this wave
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WM + i * 32 + frow;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = nw + j * 32 + 16 * h;   // 16 columns of quads 2h, 2h+1
                    const uint2 v0 = finish4(acc[i][j], 2 * h, c + 4 * fhalf);
                    const uint2 v1 = finish4(acc[i][j], 2 * h + 1, c + 8 + 4 * fhalf);
                    // lower lane: own v0 | upper's v0; upper lane: lower's v1 | own v1
                    const auto sx = __builtin_amdgcn_permlane32_swap(v0.x, v1.x, false, false);
                    const auto sy = __builtin_amdgcn_permlane32_swap(v0.y, v1.y, false, false);
                    const int n = c + 8 * fhalf;
                    if (m < M && n < N) {
                        u32x4_t o;
                        o[0] = sx[0];
                        o[1] = sy[0];
                        o[2] = sx[1];
                        o[3] = sy[1];
                        *reinterpret_cast<u32x4_t*>(Cout + (size_t)m * N + n) = o;
                    }
                }
        }
        // publish the next tile (every wave read s_next before the k-loop's
        // first barrier; the atomic has long returned)
        if (tid == 0) s_next = nx;
        if (strip) {
            const int m = m0 + BM + frow;
            if (m < M) {
#pragma unroll
                for (int b = 0; b < SB; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = nw + (wm * SB + b) * 32 + 8 * q + 4 * fhalf;
                        if (n < N)
                            *reinterpret_cast<uint2*>(Cout + (size_t)m * N + n) =
                                finish4(acc_s[b], q, n);
                    }
            }
        }
    }  // tile loop
}

// fp32 activations: LDS-tiled fp32 FMA, tile 64x64x16, 4x4 outputs per
// thread strided by 16.
constexpr int FM = 64, FN = 64, FK = 16;

template <bool RELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
    __shared__ float As[FK][FM + 4];
    __shared__ float Bs[FK][FN + 4];
    const int e = blockIdx.z;
    const int M = p.occ[e];
    const int m0 = blockIdx.y * FM;
    if (m0 >= M) return;
    const int n0 = blockIdx.x * FN;
    const int N = p.N, K = p.K;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const int lrow = tid / 4, lk = (tid % 4) * 4;
    const size_t row_e = p.row0 ? (size_t)p.row0[e] : (size_t)e * p.C;  // expert's first row
    const float* __restrict__ A = static_cast<const float*>(p.A) + row_e * K;
    const float* __restrict__ B = static_cast<const float*>(p.B) + (size_t)e * N * K;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < K; k0 += FK) {
        f32x4_t av = {0.f, 0.f, 0.f, 0.f}, bv = {0.f, 0.f, 0.f, 0.f};
        if (m0 + lrow < M && k0 + lk < K)
            av = *reinterpret_cast<const f32x4_t*>(A + (size_t)(m0 + lrow) * K + k0 + lk);
        if (n0 + lrow < N && k0 + lk < K)
            bv = *reinterpret_cast<const f32x4_t*>(B + (size_t)(n0 + lrow) * K + k0 + lk);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            As[lk + q][lrow] = av[q];
            Bs[lk + q][lrow] = bv[q];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
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
    float* __restrict__ Cout = static_cast<float*>(p.Cout) + row_e * N;
    const float* bias = p.bias ? static_cast<const float*>(p.bias) + (size_t)e * N : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            float v = acc[i][j] + (bias ? bias[n] : 0.f);
            if (RELU) v = v > 0.f ? v : 0.f;
            Cout[(size_t)m * N + n] = v;
        }
    }
}

}  // namespace

// Compute units of the current device.  The attribute is queried once per
// device and kept in a process-wide table (every writer stores the same
// value, so concurrent first calls agree).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 8)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// m-tile height: 256 when experts average at least 160 rows (each weight
// tile is then streamed once per expert and a 256x256 tile halves operand
// traffic per flop), else 128 so that lightly filled experts waste less.
int gemm_block_m(bool bf16, int S, int E, int k) {
    if (!bf16) return FM;
    const long long avg = (long long)S * k / (E > 0 ? E : 1);
    return avg >= 160 ? 256 : 128;
}

hipError_t launch_expert_gemm(const GemmParams& p, bool bf16, int bm, hipStream_t st) {
    if (p.E == 0 || p.C == 0) return hipSuccess;
    if (bf16) {
        // persistent grid: one block per CU (the LDS stages fill a CU), at most
        // one per possible tile, a multiple of the 8 XCDs
        const int bn = 256;
        const long long tiles = (long long)p.E * ceil_div(p.C, bm) * ceil_div(p.N, bn);
        const long long slots = (long long)(device_cus() / 8) * 8;
        const unsigned grid = (unsigned)(tiles < slots ? ceil_div(tiles, 8) * 8 : slots);
        // BM 256: 8 waves (2 per SIMD), so each SIMD holds one upper- and one
        // lower-half wave and a partly filled m-tile sheds MFMA work on every
        // SIMD; BM 128: 4 waves of 64 x 128
        if (bm == 256) {
            if (p.relu) gemm_bf16_kernel<256, 256, 4, true><<<grid, 512, 0, st>>>(p);
            else gemm_bf16_kernel<256, 256, 4, false><<<grid, 512, 0, st>>>(p);
        } else {
            if (p.relu) gemm_bf16_kernel<128, 256, 2, true><<<grid, 256, 0, st>>>(p);
            else gemm_bf16_kernel<128, 256, 2, false><<<grid, 256, 0, st>>>(p);
        }
    } else {
        dim3 grid((unsigned)ceil_div(p.N, FN), (unsigned)ceil_div(p.C, FM), (unsigned)p.E);
        if (p.relu)
            gemm_f32_kernel<true><<<grid, 256, 0, st>>>(p);
        else
            gemm_f32_kernel<false><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}

}  // namespace moe
