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
// bf16 path: gfx950 v_mfma_f32_32x32x16_bf16, fp32 accumulation.  Block tile
// 128x128x64, four waves in a 2x2 grid, each wave 64x64 = 2x2 MFMA tiles.
// Operand tiles are staged in LDS (rows padded by 16 bytes so that the
// 16-byte fragment reads of 8 consecutive rows fall in distinct banks) and
// double-buffered: the global loads of tile k+1 are in flight while the
// MFMAs consume tile k.  Blocks whose m-tile lies past the expert's
// occupancy exit at once, so empty experts and empty slots cost nothing
// beyond a launch slot.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

template <bool RELU>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) bf16_t As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN][LDK];

    const int e = blockIdx.z;
    const int M = p.occ[e];
    const int m0 = blockIdx.y * BM;
    if (m0 >= M) return;
    const int n0 = blockIdx.x * BN;
    const int N = p.N, K = p.K;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int wm = wave >> 1, wn = wave & 1;

    const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A) + (size_t)e * p.C * K;
    const bf16_t* __restrict__ B = static_cast<const bf16_t*>(p.B) + (size_t)e * N * K;

    // Loader: the 128x64 tile is 1024 16-byte chunks, 4 per thread; chunk
    // c covers row c/8, columns (c%8)*8 .. +8.
    u32x4_t ra[4], rb[4];
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
            ra[i] = (m0 + row < M)
                        ? *reinterpret_cast<const u32x4_t*>(A + (size_t)(m0 + row) * K + k0 + col)
                        : zero;
            rb[i] = (n0 + row < N)
                        ? *reinterpret_cast<const u32x4_t*>(B + (size_t)(n0 + row) * K + k0 + col)
                        : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
            *reinterpret_cast<u32x4_t*>(&As[buf][row][col]) = ra[i];
            *reinterpret_cast<u32x4_t*>(&Bs[buf][row][col]) = rb[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    const int KT = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    // Fragment addressing (32x32x16): lane l supplies row l%32 and the 8
    // consecutive k starting at (l/32)*8 of the 16-wide k-step.
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                a[mi] = *reinterpret_cast<const bf16x8_t*>(
                    &As[buf][wm * 64 + mi * 32 + frow][ks * 16 + fk]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                b[ni] = *reinterpret_cast<const bf16x8_t*>(
                    &Bs[buf][wn * 64 + ni * 32 + frow][ks * 16 + fk]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni],
                                                                         acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane l holds column l%32; register
    // r holds row 8*(r/4) + 4*(l/32) + r%4.
    bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.Cout) + (size_t)e * p.C * N;
    const bf16_t* bias = p.bias ? static_cast<const bf16_t*>(p.bias) + (size_t)e * N : nullptr;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (n >= N) continue;
        const float bv = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M) {
                    float v = acc[mi][ni][r] + bv;
                    if (RELU) v = v > 0.f ? v : 0.f;
                    Cout[(size_t)m * N + n] = f32_to_bf16(v);
                }
            }
        }
    }
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
    const float* __restrict__ A = static_cast<const float*>(p.A) + (size_t)e * p.C * K;
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
    float* __restrict__ Cout = static_cast<float*>(p.Cout) + (size_t)e * p.C * N;
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

int gemm_block_m(bool bf16) { return bf16 ? BM : FM; }

hipError_t launch_expert_gemm(const GemmParams& p, bool bf16, hipStream_t st) {
    if (p.E == 0 || p.C == 0) return hipSuccess;
    if (bf16) {
        dim3 grid((unsigned)ceil_div(p.N, BN), (unsigned)ceil_div(p.C, BM), (unsigned)p.E);
        if (p.relu)
            gemm_bf16_kernel<true><<<grid, 256, 0, st>>>(p);
        else
            gemm_bf16_kernel<false><<<grid, 256, 0, st>>>(p);
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
