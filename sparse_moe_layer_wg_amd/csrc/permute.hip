// Dispatch and combine: the single-GPU stand-ins for the two all-to-alls.
//
// Method: "GShard (Expert Parallelism)" (atlas), "In plain words": tokens are
// sent to the devices holding their experts by an all-to-all and returned;
// research-vault claim IX2-0404, section "WideEP", "Evidence": the results
// come back by a second all-to-all.  On one GPU the first exchange becomes a
// permute of token rows into per-expert capacity buffers [E,C,d] (or, for
// dropless routing, into compact expert segments [S*k,d]) and the second a
// gate-weighted gather back to token order.
//
// Both kernels are HBM-bound row copies: one wavefront per token, 16-byte
// vector accesses, rows of 2-14 KB, so every access is fully coalesced
// without staging through LDS.  A token's k (expert, slot) pairs are
// wave-uniform and held in scalar registers.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;  // one token per wave, 4 waves per block

// xd[idx[s,r]*stride + slot[s,r], :] = x[s, :] for kept (s,r): each row of x
// is read once and written to each of its kept destinations.  Pairs outside
// [0,E) x [0,limit) are treated as dropped.
__global__ __launch_bounds__(256) void dispatch_kernel(const u32x4_t* __restrict__ x,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const int32_t* __restrict__ slot,
                                                       u32x4_t* __restrict__ xd, int S, int nvec,
                                                       int k, int E, int stride, int limit) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(blockIdx.x * kTokPerBlock + wave);
    if (s >= S) return;
    // dst[r] < 0: assignment r absent (r >= k) or dropped
    int64_t dst[kMaxK];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        dst[r] = -1;
        if (r < k) {
            const int c = slot[(size_t)s * k + r];
            const int e = topk_idx[(size_t)s * k + r];
            if (c >= 0 && c < limit && e >= 0 && e < E)
                dst[r] = ((int64_t)e * stride + c) * nvec;
        }
    }
    const u32x4_t* src = x + (size_t)s * nvec;
    int i = lane;
    for (; i + 3 * kWave < nvec; i += 4 * kWave) {
        const u32x4_t v0 = src[i], v1 = src[i + kWave], v2 = src[i + 2 * kWave],
                      v3 = src[i + 3 * kWave];
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (dst[r] >= 0) {
                u32x4_t* o = xd + dst[r] + i;
                o[0] = v0;
                o[kWave] = v1;
                o[2 * kWave] = v2;
                o[3 * kWave] = v3;
            }
        }
    }
    for (; i < nvec; i += kWave) {
        const u32x4_t v = src[i];
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)
            if (dst[r] >= 0) xd[dst[r] + i] = v;
    }
}

// y[s] = sum over kept r of w[s,r] * out[idx[s,r]*stride + slot[s,r]] (fp32
// accumulation in rank order), rounded to the activation dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4_t* __restrict__ out,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ topk_w,
                                                      u32x4_t* __restrict__ y, int S, int nvec,
                                                      int k, int E, int stride, int limit) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int s = __builtin_amdgcn_readfirstlane(blockIdx.x * kTokPerBlock + wave);
    if (s >= S) return;
    // src[r] < 0: assignment r absent (r >= k) or dropped
    int64_t src[kMaxK];
    float wt[kMaxK];
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
        src[r] = -1;
        wt[r] = 0.f;
        if (r < k) {
            const int c = slot[(size_t)s * k + r];
            const int e = topk_idx[(size_t)s * k + r];
            if (c >= 0 && c < limit && e >= 0 && e < E) {
                src[r] = ((int64_t)e * stride + c) * nvec;
                wt[r] = topk_w[(size_t)s * k + r];
            }
        }
    }
    u32x4_t* dst = y + (size_t)s * nvec;
    for (int i = lane; i < nvec; i += kWave) {
        constexpr int NE = BF16 ? 8 : 4;
        float acc[NE];
#pragma unroll
        for (int q = 0; q < NE; ++q) acc[q] = 0.f;
        u32x4_t v[kMaxK];
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)   // each (expert, slot) row is read once
            if (src[r] >= 0) v[r] = __builtin_nontemporal_load(out + src[r] + i);
#pragma unroll
        for (int r = 0; r < kMaxK; ++r) {
            if (src[r] >= 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (BF16) {
                        acc[2 * q] = fmaf(wt[r], __uint_as_float(v[r][q] << 16), acc[2 * q]);
                        acc[2 * q + 1] =
                            fmaf(wt[r], __uint_as_float(v[r][q] & 0xffff0000u), acc[2 * q + 1]);
                    } else {
                        acc[q] = fmaf(wt[r], __uint_as_float(v[r][q]), acc[q]);
                    }
                }
            }
        }
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = BF16 ? pack_bf16x2(acc[2 * q], acc[2 * q + 1]) : __float_as_uint(acc[q]);
        __builtin_nontemporal_store(o, dst + i);   // y is not read again here
    }
}

}  // namespace

hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, const int32_t* slot,
                           void* xd, int S, int d, int k, int E, int stride, int limit,
                           int elem_bytes, hipStream_t st) {
    const int nvec = d * elem_bytes / 16;
    dispatch_kernel<<<(unsigned)ceil_div(S, kTokPerBlock), 256, 0, st>>>(
        static_cast<const u32x4_t*>(x), topk_idx, slot, static_cast<u32x4_t*>(xd), S, nvec, k, E,
        stride, limit);
    return hipGetLastError();
}

hipError_t launch_combine(const void* out, const int32_t* topk_idx, const int32_t* slot,
                          const float* topk_w, void* y, int S, int d, int k, int E, int stride,
                          int limit, bool bf16, hipStream_t st) {
    const int nvec = d * (bf16 ? 2 : 4) / 16;
    const unsigned grid = (unsigned)ceil_div(S, kTokPerBlock);
    const auto* o = static_cast<const u32x4_t*>(out);
    auto* yy = static_cast<u32x4_t*>(y);
    if (bf16)
        combine_kernel<true><<<grid, 256, 0, st>>>(o, topk_idx, slot, topk_w, yy, S, nvec, k, E,
                                                   stride, limit);
    else
        combine_kernel<false><<<grid, 256, 0, st>>>(o, topk_idx, slot, topk_w, yy, S, nvec, k, E,
                                                    stride, limit);
    return hipGetLastError();
}

}  // namespace moe
