// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kTokBlock = 64;       // tokens per routing tile (one wave of lanes)
constexpr int kMaxK = 8;            // largest supported top-k
constexpr int kMaxE = 2048;         // largest supported expert count
constexpr int kMaxEQ = kMaxE / kWave;

typedef uint16_t bf16_t;            // raw bf16 storage

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32.
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even, by gfx950's packed conversion
// (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_native_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_native_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key); -0 is
// folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide reductions on DPP lane moves (register to register, a few
// cycles each) rather than shuffles through the LDS crossbar: within each
// 16-lane row, quad_perm [1,0,3,2] and [2,3,0,1], then half-row and row
// mirrors, leave the row's result in all 16 lanes; the four rows are then
// read out as scalars (lanes 0, 16, 32, 48) and combined in that order.  All
// 64 lanes must be active.  The result is the same in every lane.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v),
                                                             static_cast<int>(v), CTRL, 0xf, 0xf,
                                                             false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(v));
    const uint32_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), l);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<kDppXor1>(v);
    v = o > v ? o : v;
    o = dpp_u64<kDppXor2>(v);
    v = o > v ? o : v;
    o = dpp_u64<kDppHalfMirror>(v);
    v = o > v ? o : v;
    o = dpp_u64<kDppMirror>(v);
    v = o > v ? o : v;
    uint64_t r = readlane_u64(v, 0);
#pragma unroll
    for (int l = 16; l < kWave; l += 16) {
        o = readlane_u64(v, l);
        r = o > r ? o : r;
    }
    return r;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v)));
    float r = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
#pragma unroll
    for (int l = 16; l < kWave; l += 16)
        r += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), l));
    return r;
}

// Largest of non-negative floats across the wave (their bit patterns order
// as unsigned integers); the result is the same in every lane.
__device__ __forceinline__ float wave_max_nonneg_f32(float v) {
    uint32_t u = __float_as_uint(v), o;
    o = dpp_u32<kDppXor1>(u);
    u = o > u ? o : u;
    o = dpp_u32<kDppXor2>(u);
    u = o > u ? o : u;
    o = dpp_u32<kDppHalfMirror>(u);
    u = o > u ? o : u;
    o = dpp_u32<kDppMirror>(u);
    u = o > u ? o : u;
    uint32_t r = __builtin_amdgcn_readlane(u, 0);
#pragma unroll
    for (int l = 16; l < kWave; l += 16) {
        o = __builtin_amdgcn_readlane(u, l);
        r = o > r ? o : r;
    }
    return __uint_as_float(r);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    auto mv = [](double x, auto ctrl_tag) {
        constexpr int C = decltype(ctrl_tag)::value;
        return __longlong_as_double(static_cast<long long>(
            dpp_u64<C>(static_cast<uint64_t>(__double_as_longlong(x)))));
    };
    v += mv(v, std::integral_constant<int, kDppXor1>{});
    v += mv(v, std::integral_constant<int, kDppXor2>{});
    v += mv(v, std::integral_constant<int, kDppHalfMirror>{});
    v += mv(v, std::integral_constant<int, kDppMirror>{});
    const auto rd = [&](int l) {
        return __longlong_as_double(static_cast<long long>(
            readlane_u64(static_cast<uint64_t>(__double_as_longlong(v)), l)));
    };
    double r = rd(0);
#pragma unroll
    for (int l = 16; l < kWave; l += 16) r += rd(l);
    return r;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
