// Device helpers shared by the gfx950 kernels of libvqkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqkv {

constexpr int kHeadDim = 128;
constexpr int kSubDim = 4;
constexpr int kNumSub = kHeadDim / kSubDim;      // 32 sub-vectors per head vector
constexpr int kWave = 64;

// log2(e) / 128: folds the 1/sqrt(D) of the scores, the 1/sqrt(D) of the
// orthonormal Hadamard matrix and the change to base-2 exponentials into one
// factor applied to the unnormalised (+-1) Walsh–Hadamard transform.
constexpr float kScoreScaleLog2 = 1.4426950408889634f / 128.0f;
constexpr float kInvSqrtD = 0.08838834764831845f;           // 1/sqrt(128)
constexpr double kInvSqrtD64 = 0.088388347648318440550;      // 1/sqrt(128)

__device__ __forceinline__ float half_bits_to_float(uint16_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}


// The value held by the lane at distance M (lane ^ M) of the wave, for one
// 32-bit word: DPP for M = 1, 2, 4, 8, a gfx950 permlane swap for 16 and 32,
// so no LDS round trip.  Every lane must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

template <int M>
__device__ __forceinline__ uint32_t lane_partner(uint32_t x, int lane) {
    if constexpr (M == 1) {
        return dpp_u32<0xB1>(x);                   // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        return dpp_u32<0x4E>(x);                   // quad_perm 2,3,0,1
    } else if constexpr (M == 4) {
        // both rotations in every lane: a DPP read from a lane that is off
        // in exec yields the fallback, so this must not become a branch
        const uint32_t down = dpp_u32<0x124>(x);   // row_ror 4: lane i - 4
        const uint32_t up = dpp_u32<0x12C>(x);     // row_ror 12: lane i + 4
        return (lane & 4) ? down : up;
    } else if constexpr (M == 8) {
        return dpp_u32<0x128>(x);                  // row_ror 8
    } else if constexpr (M == 16) {
        const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? sw[0] : sw[1];
    } else {
        static_assert(M == 32, "distance within a wave");
        const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? sw[0] : sw[1];
    }
}

template <int M>
__device__ __forceinline__ float lane_partner(float x, int lane) {
    return __builtin_bit_cast(float, lane_partner<M>(__builtin_bit_cast(uint32_t, x), lane));
}

template <int M>
__device__ __forceinline__ double lane_partner(double x, int lane) {
    uint2 u = __builtin_bit_cast(uint2, x);
    u.x = lane_partner<M>(u.x, lane);
    u.y = lane_partner<M>(u.y, lane);
    return __builtin_bit_cast(double, u);
}

// Maximum and sum over the 64 lanes of a wave, in every lane: butterfly
// stages at distance 32, 16, ..., 1 through lane_partner (no LDS round
// trip).  Each stage combines a lane with its partner symmetrically, so every
// lane ends with the same value.  Every lane must be active.
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
    const int lane = threadIdx.x & (kWave - 1);
    v = max(v, lane_partner<32>(v, lane));
    v = max(v, lane_partner<16>(v, lane));
    v = max(v, lane_partner<8>(v, lane));
    v = max(v, lane_partner<4>(v, lane));
    v = max(v, lane_partner<2>(v, lane));
    return max(v, lane_partner<1>(v, lane));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    const int lane = threadIdx.x & (kWave - 1);
    v += lane_partner<32>(v, lane);
    v += lane_partner<16>(v, lane);
    v += lane_partner<8>(v, lane);
    v += lane_partner<4>(v, lane);
    v += lane_partner<2>(v, lane);
    return v + lane_partner<1>(v, lane);
}

// One butterfly stage at lane distance M: the lane with bit M clear keeps
// a + b, the one with it set b - a (its own value being b).
template <int M, typename T>
__device__ __forceinline__ void butterfly(T& x0, T& x1, int lane) {
    const T p0 = lane_partner<M>(x0, lane), p1 = lane_partner<M>(x1, lane);
    const bool upper = (lane & M) != 0;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
}

// Unnormalised Walsh–Hadamard transform (the +-1 Sylvester matrix H') of a
// 128-vector held by one wave, two consecutive elements per lane (lane l
// holds x[2l], x[2l+1]).  Butterfly (a, b) -> (a + b, a - b) on element
// pairs at distance 1, 2, ..., 64, each add rounded once; the result is in
// natural order.  All 64 lanes must be active.
template <typename T>
__device__ __forceinline__ void fwht128(T& x0, T& x1) {
    const int lane = threadIdx.x & (kWave - 1);
    const T a = x0 + x1, b = x0 - x1;
    x0 = a;
    x1 = b;
    butterfly<1>(x0, x1, lane);
    butterfly<2>(x0, x1, lane);
    butterfly<4>(x0, x1, lane);
    butterfly<8>(x0, x1, lane);
    butterfly<16>(x0, x1, lane);
    butterfly<32>(x0, x1, lane);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, x)));
}

// max / sum over the 16 lanes of a DPP row, result in every lane of the row
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0x128>(x));   // row_ror:8
    x = fmaxf(x, dpp<0x124>(x));   // row_ror:4
    x = fmaxf(x, dpp<0x122>(x));   // row_ror:2
    x = fmaxf(x, dpp<0x121>(x));   // row_ror:1
    return x;
}
__device__ __forceinline__ float row_min16(float x) {
    x = fminf(x, dpp<0x128>(x));
    x = fminf(x, dpp<0x124>(x));
    x = fminf(x, dpp<0x122>(x));
    x = fminf(x, dpp<0x121>(x));
    return x;
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x122>(x);
    x += dpp<0x121>(x);
    return x;
}

// Squared distance ||x - c||^2 of a 4-dim sub-vector to an fp16 centroid
// (4 halves in c), in fp64 with every difference, product and sum rounded
// separately and the 4 terms summed in order, as the fp64 reference does.
__device__ __forceinline__ double sqdist4_f64(const double x[4], const uint2 c) {
    const double c0 = half_bits_to_float(c.x & 0xffffu), c1 = half_bits_to_float(c.x >> 16);
    const double c2 = half_bits_to_float(c.y & 0xffffu), c3 = half_bits_to_float(c.y >> 16);
    const double e0 = __dadd_rn(x[0], -c0), e1 = __dadd_rn(x[1], -c1);
    const double e2 = __dadd_rn(x[2], -c2), e3 = __dadd_rn(x[3], -c3);
    double d = __dmul_rn(e0, e0);
    d = __dadd_rn(d, __dmul_rn(e1, e1));
    d = __dadd_rn(d, __dmul_rn(e2, e2));
    d = __dadd_rn(d, __dmul_rn(e3, e3));
    return d;
}

// The same for an 8-dim sub-vector and an fp16 centroid of 8 halves.
__device__ __forceinline__ double sqdist8_f64(const double x[8], const uint4 c) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    double d = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t bits = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
        const double e = __dadd_rn(x[j], -static_cast<double>(half_bits_to_float(bits)));
        d = j == 0 ? __dmul_rn(e, e) : __dadd_rn(d, __dmul_rn(e, e));
    }
    return d;
}

// Lexicographic (distance, index) order: the nearest centroid, exact ties
// to the lowest index, whatever order candidates are combined in.
__device__ __forceinline__ bool nearer(double d, uint32_t i, double d0, uint32_t i0) {
    return d < d0 || (d == d0 && i < i0);
}

// Split partials of one (sequence, query head, split): running max m and
// sum l in base-2 units, unnormalised output o[128].
struct Partials {
    float* m;   // [B][Hq][S]
    float* l;   // [B][Hq][S]
    float* o;   // [B][Hq][S][128]
};

}  // namespace vqkv
