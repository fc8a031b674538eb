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

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, kWave));
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Unnormalised Walsh–Hadamard transform (the +-1 Sylvester matrix H') of a
// 128-vector held by one wave, two consecutive elements per lane
// (lane l holds x[2l], x[2l+1]).  Butterfly (a, b) -> (a + b, a - b) on
// element pairs at distance 1, 2, ..., 64; the result is in natural order.
template <typename T>
__device__ __forceinline__ void wave_fwht128(T& x0, T& x1) {
    const int lane = threadIdx.x & (kWave - 1);
    T a = x0 + x1;
    T b = x0 - x1;
    x0 = a;
    x1 = b;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const T p0 = __shfl_xor(x0, m, kWave);
        const T p1 = __shfl_xor(x1, m, kWave);
        const bool upper = (lane & m) != 0;
        x0 = upper ? p0 - x0 : x0 + p0;
        x1 = upper ? p1 - x1 : x1 + p1;
    }
}

// Split partials of one (sequence, query head, split): running max m and
// sum l in base-2 units, unnormalised output o[128].
struct Partials {
    float* m;   // [B][Hq][S]
    float* l;   // [B][Hq][S]
    float* o;   // [B][Hq][S][128]
};

}  // namespace vqkv
