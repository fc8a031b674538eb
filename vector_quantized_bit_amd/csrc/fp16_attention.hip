// Uncompressed comparator: split-K decode attention over an fp16 KV cache,
// o = softmax(q K^T / sqrt(128)) V with fp32 accumulation (VecInfer page,
// Background: KV cache and attention).  Same split partials and merge as the
// VQ kernels.
//
// Each wave owns 32-token chunks of the workgroup's range; 16 lanes share one
// token (8 channels per lane), so one 16-byte load per lane moves 4 whole
// 256-byte key (or value) rows per wave instruction.  Each 16-lane group keeps
// its own online-softmax state; groups and waves are merged at the end.
#include "launchers.hpp"

namespace vqkv {

namespace {

__device__ __forceinline__ void unpack8(const uint4 u, float f[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = half_bits_to_float(static_cast<uint16_t>(w[i] & 0xffffu));
        f[2 * i + 1] = half_bits_to_float(static_cast<uint16_t>(w[i] >> 16));
    }
}

__device__ __forceinline__ float scale_of(float m_old, float m_new) {
    return (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
}

}  // namespace

template <int G>
__global__ __launch_bounds__(256) void fp16_attention_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int num_q_heads, int num_kv_heads, int capacity,
    int context_len, int num_splits, int tokens_per_split, Partials part) {
    constexpr int CH = 32;   // tokens per wave chunk (8 per 16-lane group)
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wo[4][G][kHeadDim];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int grp = lane >> 4;      // which of the 4 tokens of a row quad
    const int sl = lane & 15;       // channels 8*sl .. 8*sl+7
    constexpr float kScale = 1.4426950408889634f * kInvSqrtD;

    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + h;
        unpack8(reinterpret_cast<const uint4*>(q + vec * kHeadDim)[sl], qf[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] *= kScale;
    }

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    const int t_begin = split * tokens_per_split;
    const int t_end = min(context_len, t_begin + tokens_per_split);
    const size_t row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity;
    const uint4* k4 = reinterpret_cast<const uint4*>(k);
    const uint4* v4 = reinterpret_cast<const uint4*>(v);

    for (int base = t_begin + wave * CH; base < t_end; base += 4 * CH) {
        float s[8][G];
        uint4 kr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = base + 4 * i + grp;
            kr[i] = (t < t_end) ? k4[(row0 + t) * (kHeadDim / 8) + sl] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float kf[8];
            unpack8(kr[i], kf);
            const bool ok = base + 4 * i + grp < t_end;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += qf[h][e] * kf[e];
                d += __shfl_xor(d, 1, kWave);
                d += __shfl_xor(d, 2, kWave);
                d += __shfl_xor(d, 4, kWave);
                d += __shfl_xor(d, 8, kWave);
                s[i][h] = ok ? d : -INFINITY;
            }
        }
        uint4 vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = base + 4 * i + grp;
            vr[i] = (t < t_end) ? v4[(row0 + t) * (kHeadDim / 8) + sl] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float cmax = s[0][h];
#pragma unroll
            for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, s[i][h]);
            const float m_new = fmaxf(m[h], cmax);
            const float a = scale_of(m[h], m_new);
            l[h] *= a;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= a;
            m[h] = m_new;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float vf[8];
            unpack8(vr[i], vf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = (s[i][h] == -INFINITY) ? 0.f : exp2f(s[i][h] - m[h]);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] += p * vf[e];
            }
        }
    }

    // merge the 4 row groups of the wave (lanes differing in bits 4 and 5)
#pragma unroll
    for (int step = 16; step <= 32; step <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], step, kWave);
            const float lo = __shfl_xor(l[h], step, kWave);
            const float mm = fmaxf(m[h], mo);
            const float a = scale_of(m[h], mm), ao = scale_of(mo, mm);
            l[h] = a * l[h] + ao * lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float oo = __shfl_xor(o[h][e], step, kWave);
                o[h][e] = a * o[h][e] + ao * oo;
            }
            m[h] = mm;
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wo[wave][h][8 * sl + e] = o[h][e];
            if (lane == 0) {
                wm[wave][h] = m[h];
                wl[wave][h] = l[h];
            }
        }
    }
    __syncthreads();
    const size_t pbase = (static_cast<size_t>(b) * num_q_heads + g * G) * num_splits + split;
    if (tid < kHeadDim) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mm = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
            float lsum = 0.f, osum = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a = scale_of(wm[w][h], mm);
                lsum += a * wl[w][h];
                osum += a * wo[w][h][tid];
            }
            const size_t pi = pbase + static_cast<size_t>(h) * num_splits;
            part.o[pi * kHeadDim + tid] = osum;
            if (tid == 0) {
                part.m[pi] = mm;
                part.l[pi] = lsum;
            }
        }
    }
}

hipError_t launch_fp16_attention_splits(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, Partials part, hipStream_t stream) {
    const dim3 grid(s.num_splits, s.num_kv_heads, s.batch);
    const int group = s.num_q_heads / s.num_kv_heads;
#define VQKV_LAUNCH(GG)                                                                       \
    case GG:                                                                                  \
        hipLaunchKernelGGL((fp16_attention_split_kernel<GG>), grid, dim3(256), 0, stream, q, k, \
                           v, s.num_q_heads, s.num_kv_heads, s.capacity, s.context_len,       \
                           s.num_splits, s.tokens_per_split, part);                            \
        break;
    switch (group) {
        VQKV_LAUNCH(1)
        VQKV_LAUNCH(2)
        VQKV_LAUNCH(3)
        VQKV_LAUNCH(4)
        VQKV_LAUNCH(5)
        VQKV_LAUNCH(6)
        VQKV_LAUNCH(7)
        VQKV_LAUNCH(8)
        default:
            return hipErrorInvalidValue;
    }
#undef VQKV_LAUNCH
    return hipGetLastError();
}

}  // namespace vqkv
