// Uncompressed comparator: split-K decode attention over an fp16 KV cache,
// o = softmax(q K^T / sqrt(128)) V with fp32 accumulation (VecInfer page,
// Background: KV cache and attention).  Same split partials and merge as the
// VQ kernels.
//
// A 16-lane DPP row owns one token at a time (8 channels per lane, one
// 16-byte load per lane per row of K or V), so a wave instruction moves 4
// whole 256-byte rows.  Each wave takes 16-token chunks (4 tokens per row);
// both K and V of a chunk are requested before any is used.  Scores are
// fp16 x fp16 dot products accumulated in fp32 (v_dot2_f32_f16) and summed
// over the row by DPP; every row keeps its own online-softmax state, merged
// across rows and waves at the end.  Registers stay near 100 per lane, so
// 4 waves per SIMD keep loads in flight.
#include "launchers.hpp"

namespace vqkv {

namespace {

typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2v_t as_half2(uint32_t w) {
    return __builtin_bit_cast(half2v_t, w);
}

__device__ __forceinline__ float scale_of(float m_old, float m_new) {
    return (m_old == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
}

}  // namespace

template <int G>
__global__ __launch_bounds__(256) void fp16_attention_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int num_q_heads, int num_kv_heads, int capacity,
    int context_len, int num_splits, int tokens_per_split, Partials part) {
    constexpr int CH = 16;   // tokens per wave chunk: 4 per 16-lane row
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wo[4][G][kHeadDim];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int grp = lane >> 4;      // row of the wave: token 4 i + grp of a chunk
    const int sl = lane & 15;       // channels 8 sl .. 8 sl + 7
    constexpr float kScale = 1.4426950408889634f * kInvSqrtD;   // base-2 scores

    uint4 qh[G];                    // q as stored (fp16), this lane's 8 channels
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + h;
        qh[h] = reinterpret_cast<const uint4*>(q + vec * kHeadDim)[sl];
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
    const int t_end = t_begin + min(tokens_per_split, context_len - t_begin);   // no int overflow
    const size_t row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity;
    const uint4* k4 = reinterpret_cast<const uint4*>(k);
    const uint4* v4 = reinterpret_cast<const uint4*>(v);

    for (int base = t_begin + wave * CH; base < t_end; base += 4 * CH) {
        uint4 kr[4], vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = base + 4 * i + grp;
            const size_t r = (row0 + min(t, t_end - 1)) * (kHeadDim / 8) + sl;
            kr[i] = k4[r];
            vr[i] = v4[r];
        }
        float s[4][G];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = base + 4 * i + grp < t_end;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = __builtin_amdgcn_fdot2(as_half2(qh[h].x), as_half2(kr[i].x), 0.f, false);
                d = __builtin_amdgcn_fdot2(as_half2(qh[h].y), as_half2(kr[i].y), d, false);
                d = __builtin_amdgcn_fdot2(as_half2(qh[h].z), as_half2(kr[i].z), d, false);
                d = __builtin_amdgcn_fdot2(as_half2(qh[h].w), as_half2(kr[i].w), d, false);
                d = row_sum16(d) * kScale;
                s[i][h] = ok ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float cmax = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
            const float m_new = fmaxf(m[h], cmax);
            if (m_new != m[h]) {
                const float a = scale_of(m[h], m_new);
                l[h] *= a;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] *= a;
                m[h] = m_new;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = (s[i][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[i][h] - m[h]);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[h][2 * e] += p * half_bits_to_float(static_cast<uint16_t>(vw[e] & 0xffffu));
                    o[h][2 * e + 1] += p * half_bits_to_float(static_cast<uint16_t>(vw[e] >> 16));
                }
            }
        }
    }

    // merge the 4 rows of the wave (lanes differing in bits 4 and 5); l is
    // the same in every lane of a row
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
