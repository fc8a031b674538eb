// Generic split-K decode attention over a VQ cache (any G <= 8, 8- or 12-bit
// key codes).  One workgroup streams one contiguous token range of one
// (sequence, KV head) and writes base-2 online-softmax partials for the G
// query heads that share that KV head.
//
// VecInfer page: Method details (VQ KV cache in attention) for the
// arithmetic; Appendix (FlashAttention block recurrence, Algorithm 1) for the
// tiled online softmax; the grid is (splits, KV heads, batch) in the spirit of
// the page's (batch_size, num_heads, num_splits) grid.
//
// Per tile of 256 tokens:
//   A. thread t loads token t's key-code row from HBM, looks each code up in
//      the LDS copy of C_k and dots the centroid with q~ (scores in base-2
//      units; q~ is computed in the prologue by a wave FWHT);
//   B. block max, rescale factors, p = 2^(s - m) into LDS;
//   C. thread (position, slice) accumulates p-weighted V centroids for all G
//      heads of its 4 output channels over the tile's tokens of its slice.
#include <type_traits>

#include "launchers.hpp"

namespace vqkv {

namespace {

template <int KBITS>
struct KCodebookLds {
    // 8-bit codebooks are expanded to fp32 (4 KiB); 12-bit ones stay fp16
    // (32 KiB) and are widened at each lookup.
    using Entry = typename std::conditional<KBITS == 8, float4, uint2>::type;
};

__device__ __forceinline__ float4 widen(const float4 c) { return c; }
__device__ __forceinline__ float4 widen(const uint2 c) {
    return make_float4(half_bits_to_float(c.x & 0xffffu), half_bits_to_float(c.x >> 16),
                       half_bits_to_float(c.y & 0xffffu), half_bits_to_float(c.y >> 16));
}

template <int KBITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int p) {
    if constexpr (KBITS == 8) {
        return (w[p >> 2] >> ((p & 3) * 8)) & 0xffu;
    } else {
        const int bit = 12 * p;
        const int lo = bit >> 5;
        const int sh = bit & 31;
        uint32_t v = w[lo] >> sh;
        if (sh > 20) v |= w[lo + 1] << (32 - sh);
        return v & 0xfffu;
    }
}

}  // namespace

template <int G, int KBITS>
__global__ __launch_bounds__(256) void vq_attention_split_kernel(
    const void* __restrict__ q, int q_f32, const float* __restrict__ lambda,
    const uint16_t* __restrict__ cb_k, const uint16_t* __restrict__ cb_v,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v, int num_q_heads,
    int num_kv_heads, int capacity, int context_len, int num_splits, int tokens_per_split,
    Partials part) {
    constexpr int KROW = kNumSub * KBITS / 8;          // bytes per key-code row
    constexpr int KWORDS = KROW / 4;
    constexpr int KENT = 1 << KBITS;
    using KEntry = typename KCodebookLds<KBITS>::Entry;

    __shared__ float qs[G][kHeadDim];
    __shared__ KEntry ck[KENT];
    __shared__ float4 cv[256];
    __shared__ uint4 vtile[kVqTile * 2];
    __shared__ float pt[kVqTile * G];
    __shared__ float red[4][G];
    __shared__ float obuf[8][kHeadDim];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // ---- prologue: codebooks into LDS, q~ for the G heads -------------------
    {
        const uint2* src = reinterpret_cast<const uint2*>(cb_k) + static_cast<size_t>(g) * KENT;
        for (int i = tid; i < KENT; i += 256) {
            const uint2 raw = src[i];
            if constexpr (KBITS == 8) ck[i] = widen(raw); else ck[i] = raw;
        }
        const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
        cv[tid] = widen(vsrc[tid]);
    }
    for (int h = wave; h < G; h += 4) {
        const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + h;
        float x0, x1;
        if (q_f32) {
            const float2 v = reinterpret_cast<const float2*>(q)[vec * (kHeadDim / 2) + lane];
            x0 = v.x;
            x1 = v.y;
        } else {
            const uint32_t w = reinterpret_cast<const uint32_t*>(q)[vec * (kHeadDim / 2) + lane];
            x0 = half_bits_to_float(static_cast<uint16_t>(w & 0xffffu));
            x1 = half_bits_to_float(static_cast<uint16_t>(w >> 16));
        }
        const float2 l = reinterpret_cast<const float2*>(lambda + g * kHeadDim)[lane];
        x0 *= l.x;
        x1 *= l.y;
        wave_fwht128(x0, x1);
        qs[h][2 * lane] = x0 * kScoreScaleLog2;
        qs[h][2 * lane + 1] = x1 * kScoreScaleLog2;
    }
    __syncthreads();

    const int t_begin = split * tokens_per_split;
    const int t_end = min(context_len, t_begin + tokens_per_split);
    const size_t stream_row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity;

    float m_run[G], l_part[G], acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_part[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][j] = 0.f;
    }
    const int pos = tid & 31;
    const int slice = tid >> 5;

    for (int tile = t_begin; tile < t_end; tile += kVqTile) {
        const int n_tile = min(kVqTile, t_end - tile);
        const bool valid = tid < n_tile;
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
        // ---- A: scores ------------------------------------------------------
        if (valid) {
            const size_t row = stream_row0 + tile + tid;
            uint32_t w[KWORDS];
            const uint4* kr = reinterpret_cast<const uint4*>(codes_k + row * KROW);
#pragma unroll
            for (int i = 0; i < KWORDS / 4; ++i) {
                const uint4 u = kr[i];
                w[4 * i] = u.x;
                w[4 * i + 1] = u.y;
                w[4 * i + 2] = u.z;
                w[4 * i + 3] = u.w;
            }
            const uint4* vr = reinterpret_cast<const uint4*>(codes_v + row * kNumSub);
            vtile[2 * tid] = vr[0];
            vtile[2 * tid + 1] = vr[1];
#pragma unroll
            for (int p = 0; p < kNumSub; ++p) {
                const float4 c = widen(ck[code_at<KBITS>(w, p)]);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float4 qq = *reinterpret_cast<const float4*>(&qs[h][4 * p]);
                    s[h] += qq.x * c.x + qq.y * c.y + qq.z * c.z + qq.w * c.w;
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = -INFINITY;
        }
        // ---- B: online softmax ---------------------------------------------
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float wm = wave_max(s[h]);
            if (lane == 0) red[wave][h] = wm;
        }
        __syncthreads();
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float tmax = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
            const float m_new = fmaxf(m_run[h], tmax);       // finite: the tile has a token
            alpha[h] = exp2f(m_run[h] - m_new);               // 0 on the first tile
            const float p = valid ? exp2f(s[h] - m_new) : 0.f;
            pt[tid * G + h] = p;
            l_part[h] = l_part[h] * alpha[h] + p;
            m_run[h] = m_new;
        }
        __syncthreads();
        // ---- C: p-weighted V centroids ---------------------------------------
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[h][j] *= alpha[h];
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(vtile);
        for (int t = slice; t < n_tile; t += 8) {
            const float4 c = cv[vb[t * kNumSub + pos]];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = pt[t * G + h];
                acc[h][0] += p * c.x;
                acc[h][1] += p * c.y;
                acc[h][2] += p * c.z;
                acc[h][3] += p * c.w;
            }
        }
        __syncthreads();
    }

    // ---- epilogue: block-reduce l and o, write the split partials ----------
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float ws = wave_sum(l_part[h]);
        if (lane == 0) red[wave][h] = ws;
    }
    __syncthreads();
    const size_t pbase = (static_cast<size_t>(b) * num_q_heads + g * G) * num_splits + split;
    if (tid == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            part.m[pbase + static_cast<size_t>(h) * num_splits] = m_run[h];
            part.l[pbase + static_cast<size_t>(h) * num_splits] =
                red[0][h] + red[1][h] + red[2][h] + red[3][h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        *reinterpret_cast<float4*>(&obuf[slice][4 * pos]) =
            make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        __syncthreads();
        if (tid < kHeadDim) {
            float o = 0.f;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) o += obuf[sl][tid];
            part.o[(pbase + static_cast<size_t>(h) * num_splits) * kHeadDim + tid] = o;
        }
        __syncthreads();
    }
}

namespace {

template <int KBITS>
hipError_t launch_g(int group, dim3 grid, const AttnShape& s, const void* q, bool q_f32,
                    const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                    const uint8_t* codes_k, const uint8_t* codes_v, Partials part,
                    hipStream_t stream) {
#define VQKV_LAUNCH(GG)                                                                     \
    case GG:                                                                                \
        hipLaunchKernelGGL((vq_attention_split_kernel<GG, KBITS>), grid, dim3(256), 0,      \
                           stream, q, q_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v, \
                           s.num_q_heads, s.num_kv_heads, s.capacity, s.context_len,        \
                           s.num_splits, s.tokens_per_split, part);                          \
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

}  // namespace

hipError_t launch_vq_attention_splits(const AttnShape& s, int k_bits, const void* q, bool q_f32,
                                      const float* lambda, const uint16_t* cb_k,
                                      const uint16_t* cb_v, const uint8_t* codes_k,
                                      const uint8_t* codes_v, Partials part,
                                      hipStream_t stream) {
    const dim3 grid(s.num_splits, s.num_kv_heads, s.batch);
    const int group = s.num_q_heads / s.num_kv_heads;
    if (k_bits == 8)
        return launch_g<8>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k, codes_v, part,
                           stream);
    return launch_g<12>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k, codes_v, part,
                        stream);
}

// ---- cross-split log-sum-exp merge (one workgroup per (sequence, q head)) ----
__global__ __launch_bounds__(128) void merge_splits_kernel(int num_splits, Partials part,
                                                           float* __restrict__ out) {
    const size_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* m = part.m + bh * num_splits;
    const float* l = part.l + bh * num_splits;
    const float* o = part.o + bh * num_splits * kHeadDim;
    float mx = -INFINITY;
    for (int s = 0; s < num_splits; ++s) mx = fmaxf(mx, m[s]);
    float den = 0.f, num = 0.f;
    for (int s = 0; s < num_splits; ++s) {
        const float ms = m[s];
        const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
        den += w * l[s];
        num += w * o[static_cast<size_t>(s) * kHeadDim + d];
    }
    out[bh * kHeadDim + d] = num / den;
}

hipError_t launch_merge_splits(int batch, int num_q_heads, int num_splits, Partials part,
                               float* out, hipStream_t stream) {
    hipLaunchKernelGGL(merge_splits_kernel, dim3(batch * num_q_heads), dim3(kHeadDim), 0, stream,
                       num_splits, part, out);
    return hipGetLastError();
}

}  // namespace vqkv
