// Split-K decode attention over a VQ cache on the gfx950 matrix cores.
//
// What is computed (VecInfer page, Method details, "VQ KV cache in attention"):
//   s = q~ VQ^-1(K~_q, C_k)^T / sqrt(D),  p = softmax(s),  o = p VQ^-1(V_q, C_v)
// with q~ = q diag(lambda) H_D.  The tiled online softmax follows the page's
// Appendix (FlashAttention block recurrence, Algorithm 1): running max m,
// running sum l, rescaled output accumulator, final o / l.
//
// How it maps to gfx950 (one workgroup = 8 waves = one contiguous token range
// of one (sequence, KV head); one wave = 32-token tiles):
//  * Both products are dense contractions once a centroid is looked up, so
//    both run on v_mfma_f32_16x16x32_f16.  The 16 MFMA rows are (head, part):
//    every fp32 operand that is not exact in fp16 (q~ and p) is split into
//    hi = fp16(x) and lo = fp16(x - hi) and the two rows are summed after the
//    product; codebook entries are fp16 already.  Accuracy is that of fp32.
//  * Scores: B operand = the 8 fp16 values of two key centroids per lane,
//    read from LDS with one 8-byte gather each.
//  * Values: the MFMA wants 8 tokens x 1 channel per lane, a gather gives
//    1 token x 4 channels.  ds_read_b64_tr_b16 does both at once: every lane
//    supplies the address of one centroid and the hardware returns, to lane
//    16G+4a+e, channel e of the centroids fetched by lanes 16G+4k+a, k=0..3.
//  * The codebooks live in a 64 KiB LDS table with one 256-byte row per code:
//    16 copies of the key centroid then 16 copies of the value centroid, so
//    lane n of every 16-lane group reads its own copy (slot n): the gathers
//    are bank-conflict free for any codes, and the address
//    (code << 8) | slot is one v_perm_b32 of the loaded code bytes.  (12-bit
//    key codebooks, 4096 x 8 B, fill the 16 key slots of all 256 rows.)
//  * Code rows stay token-major in HBM; every load is 8 contiguous bytes per
//    lane and the scores and values each read a wave's tile once.
//  * The cross-split log-sum-exp merge runs in the same kernel: the last
//    workgroup of each (sequence, KV head) to finish (device-scope atomic
//    ticket) merges all split partials for its G heads.
#include "launchers.hpp"

namespace vqkv {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kTok = 32;                  // tokens per wave tile
constexpr float kTau = 8.0f;              // lazy-rescale slack (log2 units)
constexpr int kRow = 256;                 // bytes per code row of the LDS table
constexpr int kVOff = 128;                // value slots start here in a row

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// ds_read_b64_tr_b16 at an LDS byte address
__device__ __forceinline__ half4_t read_tr16(const uint8_t* p) {
    return __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a DPP row, result in every lane of the row
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0x128>(x));   // row_ror:8
    x = fmaxf(x, dpp<0x124>(x));   // row_ror:4
    x = fmaxf(x, dpp<0x122>(x));   // row_ror:2
    x = fmaxf(x, dpp<0x121>(x));   // row_ror:1
    return x;
}
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x122>(x);
    x += dpp<0x121>(x);
    return x;
}

// LDS address (code << 8) | slot, code = byte k of w: one v_perm_b32
template <int K>
__device__ __forceinline__ uint32_t row_addr(uint32_t w, uint32_t slot) {
    return __builtin_amdgcn_perm(w, slot, 0x0C0C0000u | ((4u + K) << 8));
}

__device__ __forceinline__ half8_t cat(uint2 a, uint2 b) {
    return __builtin_bit_cast(half8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// 2^x with the hardware exponential (results below 2^-126 flush to 0, which
// only drops weights that are negligible next to the running sum >= 1)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float rescale_factor(float m_old, float m_new) {
    return (m_new == -INFINITY) ? 1.f : fast_exp2(m_old - m_new);
}

// hi/lo fp16 pair of x (two halves packed: lo half = hi part, high half = lo part)
__device__ __forceinline__ uint32_t split_hi_lo(float x) {
    const _Float16 hi = static_cast<_Float16>(x);
    const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) << 16);
}

// the 8 key codes of positions 8*grp .. 8*grp+7 of one token
template <int KBITS>
struct KChunk;

template <>
struct KChunk<8> {
    uint2 w;
    __device__ void load(const uint8_t* row, int grp) {
        w = *reinterpret_cast<const uint2*>(row + 8 * grp);
    }
    __device__ void clear() { w = make_uint2(0, 0); }
    // LDS address of the key centroid for position 8*grp + i
    template <int I>
    __device__ uint32_t addr(uint32_t slot) const {
        return row_addr<I & 3>(I < 4 ? w.x : w.y, slot);
    }
};

template <>
struct KChunk<12> {
    uint32_t w0, w1, w2;   // 96 bits: 8 codes of 12 bits, little-endian
    __device__ void load(const uint8_t* row, int grp) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 12 * grp);
        w0 = p[0];
        w1 = p[1];
        w2 = p[2];
    }
    __device__ void clear() { w0 = w1 = w2 = 0; }
    template <int I>
    __device__ uint32_t addr(uint32_t slot) const {
        constexpr int bit = 12 * I, lo = bit >> 5, sh = bit & 31;
        const uint32_t a = lo == 0 ? w0 : (lo == 1 ? w1 : w2);
        uint32_t code;
        if constexpr (sh + 12 <= 32) {
            code = __builtin_amdgcn_ubfe(a, sh, 12);
        } else {
            const uint32_t b = lo == 0 ? w1 : w2;
            code = __builtin_amdgcn_alignbit(b, a, sh) & 0xfffu;
        }
        // entry e of a 4096-entry table sits at row e >> 4, key slot e & 15
        (void)slot;
        return ((code & 0xff0u) << 4) | ((code & 0xfu) << 3);
    }
};

}  // namespace

template <int G, int KBITS>
__global__ __launch_bounds__(kWaves * 64, 4) void vq_attention_mfma_kernel(
    const void* __restrict__ q, int q_f32, const float* __restrict__ lambda,
    const uint16_t* __restrict__ cb_k, const uint16_t* __restrict__ cb_v,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v, int num_q_heads,
    int num_kv_heads, int capacity, int context_len, int num_splits, int tokens_per_split,
    Partials part, uint32_t* __restrict__ tickets, float* __restrict__ out) {
    static_assert(G >= 1 && G <= 8, "2G MFMA rows");
    constexpr int KROW = kNumSub * KBITS / 8;

    __shared__ __attribute__((aligned(16))) uint8_t tab[256 * kRow];
    __shared__ __attribute__((aligned(16))) uint2 pbuf[kWaves][kTok * 4];   // [token][16 rows] fp16
    __shared__ half8_t qa[4][64];
    // q~ (fp32) lives in the p buffers during the prologue
    static_assert(sizeof(float) * G * kHeadDim <= sizeof(uint2) * kWaves * kTok * 4, "qsh fits");
    float (*qsh)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(&pbuf[0][0]);
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ uint32_t last_flag;

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, n = lane & 15;

    // ---- prologue: codebook table, q~ --------------------------------------
    {
        const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
        const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
        if constexpr (KBITS == 8) {
            const int code = tid >> 1;
            const uint2 c = (tid & 1) ? vsrc[code] : ksrc[code];
            uint4* dst = reinterpret_cast<uint4*>(tab + code * kRow + (tid & 1) * kVOff);
            const uint4 cc = make_uint4(c.x, c.y, c.x, c.y);
#pragma unroll
            for (int s = 0; s < 8; ++s) dst[s] = cc;
        } else {
            for (int e = tid; e < 4096; e += kWaves * 64)
                *reinterpret_cast<uint2*>(tab + (e >> 4) * kRow + (e & 15) * 8) = ksrc[e];
            if (tid < 256) {
                const uint2 c = vsrc[tid];
                uint4* dst = reinterpret_cast<uint4*>(tab + tid * kRow + kVOff);
                const uint4 cc = make_uint4(c.x, c.y, c.x, c.y);
#pragma unroll
                for (int s = 0; s < 8; ++s) dst[s] = cc;
            }
        }
    }
    if (wave < G) {
        const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + wave;
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
        qsh[wave][2 * lane] = x0 * kScoreScaleLog2;
        qsh[wave][2 * lane + 1] = x1 * kScoreScaleLog2;
    }
    __syncthreads();

    // score A operand, shared by all waves through LDS: lane (16 grp + r)
    // holds row r = 2h + part of q~ for dims 32 grp + 8 kk + e (K-step kk,
    // element e); part 0 = hi, 1 = lo; rows of heads >= G are zero
    if (wave == 0) {
        const int r = n;
        const int h = r >> 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            half8_t a;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = 0.f;
                if (h < G) x = qsh[h][32 * grp + 8 * kk + e];
                const _Float16 hi = static_cast<_Float16>(x);
                a[e] = (r & 1) ? static_cast<_Float16>(x - static_cast<float>(hi)) : hi;
            }
            qa[kk][lane] = a;
        }
    }
    __syncthreads();

    const int t_begin = split * tokens_per_split;
    const int t_end = min(context_len, t_begin + tokens_per_split);
    const size_t row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity;
    const uint8_t* kbase = codes_k + row0 * KROW;
    const uint8_t* vbase = codes_v + row0 * kNumSub;
    const uint32_t kslot = static_cast<uint32_t>(n) * 8;
    const uint32_t vslot = kVOff + static_cast<uint32_t>(n) * 8;
    const int kq = n >> 2, aq4 = n & 3;   // fetch-lane split of n for the transposed reads

    // heads of this lane's MFMA output rows: rows 4 grp .. 4 grp + 3 = (hA hi,
    // hA lo, hB hi, hB lo)
    const int hA = 2 * grp, hB = 2 * grp + 1;
    const bool validA = hA < G, validB = hB < G;

    float mA = -INFINITY, mB = -INFINITY, lA = 0.f, lB = 0.f;
    float4_t oacc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    uint2* pw = pbuf[wave];
    const uint8_t* pw_bytes = reinterpret_cast<const uint8_t*>(pw);

    // Code loads: 8 bytes per lane per chunk, rows clamped into the split so
    // every load is unconditional (masked tokens are discarded by the scores).
    // (uniform 64-bit base of the split + 32-bit per-lane offsets)
    const uint8_t* ksplit = kbase + static_cast<size_t>(t_begin) * KROW;
    const uint8_t* vsplit = vbase + static_cast<size_t>(t_begin) * kNumSub;
    const int t_last = t_end - 1 - t_begin;
    auto load_tile = [&](int tile, KChunk<KBITS>* kk_, uint2* vv_) {
        const int rel = tile - t_begin;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const uint32_t t = static_cast<uint32_t>(min(rel + 16 * sb + n, t_last));
            kk_[sb].load(ksplit + t * KROW, grp);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t t = static_cast<uint32_t>(min(rel + 8 * grp + 4 * j + kq, t_last));
            vv_[j] = *reinterpret_cast<const uint2*>(vsplit + t * kNumSub + 8 * aq4);
        }
    };

    auto compute_tile = [&](int tile, const KChunk<KBITS>* kc, const uint2* vc) {
        // ---- scores: 2 blocks of 16 tokens, 4 K-steps of 32 dims ------------
        float4_t sacc[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            sacc[sb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; kk += 2) {
                uint2 kg[4];
                if (kk == 0) {
                    kg[0] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<0>(kslot));
                    kg[1] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<1>(kslot));
                    kg[2] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<2>(kslot));
                    kg[3] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<3>(kslot));
                } else {
                    kg[0] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<4>(kslot));
                    kg[1] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<5>(kslot));
                    kg[2] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<6>(kslot));
                    kg[3] = *reinterpret_cast<const uint2*>(tab + kc[sb].template addr<7>(kslot));
                }
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk][lane], cat(kg[0], kg[1]),
                                                                  sacc[sb], 0, 0, 0);
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk + 1][lane], cat(kg[2], kg[3]),
                                                                  sacc[sb], 0, 0, 0);
            }
        }

        // ---- online softmax (base 2) -----------------------------------------
        float sA[2], sB[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const bool live = tile + 16 * sb + n < t_end;
            sA[sb] = (validA && live) ? sacc[sb][0] + sacc[sb][1] : -INFINITY;
            sB[sb] = (validB && live) ? sacc[sb][2] + sacc[sb][3] : -INFINITY;
        }
        const float tA = row_max16(fmaxf(sA[0], sA[1]));
        const float tB = row_max16(fmaxf(sB[0], sB[1]));
        if (__builtin_amdgcn_ballot_w64(tA > mA + kTau || tB > mB + kTau) != 0) {
            const float nA = fmaxf(mA, tA), nB = fmaxf(mB, tB);
            const float fA = rescale_factor(mA, nA), fB = rescale_factor(mB, nB);
            mA = nA;
            mB = nB;
            lA *= fA;
            lB *= fB;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                oacc[c][0] *= fA;
                oacc[c][1] *= fA;
                oacc[c][2] *= fB;
                oacc[c][3] *= fB;
            }
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            // 0 for masked tokens; padded rows (head >= G) stay 0 too
            const float pA = validA ? fast_exp2(sA[sb] - mA) : 0.f;
            const float pB = validB ? fast_exp2(sB[sb] - mB) : 0.f;
            lA += pA;
            lB += pB;
            // token 16 sb + n, rows 4 grp .. 4 grp + 3
            pw[(16 * sb + n) * 4 + grp] = make_uint2(split_hi_lo(pA), split_hi_lo(pB));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // V A operand: lane (16 grp + r) gets p rows r of tokens 8 grp .. 8 grp + 7
        half8_t ap;
        {
            const half4_t x0 = read_tr16(pw_bytes + (8 * grp + kq) * 32 + aq4 * 8);
            const half4_t x1 = read_tr16(pw_bytes + (8 * grp + 4 + kq) * 32 + aq4 * 8);
            ap = half8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }

        // ---- values: 8 N-tiles of 16 channels, gathered 2 tiles at a time ------
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint32_t w0 = (q4 < 2) ? vc[0].x : vc[0].y;
            const uint32_t w1 = (q4 < 2) ? vc[1].x : vc[1].y;
            half4_t x[2][2];
            if ((q4 & 1) == 0) {
                x[0][0] = read_tr16(tab + row_addr<0>(w0, vslot));
                x[0][1] = read_tr16(tab + row_addr<0>(w1, vslot));
                x[1][0] = read_tr16(tab + row_addr<1>(w0, vslot));
                x[1][1] = read_tr16(tab + row_addr<1>(w1, vslot));
            } else {
                x[0][0] = read_tr16(tab + row_addr<2>(w0, vslot));
                x[0][1] = read_tr16(tab + row_addr<2>(w1, vslot));
                x[1][0] = read_tr16(tab + row_addr<3>(w0, vslot));
                x[1][1] = read_tr16(tab + row_addr<3>(w1, vslot));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const half8_t bv = half8_t{x[i][0][0], x[i][0][1], x[i][0][2], x[i][0][3],
                                           x[i][1][0], x[i][1][1], x[i][1][2], x[i][1][3]};
                oacc[2 * q4 + i] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, bv, oacc[2 * q4 + i], 0, 0, 0);
            }
        }
    };

    // two register sets, alternating: load the next tile, then compute the
    // current one, so one tile of code loads is always in flight
    const int stride = kWaves * kTok;
    int tile = t_begin + wave * kTok;
    if (tile < t_end) {
        KChunk<KBITS> kA[2], kB[2];
        uint2 vA[2], vB[2];
        load_tile(tile, kA, vA);
        for (;;) {
            load_tile(tile + stride, kB, vB);
            compute_tile(tile, kA, vA);
            tile += stride;
            if (tile >= t_end) break;
            load_tile(tile + stride, kA, vA);
            compute_tile(tile, kB, vB);
            tile += stride;
            if (tile >= t_end) break;
        }
    }

    // ---- merge the 8 waves of the workgroup ----------------------------------
    lA = row_sum16(lA);
    lB = row_sum16(lB);
    __syncthreads();                                      // everyone is done with tab
    float* obuf = reinterpret_cast<float*>(tab);          // [kWaves][G][128]
    if (n == 0) {
        if (validA) { wm[wave][hA] = mA; wl[wave][hA] = lA; }
        if (validB) { wm[wave][hB] = mB; wl[wave][hB] = lB; }
    }
    // lane (16 grp + 4 a + e), tile c: channel 32 a + 4 c + e; rows (hA, hB) hi + lo
    {
        const int a = n >> 2, e = n & 3;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int d = 32 * a + 4 * c + e;
            if (validA) obuf[(wave * G + hA) * kHeadDim + d] = oacc[c][0] + oacc[c][1];
            if (validB) obuf[(wave * G + hB) * kHeadDim + d] = oacc[c][2] + oacc[c][3];
        }
    }
    __syncthreads();
    const size_t pbase = (static_cast<size_t>(b) * num_q_heads + g * G) * num_splits + split;
    for (int i = tid; i < G * kHeadDim; i += kWaves * 64) {
        const int h = i / kHeadDim, d = i % kHeadDim;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][h]);
        float ls = 0.f, os = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (wm[w][h] == -INFINITY) ? 0.f : exp2f(wm[w][h] - mx);
            ls += f * wl[w][h];
            os += f * obuf[(w * G + h) * kHeadDim + d];
        }
        const size_t pi = pbase + static_cast<size_t>(h) * num_splits;
        part.o[pi * kHeadDim + d] = os;
        if (d == 0) {
            part.m[pi] = mx;
            part.l[pi] = ls;
        }
    }

    // ---- last workgroup of this (sequence, KV head) merges all splits -------
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t prev = atomicAdd(&tickets[static_cast<size_t>(b) * num_kv_heads + g], 1u);
        last_flag = (prev == static_cast<uint32_t>(num_splits - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (last_flag == 0u) return;
    __threadfence();
    const size_t hbase = (static_cast<size_t>(b) * num_q_heads + g * G) * num_splits;
    for (int i = tid; i < G * kHeadDim; i += kWaves * 64) {
        const int h = i / kHeadDim, d = i % kHeadDim;
        const float* m = part.m + hbase + static_cast<size_t>(h) * num_splits;
        const float* l = part.l + hbase + static_cast<size_t>(h) * num_splits;
        const float* o = part.o + (hbase + static_cast<size_t>(h) * num_splits) * kHeadDim + d;
        float mx = -INFINITY;
        for (int s = 0; s < num_splits; ++s) mx = fmaxf(mx, m[s]);
        float den = 0.f, num = 0.f;
        for (int s = 0; s < num_splits; ++s) {
            const float ms = m[s];
            const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
            den += f * l[s];
            num += f * o[static_cast<size_t>(s) * kHeadDim];
        }
        out[(static_cast<size_t>(b) * num_q_heads + g * G + h) * kHeadDim + d] = num / den;
    }
    if (tid == 0) tickets[static_cast<size_t>(b) * num_kv_heads + g] = 0u;   // ready for the next call
}

namespace {

template <int KBITS>
hipError_t launch_mfma_g(int group, dim3 grid, const AttnShape& s, const void* q, bool q_f32,
                         const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                         const uint8_t* codes_k, const uint8_t* codes_v, Partials part,
                         uint32_t* tickets, float* out, hipStream_t stream) {
#define VQKV_LAUNCH(GG)                                                                        \
    case GG:                                                                                   \
        hipLaunchKernelGGL((vq_attention_mfma_kernel<GG, KBITS>), grid, dim3(kWaves * 64), 0,  \
                           stream, q, q_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,    \
                           s.num_q_heads, s.num_kv_heads, s.capacity, s.context_len,           \
                           s.num_splits, s.tokens_per_split, part, tickets, out);              \
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

hipError_t launch_vq_attention_fused(const AttnShape& s, int k_bits, const void* q, bool q_f32,
                                     const float* lambda, const uint16_t* cb_k,
                                     const uint16_t* cb_v, const uint8_t* codes_k,
                                     const uint8_t* codes_v, Partials part, uint32_t* tickets,
                                     float* out, hipStream_t stream) {
    const dim3 grid(s.num_splits, s.num_kv_heads, s.batch);
    const int group = s.num_q_heads / s.num_kv_heads;
    if (k_bits == 8)
        return launch_mfma_g<8>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k, codes_v,
                                part, tickets, out, stream);
    return launch_mfma_g<12>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k, codes_v,
                             part, tickets, out, stream);
}

}  // namespace vqkv
