// Nearest-centroid encoder for appended tokens.
//
// VecInfer page, Method details (VQ KV cache in attention): a new key gets
// the online dual transform k~ = k diag(lambda)^-1 H_D and is quantised with
// C_k; its value is quantised untransformed with C_v; the codes are
// concatenated to the cache.  Background (VQ principle): every 4-channel
// sub-vector x gets j* = argmin_j ||x - C_j||^2.
//
// The decision is the one the fp64 reference takes (squared distances in
// fp64 with every difference, product and sum rounded separately, exact ties
// to the lowest index), found by the certified matrix-core search of
// nearest_search.hpp with the transformed keys and the values rounded to fp32
// for the scores and kept in fp64 for the few exact distances.
//
// One 512-thread workgroup encodes up to 8 tokens of one (sequence, KV
// head): 256 key and 256 value sub-vectors, 16 row blocks each, spread over
// the 8 waves.  Codebooks (-2c by channel, fp32) and their bound-scaled
// squared norms are staged in LDS.
#include "launchers.hpp"
#include "nearest_search.hpp"

namespace vqkv {

namespace {

constexpr int kEncThreads = 512;
constexpr int kEncWaves = kEncThreads / kWave;     // 8
constexpr int kEncTok = 8;                          // tokens per workgroup
constexpr int kEncBlocks = kEncTok * kNumSub / 16;  // row blocks per tensor
// Threads of the d = 4 encoder: with 4096-entry C_k its tables (about
// 120 KiB of LDS) allow one workgroup per CU, so it takes 16 waves, one key
// row block each, to keep 4 waves on every SIMD; with 256 entries several
// 8-wave workgroups share a CU.
template <int KBITS>
constexpr int kEncThreadsOf = KBITS == 12 ? 1024 : 512;


__device__ __forceinline__ double load_elem(const void* p, bool f32, size_t i) {
    if (f32) return static_cast<double>(reinterpret_cast<const float*>(p)[i]);
    return static_cast<double>(half_bits_to_float(reinterpret_cast<const uint16_t*>(p)[i]));
}

// The nearest centroid of sub-vector rb*16 + lane % 16 of `xs` ([8 tokens]
// [128] fp64 = [256 sub-vectors][4]) among NENT fp16 centroids staged as -2c
// by channel (m2) and bound-scaled squared norms (cu, cd).
template <int NENT>
__device__ __forceinline__ uint32_t search_rows(const float* m2, const float* cu,
                                                const float* cd, const double (*xs)[kHeadDim],
                                                int rb, int lane) {
    const double* x = &xs[0][0] + (rb * 16 + (lane & 15)) * 4;
    const float b = static_cast<float>(x[lane >> 4]);   // B operand: channel lane / 16
    float xx = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float v = static_cast<float>(x[j]);
        xx += v * v;
    }
    // the fp16 centroid, recovered exactly from -2c; the distance rounded as
    // the fp64 reference rounds it
    const auto exact = [&](uint32_t nc) {
        double dd = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double c = -0.5 * static_cast<double>(m2[j * kSearchStride<NENT> + nc]);
            const double e = __dadd_rn(x[j], -c);
            dd = j == 0 ? __dmul_rn(e, e) : __dadd_rn(dd, __dmul_rn(e, e));
        }
        return dd;
    };
    return nearest16<NENT>(m2, cu, cd, b, row_bound(xx), lane, exact);
}

}  // namespace

template <int KBITS>
__global__ __launch_bounds__(kEncThreadsOf<KBITS>) void encode_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    constexpr int KENT = 1 << KBITS;
    constexpr int KROW = kNumSub * KBITS / 8;
    constexpr int kThr = kEncThreadsOf<KBITS>, kWv = kThr / kWave;
    // -2c by channel ([4][E], exact in fp32) and ||c||^2, per tensor
    __shared__ float km2[4 * kSearchStride<KENT>];
    __shared__ float vm2[4 * kSearchStride<256>];
    // ||c||^2 (1 + 2^-16), ||c||^2 (1 - 2^-16), read as float4
    __shared__ __align__(16) float kcu[KENT];
    __shared__ __align__(16) float kcd[KENT];
    __shared__ __align__(16) float vcu[256];
    __shared__ __align__(16) float vcd[256];
    __shared__ double xs[2][kEncTok][kHeadDim];       // transformed keys, values (fp64)
    __shared__ uint16_t code[2][kEncTok][kNumSub];

    const int t0 = blockIdx.x * kEncTok, g = blockIdx.y, b = blockIdx.z;
    const int ntok = min(kEncTok, num_new - t0);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool f32 = kv_f32 != 0;

    // codebooks (-2c by channel) and squared norms
    const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
    const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
    // every load is issued before any is used (one latency, not one per entry)
    constexpr int KPER = (KENT + kThr - 1) / kThr;
    uint2 kc[KPER];
#pragma unroll
    for (int j = 0; j < KPER; ++j) kc[j] = ksrc[min(tid + j * kThr, KENT - 1)];
    const uint2 vc = vsrc[tid & 255];
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
        const int i = tid + j * kThr;
        if (i < KENT) {
            km2[0 * kSearchStride<KENT> + i] = -2.f * half_bits_to_float(kc[j].x & 0xffffu);
            km2[1 * kSearchStride<KENT> + i] = -2.f * half_bits_to_float(kc[j].x >> 16);
            km2[2 * kSearchStride<KENT> + i] = -2.f * half_bits_to_float(kc[j].y & 0xffffu);
            km2[3 * kSearchStride<KENT> + i] = -2.f * half_bits_to_float(kc[j].y >> 16);
            const float nn = norm2(kc[j]);
            kcu[i] = nn * kBoundUp;
            kcd[i] = nn * kBoundDown;
        }
    }
    if (tid < 256) {
        vm2[0 * kSearchStride<256> + tid] = -2.f * half_bits_to_float(vc.x & 0xffffu);
        vm2[1 * kSearchStride<256> + tid] = -2.f * half_bits_to_float(vc.x >> 16);
        vm2[2 * kSearchStride<256> + tid] = -2.f * half_bits_to_float(vc.y & 0xffffu);
        vm2[3 * kSearchStride<256> + tid] = -2.f * half_bits_to_float(vc.y >> 16);
        const float nn = norm2(vc);
        vcu[tid] = nn * kBoundUp;
        vcd[tid] = nn * kBoundDown;
    }

    // k / lambda in fp64, the +-1 Walsh–Hadamard transform, then 1/sqrt(128);
    // values as they are.  Rows of tokens past num_new are zero.
    const float* lam = lambda + g * kHeadDim;
    for (int t = wave; t < kEncTok; t += kWv) {
        const bool live = t < ntok;
        const size_t in_row = (static_cast<size_t>(b) * num_kv_heads + g) * num_new + t0 +
                              (live ? t : 0);
        double x0 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane) /
                    static_cast<double>(lam[2 * lane]);
        double x1 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane + 1) /
                    static_cast<double>(lam[2 * lane + 1]);
        fwht128(x0, x1);
        xs[0][t][2 * lane] = live ? x0 * kInvSqrtD64 : 0.0;
        xs[0][t][2 * lane + 1] = live ? x1 * kInvSqrtD64 : 0.0;
        xs[1][t][2 * lane] = live ? load_elem(v_new, f32, in_row * kHeadDim + 2 * lane) : 0.0;
        xs[1][t][2 * lane + 1] =
            live ? load_elem(v_new, f32, in_row * kHeadDim + 2 * lane + 1) : 0.0;
    }
    __syncthreads();

    // row block jobs: keys then values; sub-vector r = 32 token + position
    for (int job = wave; job < 2 * kEncBlocks; job += kWv) {
        const int tt = job / kEncBlocks, rb = job % kEncBlocks;
        if (rb * 16 >= ntok * kNumSub) continue;   // whole block past the last token
        const uint32_t cd = tt == 0 ? search_rows<KENT>(km2, kcu, kcd, xs[0], rb, lane)
                                    : search_rows<256>(vm2, vcu, vcd, xs[1], rb, lane);
        const int r = rb * 16 + lane;
        if (lane < 16) code[tt][r >> 5][r & 31] = static_cast<uint16_t>(cd);
    }
    __syncthreads();

    // codes of the live tokens to their slots
    const size_t out0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + t0;
    {
        const int t = tid / kNumSub, pos = tid % kNumSub;   // 8 tokens x 32 positions (tid < 256)
        if (t < ntok) codes_v[(out0 + t) * kNumSub + pos] = static_cast<uint8_t>(code[1][t][pos]);
        if constexpr (KBITS == 8) {
            if (t < ntok) codes_k[(out0 + t) * KROW + pos] = static_cast<uint8_t>(code[0][t][pos]);
        }
    }
    if constexpr (KBITS == 12) {
        // byte j of a row holds bits [8j, 8j + 8) of the little-endian 12-bit stream
        for (int e = tid; e < ntok * KROW; e += kThr) {
            const int t = e / KROW, j = e % KROW;
            const int bit = 8 * j, i0 = bit / 12, sh = bit % 12;
            uint32_t v = static_cast<uint32_t>(code[0][t][i0]) >> sh;
            if (sh > 4) v |= static_cast<uint32_t>(code[0][t][i0 + 1]) << (12 - sh);
            codes_k[(out0 + t) * KROW + j] = static_cast<uint8_t>(v & 0xffu);
        }
    }
}

// The d = 8 layout (16 sub-vectors of 8 channels, C_k and C_v of 4096
// entries, 24-byte rows of 12-bit codes): 16 tokens per workgroup, one per wave,
// searched with nearest16_d8 against the fp16 codebook in LDS.  A 4096 x 8
// table with its two norm tables takes 96 KiB, so keys and values are
// searched one after the other with the same LDS.
constexpr int kEnc8Ent = 4096;
constexpr int kEnc8Pos = kHeadDim / 8;           // 16 sub-vectors per vector
constexpr int kEnc8Row = kEnc8Pos * 12 / 8;      // 24 bytes per code row
// One token per wave, 16 per workgroup: the tables leave room for one
// workgroup per CU, and 16 waves keep 4 on every SIMD.
constexpr int kEnc8Tok = 16;
constexpr int kEnc8Waves = kEnc8Tok;
constexpr int kEnc8Threads = kEnc8Waves * kWave;

__global__ __launch_bounds__(kEnc8Threads) void encode_append8_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    __shared__ __align__(16) uint16_t ctab[kEnc8Ent * 8];   // one codebook, fp16 as stored
    __shared__ __align__(16) float cu[kEnc8Ent];            // ||c||^2 (1 + 2^-16)
    __shared__ __align__(16) float cd[kEnc8Ent];            // ||c||^2 (1 - 2^-16)
    __shared__ double xs[2][kEnc8Tok][kHeadDim];             // transformed keys, values (fp64)
    __shared__ uint16_t code[2][kEnc8Tok][kEnc8Pos];

    const int t0 = blockIdx.x * kEnc8Tok, g = blockIdx.y, b = blockIdx.z;
    const int ntok = min(kEnc8Tok, num_new - t0);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool f32 = kv_f32 != 0;

    // k / lambda in fp64, the +-1 Walsh–Hadamard transform, then 1/sqrt(128);
    // values as they are.  Rows of tokens past num_new are zero.
    const float* lam = lambda + g * kHeadDim;
    for (int t = wave; t < kEnc8Tok; t += kEnc8Waves) {
        const bool live = t < ntok;
        const size_t in_row = (static_cast<size_t>(b) * num_kv_heads + g) * num_new + t0 +
                              (live ? t : 0);
        double x0 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane) /
                    static_cast<double>(lam[2 * lane]);
        double x1 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane + 1) /
                    static_cast<double>(lam[2 * lane + 1]);
        fwht128(x0, x1);
        xs[0][t][2 * lane] = live ? x0 * kInvSqrtD64 : 0.0;
        xs[0][t][2 * lane + 1] = live ? x1 * kInvSqrtD64 : 0.0;
        xs[1][t][2 * lane] = live ? load_elem(v_new, f32, in_row * kHeadDim + 2 * lane) : 0.0;
        xs[1][t][2 * lane + 1] =
            live ? load_elem(v_new, f32, in_row * kHeadDim + 2 * lane + 1) : 0.0;
    }

    for (int tt = 0; tt < 2; ++tt) {
        if (tt == 1) __syncthreads();   // every search of the key table is done
        const uint4* src = reinterpret_cast<const uint4*>(tt == 0 ? cb_k : cb_v) +
                           static_cast<size_t>(g) * kEnc8Ent;
        for (int i = tid; i < kEnc8Ent; i += kEnc8Threads) {
            const uint4 c = src[i];
            reinterpret_cast<uint4*>(ctab)[i] = c;
            const uint32_t w[4] = {c.x, c.y, c.z, c.w};
            float nn = 0.f;   // the squares of fp16 values are exact in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = half_bits_to_float(static_cast<uint16_t>(w[j] & 0xffffu));
                const float hi = half_bits_to_float(static_cast<uint16_t>(w[j] >> 16));
                nn += lo * lo;
                nn += hi * hi;
            }
            cu[i] = nn * kBoundUp;
            cd[i] = nn * kBoundDown;
        }
        __syncthreads();
        // wave w: the 16 sub-vectors of token w (position lane % 16)
        const int tok = wave, pos = lane & 15;
        static_assert(kEnc8Waves == kEnc8Tok && kEnc8Pos == 16, "one token per wave");
        if (tok < ntok) {   // uniform
            const double* x = &xs[tt][tok][8 * pos];
            const int gq = lane >> 4;
            const float b0 = -2.f * static_cast<float>(x[2 * gq]);
            const float b1 = -2.f * static_cast<float>(x[2 * gq + 1]);
            float xx = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = static_cast<float>(x[j]);
                xx += v * v;
            }
            double xd[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xd[j] = x[j];
            const auto exact = [&](uint32_t nc) {
                return sqdist8_f64(xd, reinterpret_cast<const uint4*>(ctab)[nc]);
            };
            const uint32_t c = nearest16_d8<kEnc8Ent>(ctab, cu, cd, b0, b1, row_bound(xx), lane,
                                                      exact);
            if (lane < 16) code[tt][tok][pos] = static_cast<uint16_t>(c);
        }
    }
    __syncthreads();

    // the live tokens' rows: byte j holds bits [8j, 8j + 8) of the 12-bit stream
    const size_t out0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + t0;
    for (int e = tid; e < 2 * ntok * kEnc8Row; e += kEnc8Threads) {
        const int tt = e / (ntok * kEnc8Row), rem = e % (ntok * kEnc8Row);
        const int t = rem / kEnc8Row, j = rem % kEnc8Row;
        const int bit = 8 * j, i0 = bit / 12, sh = bit % 12;
        uint32_t v = static_cast<uint32_t>(code[tt][t][i0]) >> sh;
        if (sh > 4) v |= static_cast<uint32_t>(code[tt][t][i0 + 1]) << (12 - sh);
        (tt == 0 ? codes_k : codes_v)[(out0 + t) * kEnc8Row + j] = static_cast<uint8_t>(v & 0xffu);
    }
}

hipError_t launch_encode_append(int k_bits, int sub_dim, const void* k_new, const void* v_new,
                                bool kv_f32, const float* lambda, const uint16_t* cb_k,
                                const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v,
                                int batch, int num_kv_heads, int capacity, int cur_len,
                                int num_new, hipStream_t stream) {
    const dim3 grid((num_new + kEncTok - 1) / kEncTok, num_kv_heads, batch);
    const dim3 grid8((num_new + kEnc8Tok - 1) / kEnc8Tok, num_kv_heads, batch);
    if (sub_dim == 8)
        hipLaunchKernelGGL(encode_append8_kernel, grid8, dim3(kEnc8Threads), 0, stream, k_new, v_new,
                           kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v, num_kv_heads,
                           capacity, cur_len, num_new);
    else if (k_bits == 8)
        hipLaunchKernelGGL(encode_append_kernel<8>, grid, dim3(kEncThreadsOf<8>), 0, stream, k_new,
                           v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,
                           num_kv_heads, capacity, cur_len, num_new);
    else
        hipLaunchKernelGGL(encode_append_kernel<12>, grid, dim3(kEncThreadsOf<12>), 0, stream, k_new,
                           v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,
                           num_kv_heads, capacity, cur_len, num_new);
    return hipGetLastError();
}

}  // namespace vqkv
