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
// to the lowest index), found by the certified fp16 hi/lo matrix-core search
// of nearest_search.hpp, with the transformed keys and the values kept in
// fp64 for the few exact distances.
//
// One 512-thread workgroup (1024 with 12-bit keys) encodes up to 8 tokens
// (4 for short appends, 16 for prompts) of one (sequence, KV head): 32 key
// and 32 value sub-vectors a token, in row blocks of 16, spread over the
// waves.  The codebooks
// (fp16, as stored) and their squared norms are staged in LDS.
#include "launchers.hpp"
#include "nearest_search.hpp"

namespace vqkv {

namespace {

// Tokens per workgroup: 8; 4 where the launch with 8 would leave CUs
// without a workgroup (short appends), since a workgroup of 4 tokens gives
// each wave one search job instead of two; 16 where 8 would give more than
// 8 workgroups a CU (prompts), which spreads each workgroup's fixed work
// (tables, scales, barriers) over twice the tokens.
constexpr int kEncTok = 8;
constexpr int kEncTokSmall = 4;
constexpr int kEncTokLarge = 16;
constexpr int kEncFill = 256;   // workgroups that fill the chip (one per CU)
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

// The nearest centroids of the 16 sub-vectors of each of the NC row blocks
// rb0 .. rb0 + NC - 1 of `xs` ([tokens][128] fp64: 32 sub-vectors of 4 a token)
// among NENT fp16 centroids c16 (the codebook as stored), with the norm terms
// of hilo_norm_terms at scale sc in cu / cd (dmax: their largest
// difference): fp16 hi/lo matrix-core scores, certified
// (nearest_search.hpp), fp64 distances for the few candidates.
// Every centroid block's A operand and norm terms are read from LDS once for
// all NC products; lane l % 16 of row block j gets out[j].
template <int NENT, int NC>
__device__ __forceinline__ void search_rows_cols(const uint2* c16, const float* cu,
                                                 const float* cd, float sc, float dmax,
                                                 const double (*xs)[kHeadDim], int rb0, int lane,
                                                 uint32_t (&out)[NC]) {
    const double* x0 = &xs[0][0] + (rb0 * 16 + (lane & 15)) * 4;   // row block j at + 64 j
    BlockD4HN<NC> block;
    block.arow = c16 + (lane & 15);
    float ex[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const double* x = x0 + 64 * j;
        block.b[j] = hilo_rows<4, h4_t>(x, lane, sc);
        float xx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = static_cast<float>(x[i]);
            xx += v * v;
        }
        ex[j] = row_bound_h(xx) * sc;
    }
    // the distance rounded as the fp64 reference rounds it
    const auto exact = [&](int j, uint32_t nc) { return sqdist4_f64(x0 + 64 * j, c16[nc]); };
    nearest16_cols<NENT, NC, NC == 1 ? kSearchUnroll : 4>(cu, cd, block, ex, dmax, lane, exact,
                                                          out);
}

// The largest |2x| over the n values of xs, reduced over the workgroup
// (red: kThr / 64 floats of LDS); every thread gets it.
template <int kThr>
__device__ __forceinline__ float block_absmax2(const double* xs, int n, float* red, int tid) {
    float m = 0.f;
    for (int i = tid; i < n; i += kThr) m = fmaxf(m, fabsf(-2.f * static_cast<float>(xs[i])));
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kThr / kWave; ++w) r = fmaxf(r, red[w]);
    return r;
}

}  // namespace

template <int KBITS, int TOK>
__global__ __launch_bounds__(kEncThreadsOf<KBITS>) void encode_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    constexpr int KENT = 1 << KBITS;
    constexpr int KROW = kNumSub * KBITS / 8;
    constexpr int kThr = kEncThreadsOf<KBITS>, kWv = kThr / kWave;
    // the codebooks as stored (fp16) and their norm terms at this
    // workgroup's scale (hilo_norm_terms), per tensor
    __shared__ __align__(16) uint2 kc16[KENT];
    __shared__ __align__(16) uint2 vc16[256];
    __shared__ __align__(16) float kcu[KENT];
    __shared__ __align__(16) float kcd[KENT];
    __shared__ __align__(16) float vcu[256];
    __shared__ __align__(16) float vcd[256];
    __shared__ float red[3][kThr / kWave];
    __shared__ double xs[2][TOK][kHeadDim];       // transformed keys, values (fp64)
    __shared__ uint16_t code[2][TOK][kNumSub];
    constexpr int kBlocks = TOK * kNumSub / 16;   // row blocks per tensor
    static_assert(TOK * kNumSub <= kThr, "one thread per (token, position) writes the codes");

    const int t0 = blockIdx.x * TOK, g = blockIdx.y, b = blockIdx.z;
    const int ntok = min(TOK, num_new - t0);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool f32 = kv_f32 != 0;

    const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
    const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
    // every load is issued before any is used (one latency, not one per entry)
    constexpr int KPER = (KENT + kThr - 1) / kThr;
    uint2 kc[KPER];
#pragma unroll
    for (int j = 0; j < KPER; ++j) kc[j] = ksrc[min(tid + j * kThr, KENT - 1)];
    const uint2 vc = vsrc[tid & 255];
    // k / lambda in fp64, the +-1 Walsh–Hadamard transform, then 1/sqrt(128);
    // values as they are.  Rows of tokens past num_new are zero.
    const float* lam = lambda + g * kHeadDim;
    for (int t = wave; t < TOK; t += kWv) {
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
    // one scale per tensor for the workgroup's hi/lo rows, and the tables
    const float ksc = hilo_scale(block_absmax2<kThr>(&xs[0][0][0], TOK * kHeadDim, red[0], tid));
    const float vsc = hilo_scale(block_absmax2<kThr>(&xs[1][0][0], TOK * kHeadDim, red[1], tid));
    float dk = 0.f;   // the largest difference of C_k's two norm terms
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
        const int i = tid + j * kThr;
        if (i < KENT) {
            kc16[i] = kc[j];
            const float2 t = hilo_norm_terms(norm2(kc[j]), l1_4(kc[j]), ksc);
            kcu[i] = t.x;
            kcd[i] = t.y;
            dk = fmaxf(dk, t.x - t.y);
        }
    }
    dk = wave_max(dk);
    if (lane == 0) red[2][wave] = dk;
    if (tid < 256) {
        vc16[tid] = vc;
        const float2 t = hilo_norm_terms(norm2(vc), l1_4(vc), vsc);
        vcu[tid] = t.x;
        vcd[tid] = t.y;
    }
    __syncthreads();
    float kdmax = 0.f;
#pragma unroll
    for (int w = 0; w < kWv; ++w) kdmax = fmaxf(kdmax, red[2][w]);

    // jobs of row blocks, keys then values; sub-vector r = 32 token +
    // position.  A wave searches the blocks of a job together, so the LDS
    // reads of the tables serve every block of the job.  4096-entry keys keep
    // one block a job: pairs would leave half of the 16 waves without a key
    // job (measured 18% slower).
    constexpr int kPairK = KBITS == 12 ? 1 : 2, kPairV = 2;
    constexpr int kJobsK = kBlocks / kPairK, kJobsV = kBlocks / kPairV;
    const auto put = [&](int tt, int rb, uint32_t cd) {
        const int r = rb * 16 + lane;
        if (lane < 16) code[tt][r >> 5][r & 31] = static_cast<uint16_t>(cd);
    };
    for (int job = wave; job < kJobsK + kJobsV; job += kWv) {
        const bool key = job < kJobsK;
        const int rb0 = key ? job * kPairK : (job - kJobsK) * kPairV;
        if (rb0 * 16 >= ntok * kNumSub) continue;   // every block past the last token
        if (key) {
            uint32_t cd[kPairK];
            search_rows_cols<KENT, kPairK>(kc16, kcu, kcd, ksc, kdmax, xs[0], rb0, lane, cd);
#pragma unroll
            for (int j = 0; j < kPairK; ++j) put(0, rb0 + j, cd[j]);
        } else {
            uint32_t cd[kPairV];
            search_rows_cols<256, kPairV>(vc16, vcu, vcd, vsc, 0.f, xs[1], rb0, lane, cd);
#pragma unroll
            for (int j = 0; j < kPairV; ++j) put(1, rb0 + j, cd[j]);
        }
    }
    __syncthreads();

    // codes of the live tokens to their slots
    const size_t out0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + t0;
    {
        const int t = tid / kNumSub, pos = tid % kNumSub;   // TOK tokens x 32 positions
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
// searched with fp16 hi/lo scores against the fp16 codebook in LDS.  A 4096 x 8
// table with its norm table takes 80 KiB, so keys and values are searched
// one after the other with the same LDS.
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
    // its norm terms at the workgroup's scale for the tensor (hilo_norm_terms)
    __shared__ __align__(16) float cu[kEnc8Ent];
    __shared__ __align__(16) float cd[kEnc8Ent];
    __shared__ float red[3][kEnc8Waves];
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

    __syncthreads();
    // one scale per tensor for the workgroup's hi/lo rows
    float scale[2];
    for (int tt = 0; tt < 2; ++tt)
        scale[tt] = hilo_scale(block_absmax2<kEnc8Threads>(&xs[tt][0][0], kEnc8Tok * kHeadDim,
                                                           red[tt], tid));
    for (int tt = 0; tt < 2; ++tt) {
        if (tt == 1) __syncthreads();   // every search of the key table is done
        const uint4* src = reinterpret_cast<const uint4*>(tt == 0 ? cb_k : cb_v) +
                           static_cast<size_t>(g) * kEnc8Ent;
        float dm = 0.f;
        for (int i = tid; i < kEnc8Ent; i += kEnc8Threads) {
            const uint4 c = src[i];
            reinterpret_cast<uint4*>(ctab)[i] = c;
            const uint32_t w[4] = {c.x, c.y, c.z, c.w};
            float nn = 0.f, l1 = 0.f;   // the squares of fp16 values are exact in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = half_bits_to_float(static_cast<uint16_t>(w[j] & 0xffffu));
                const float hi = half_bits_to_float(static_cast<uint16_t>(w[j] >> 16));
                nn += lo * lo;
                nn += hi * hi;
                l1 += fabsf(lo) + fabsf(hi);
            }
            const float2 t = hilo_norm_terms(nn, l1, scale[tt]);
            cu[i] = t.x;
            cd[i] = t.y;
            dm = fmaxf(dm, t.x - t.y);
        }
        dm = wave_max(dm);
        if (lane == 0) red[2][wave] = dm;
        __syncthreads();
        float dmax = 0.f;   // the largest difference of the two norm terms
#pragma unroll
        for (int w = 0; w < kEnc8Waves; ++w) dmax = fmaxf(dmax, red[2][w]);
        // wave w: the 16 sub-vectors of token w (position lane % 16)
        const int tok = wave, pos = lane & 15;
        static_assert(kEnc8Waves == kEnc8Tok && kEnc8Pos == 16, "one token per wave");
        if (tok < ntok) {   // uniform
            const double* x = &xs[tt][tok][8 * pos];
            float xx = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = static_cast<float>(x[j]);
                xx += v * v;
            }
            double xd[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xd[j] = x[j];
            const auto exact = [&](int, uint32_t nc) {
                return sqdist8_f64(xd, reinterpret_cast<const uint4*>(ctab)[nc]);
            };
            // fp16 hi/lo matrix-core scores in units of the workgroup's 2^s;
            // groups of 4 blocks, their operands requested before the products
            const float sc = scale[tt];
            BlockD8HN<1> block;
            block.arow = reinterpret_cast<const uint4*>(ctab) + (lane & 15);
            block.b[0] = hilo_rows<8, h8_t>(xd, lane, sc);
            const float ex[1] = {row_bound_h(xx) * sc};
            uint32_t c[1];
            nearest16_cols<kEnc8Ent, 1, 4>(cu, cd, block, ex, dmax, lane, exact, c);
            if (lane < 16) code[tt][tok][pos] = static_cast<uint16_t>(c[0]);
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

// Short appends in the d = 8 layout: one token per workgroup, its 4096
// centroids of each tensor spread over the 16 waves (codes8_one_token, the
// search of the decode step's new token), so that a few tokens still occupy
// many CUs.  The decisions are those of encode_append8_kernel.
// LDS: C_k and C_v as stored (64 KiB each), the norms, the exchanges.
__global__ __launch_bounds__(1024) void encode_token8_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    constexpr int kTab = kEnc8Ent * 16;   // bytes of one codebook
    __shared__ __align__(16) uint8_t tab[2 * kTab];
    __shared__ __align__(16) float nrm[kEnc8Ent];
    __shared__ __align__(16) uint8_t xbuf[4096];
    __shared__ double xnew[2][kHeadDim];   // transformed key, value (fp64)
    __shared__ uint32_t newc[2][kNumSub];

    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const bool f32 = kv_f32 != 0;
    const uint4* ksrc = reinterpret_cast<const uint4*>(cb_k) + static_cast<size_t>(g) * kEnc8Ent;
    const uint4* vsrc = reinterpret_cast<const uint4*>(cb_v) + static_cast<size_t>(g) * kEnc8Ent;
    for (int i = tid; i < kEnc8Ent; i += 1024) {
        reinterpret_cast<uint4*>(tab)[i] = ksrc[i];
        reinterpret_cast<uint4*>(tab + kTab)[i] = vsrc[i];
    }
    // k / lambda in fp64, the +-1 Walsh–Hadamard transform, then 1/sqrt(128)
    // (wave 0); the value as it is (wave 1)
    if (wave < 2) {
        const size_t in_row = (static_cast<size_t>(b) * num_kv_heads + g) * num_new + t;
        const void* src = wave == 0 ? k_new : v_new;
        double x0 = load_elem(src, f32, in_row * kHeadDim + 2 * lane);
        double x1 = load_elem(src, f32, in_row * kHeadDim + 2 * lane + 1);
        if (wave == 0) {
            const float* lam = lambda + g * kHeadDim;
            x0 = x0 / static_cast<double>(lam[2 * lane]);
            x1 = x1 / static_cast<double>(lam[2 * lane + 1]);
            fwht128(x0, x1);
            x0 *= kInvSqrtD64;
            x1 *= kInvSqrtD64;
        }
        xnew[wave][2 * lane] = x0;
        xnew[wave][2 * lane + 1] = x1;
    }
    __syncthreads();
    codes8_one_token(tab, kTab, nrm, xbuf, xnew, newc, tid, lane, wave);
    // the two 24-byte rows: byte j holds bits [8j, 8j + 8) of the 12-bit stream
    const size_t row = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + t;
    if (tid < 2 * kEnc8Row) {
        const int tsel = tid / kEnc8Row, j = tid % kEnc8Row;
        const int bit = 8 * j, i0 = bit / 12, sh = bit % 12;
        uint32_t v = newc[tsel][i0] >> sh;
        if (sh > 4) v |= newc[tsel][i0 + 1] << (12 - sh);
        (tsel ? codes_v : codes_k)[row * kEnc8Row + j] = static_cast<uint8_t>(v & 0xffu);
    }
}

hipError_t launch_encode_append(int k_bits, int sub_dim, const void* k_new, const void* v_new,
                                bool kv_f32, const float* lambda, const uint16_t* cb_k,
                                const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v,
                                int batch, int num_kv_heads, int capacity, int cur_len,
                                int num_new, hipStream_t stream) {
    const dim3 grid8((num_new + kEnc8Tok - 1) / kEnc8Tok, num_kv_heads, batch);
    if (sub_dim == 8) {
        // a token a workgroup where 16-token workgroups would leave CUs idle
        if (static_cast<long long>(grid8.x) * num_kv_heads * batch < kEncFill)
            hipLaunchKernelGGL(encode_token8_kernel, dim3(num_new, num_kv_heads, batch), dim3(1024),
                               0, stream, k_new, v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k,
                               codes_v, num_kv_heads, capacity, cur_len, num_new);
        else
            hipLaunchKernelGGL(encode_append8_kernel, grid8, dim3(kEnc8Threads), 0, stream, k_new,
                               v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,
                               num_kv_heads, capacity, cur_len, num_new);
        return hipGetLastError();
    }
    const long long full = static_cast<long long>((num_new + kEncTok - 1) / kEncTok) *
                           num_kv_heads * batch;
    const bool small = full < kEncFill;
    const bool large = full >= 8 * kEncFill;
    const int tok = small ? kEncTokSmall : (large ? kEncTokLarge : kEncTok);
    const dim3 grid((num_new + tok - 1) / tok, num_kv_heads, batch);
    const auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, k_new, v_new, kv_f32 ? 1 : 0,
                           lambda, cb_k, cb_v, codes_k, codes_v, num_kv_heads, capacity, cur_len,
                           num_new);
    };
    if (k_bits == 8) {
        if (small) launch(encode_append_kernel<8, kEncTokSmall>, kEncThreadsOf<8>);
        else if (large) launch(encode_append_kernel<8, kEncTokLarge>, kEncThreadsOf<8>);
        else launch(encode_append_kernel<8, kEncTok>, kEncThreadsOf<8>);
    } else {
        if (small) launch(encode_append_kernel<12, kEncTokSmall>, kEncThreadsOf<12>);
        else if (large) launch(encode_append_kernel<12, kEncTokLarge>, kEncThreadsOf<12>);
        else launch(encode_append_kernel<12, kEncTok>, kEncThreadsOf<12>);
    }
    return hipGetLastError();
}

}  // namespace vqkv
