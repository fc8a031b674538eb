// Split-K decode attention over a VQ cache on the gfx950 matrix cores.
//
// What is computed (VecInfer page, Method details, "VQ KV cache in attention"):
//   s = q~ VQ^-1(K~_q, C_k)^T / sqrt(D),  p = softmax(s),  o = p VQ^-1(V_q, C_v)
// with q~ = q diag(lambda) H_D.  The tiled online softmax follows the page's
// Appendix (FlashAttention block recurrence, Algorithm 1): running max m,
// running sum l, rescaled output accumulator, final o / l.
//
// How it maps to gfx950.  One workgroup (16 waves, one per CU) streams one
// contiguous token range of one (sequence, KV head); each wave takes 32-token
// tiles in turn.
//  * Both products are dense contractions once a centroid is looked up, so
//    both run on v_mfma_f32_16x16x32_f16.  The 16 MFMA rows are (head, part):
//    q~ and p, the operands that are not exact in fp16, are split into a
//    high and a low fp16 part on separate rows that are summed after the
//    product; codebook entries are fp16 already.  Row 4j + i holds
//    (head 2j, hi), (head 2j+1, hi), (head 2j, lo), (head 2j+1, lo) for
//    i = 0..3, so G <= 8 heads fit; rows of heads >= G are zero.
//      - q~ of each head is first scaled by a power of two 2^e that puts its
//        largest element in [2^14, 2^15): hi = fp16(x 2^e), lo =
//        fp16(x 2^e - hi), and the head's scores are multiplied by 2^-e.
//        Any finite q~ fits fp16 this way, and both parts stay normal
//        numbers for every element within 2^-17 of the largest.
//      - p = 2^(s - m) <= 2^8 is split as hi = fp16_rtz(p) and lo =
//        fp16_rtz((p - hi) 2^16); the low rows are scaled by 2^-16 when the
//        waves fold.  So hi + lo 2^-16 is within 2^-20 p + 2^-40 of p: a
//        weight far below the running maximum keeps its own relative
//        precision instead of being truncated at the fp16 subnormal step.
//  * Scores: the B operand is two key centroids (8 fp16) per lane, each one
//    8-byte LDS gather.
//  * Values: the MFMA wants 8 tokens x 1 channel per lane, a gather gives
//    1 token x 4 channels.  ds_read_b64_tr_b16 does both at once: every lane
//    supplies the address of one centroid and lane 16G+4a+e receives channel
//    e of the centroids fetched by lanes 16G+4k+a, k = 0..3.
//  * Codebooks live in LDS as two 64 KiB tables, keys then values, with one
//    256-byte row per code holding 32 copies of the centroid: lane l reads
//    copy l mod 32, so the 32 lanes one LDS cycle serves always hit 64
//    distinct banks — no bank conflicts for any codes — and the address
//    (code << 8) | slot is a single v_perm_b32 of the loaded code bytes.
//    (A 12-bit key codebook, 4096 x 8 B, is stored once, unreplicated.)
//  * Code rows stay token-major in HBM.  Loads are raw buffer loads of 8
//    (or 12) contiguous bytes per lane: the split's rows form the buffer
//    range, so rows past the split's end read as zero without any clamp.
//    One register set: once a tile's key gathers are issued its key-code
//    registers take the next tile's key codes, and likewise the value codes
//    after the value gathers, so the next tile's loads are in flight while
//    the rest of the tile is computed.
//  * Tiles are handed to waves dynamically (LDS counter), so the tokens a
//    wave folds into its online softmax depend on timing: results agree run
//    to run to fp32 rounding, not bit for bit.  In deterministic mode
//    (vq_set_deterministic) wave w takes tiles w, w + 16, ... instead, and
//    every launch with the same inputs gives the same bits (2-3% slower at
//    the 196608-token layer).
//  * The workgroup folds its 16 wave states in LDS and leaves one base-2
//    partial (m, l, o); a second, small kernel merges the splits by
//    log-sum-exp.  Merging the splits inside this kernel would need a
//    device-scope release per workgroup, which writes back the XCD's L2 and
//    costs more than the extra launch.
#include <type_traits>

#include "launchers.hpp"
#include "nearest_search.hpp"

namespace vqkv {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int kWaves = kVqWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kTok = 32;                  // tokens per wave tile
constexpr int kStride = kWaves * kTok;    // tokens per workgroup sweep
constexpr float kTau = 8.0f;              // lazy-rescale slack (log2 units)
constexpr float kLoScale = 65536.0f;      // low part of p, scaled: (p - hi) 2^16
constexpr float kLoUnscale = 1.0f / 65536.0f;
constexpr int kTable = 65536;             // bytes of one codebook table
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw (untyped) buffer, gfx9

static_assert(kStride == kVqTile && kTok == kVqTileGrain, "split planning matches the tiles");

// LDS address bytes [slot.b2 : code : slot.b0], code = byte K of w
template <int K>
__device__ __forceinline__ uint32_t row_addr(uint32_t w, uint32_t slot) {
    return __builtin_amdgcn_perm(w, slot, 0x0C020000u | ((4u + K) << 8));
}

__device__ __forceinline__ half8_t cat(uint2 a, uint2 b) {
    return __builtin_bit_cast(half8_t, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ half8_t cat(half4_t a, half4_t b) {
    return half8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ half4_t read_tr16(const uint8_t* p) {
    return __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p));
}

// 2^x on the hardware exponential (results below 2^-126 flush to 0, which
// only drops weights negligible next to the running sum, itself >= 1)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float rescale_factor(float m_old, float m_new) {
    return (m_old == m_new) ? 1.f : fast_exp2(m_old - m_new);
}

// Lanes 0-31 of a, then lanes 0-31 of b (in lanes 32-63): one permlane swap.
__device__ __forceinline__ float lo_halves(float a, float b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(__builtin_amdgcn_permlane32_swap(
        __builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), false, false)[0]));
}

__device__ __forceinline__ uint32_t pack_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ __forceinline__ float lo_half_to_float(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float hi_half_to_float(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// The 8 key codes of positions 8 grp .. 8 grp + 7 of one token, and the LDS
// address of the key centroid of position 8 grp + I.
template <int KBITS>
struct KChunk;

template <>
struct KChunk<8> {
    uint2 w;
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        w = make_uint2(v[0], v[1]);
    }
    __device__ void set(const uint8_t* p) { w = *reinterpret_cast<const uint2*>(p); }
    template <int I>
    __device__ uint32_t addr(uint32_t slot) const {
        return row_addr<I & 3>(I < 4 ? w.x : w.y, slot);
    }
};

template <>
struct KChunk<12> {
    uint32_t w0, w1, w2;   // 96 bits: 8 codes of 12 bits, little-endian
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
        w0 = v[0];
        w1 = v[1];
        w2 = v[2];
    }
    __device__ void set(const uint8_t* p) {
        const uint32_t* u = reinterpret_cast<const uint32_t*>(p);
        w0 = u[0];
        w1 = u[1];
        w2 = u[2];
    }
    template <int I>
    __device__ uint32_t addr(uint32_t) const {
        constexpr int bit = 12 * I, lo = bit >> 5, sh = bit & 31;
        const uint32_t a = lo == 0 ? w0 : (lo == 1 ? w1 : w2);
        uint32_t code;
        if constexpr (sh + 12 <= 32) {
            code = __builtin_amdgcn_ubfe(a, sh, 12);
        } else {
            const uint32_t b = lo == 0 ? w1 : w2;
            code = __builtin_amdgcn_alignbit(b, a, sh) & 0xfffu;
        }
        return code << 3;   // unreplicated 4096 x 8 B table at the start of LDS
    }
};

// Four 12-bit codes, positions 4 j .. 4 j + 3, of one 24-byte row of the
// d = 8 layout (16 codes of 12 bits): bytes [6 j, 6 j + 6).  They are read as
// the dword-aligned 8 bytes at 12 (j / 2) + 4 (j % 2) and shifted down by
// 16 (j % 2) bits when used (a shift at load time would wait for the load).
struct Chunk8 {
    uint32_t x, y;
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        x = v[0];
        y = v[1];
    }
    // the 4 codes, given the lane's shift (0 or 16)
    __device__ void codes(uint32_t sh, uint32_t c[4]) const {
        const uint32_t lo = __builtin_amdgcn_alignbit(y, x, sh), hi = y >> sh;
        c[0] = lo & 0xfffu;
        c[1] = (lo >> 12) & 0xfffu;
        c[2] = __builtin_amdgcn_alignbit(hi, lo, 24) & 0xfffu;
        c[3] = (hi >> 4) & 0xfffu;
    }
};

// The 32 key codes (bytes) of one token, for the lookup-table score path.
struct LutCodes {
    uint32_t w[8];
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = a[i];
            w[4 + i] = b[i];
        }
    }
};

}  // namespace

// Inputs of the new-token workgroups: q~ of head `wave` (fp32, base-2 score
// scale, two elements per lane) for waves < G; the new key transformed,
// k diag(lambda)^-1 H_D in fp64 (wave 8), and the new value as is (wave 9),
// into xnew.
template <int G>
__device__ __forceinline__ void new_token_inputs(const void* q, int q_f32, const float* lambda,
                                                 const void* k_new, const void* v_new, int kv_f32,
                                                 int num_q_heads, int num_kv_heads, int g, int b,
                                                 int wave, int lane, float& x0, float& x1,
                                                 double (*xnew)[kHeadDim]) {
    x0 = 0.f;
    x1 = 0.f;
    if (wave < G) {
        const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + wave;
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(q) +
                             (q_f32 ? vec * kHeadDim + 2 * lane : vec * (kHeadDim / 2) + lane);
        const float2 lam2 = reinterpret_cast<const float2*>(lambda + g * kHeadDim)[lane];
        x0 = (q_f32 ? __builtin_bit_cast(float, qw[0]) : half_bits_to_float(qw[0] & 0xffffu)) *
             lam2.x;
        x1 = (q_f32 ? __builtin_bit_cast(float, qw[1]) : half_bits_to_float(qw[0] >> 16)) *
             lam2.y;
        fwht128(x0, x1);
        x0 *= kScoreScaleLog2;
        x1 *= kScoreScaleLog2;
    } else if (wave == 8 || wave == 9) {
        // k / lambda in fp64 with the +-1 transform and 1/sqrt(128) (wave 8);
        // the value as is (wave 9)
        const size_t row = static_cast<size_t>(b) * num_kv_heads + g;
        const void* src = wave == 8 ? k_new : v_new;
        double y0, y1;
        if (kv_f32) {
            const float2 v = reinterpret_cast<const float2*>(src)[row * (kHeadDim / 2) + lane];
            y0 = v.x;
            y1 = v.y;
        } else {
            const uint32_t w = reinterpret_cast<const uint32_t*>(src)[row * (kHeadDim / 2) + lane];
            y0 = half_bits_to_float(w & 0xffffu);
            y1 = half_bits_to_float(w >> 16);
        }
        if (wave == 8) {
            const float* lam = lambda + g * kHeadDim;
            y0 = y0 / static_cast<double>(lam[2 * lane]);
            y1 = y1 / static_cast<double>(lam[2 * lane + 1]);
            fwht128(y0, y1);
            y0 *= kInvSqrtD64;
            y1 *= kInvSqrtD64;
        }
        xnew[wave - 8][2 * lane] = y0;
        xnew[wave - 8][2 * lane + 1] = y1;
    }
}

// LDS of the new-token workgroup with 12-bit keys (offsets into `tab`):
// C_k as stored (fp16, 8 bytes an entry) with its norm terms (upper, lower),
// C_v likewise, and the exchanges of the search.
constexpr int kNtKu = 4096 * 8;
constexpr int kNtKd = kNtKu + 4096 * 4;
constexpr int kNtV = kNtKd + 4096 * 4;
constexpr int kNtVu = kNtV + 256 * 8;
constexpr int kNtVd = kNtVu + 256 * 4;
constexpr int kNtX = kNtVd + 256 * 4;
constexpr int kNtXBytes = 64 * 4 + 2 * kWaves * 16 * 8 + 2 * kWaves * 16 * 4 + 2 * kWaves * 4;
static_assert(kNtX + kNtXBytes <= 2 * kTable, "the 12-bit new-token tables fit the LDS tables");

// C_k (4096 entries) and C_v (256) of the new-token workgroup with 12-bit
// keys, loaded before the token's inputs are known and written to LDS by
// new_token_codes12 with their norm terms.
struct Codes12Tables {
    uint2 k[4096 / kThreads];
    uint2 v;
};
__device__ __forceinline__ Codes12Tables load_codes12(const uint2* __restrict__ ksrc,
                                                      const uint2* __restrict__ vsrc, int tid) {
    Codes12Tables t;
#pragma unroll
    for (int j = 0; j < 4096 / kThreads; ++j) t.k[j] = ksrc[tid + j * kThreads];
    t.v = vsrc[tid & 255];
    return t;
}

// Float keys whose unsigned order is the float order (finite values).
__device__ __forceinline__ uint32_t ordered_key(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u >> 31) != 0 ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_key(uint32_t k) {
    return __builtin_bit_cast(float, (k >> 31) != 0 ? (k & 0x7fffffffu) : ~k);
}

// The codes of the appended token for 4096-entry C_k and 256-entry C_v
// (d = 4), found by the certified fp16 hi/lo search of nearest_search.hpp
// with one scale per tensor (the token's largest |2x|, which every wave
// finds for itself), so that the norm terms are scaled once as the tables
// are written.  Wave w takes the 16 sub-vectors of column block w / 8 and,
// with k = w % 8, key centroid blocks 32 k .. 32 k + 31 and value blocks
// 2 k, 2 k + 1.  Pass-1 minima meet in LDS as atomic minima (the
// thresholds); the second pass evaluates each candidate (a score within the
// bound of the threshold, about one a sub-vector) in fp64 as it finds it,
// and the waves' fp64 minima meet in LDS.  The decisions are those of the
// fp64 scan: ties to the lowest index.
//   tabs   the codebooks of load_codes12; tab receives the tables, exchanges at kNtX
//   xnew   the transformed key and the value (fp64); codes[t][32] receives the codes
// Ends with a barrier; codes is then visible to the whole workgroup.
__device__ __forceinline__ void new_token_codes12(const Codes12Tables& tabs, uint8_t* tab,
                                                  const double (*xnew)[kHeadDim],
                                                  uint32_t (*codes)[kNumSub], int tid, int lane,
                                                  int wave) {
    constexpr int kCb = 8;   // waves per column block
    static_assert(kThreads == 1024 && 4096 == kCb * 32 * 16 && 256 == kCb * 2 * 16,
                  "32 key blocks and 2 value blocks a wave");
    uint32_t* wthr = reinterpret_cast<uint32_t*>(tab + kNtX);               // [2][32] keys
    double* wbd = reinterpret_cast<double*>(tab + kNtX + 256);              // [2][16 waves][16]
    uint32_t* wbi = reinterpret_cast<uint32_t*>(tab + kNtX + 256 + 2 * kWaves * 16 * 8);
    float* wdm = reinterpret_cast<float*>(wbi + 2 * kWaves * 16);          // [2][16 waves]
    // one scale per tensor: the largest |2x| of the token's 128 channels
    float sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float m = fmaxf(fabsf(-2.f * static_cast<float>(xnew[t][lane])),
                              fabsf(-2.f * static_cast<float>(xnew[t][lane + 64])));
        sc[t] = hilo_scale(wave_max(m));
    }
    // the tables with their norm terms at these scales, and each wave's
    // largest difference of the two norm terms (for the skip of pass 2)
    float dk = 0.f;
#pragma unroll
    for (int j = 0; j < 4096 / kThreads; ++j) {
        const int i = tid + j * kThreads;
        const uint2 c = tabs.k[j];
        const float2 nt = hilo_norm_terms(norm2(c), l1_4(c), sc[0]);
        reinterpret_cast<uint2*>(tab)[i] = c;
        reinterpret_cast<float*>(tab + kNtKu)[i] = nt.x;
        reinterpret_cast<float*>(tab + kNtKd)[i] = nt.y;
        dk = fmaxf(dk, nt.x - nt.y);
    }
    dk = wave_max(dk);
    if (lane == 0) wdm[wave] = dk;
    if (tid < 256) {   // waves 0-3
        const float2 nt = hilo_norm_terms(norm2(tabs.v), l1_4(tabs.v), sc[1]);
        reinterpret_cast<uint2*>(tab + kNtV)[tid] = tabs.v;
        reinterpret_cast<float*>(tab + kNtVu)[tid] = nt.x;
        reinterpret_cast<float*>(tab + kNtVd)[tid] = nt.y;
        const float dv = wave_max(nt.x - nt.y);
        if (lane == 0) wdm[kWaves + wave] = dv;
    }
    if (tid < 2 * kNumSub) wthr[tid] = 0xffffffffu;
    wave = __builtin_amdgcn_readfirstlane(wave);   // scalar: block bounds and loop counters in SGPRs
    const int cb = wave / kCb, wk = wave % kCb, sv = 16 * cb + (lane & 15), q4 = 4 * (lane >> 4);
    BlockD4HN<1> bk, bv;
    bk.arow = reinterpret_cast<const uint2*>(tab) + (lane & 15);
    bv.arow = reinterpret_cast<const uint2*>(tab + kNtV) + (lane & 15);
    bk.b[0] = hilo_rows<4, h4_t>(&xnew[0][4 * sv], lane, sc[0]);
    bv.b[0] = hilo_rows<4, h4_t>(&xnew[1][4 * sv], lane, sc[1]);
    float bound[2];   // the row bound of the lane's sub-vector at the tensor's scale
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float xx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = static_cast<float>(xnew[t][4 * sv + i]);
            xx += v * v;
        }
        bound[t] = row_bound_h(xx) * sc[t];
    }
    struct Col {
        const f32x4_t* p;
        __device__ f32x4_t operator()(int blk) const { return p[blk * 4]; }
    };
    const Col kup{reinterpret_cast<const f32x4_t*>(tab + kNtKu) + lane / 16};
    const Col kdown{reinterpret_cast<const f32x4_t*>(tab + kNtKd) + lane / 16};
    const Col vup{reinterpret_cast<const f32x4_t*>(tab + kNtVu) + lane / 16};
    const Col vdown{reinterpret_cast<const f32x4_t*>(tab + kNtVd) + lane / 16};
    const auto kexact = [&](int, uint32_t nc) {
        return sqdist4_f64(&xnew[0][4 * sv], reinterpret_cast<const uint2*>(tab)[nc]);
    };
    const auto vexact = [&](int, uint32_t nc) {
        return sqdist4_f64(&xnew[1][4 * sv], reinterpret_cast<const uint2*>(tab + kNtV)[nc]);
    };
    const int kb0 = 32 * wk, kb1 = kb0 + 32, vb0 = 2 * wk, vb1 = vb0 + 2;
    __syncthreads();   // tables and threshold slots written

    // pass 1: the thresholds, and this lane's minimum over each run of 4 key
    // blocks and over its 2 value blocks
    float gk[8], gv[1];
    {
        search_pass1_groups<kSearchUnroll, 4, 4>(bk, kup, kb0, gk);
        search_pass1_groups<2, 2, 1>(bv, vup, vb0, gv);
        float sk = fminf(fminf(fminf(gk[0], gk[1]), fminf(gk[2], gk[3])),
                         fminf(fminf(gk[4], gk[5]), fminf(gk[6], gk[7])));
        float sv1 = gv[0];
        sk = fminf(sk, lane_partner<16>(sk, lane));
        sk = fminf(sk, lane_partner<32>(sk, lane));
        sv1 = fminf(sv1, lane_partner<16>(sv1, lane));
        sv1 = fminf(sv1, lane_partner<32>(sv1, lane));
        if (lane < 16) {
            atomicMin(&wthr[sv], ordered_key(sk));
            atomicMin(&wthr[32 + sv], ordered_key(sv1));
        }
    }
    __syncthreads();
    const float thk[1] = {from_ordered_key(wthr[sv]) + bound[0]};
    const float thv[1] = {from_ordered_key(wthr[32 + sv]) + bound[1]};
    float dmk = 0.f, dmv = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) dmk = fmaxf(dmk, wdm[w]);
#pragma unroll
    for (int w = 0; w < 4; ++w) dmv = fmaxf(dmv, wdm[kWaves + w]);
    // the runs where some lane of the wave may have a candidate
    const uint32_t needk = pass3_need(gk, thk[0], dmk, bound[0]);
    const uint32_t needv = pass3_need(gv, thv[0], dmv, bound[1]);

    // pass 2: fp64 distances of every candidate; the lexicographic minimum
    // over the 4 lanes of a sub-vector, then over the waves of its block
    {
        double bd[1];
        uint32_t bi[1];
        search_pass3_cols<1, 4>(bk, kdown, kb0, kb1, thk, q4, kexact, bd, bi, needk);
        take_lanes16_32(bd[0], bi[0], lane);
        if (lane < 16) {
            wbd[wave * 16 + lane] = bd[0];
            wbi[wave * 16 + lane] = bi[0];
        }
        search_pass3_cols<1, 2>(bv, vdown, vb0, vb1, thv, q4, vexact, bd, bi, needv);
        take_lanes16_32(bd[0], bi[0], lane);
        if (lane < 16) {
            wbd[(kWaves + wave) * 16 + lane] = bd[0];
            wbi[(kWaves + wave) * 16 + lane] = bi[0];
        }
    }
    __syncthreads();
    if (tid < 2 * kNumSub) {   // tensor tid / 32, sub-vector tid % 32 (column block, column)
        const int t = tid >> 5, sub = tid & 31, w0 = (sub / 16) * kCb, c = sub & 15;
        const double* d = wbd + (t * kWaves + w0) * 16 + c;
        const uint32_t* ix = wbi + (t * kWaves + w0) * 16 + c;
        double d0 = d[0];
        uint32_t i0 = ix[0];
#pragma unroll
        for (int w = 1; w < kCb; ++w) {
            if (nearer(d[w * 16], ix[w * 16], d0, i0)) {
                d0 = d[w * 16];
                i0 = ix[w * 16];
            }
        }
        codes[t][sub] = i0 & (t == 0 ? 4095u : 255u);   // (a code always exists for finite inputs)
    }
    __syncthreads();
}

// The appended token of one (sequence, KV head), handled by one extra
// workgroup of the split kernel while the others attend over the cached
// tokens (VecInfer page, Method details, "VQ KV cache in attention": each
// newly arrived key takes the online dual transform k~ = k diag(lambda)^-1
// H_D and is quantised with C_k, its value with C_v, and both are
// concatenated to the cache before the query attends).
//  1. Codes: the nearest centroid of each 4-dim sub-vector (Background, VQ
//     principle), distances in fp64 with every operation rounded separately,
//     ties to the lowest index: the decisions of vq_encode_append.  For a
//     256-entry codebook thread (slice, pos) scans centroids slice,
//     slice + 32, ... of sub-vector pos, and the 32 slices are combined by
//     the lexicographic (distance, index) minimum.  With 12-bit keys both
//     tensors take the matrix-core search of new_token_codes12.  The codes
//     are written to the cache slot append_pos.
//  2. Its attention partial, as one more split of one token: m = x (its
//     base-2 score), l = 1, o = its dequantised value, at split index `slot`.
// LDS: the codebooks unreplicated in `tab` (keys at 0, values at 32 KiB; with
// 12-bit keys the tables and exchanges of new_token_codes12), the scratch of
// the 256-entry scans' combination in `scratch` (the p buffers).
template <int G, int KBITS>
__device__ __forceinline__ void new_token_workgroup(
    const void* q, int q_f32, const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
    const void* k_new, const void* v_new, int kv_f32, int num_q_heads, int num_kv_heads, int g,
    int b, int capacity, int append_pos, uint8_t* new_codes_k, uint8_t* new_codes_v,
    Partials part, int part_stride, int slot, uint8_t* tab, uint8_t* scratch,
    double (*xnew)[kHeadDim], uint32_t (*newc)[kNumSub]) {
    constexpr int KENT = 1 << KBITS;
    constexpr int kVtab = KBITS == 12 ? kNtV : 32768;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
    const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
    Codes12Tables tabs12;
    if constexpr (KBITS == 12) {
        tabs12 = load_codes12(ksrc, vsrc, tid);
    } else {
        for (int i = tid; i < KENT; i += kThreads) reinterpret_cast<uint2*>(tab)[i] = ksrc[i];
        if (tid < 256) reinterpret_cast<uint2*>(tab + kVtab)[tid] = vsrc[tid];
    }

    float x0, x1;
    new_token_inputs<G>(q, q_f32, lambda, k_new, v_new, kv_f32, num_q_heads, num_kv_heads, g, b,
                        wave, lane, x0, x1, xnew);
    __syncthreads();

    // 1. codes
    const size_t row = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + append_pos;
    if constexpr (KBITS == 12) {
        new_token_codes12(tabs12, tab, xnew, newc, tid, lane, wave);
        // byte j of the key row holds bits [8j, 8j + 8) of the 12-bit stream
        if (tid < 48) {
            const int bit = 8 * tid, i0 = bit / 12, sh = bit % 12;
            uint32_t v = newc[0][i0] >> sh;
            if (sh > 4) v |= newc[0][i0 + 1] << (12 - sh);
            new_codes_k[row * 48 + tid] = static_cast<uint8_t>(v & 0xffu);
        } else if (tid >= 64 && tid < 64 + kNumSub) {
            new_codes_v[row * kNumSub + tid - 64] = static_cast<uint8_t>(newc[1][tid - 64]);
        }
    } else {
        // fp64 scans of the 256-entry tables: thread (slice, pos) takes
        // centroids slice, slice + 32, ... of sub-vector pos
        const int pos = tid & 31, slice = tid >> 5;
        double xk[4], xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xk[i] = xnew[0][4 * pos + i];
            xv[i] = xnew[1][4 * pos + i];
        }
        double dk = INFINITY, dv = INFINITY;
        uint32_t ik = 0, iv = 0;
        for (int c = slice; c < KENT; c += 32) {
            const double d = sqdist4_f64(xk, reinterpret_cast<const uint2*>(tab)[c]);
            if (d < dk) {
                dk = d;
                ik = static_cast<uint32_t>(c);
            }
        }
#pragma unroll 2
        for (int c = slice; c < 256; c += 32) {
            const double d = sqdist4_f64(xv, reinterpret_cast<const uint2*>(tab + kVtab)[c]);
            if (d < dv) {
                dv = d;
                iv = static_cast<uint32_t>(c);
            }
        }
        {
            const double dk2 = __shfl_xor(dk, 32, kWave), dv2 = __shfl_xor(dv, 32, kWave);
            const uint32_t ik2 = __shfl_xor(ik, 32, kWave), iv2 = __shfl_xor(iv, 32, kWave);
            if (nearer(dk2, ik2, dk, ik)) {
                dk = dk2;
                ik = ik2;
            }
            if (nearer(dv2, iv2, dv, iv)) {
                dv = dv2;
                iv = iv2;
            }
        }
        // [tensor][wave][pos]: lanes 0..31 report keys, 32..63 values
        double* sd = reinterpret_cast<double*>(scratch);
        uint32_t* si = reinterpret_cast<uint32_t*>(sd + 2 * kWaves * 32);
        const int tsel = lane >> 5;
        sd[(tsel * kWaves + wave) * 32 + pos] = tsel ? dv : dk;
        si[(tsel * kWaves + wave) * 32 + pos] = tsel ? iv : ik;
        __syncthreads();
        if (tid < 64) {
            double d0 = sd[tsel * kWaves * 32 + pos];
            uint32_t i0 = si[tsel * kWaves * 32 + pos];
            for (int w = 1; w < kWaves; ++w) {
                const double d = sd[(tsel * kWaves + w) * 32 + pos];
                const uint32_t i = si[(tsel * kWaves + w) * 32 + pos];
                if (nearer(d, i, d0, i0)) {
                    d0 = d;
                    i0 = i;
                }
            }
            newc[tsel][pos] = i0;
            (tsel ? new_codes_v : new_codes_k)[row * kNumSub + pos] = static_cast<uint8_t>(i0);
        }
        __syncthreads();
    }

    // 2. the one-token partial of each query head: lane l holds dims 2l, 2l + 1,
    //    components 2 (l % 2), + 1 of sub-vector l / 2
    if (wave < G) {
        const int j = lane >> 1, comp = 2 * (lane & 1);
        // (C_k sits at the start of tab as stored, for 8- and 12-bit keys)
        const uint2 kc = reinterpret_cast<const uint2*>(tab)[newc[0][j]];
        const uint32_t kw = comp ? kc.y : kc.x;
        const float k0 = half_bits_to_float(kw & 0xffffu);
        const float k1 = half_bits_to_float(kw >> 16);
        const uint2 vc = reinterpret_cast<const uint2*>(tab + kVtab)[newc[1][j]];
        const uint32_t vw = comp ? vc.y : vc.x;
        const float x = wave_sum(x0 * k0 + x1 * k1);
        const size_t pi = (static_cast<size_t>(b) * num_q_heads + g * G + wave) * part_stride + slot;
        part.o[pi * kHeadDim + 2 * lane] = half_bits_to_float(vw & 0xffffu);
        part.o[pi * kHeadDim + 2 * lane + 1] = half_bits_to_float(vw >> 16);
        if (lane == 0) {
            part.m[pi] = x;
            part.l[pi] = 1.f;
        }
    }
}

// The appended token in the d = 8 layout (16 sub-vectors of 8 channels; C_k
// and C_v of 4096 entries; 24-byte rows of 12-bit codes), with the decisions
// of new_token_workgroup, found by the certified matrix-core search of
// nearest_search.hpp spread over the workgroup: the 16 sub-vectors of a
// tensor are one MFMA column block, and wave w scans centroids 256 w ..
// 256 w + 255.  Per tensor: the waves' pass-1 minima meet in LDS (the
// threshold), then the fp64 minima over their candidates.
// LDS: C_k in `tab`, C_v 64 KiB above; ||c||^2 of the current tensor in
// `scratch` (16 KiB); the exchanges in `xbuf` (4 KiB).
template <int G>
__device__ __forceinline__ void new_token_workgroup8(
    const void* q, int q_f32, const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
    const void* k_new, const void* v_new, int kv_f32, int num_q_heads, int num_kv_heads, int g,
    int b, int capacity, int append_pos, uint8_t* new_codes_k, uint8_t* new_codes_v,
    Partials part, int part_stride, int slot, uint8_t* tab, uint8_t* scratch, uint8_t* xbuf,
    double (*xnew)[kHeadDim], uint32_t (*newc)[kNumSub]) {
    constexpr int kEnt = 4096, kPos = kHeadDim / 8, kRow = kPos * 12 / 8;   // 16 codes, 24 B
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint4* ksrc = reinterpret_cast<const uint4*>(cb_k) + static_cast<size_t>(g) * kEnt;
    const uint4* vsrc = reinterpret_cast<const uint4*>(cb_v) + static_cast<size_t>(g) * kEnt;
    const uint4* kt = reinterpret_cast<const uint4*>(tab);
    const uint4* vt = reinterpret_cast<const uint4*>(tab + kTable);
    for (int i = tid; i < kEnt; i += kThreads) {
        reinterpret_cast<uint4*>(tab)[i] = ksrc[i];
        reinterpret_cast<uint4*>(tab + kTable)[i] = vsrc[i];
    }
    float x0, x1;
    new_token_inputs<G>(q, q_f32, lambda, k_new, v_new, kv_f32, num_q_heads, num_kv_heads, g, b,
                        wave, lane, x0, x1, xnew);
    __syncthreads();

    // 1. codes, one tensor after the other
    static_assert(kThreads == 1024, "16 waves of 256 centroids");
    codes8_one_token(tab, kTable, reinterpret_cast<float*>(scratch), xbuf, xnew, newc, tid, lane,
                     wave);
    const size_t row = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + append_pos;
    if (tid < 2 * kRow) {   // byte j of a row holds bits [8j, 8j + 8) of the 12-bit stream
        const int tsel = tid / kRow, j = tid % kRow;
        const int bit = 8 * j, i0 = bit / 12, sh = bit % 12;
        uint32_t v = newc[tsel][i0] >> sh;
        if (sh > 4) v |= newc[tsel][i0 + 1] << (12 - sh);
        (tsel ? new_codes_v : new_codes_k)[row * kRow + j] = static_cast<uint8_t>(v & 0xffu);
    }

    // 2. the one-token partial of each query head: lane l holds dims 2l, 2l + 1,
    //    halves 2 (l % 4), + 1 of sub-vector l / 4
    if (wave < G) {
        const int j = lane >> 2, word = lane & 3;
        const uint4 kc = kt[newc[0][j]], vc = vt[newc[1][j]];
        const uint32_t kw = word == 0 ? kc.x : (word == 1 ? kc.y : (word == 2 ? kc.z : kc.w));
        const uint32_t vw = word == 0 ? vc.x : (word == 1 ? vc.y : (word == 2 ? vc.z : vc.w));
        const float x = wave_sum(x0 * half_bits_to_float(kw & 0xffffu) +
                                 x1 * half_bits_to_float(kw >> 16));
        const size_t pi = (static_cast<size_t>(b) * num_q_heads + g * G + wave) * part_stride + slot;
        part.o[pi * kHeadDim + 2 * lane] = half_bits_to_float(vw & 0xffffu);
        part.o[pi * kHeadDim + 2 * lane + 1] = half_bits_to_float(vw >> 16);
        if (lane == 0) {
            part.m[pi] = x;
            part.l[pi] = 1.f;
        }
    }
}

// Sum over the L lanes of an aligned group (L = 16 or 32), in every lane of
// the group.
template <int L>
__device__ __forceinline__ float group_sum(float v, int lane) {
    static_assert(L == 16 || L == 32, "lane group");
    if constexpr (L == 32) v += lane_partner<16>(v, lane);
    v += lane_partner<8>(v, lane);
    v += lane_partner<4>(v, lane);
    v += lane_partner<2>(v, lane);
    return v + lane_partner<1>(v, lane);
}

// The residual-window workgroup of one (sequence, KV head), for a decode
// step that keeps the most recent tokens in full precision (VecInfer page,
// Experiments: a residual of 128 full-precision tokens beside the VQ cache;
// HACK page: the last, not yet full block stays in fp16 and is multiplied in
// fp16 within the same attention).  It replaces the new-token workgroup.
//  1. The new token's k and v, rounded to fp16, go to window slot win_len.
//  2. The G query heads attend over window tokens 0 .. win_len with raw
//     keys: q . k / sqrt(D), which equals q~ . k~ (H_D orthonormal), so the
//     window needs no transform.  Wave w takes 16-token blocks w, w + 16, ...
//     on the matrix cores: scores from the heads' q (fp16 as given; fp32 as
//     fp16 hi and lo rows with one power-of-two scale per head, undone after
//     the product) against the window's key rows, an online softmax per
//     head, and the weights as fp16 hi and lo (times 2^16) rows against the
//     block's value rows staged in LDS.  Slot win_len holds the new token,
//     taken from k_new / v_new (the lanes that load it store it); slots past
//     win_len are masked.  Waves past the last block
//     (all but 8 for a 128-token window) do no work.
//  3. The states of the waves with tokens fold in LDS into one partial
//     (m, l, o) at split index `slot`, in the base-2 units of the code
//     splits.
// LDS (`lds`, the 128 KiB of the codebook tables): per wave 16 value rows at
// a stride of 136 halves (which afterwards hold the wave's G x 128 outputs),
// the waves' m and l, per wave a 16 x 16 fp16 weight tile and 8 head scales.
template <int G>
__device__ __forceinline__ void window_workgroup(
    const void* q, int q_f32, const void* k_new, const void* v_new, int kv_f32, int num_q_heads,
    int num_kv_heads, int g, int b, uint16_t* win_k, uint16_t* win_v, int win_len, int win_cap,
    Partials part, int part_stride, int slot, float* lds) {
    static_assert(G >= 1 && G <= 8, "2 G rows of one 16-row product");
    constexpr float kScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)
    constexpr int kWords = kHeadDim / 2;                                  // fp16 pairs per row
    constexpr int kVs = kHeadDim + 8;                                     // staged value row stride
    constexpr int kWaveBytes = 16 * kVs * 2;                              // 4352
    static_assert(G * kHeadDim * 4 <= kWaveBytes, "a wave's outputs fit its staging rows");
    constexpr int kFm = kWaves * kWaveBytes, kPt = kFm + 2 * kWaves * 8 * 4,
                  kSc = kPt + kWaves * 16 * 16 * 2, kEnd = kSc + kWaves * 8 * 4;
    static_assert(kEnd <= 2 * kTable, "the window's LDS fits the tables");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, n = lane & 15;
    const size_t stream = static_cast<size_t>(b) * num_kv_heads + g;
    const uint16_t* wk = win_k + stream * win_cap * kHeadDim;
    const uint16_t* wv = win_v + stream * win_cap * kHeadDim;
    uint8_t* base = reinterpret_cast<uint8_t*>(lds);
    uint16_t* vst = reinterpret_cast<uint16_t*>(base + wave * kWaveBytes);
    float* fm = reinterpret_cast<float*>(base + kFm);   // [kWaves][8] m, then [kWaves][8] l
    float* fl = fm + kWaves * 8;
    uint16_t* pt = reinterpret_cast<uint16_t*>(base + kPt) + wave * 256;   // [16 rows][16 tokens]
    float* sinv = reinterpret_cast<float*>(base + kSc) + wave * 8;         // 2^-e per head

    // the new token as the window stores it (fp16, round to nearest even),
    // two channels
    const auto new_pair = [&](const void* src, int c2) {   // channels 2 c2, 2 c2 + 1
        if (kv_f32) {
            const float2 a = reinterpret_cast<const float2*>(src)[stream * kWords + c2];
            return __builtin_bit_cast(uint32_t, half2_t{static_cast<_Float16>(a.x),
                                                        static_cast<_Float16>(a.y)});
        }
        return reinterpret_cast<const uint32_t*>(src)[stream * kWords + c2];
    };
    // 16 bytes of window row `row` (slot win_len and beyond: the new token)
    const auto row16 = [&](const uint16_t* win, const void* src, int row, int c0) {
        if (row < win_len)
            return *reinterpret_cast<const uint4*>(win + static_cast<size_t>(row) * kHeadDim + c0);
        return make_uint4(new_pair(src, c0 / 2), new_pair(src, c0 / 2 + 1), new_pair(src, c0 / 2 + 2),
                          new_pair(src, c0 / 2 + 3));
    };
    // waves past the window's last block hold no tokens: they skip to the
    // fold, which reads the first nw states only
    const int nw = min(kWaves, win_len / 16 + 1);
    if (wave < nw) {
        // a block's rows in registers: the key B operands of lane (16 grp + n)
        // (token 16 blk + n, channels 32 kk + 8 grp .. + 7) and the value rows
        // lane l copies to LDS (token l / 4, channels 32 (l % 4) + 8 j .. + 7);
        // the wave's first block is requested before the query, so the two
        // memory latencies overlap
        uint4 kb[4], vb[4];
        const int tk = 16 * wave + n, tv = 16 * wave + (lane >> 2);
        if (!kv_f32) {   // fp16 new token: one load per operand, no branch
            const uint16_t* rk = tk < win_len ? wk + static_cast<size_t>(tk) * kHeadDim
                                              : static_cast<const uint16_t*>(k_new) + stream * kHeadDim;
            const uint16_t* rv = tv < win_len ? wv + static_cast<size_t>(tv) * kHeadDim
                                              : static_cast<const uint16_t*>(v_new) + stream * kHeadDim;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kb[kk] = *reinterpret_cast<const uint4*>(rk + 32 * kk + 8 * grp);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vb[j] = *reinterpret_cast<const uint4*>(rv + 32 * (lane & 3) + 8 * j);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kb[kk] = row16(wk, k_new, tk, 32 * kk + 8 * grp);
#pragma unroll
            for (int j = 0; j < 4; ++j) vb[j] = row16(wv, v_new, tv, 32 * (lane & 3) + 8 * j);
        }

        // score A operands: lane (16 grp + r) holds row r (head r % 8, hi for
        // r < 8, lo after) at channels 32 kk + 8 grp .. + 7.  An fp16 query is
        // its own hi row (lo rows zero, products exact in fp32); an fp32 one
        // is scaled by 2^e per head (its largest |q| to [2^14, 2^15)) and
        // split into fp16 hi and lo, the scale undone after the product.
        // inv[r]: the factor from a score row to log2 units
        const int hr = n & 7;
        const bool hi_row = n < 8, live_row = hr < G;
        const size_t qrow =
            (static_cast<size_t>(b) * num_q_heads + g * G + min(hr, G - 1)) * kHeadDim + 8 * grp;
        // output rows of lane (16 grp + n): 4 grp + r, head hq + r (hi rows in
        // groups 0 and 1, lo rows in 2 and 3)
        const int hq = 4 * (grp & 1);
        half8_t aq[4];
        float inv[4];
        if (!q_f32) {
            const uint16_t* qh = static_cast<const uint16_t*>(q) + qrow;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4 u = *reinterpret_cast<const uint4*>(qh + 32 * kk);
                aq[kk] = __builtin_bit_cast(half8_t, (hi_row && live_row) ? u : make_uint4(0, 0, 0, 0));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) inv[r] = kScale;
        } else {
            // all of the lane's query words are requested before any is used
            const float* qf = static_cast<const float*>(q) + qrow;
            float qv[4][8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 u = *reinterpret_cast<const float4*>(qf + 32 * kk);
                const float4 v = *reinterpret_cast<const float4*>(qf + 32 * kk + 4);
                const float t[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) qv[kk][j] = t[j];
            }
            float amax = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(qv[kk][j]));
            // the 8 lanes of a head: n and n ^ 8, in every lane group
            amax = fmaxf(amax, lane_partner<8>(amax, lane));
            amax = fmaxf(amax, lane_partner<16>(amax, lane));
            amax = fmaxf(amax, lane_partner<32>(amax, lane));
            const int ex = min(15 - __builtin_amdgcn_frexp_expf(amax), 126);
            if (lane < 8) sinv[lane] = __builtin_amdgcn_ldexpf(kScale, -ex);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = __builtin_amdgcn_ldexpf(qv[kk][j], ex);
                    const _Float16 h = static_cast<_Float16>(x);
                    const _Float16 l = static_cast<_Float16>(x - static_cast<float>(h));
                    aq[kk][j] = live_row ? (hi_row ? h : l) : static_cast<_Float16>(0.f);
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int r = 0; r < 4; ++r) inv[r] = sinv[hq + r];
        }

        float m[4], l[4];
        float4_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};

        // one block; kPre: its rows are in kb / vb, else they are loaded here
        const auto block = [&](int blk, auto pre) {
            constexpr bool kPre = decltype(pre)::value;
            // the block's value rows into this wave's LDS rows; in a wave's
            // first block the lanes that hold the new token's fp16 k and v
            // also store them to window slot win_len
            uint16_t* slot_k = win_k + (stream * win_cap + win_len) * kHeadDim;
            uint16_t* slot_v = win_v + (stream * win_cap + win_len) * kHeadDim;
            const int tv = 16 * blk + (lane >> 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c0 = 32 * (lane & 3) + 8 * j;
                const uint4 vr = kPre ? vb[j] : row16(wv, v_new, tv, c0);
                *reinterpret_cast<uint4*>(vst + (lane >> 2) * kVs + c0) = vr;
                if (kPre && tv == win_len) *reinterpret_cast<uint4*>(slot_v + c0) = vr;
            }
            // scores of token t = 16 blk + n
            const int t = 16 * blk + n;
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int c0 = 32 * kk + 8 * grp;
                const uint4 kr = kPre ? kb[kk] : row16(wk, k_new, t, c0);
                if (kPre && t == win_len) *reinterpret_cast<uint4*>(slot_k + c0) = kr;
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[kk], __builtin_bit_cast(half8_t, kr), s,
                                                           0, 0, 0);
            }
            // hi + lo rows: every lane then holds heads hq .. hq + 3 of token n
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = s[r] + lane_partner<32>(s[r], lane);
                x[r] = t <= win_len ? v * inv[r] : -INFINITY;
            }
            float f[4], pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mn = fmaxf(m[r], row_max16(x[r]));   // finite: token 16 blk is live
                f[r] = (m[r] == -INFINITY) ? 0.f : fast_exp2(m[r] - mn);
                pv[r] = fast_exp2(x[r] - mn);
                l[r] = l[r] * f[r] + pv[r];
                m[r] = mn;
            }
            // weights tile: row 4 grp + r, column n; hi parts round toward zero,
            // lo = (p - hi) 2^16 (groups 2 and 3)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const _Float16 ph =
                    __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv[r], 0.f))[0];
                const _Float16 pl = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(
                                        (pv[r] - static_cast<float>(ph)) * kLoScale, 0.f))[0];
                pt[(4 * grp + r) * 16 + n] = __builtin_bit_cast(uint16_t, grp < 2 ? ph : pl);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[c][r] *= f[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // value product: A = weight rows (tokens 4 grp .. + 3), B = value
            // rows of the same tokens at channel 16 c + n
            const half4_t ap = *reinterpret_cast<const half4_t*>(pt + n * 16 + 4 * grp);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                half4_t bv;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bv[j] = __builtin_bit_cast(_Float16, vst[(4 * grp + j) * kVs + 16 * c + n]);
                o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap, bv, o[c], 0, 0, 0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        block(wave, std::true_type{});
        for (int blk = wave + kWaves; 16 * blk <= win_len; blk += kWaves)
            block(blk, std::false_type{});
        // past the first blocks (windows over 256 tokens) wave 0 stores the
        // new token, two channels per lane
        if (win_len >= 16 * kWaves && wave == 0) {
            reinterpret_cast<uint32_t*>(win_k)[(stream * win_cap + win_len) * kWords + lane] =
                new_pair(k_new, lane);
            reinterpret_cast<uint32_t*>(win_v)[(stream * win_cap + win_len) * kWords + lane] =
                new_pair(v_new, lane);
        }
        // the wave's state: l summed over its lanes' tokens, o = hi + lo 2^-16
        // rows (lanes 0-31), into its staging rows and the m / l arrays
        float* fo = reinterpret_cast<float*>(vst);   // [G][128]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ls = row_sum16(l[r]);
            const int h = hq + r;
            if (lane < 32 && n == 0 && h < G) {
                fm[wave * 8 + h] = m[r];
                fl[wave * 8 + h] = ls;
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = fmaf(lane_partner<32>(o[c][r], lane), kLoUnscale, o[c][r]);
                if (lane < 32 && hq + r < G) fo[(hq + r) * kHeadDim + 16 * c + n] = v;
            }
    }
    __syncthreads();
    for (int i = tid; i < G * kHeadDim; i += kThreads) {
        const int h = i / kHeadDim, d = i % kHeadDim;
        float mx = -INFINITY;
        for (int w = 0; w < nw; ++w) mx = fmaxf(mx, fm[w * 8 + h]);
        float ls = 0.f, os = 0.f;
        for (int w = 0; w < nw; ++w) {
            const float fw = fast_exp2(fm[w * 8 + h] - mx);   // every state holds a token
            ls += fw * fl[w * 8 + h];
            os += fw * reinterpret_cast<const float*>(base + w * kWaveBytes)[h * kHeadDim + d];
        }
        const size_t pi = (static_cast<size_t>(b) * num_q_heads + g * G + h) * part_stride + slot;
        part.o[pi * kHeadDim + d] = os;
        if (d == 0) {
            part.m[pi] = mx;
            part.l[pi] = ls;
        }
    }
}

template <int G, int KBITS, int SUB, bool LUT>
__global__ __launch_bounds__(kThreads, 1) void vq_attention_mfma_kernel(
    const void* __restrict__ q, int q_f32, const float* __restrict__ lambda,
    const uint16_t* __restrict__ cb_k, const uint16_t* __restrict__ cb_v,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v, int num_q_heads,
    int num_kv_heads, int capacity, int context_len, int num_splits, int tokens_per_split,
    Partials part, const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    int append_pos, uint8_t* __restrict__ new_codes_k, uint8_t* __restrict__ new_codes_v,
    int part_stride, uint16_t* __restrict__ win_k, uint16_t* __restrict__ win_v, int win_len,
    int win_cap, int fold, int static_tiles) {
    static_assert(G >= 1 && G <= 8, "2G MFMA rows");
    // G <= 4: the rows of every head are in lanes 0-31 of an MFMA result, so
    // the softmax packs a tile's two 16-token blocks into one set of lanes
    constexpr bool kPack = G <= 4;
    constexpr int kSb = kPack ? 1 : 2;   // 16-token score blocks per lane and tile
    // SUB = 8: the 1.5-bit layout, 16 sub-vectors of 8 channels per vector,
    // 4096-entry C_k and C_v (64 KiB each, unreplicated), 24-byte rows of
    // 12-bit codes for K and V
    constexpr bool kD8 = SUB == 8;
    static_assert(SUB == 4 || (SUB == 8 && KBITS == 12), "d = 4, or d = 8 with 12-bit codes");
    // LUT: the lookup-table score path (8-bit keys, d = 4, G <= 4): scores
    // are sums over the 32 positions of LUT[pos][code][head] = q~ . C_k[code]
    // entries instead of matrix-core products; values as below, from a
    // 4-copy table (the LUT takes the 128 KiB of the replicated tables)
    static_assert(!LUT || (KBITS == 8 && SUB == 4 && G <= 4), "LUT scores: 8-bit keys, d = 4, G <= 4");
    constexpr int KROW = kD8 ? 24 : kNumSub * KBITS / 8;
    constexpr int VROW = kD8 ? 24 : kNumSub;

    __shared__ __attribute__((aligned(16))) uint8_t tab[2 * kTable];       // keys | values
    __shared__ __attribute__((aligned(16))) uint2 pbuf[kWaves][kTok * 4];  // [token][16 rows] fp16
    __shared__ half8_t qa[4][64];
    __shared__ float qsc[8];   // per head: 2^-e, the inverse of q~'s scale in qa
    __shared__ float wmT[G][kWaves], wlT[G][kWaves];   // per head and wave: m, rescaled l
    __shared__ uint32_t tile_ctr;   // next 32-token tile of the split to hand out
    // appended token (new-token workgroup): transformed key and value (fp64)
    __shared__ double xnew[2][kHeadDim];
    __shared__ uint32_t newc[2][kNumSub];   // its key and value codes
    // LUT: the value table (4 copies of 256 x 8 B) and q~ in fp32 (base-2 scale)
    __shared__ __attribute__((aligned(16))) uint8_t vtab4[LUT ? 4 * 256 * 8 : 16];
    __shared__ __attribute__((aligned(16))) float qf[LUT ? G : 1][LUT ? kHeadDim : 1];

    // A 1-D grid, split-major: the workgroups of split s of every stream
    // (sequence, KV head) follow those of split s - 1, and the extra
    // workgroups (split == num_splits: the new token or the window) come
    // last, so every split workgroup is dispatched before any of them.  With
    // `fold` there are no extra workgroups: the last split of a stream
    // encodes the new token (or attends over the window) first, then attends
    // over its own tokens.
    const int extra = (append_pos >= 0 && !fold) ? 1 : 0;
    const int streams = static_cast<int>(gridDim.x) / (num_splits + extra);
    const int split = static_cast<int>(blockIdx.x) / streams;
    const int stream_id = static_cast<int>(blockIdx.x) - split * streams;
    const int g = stream_id % num_kv_heads, b = stream_id / num_kv_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: tile indices stay in SGPRs
    if (append_pos >= 0 && split == num_splits - 1 + extra && win_k != nullptr) {   // the window
        window_workgroup<G>(q, q_f32, k_new, v_new, kv_f32, num_q_heads, num_kv_heads, g, b, win_k,
                            win_v, win_len, win_cap, part, part_stride, num_splits,
                            reinterpret_cast<float*>(tab));
        if (extra) return;
        __syncthreads();   // the LDS is free for the split
    } else if (append_pos >= 0 && split == num_splits - 1 + extra) {   // the new token
        if constexpr (kD8)
            new_token_workgroup8<G>(q, q_f32, lambda, cb_k, cb_v, k_new, v_new, kv_f32,
                                    num_q_heads, num_kv_heads, g, b, capacity, append_pos, new_codes_k,
                                    new_codes_v, part, part_stride, num_splits, tab,
                                    reinterpret_cast<uint8_t*>(&pbuf[0][0]),
                                    reinterpret_cast<uint8_t*>(&qa[0][0]), xnew, newc);
        else
            new_token_workgroup<G, KBITS>(q, q_f32, lambda, cb_k, cb_v, k_new, v_new, kv_f32,
                                          num_q_heads, num_kv_heads, g, b, capacity, append_pos,
                                          new_codes_k, new_codes_v, part, part_stride,
                                          num_splits, tab,
                                          reinterpret_cast<uint8_t*>(&pbuf[0][0]), xnew, newc);
        if (extra) return;
        __syncthreads();   // the LDS is free for the split
    }
    const int grp = lane >> 4, n = lane & 15;
    const int kq = n >> 2, aq4 = n & 3;   // fetch-lane split of n for the transposed reads

    const int t_begin = split * tokens_per_split;
    const int t_len = min(tokens_per_split, context_len - t_begin);   // no int overflow
    const size_t row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + t_begin;
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes_k + row0 * KROW), 0, t_len * KROW, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes_v + row0 * VROW), 0, t_len * VROW, kBufferWord3);
    // per-lane byte offsets of the chunks inside a tile (d = 8: the dword-
    // aligned 8 bytes that hold codes 4 j .. 4 j + 3, and the shift to them)
    const uint32_t koff0 = static_cast<uint32_t>(
        n * KROW + (kD8 ? 12 * (grp >> 1) + 4 * (grp & 1) : (KBITS == 8 ? 8 : 12) * grp));
    const uint32_t koff1 = koff0 + 16 * KROW;
    const uint32_t voff0 = static_cast<uint32_t>(
        (8 * grp + kq) * VROW + (kD8 ? 12 * (aq4 >> 1) + 4 * (aq4 & 1) : 8 * aq4));
    const uint32_t voff1 = voff0 + 4 * VROW;
    const uint32_t ksh = 16u * static_cast<uint32_t>(grp & 1);   // d = 8 only
    // LUT: lane 16 grp + n scores token 16 (grp / 2) + n (the packed softmax's
    // token) for heads 2 (grp % 2), + 1 over all 32 positions
    const uint32_t koffL = static_cast<uint32_t>((16 * (grp >> 1) + n) * KROW);
    const uint32_t vsh = 16u * static_cast<uint32_t>(aq4 & 1);

    // ---- prologue ----------------------------------------------------------
    if (tid == 0) tile_ctr = kWaves;   // tiles 0 .. kWaves-1 go to waves 0 .. kWaves-1
    // Every prologue load is unconditional (indices clamped into range, code
    // loads range-checked), so the waits that follow can count outstanding
    // loads instead of draining them: codebook entries, q and lambda go out
    // first (they gate the tables and q~), then the first tile of codes, which
    // stays in flight while the tables are built.
    const uint2* vsrc = reinterpret_cast<const uint2*>(cb_v) + static_cast<size_t>(g) * 256;
    const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
    uint2 centroid;
    uint2 kcent[KBITS == 8 ? 1 : 4];
    uint4 cent8[kD8 ? 8 : 1];   // d = 8: entries tid + 1024 i of C_k (i < 4), C_v (i >= 4)
    if constexpr (kD8) {
        const uint4* k8 = reinterpret_cast<const uint4*>(cb_k) + static_cast<size_t>(g) * 4096;
        const uint4* v8 = reinterpret_cast<const uint4*>(cb_v) + static_cast<size_t>(g) * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cent8[i] = k8[tid + i * kThreads];
            cent8[4 + i] = v8[tid + i * kThreads];
        }
    } else if constexpr (LUT) {
        // thread: C_k entry tid % 256 (its LUT entries), C_v entry tid % 256
        kcent[0] = ksrc[tid & 255];
        centroid = vsrc[tid & 255];
    } else if constexpr (KBITS == 8) {
        // thread: code = tid / 4, table = (tid / 2) % 2, slots 16 (tid % 2) .. + 15
        centroid = ((tid >> 1) & 1) ? vsrc[tid >> 2] : ksrc[tid >> 2];
    } else {
        centroid = vsrc[(tid >> 1) & 255];                  // used by tid < 512
#pragma unroll
        for (int i = 0; i < 4; ++i) kcent[i] = ksrc[tid + i * kThreads];
    }
    // q row of head min(wave, G - 1), two consecutive elements per lane: as
    // fp32, words 2 lane and 2 lane + 1; as fp16, both halves of word lane
    const size_t vec = static_cast<size_t>(b) * num_q_heads + g * G + min(wave, G - 1);
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(q) +
                         (q_f32 ? vec * kHeadDim + 2 * lane : vec * (kHeadDim / 2) + lane);
    const uint32_t qw0 = qw[0];
    const uint32_t qw1 = qw[q_f32 ? 1 : 0];
    const float2 lam2 = reinterpret_cast<const float2*>(lambda + g * kHeadDim)[lane];
    using KC = std::conditional_t<kD8, Chunk8, std::conditional_t<LUT, LutCodes, KChunk<KBITS>>>;
    using VC = std::conditional_t<kD8, Chunk8, uint2>;
    KC kA[2];
    VC vA[2];
    // (the whole offset goes in the VGPR operand: the buffer range check
    // covers the VGPR offset, not the scalar one)
    auto load_k = [&](int rel, KC* kk_) {
        const uint32_t ks = static_cast<uint32_t>(rel * KROW);
        if constexpr (LUT) {
            kk_[0].load(krsrc, koffL + ks);
        } else if constexpr (kD8) {
            kk_[0].load(krsrc, koff0 + ks);
            kk_[1].load(krsrc, koff1 + ks);
        } else {
            kk_[0].load(krsrc, koff0 + ks, 0);
            kk_[1].load(krsrc, koff1 + ks, 0);
        }
    };
    auto load_v = [&](int rel, VC* vv_) {
        const uint32_t vs = static_cast<uint32_t>(rel * VROW);
        if constexpr (kD8) {
            vv_[0].load(vrsrc, voff0 + vs);
            vv_[1].load(vrsrc, voff1 + vs);
        } else {
            const auto v0 = __builtin_amdgcn_raw_buffer_load_b64(vrsrc, voff0 + vs, 0, 0);
            const auto v1 = __builtin_amdgcn_raw_buffer_load_b64(vrsrc, voff1 + vs, 0, 0);
            vv_[0] = make_uint2(v0[0], v0[1]);
            vv_[1] = make_uint2(v1[0], v1[1]);
        }
    };
    auto load_tile = [&](int rel, KC* kk_, VC* vv_) {
        load_k(rel, kk_);
        load_v(rel, vv_);
    };
    load_tile(wave * kTok, kA, vA);   // past the split's end: range-checked, reads zeros
    __builtin_amdgcn_sched_barrier(0);   // keep the table writes (and their wait) below

    {
        const uint4 cc = make_uint4(centroid.x, centroid.y, centroid.x, centroid.y);
        // A thread fills half a row (8 x 16 B).  Its 16-B slots are taken in
        // an order rotated by tid / 2, so any 16 consecutive lanes store to
        // 16 distinct 16-B bank groups: without the rotation every lane of a
        // half row hits the same four banks, and the table build took longer
        // than the rest of the prologue.
        const int rot = tid >> 1;
        if constexpr (LUT) {   // the 4-copy value table; the LUT follows q~
            if (tid < 256) {
                reinterpret_cast<uint4*>(vtab4)[2 * tid] = cc;
                reinterpret_cast<uint4*>(vtab4)[2 * tid + 1] = cc;
            }
        } else if constexpr (kD8) {   // C_k then C_v, 16-byte entries, stored once
            // The value table is read 8 bytes (half an entry) at a time: an
            // entry whose code has bit 4 set keeps its halves swapped, so the
            // reads of one half over random codes spread over all 32 bank
            // pairs instead of 16 (entry tid + 1024 i has bit 4 of tid).
            const bool swap_halves = (tid & 16) != 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                reinterpret_cast<uint4*>(tab)[tid + i * kThreads] = cent8[i];
                const uint4 v = cent8[4 + i];
                reinterpret_cast<uint4*>(tab + kTable)[tid + i * kThreads] =
                    swap_halves ? make_uint4(v.z, v.w, v.x, v.y) : v;
            }
        } else if constexpr (KBITS == 8) {
            uint4* dst = reinterpret_cast<uint4*>(tab + ((tid >> 1) & 1) * kTable +
                                                  (tid >> 2) * 256 + (tid & 1) * 128);
#pragma unroll
            for (int s = 0; s < 8; ++s) dst[(s + rot) & 7] = cc;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint2*>(tab + (tid + i * kThreads) * 8) = kcent[i];
            if (tid < 512) {
                uint4* dst = reinterpret_cast<uint4*>(tab + kTable + (tid >> 1) * 256 + (tid & 1) * 128);
#pragma unroll
                for (int s = 0; s < 8; ++s) dst[(s + rot) & 7] = cc;
            }
        }
    }
    if constexpr (kPack) {   // p rows 8-15 (heads 4-7) are never written: keep them zero
        reinterpret_cast<uint4*>(&pbuf[0][0])[tid] = make_uint4(0u, 0u, 0u, 0u);
        static_assert(sizeof(pbuf) == kThreads * sizeof(uint4), "one 16-byte store per thread");
    }
    // Waves 0 .. G - 1 transform head `wave`; waves G .. 7 leave zeros.  Waves
    // 0 .. 7 then write their rows straight into the score A operand, shared
    // by every wave: lane (16 qg + r) of K-step kk holds row r for dims
    // 32 qg + 8 kk + e, e = 0 .. 7, where row r is head 2 (r / 4) + r % 2, its
    // fp16 high part for r % 4 < 2, else the low part (x - hi rounded to
    // fp16), both of x 2^e (the head's largest element in [2^14, 2^15); 2^-e
    // goes to qsc).  This lane's dims 2 lane, 2 lane + 1 are elements
    // e = 2 (lane % 4), + 1 of entry qg = lane / 16, kk = lane % 16 / 4.
    // Only G waves (one per SIMD at G = 4) run the butterflies: with every
    // wave transforming, the 16 copies took most of the prologue.  The empty
    // asm keeps the q loads (issued first, every wave) ahead of the branch,
    // so they are not sunk behind the tile loads.
    asm volatile("" ::"v"(qw0), "v"(qw1), "v"(lam2.x), "v"(lam2.y));
    if (wave < 8) {
        float x0 = 0.f, x1 = 0.f;
        if (wave < G) {
            x0 = (q_f32 ? __builtin_bit_cast(float, qw0) : lo_half_to_float(qw0)) * lam2.x;
            x1 = (q_f32 ? __builtin_bit_cast(float, qw1) : hi_half_to_float(qw0)) * lam2.y;
            fwht128(x0, x1);
            x0 *= kScoreScaleLog2;
            x1 *= kScoreScaleLog2;
        }
        if constexpr (LUT) {   // q~ in fp32 for the LUT build; scores come unscaled
            if (wave < G) {
                qf[wave][2 * lane] = x0;
                qf[wave][2 * lane + 1] = x1;
            }
            if (lane == 0) qsc[wave] = 1.f;
        } else {
            const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
            const int ex = min(15 - __builtin_amdgcn_frexp_expf(amax), 126);
            x0 = __builtin_amdgcn_ldexpf(x0, ex);
            x1 = __builtin_amdgcn_ldexpf(x1, ex);
            if (lane == 0) qsc[wave] = __builtin_amdgcn_ldexpf(1.f, -ex);
            const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
            const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
            const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
            const int r = 4 * (wave >> 1) + (wave & 1);
            const int kk = (lane & 15) >> 2, qg = lane >> 4;
            uint32_t* row = reinterpret_cast<uint32_t*>(&qa[kk][16 * qg + r]) + (lane & 3);
            row[0] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
            row[8] = __builtin_bit_cast(uint32_t, half2_t{l0, l1});   // row r + 2
        }
    }
    __syncthreads();
    if constexpr (LUT) {
        // The lookup table (VecInfer page, Appendix, Algorithm 1: the table of
        // the query against C_k, then scores as sums of its entries):
        // LUT[pos][code] holds q~_h[4 pos .. 4 pos + 3] . C_k[code] for heads
        // h = 0 .. 3 (zero for h >= G), base-2 score units, 16 bytes per entry.
        // Thread: code tid % 256, positions tid / 256 + 4 k.
        const uint2 c = kcent[0];
        const float c0 = lo_half_to_float(c.x), c1 = hi_half_to_float(c.x);
        const float c2 = lo_half_to_float(c.y), c3 = hi_half_to_float(c.y);
        const int code = tid & 255;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int pos = (tid >> 8) + 4 * k;
            float e[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                e[h] = 0.f;
                if (h < G) {
                    const float4_t qv = *reinterpret_cast<const float4_t*>(&qf[h][4 * pos]);
                    e[h] = fmaf(qv[3], c3, fmaf(qv[2], c2, fmaf(qv[1], c1, qv[0] * c0)));
                }
            }
            reinterpret_cast<float4_t*>(tab)[pos * 256 + code] = float4_t{e[0], e[1], e[2], e[3]};
        }
        __syncthreads();
    }

    // MFMA rows of lane 16 grp + n: 4 grp .. 4 grp + 3 = (hA hi, hB hi, hA lo, hB lo)
    const int hA = 2 * grp, hB = 2 * grp + 1;
    // softmax state of the lane: heads sh, sh + 1 for token tok0 + n of each
    // 16-token block it holds (see the online softmax below)
    const int sh = kPack ? 2 * (grp & 1) : hA;
    const int tok0 = kPack ? 16 * (grp >> 1) : 0;
    // heads >= G start at m = +inf, so their p = 2^(s - m) is 0 with no mask
    float mA = sh < G ? -INFINITY : INFINITY;
    float mB = sh + 1 < G ? -INFINITY : INFINITY;
    float lA = 0.f, lB = 0.f;
    // MFMA scores are s 2^e: rsA, rsB = 2^-e of the lane's heads; m and l are
    // in base-2 units, the rescale thresholds (m + tau) 2^e in MFMA units
    const float rsA = qsc[sh], rsB = qsc[sh + 1];
    const float scA = 1.f / rsA, scB = 1.f / rsB;   // exact: powers of two
    float thA = (mA + kTau) * scA, thB = (mB + kTau) * scB;
    float4_t oacc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    // p tile of a wave: the 8-byte chunk (token t, rows 4 rb .. 4 rb + 3) sits
    // in slot 4 t' + (rb ^ 2 o), with o = bit 3 of t and t' = t ^ 4 o.  With
    // the plain [token][row] order the chunk writes of a 16-lane group hit
    // every bank pair twice and the transposed reads of lanes 0-15 and 16-31
    // shared banks (measured: 32 and 4 LDS cycles per instruction); with the
    // swizzle every 16- or 32-lane write group and every 32-lane read group
    // covers distinct banks (8 and 2 cycles).
    uint2* pw = pbuf[wave];
    // the score A operand stays in registers for the whole loop
    const half8_t qr[4] = {qa[0][lane], qa[1][lane], qa[2][lane], qa[3][lane]};
    const uint8_t* pw_bytes = reinterpret_cast<const uint8_t*>(pw);
    const int ow = (n >> 3) & 1, orr = grp & 1;
    const int rbw = kPack ? (grp & 1) : grp;   // row block (head pair) this lane writes
    const int pslot_w = 4 * tok0 + 4 * (n ^ (ow << 2)) + (rbw ^ (2 * ow));   // token tok0 + n (+ 64: + 16)
    const uint32_t pread0 = 8u * (4 * (8 * grp + 4 * orr + kq) + (aq4 ^ (2 * orr)));        // tokens 8 grp + kq
    const uint32_t pread1 = 8u * (4 * (8 * grp + 4 * (orr ^ 1) + kq) + (aq4 ^ (2 * orr)));  // tokens 8 grp + 4 + kq
    const uint32_t kslot = static_cast<uint32_t>(lane & 31) * 8;               // key table
    const uint32_t vslot = 0x10000u | (static_cast<uint32_t>(lane & 31) * 8);  // value table
    const uint32_t vcopy = static_cast<uint32_t>(lane & 3) * 8;                // LUT: value copy

    auto compute_tile = [&](int rel_, KC* kc, VC* vc, int nrel) {
        // ---- scores: 2 blocks of 16 tokens, 4 K-steps of 32 dims ------------
        float4_t sacc[2];
        float lutA = 0.f, lutB = 0.f;   // LUT: the lane's scores of heads sh, sh + 1
        if constexpr (LUT) {
            // one 8-byte read per position: the lane's head pair of entry
            // (pos, code), summed in position order
            const uint8_t* lrow = tab + 8 * (grp & 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t w = kc[0].w[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t code = (w >> (8 * k)) & 0xffu;
                    const float2 e = *reinterpret_cast<const float2*>(lrow + (4 * i + k) * 4096 +
                                                                      code * 16);
                    lutA += e.x;
                    lutB += e.y;
                }
            }
        } else if constexpr (kD8) {
            // K-step kk of lane (16 grp + n): dims 32 grp + 8 kk .. + 7 of its
            // token = the centroid of code kk of its chunk, one 16-byte gather
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                uint32_t c[4];
                kc[sb].codes(ksh, c);
                half8_t kg[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    kg[kk] = *reinterpret_cast<const half8_t*>(tab + (c[kk] << 4));
                sacc[sb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qr[kk], kg[kk], sacc[sb],
                                                                      0, 0, 0);
            }
        } else
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
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qr[kk], cat(kg[0], kg[1]),
                                                                  sacc[sb], 0, 0, 0);
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qr[kk + 1], cat(kg[2], kg[3]),
                                                                  sacc[sb], 0, 0, 0);
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        // this tile's key codes are consumed: the next tile's go into the same registers
        load_k(nrel, kc);
        __builtin_amdgcn_sched_barrier(0);
        // ---- online softmax (base 2) -----------------------------------------
        // With G <= 4 every head's rows sit in lanes 0-31, so the scores of
        // tokens 16-31 move to lanes 32-63 (one permlane swap) and the
        // softmax runs once per tile: lane 16 grp + n then holds token
        // 16 (grp / 2) + n of heads 2 (grp % 2) and 2 (grp % 2) + 1.
        float sA[kSb], sB[kSb];
        if constexpr (LUT) {
            sA[0] = lutA;
            sB[0] = lutB;
        } else if constexpr (kPack) {
            sA[0] = lo_halves(sacc[0][0] + sacc[0][2], sacc[1][0] + sacc[1][2]);
            sB[0] = lo_halves(sacc[0][1] + sacc[0][3], sacc[1][1] + sacc[1][3]);
        } else {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                sA[sb] = sacc[sb][0] + sacc[sb][2];
                sB[sb] = sacc[sb][1] + sacc[sb][3];
            }
        }
        if (__builtin_expect(rel_ + kTok > t_len, 0)) {   // the split's last, partial tile
#pragma unroll
            for (int sb = 0; sb < kSb; ++sb) {
                const bool live = rel_ + tok0 + 16 * sb + n < t_len;
                sA[sb] = live ? sA[sb] : -INFINITY;
                sB[sb] = live ? sB[sb] : -INFINITY;
            }
        }
        // A row's maximum exceeds m + tau exactly when one of its scores
        // does, so the rescale test needs no row reduction; the row maxima
        // are formed only on the (rare) rescale.
        // (one wave ballot per comparison: the masks combine in SGPRs)
        uint64_t over = 0;
#pragma unroll
        for (int sb = 0; sb < kSb; ++sb)
            over |= __builtin_amdgcn_ballot_w64(sA[sb] > thA) | __builtin_amdgcn_ballot_w64(sB[sb] > thB);
        if (over != 0) {
            float cA = sA[0], cB = sB[0];
            if constexpr (!kPack) {
                cA = fmaxf(sA[0], sA[1]);
                cB = fmaxf(sB[0], sB[1]);
            }
            cA = row_max16(cA);
            cB = row_max16(cB);
            if constexpr (kPack) {   // the same heads' other 16 tokens
                cA = fmaxf(cA, lane_partner<32>(cA, lane));
                cB = fmaxf(cB, lane_partner<32>(cB, lane));
            }
            const float nA = fmaxf(mA, cA * rsA), nB = fmaxf(mB, cB * rsB);
            const float fA = rescale_factor(mA, nA), fB = rescale_factor(mB, nB);
            mA = nA;
            mB = nB;
            thA = (nA + kTau) * scA;
            thB = (nB + kTau) * scB;
            lA *= fA;
            lB *= fB;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                oacc[c][0] *= fA;
                oacc[c][1] *= fB;
                oacc[c][2] *= fA;
                oacc[c][3] *= fB;
            }
        }
#pragma unroll
        for (int sb = 0; sb < kSb; ++sb) {
            const float pA = fast_exp2(fmaf(sA[sb], rsA, -mA));
            const float pB = fast_exp2(fmaf(sB[sb], rsB, -mB));
            lA += pA;
            lB += pB;
            // hi parts round toward zero; the remainders are exact in fp32,
            // and so are they times 2^16 (below 2^14: no fp16 overflow)
            const uint32_t hi = pack_rtz(pA, pB);
            const uint32_t lo = pack_rtz((pA - lo_half_to_float(hi)) * kLoScale,
                                         (pB - hi_half_to_float(hi)) * kLoScale);
            pw[pslot_w + 64 * sb] = make_uint2(hi, lo);   // this lane's token, rows of its heads
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // V A operand: lane (16 grp + r) gets p row r of tokens 8 grp .. 8 grp + 7
        const half8_t ap = cat(read_tr16(pw_bytes + pread0), read_tr16(pw_bytes + pread1));

        // ---- values: 8 N-tiles of 16 channels, gathered 2 tiles at a time ------
        // N-tile c, column 4a + e is channel 4 (8a + c) + e = 32 a + 4 c + e
        if constexpr (kD8) {
            // channel 32 a + 4 c + e is element 4 (c % 2) + e of the centroid
            // of code c / 2 of the chunk (positions 4 a ..): the fetching lane
            // points the transposing read at that half of the 16-byte entry
            // (halves swapped where bit 4 of the code is set: bit 3 of the
            // address flips)
            uint32_t c0[4], c1[4];
            vc[0].codes(vsh, c0);
            vc[1].codes(vsh, c1);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t a0 = kTable + (c0[q4] << 4), a1 = kTable + (c1[q4] << 4);
                const uint32_t f0 = (c0[q4] >> 1) & 8u, f1 = (c1[q4] >> 1) & 8u;
                half4_t x[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    x[i][0] = read_tr16(tab + ((a0 + 8 * i) ^ f0));
                    x[i][1] = read_tr16(tab + ((a1 + 8 * i) ^ f1));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    oacc[2 * q4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        ap, cat(x[i][0], x[i][1]), oacc[2 * q4 + i], 0, 0, 0);
            }
        } else
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint32_t w0 = (q4 < 2) ? vc[0].x : vc[0].y;
            const uint32_t w1 = (q4 < 2) ? vc[1].x : vc[1].y;
            half4_t x[2][2];
            if constexpr (LUT) {   // the 4-copy table: 32-byte rows, copy lane % 4
                const int b0 = (q4 & 1) ? 2 : 0;
                x[0][0] = read_tr16(vtab4 + ((((w0 >> (8 * b0)) & 0xffu) << 5) | vcopy));
                x[0][1] = read_tr16(vtab4 + ((((w1 >> (8 * b0)) & 0xffu) << 5) | vcopy));
                x[1][0] = read_tr16(vtab4 + ((((w0 >> (8 * b0 + 8)) & 0xffu) << 5) | vcopy));
                x[1][1] = read_tr16(vtab4 + ((((w1 >> (8 * b0 + 8)) & 0xffu) << 5) | vcopy));
            } else if ((q4 & 1) == 0) {
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
            for (int i = 0; i < 2; ++i)
                oacc[2 * q4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    ap, cat(x[i][0], x[i][1]), oacc[2 * q4 + i], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_v(nrel, vc);   // and the value codes
    };

    // Tiles are handed out from an LDS counter as waves become free: the SIMD
    // issue arbiter favours older waves, so a fixed interleave leaves the
    // youngest waves with a long tail (it is used only in deterministic mode).  A single register set holds a tile's
    // codes and is refilled during the tile (a second set, alternated by
    // unrolling, made the compiler copy the 32 output accumulators on every
    // other tile).
    auto grab = [&]() -> int {
        uint32_t v = 0;
        if (lane == 0) v = atomicAdd(&tile_ctr, 1u);
        return static_cast<int>(__builtin_amdgcn_readfirstlane(v));
    };
    int cur = wave;
    while (cur * kTok < t_len) {
        const int nxt = static_tiles ? cur + kWaves : grab();
        compute_tile(cur * kTok, kA, vA, nxt * kTok);
        cur = nxt;
    }

    // ---- fold the waves' states, leave one partial per split ----------------
    // lane (16 grp + 4 a + e), N-tile c holds channel 32 a + 4 c + e of rows
    // (hA hi, hB hi, hA lo, hB lo); a wave that got no tile has m = -inf.
    //  1. every wave publishes its m per head;
    //  2. every wave reads the maxima M over the waves, rescales its l and o by
    //     2^(m - M) in registers and stores them lane by lane (no bank
    //     conflicts: a channel-major store had four-way conflicts and took
    //     longer than the rest of the fold);
    //  3. the partial is then a plain sum over the waves.
    lA = row_sum16(lA);
    lB = row_sum16(lB);
    if constexpr (kPack) {   // the same heads' sums over the other 16-token blocks
        lA += lane_partner<32>(lA, lane);
        lB += lane_partner<32>(lB, lane);
    }
    if (n == 0) {
        if (hA < G) wmT[hA][wave] = mA;
        if (hB < G) wmT[hB][wave] = mB;
    }
    __syncthreads();   // the m are complete, and every wave is done with tab
    float MA = -INFINITY, MB = -INFINITY;
    {
        // lane row r reduces heads r and r + 4 over the 16 waves
        const float mr0 = row_max16(wmT[min(grp, G - 1)][n]);
        const float mr1 = row_max16(wmT[min(grp + 4, G - 1)][n]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mh = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h < 4 ? mr0 : mr1), 16 * (h & 3)));
            MA = (hA == h) ? mh : MA;
            MB = (hB == h) ? mh : MB;
        }
    }
    const float fA = (hA < G && mA != -INFINITY) ? fast_exp2(mA - MA) : 0.f;
    const float fB = (hB < G && mB != -INFINITY) ? fast_exp2(mB - MB) : 0.f;
    constexpr int kLanes = 16 * ((G + 1) / 2);   // lanes holding rows of real heads
    float2* obuf = reinterpret_cast<float2*>(tab);   // [kWaves][8][kLanes] (head hA, head hB)
    if (lane < kLanes) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            obuf[(wave * 8 + c) * kLanes + lane] =
                make_float2(fA * fmaf(oacc[c][2], kLoUnscale, oacc[c][0]),
                            fB * fmaf(oacc[c][3], kLoUnscale, oacc[c][1]));
    }
    if (n == 0) {
        if (hA < G) wlT[hA][wave] = fA * lA;
        if (hB < G) wlT[hB][wave] = fB * lB;
    }
    __syncthreads();
    const size_t pbase = (static_cast<size_t>(b) * num_q_heads + g * G) * part_stride + split;
    constexpr int kItems = 8 * kLanes * 2;   // (N-tile, lane, head of the lane's pair)
    static_assert(kItems <= kThreads, "one fold item per thread");
    if (tid < kItems) {
        const int comp = tid & 1, ln = (tid >> 1) % kLanes, c = (tid >> 1) / kLanes;
        const float* src = reinterpret_cast<const float*>(obuf) + (c * kLanes + ln) * 2 + comp;
        float os = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) os += src[w * 8 * kLanes * 2];
        const int h = 2 * (ln >> 4) + comp;
        if (h < G) {
            const int d = 32 * ((ln & 15) >> 2) + 4 * c + (ln & 3);
            part.o[(pbase + static_cast<size_t>(h) * part_stride) * kHeadDim + d] = os;
        }
    }
    if (tid < G) {
        float mx = -INFINITY, ls = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mx = fmaxf(mx, wmT[tid][w]);
            ls += wlT[tid][w];
        }
        const size_t pi = pbase + static_cast<size_t>(tid) * part_stride;
        part.m[pi] = mx;
        part.l[pi] = ls;
    }
}

namespace {

template <int KBITS, int SUB, bool LUT>
hipError_t launch_mfma_g(int group, dim3 grid, const AttnShape& s, const void* q, bool q_f32,
                         const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                         const uint8_t* codes_k, const uint8_t* codes_v, Partials part,
                         const AppendArgs& ap, hipStream_t stream) {
    // with an append, one more workgroup per (sequence, KV head) encodes the
    // new token (or, folded, the last split does) and leaves its one-token
    // partial at split index num_splits
    const bool app = ap.k_new != nullptr;
    const bool fold = app && ap.fold;
    const int pos = app ? ap.append_pos : -1;
    const int stride = s.num_splits + (app ? 1 : 0);
    const dim3 full((grid.x + (app && !fold ? 1 : 0)) * grid.y * grid.z);   // split-major
    if (fold && s.num_splits < 1) return hipErrorInvalidValue;
#define VQKV_LAUNCH(GG)                                                                       \
    case GG:                                                                                  \
        if constexpr (!LUT || GG <= 4)                                                        \
            hipLaunchKernelGGL((vq_attention_mfma_kernel<GG, KBITS, SUB, LUT && GG <= 4>),    \
                               full, dim3(kThreads), 0, stream, q, q_f32 ? 1 : 0, lambda,     \
                               cb_k, cb_v, codes_k, codes_v, s.num_q_heads, s.num_kv_heads,   \
                               s.capacity, s.context_len, s.num_splits, s.tokens_per_split,   \
                               part, ap.k_new, ap.v_new, ap.kv_f32 ? 1 : 0, pos, ap.codes_k,  \
                               ap.codes_v, stride, ap.win_k, ap.win_v, ap.win_len, ap.win_cap, \
                               fold ? 1 : 0, deterministic() ? 1 : 0);                        \
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

hipError_t launch_vq_attention(const AttnShape& s, int k_bits, int sub_dim, const void* q,
                               bool q_f32, const float* lambda, const uint16_t* cb_k,
                               const uint16_t* cb_v, const uint8_t* codes_k,
                               const uint8_t* codes_v, Partials part, const AppendArgs& append,
                               hipStream_t stream) {
    const dim3 grid(s.num_splits, s.num_kv_heads, s.batch);
    const int group = s.num_q_heads / s.num_kv_heads;
    if (sub_dim == 8)
        return launch_mfma_g<12, 8, false>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k,
                                           codes_v, part, append, stream);
    if (k_bits == 12)
        return launch_mfma_g<12, 4, false>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k,
                                           codes_v, part, append, stream);
    // the lookup-table score path where selected (8-bit keys, G <= 4)
    if (score_method() == kScoresLut && group <= 4)
        return launch_mfma_g<8, 4, true>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k,
                                         codes_v, part, append, stream);
    return launch_mfma_g<8, 4, false>(group, grid, s, q, q_f32, lambda, cb_k, cb_v, codes_k,
                                      codes_v, part, append, stream);
}

}  // namespace vqkv
