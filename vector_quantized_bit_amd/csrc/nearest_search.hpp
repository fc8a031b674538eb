// Certified nearest-centroid search for 16 sub-vectors of dimension 4 or 8
// on the matrix cores, shared by the encoders, the decode step's new token
// and K-Means.
//
// VecInfer page, Background (VQ principle): each sub-vector x gets
// j* = argmin_j ||x - C_j||^2.  The decision taken is the fp64 one: squared
// distance with every difference, product and sum rounded separately, in
// channel order; exact ties to the lowest index.
//
// Scores s(c) = ||c||^2 - 2 x.c come from v_mfma_f32_16x16x4_f32 with the
// centroids as the 16 rows (A: -2c), the sub-vectors as the 16 columns (B)
// and the 4 channels as the contraction; the accumulator input is the
// centroids' squared norms, read from LDS straight into the C registers.
// ||x||^2 is common to a column and left out.  With u = 2^-24, s(c) is within
// about 12 u (||x||^2 + ||c||^2) of the exact ||x - c||^2 - ||x||^2 when x
// and c enter the matrix cores rounded to fp32; the bound used, E(c) =
// 2^-16 (||x||^2 + ||c||^2) + 1e-30, has a margin of about 20x.
//   pass 1: thr = min_c (s(c) + E(c))          (per sub-vector)
//   pass 2: candidates are the c with s(c) - E(c) <= thr; the exact nearest
//           centroid is always one of them.
// A sub-vector with exactly one candidate has its answer without any fp64
// work.  Only a wave in which some sub-vector has two or more candidates
// evaluates the fp64 distances of the candidates and takes the
// lexicographic (distance, index) minimum.
//
// Lane l holds sub-vector l % 16 and, of every 16 centroids, the 4 rows
// 4 (l / 16) .. 4 (l / 16) + 3: the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 share a
// sub-vector and together see all centroids.  The ||c||^2 (1 + 2^-16) and
// ||c||^2 (1 - 2^-16) terms (the per-centroid part of E folded into the
// accumulator input) come precomputed from LDS; the per-sub-vector part
// 2 * 2^-16 ||x||^2 + 1e-30 is the caller's ex.
#pragma once

#include "device_common.hpp"

namespace vqkv {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Row stride of the -2c tables: 16 floats of padding put the 4 channel rows
// on different banks for the 64 lanes of one B-operand read.
template <int NENT>
constexpr int kSearchStride = NENT + 16;

constexpr float kBoundUp = 1.0f + 0x1p-16f;
constexpr float kBoundDown = 1.0f - 0x1p-16f;

// ||c||^2 of a 4-dim fp16 centroid: the squares are exact in fp32, the sums
// rounded
__device__ __forceinline__ float norm2(const uint2 c) {
    const float c0 = half_bits_to_float(c.x & 0xffffu), c1 = half_bits_to_float(c.x >> 16);
    const float c2 = half_bits_to_float(c.y & 0xffffu), c3 = half_bits_to_float(c.y >> 16);
    return (c0 * c0 + c1 * c1) + (c2 * c2 + c3 * c3);
}

// ex[i] of a row from its fp32 squared norm
__device__ __forceinline__ float row_bound(float xx) { return 2.f * (0x1p-16f * xx) + 1e-30f; }

// The nearest of NENT centroids for 16 sub-vectors (one MFMA column block).
//   m2   [4][kSearchStride<NENT>] fp32: -2 fl32(c) by channel
//   ccu, ccd [NENT] fp32, 16-byte aligned: fl32(||c||^2) (1 + 2^-16), (1 - 2^-16)
//   b    this lane's B operand: channel lane / 16 of sub-vector lane % 16
//   ex   the bound term of sub-vector lane % 16
//   exact(c) -> double: the fp64 distance of sub-vector lane % 16 to centroid c
// Returns the nearest centroid of sub-vector lane % 16 (in all 4 of its
// lanes; 0xffffffff only for a sub-vector with no candidate, which finite
// inputs never produce).  Every lane of the wave must be active; all
// branches below are uniform except each lane's loop over its own hits in a
// group, which holds no cross-lane operation.
//
// The encoders and the one-token searches of the decode step use the fp16
// hi/lo form below (BlockD4HN, BlockD8HN, BlockD8H): the centroids enter the matrix
// cores as the codebook stores them (fp16) and the sub-vector as a scaled
// hi/lo fp16 pair, with their own certified bound (2^-15).  The fp32 form
// above remains in K-Means (BlockF32D8 for 8-dim samples).
// The passes over centroid blocks [b0, b1) (16 centroids each; b1 - b0 a
// multiple of 8).  block(blk, c) is the MFMA score of block blk with
// accumulator input c; cup(blk) / cdown(blk) give the lane's 4 norm terms
// ||c||^2 (1 + 2^-16) / (1 - 2^-16).
constexpr int kSearchUnroll = 8;
static_assert(kSearchUnroll * 4 <= 32, "a group's hits fit one 32-bit mask");

// the minimum of one group's scores in this lane
__device__ __forceinline__ float group_min(const f32x4_t (&d)[kSearchUnroll]) {
    float m = INFINITY;
#pragma unroll
    for (int u = 0; u < kSearchUnroll; ++u)
        m = fminf(m, fminf(fminf(d[u][0], d[u][1]), fminf(d[u][2], d[u][3])));
    return m;
}

// pass 1: this lane's minimum of s(c) + E(c) (without the ||x||^2 part)
template <typename Block, typename Cop>
__device__ __forceinline__ float search_pass1(Block block, Cop cup, int b0, int b1) {
    float smin = INFINITY;
#pragma nounroll
    for (int blk = b0; blk < b1; blk += kSearchUnroll) {
        f32x4_t d[kSearchUnroll];
#pragma unroll
        for (int u = 0; u < kSearchUnroll; ++u) d[u] = block(blk + u, cup(blk + u));
        smin = fminf(smin, group_min(d));
    }
    return smin;
}

// pass 1 over NR groups of kSearchUnroll blocks from b0, unrolled: rmin[i]
// is this lane's minimum over group i (for the need masks of passes 2 and 3,
// as with search_pass1_groups and pass3_need)
template <int NR, typename Block, typename Cop>
__device__ __forceinline__ void search_pass1_runs(Block block, Cop cup, int b0,
                                                  float (&rmin)[NR]) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int blk = b0 + i * kSearchUnroll;
        f32x4_t d[kSearchUnroll];
#pragma unroll
        for (int u = 0; u < kSearchUnroll; ++u) d[u] = block(blk + u, cup(blk + u));
        rmin[i] = group_min(d);
        // one group's operands at a time (the unrolled loop would otherwise
        // request every group's at once)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// pass 2: how many of this lane's centroids have s(c) - E(c) <= thr, and the
// row (16 blk + r, without the lane's 4 (lane / 16)) of the last of them.
// kSkip: a group of 8 blocks without a hit in the whole wave is skipped after
// one ballot, and within a group only the blocks with a hit in some lane are
// counted, which pays where hits are sparse (a wave over 1024 or more
// centroids) and costs a little where nearly every block has one.
// need (wave-uniform): bit i set for the groups i of kSearchUnroll blocks
// from b0 that may hold a candidate; the others are skipped.
template <bool kSkip, typename Block, typename Cop>
__device__ __forceinline__ void search_pass2(Block block, Cop cdown, int b0, int b1, float thr,
                                             int& cnt, int& cand, uint32_t need = 0xffffffffu) {
    cnt = 0;
    cand = -1;
#pragma nounroll
    for (int blk = b0; blk < b1; blk += kSearchUnroll) {
        if (((need >> ((blk - b0) / kSearchUnroll)) & 1u) == 0) continue;
        f32x4_t d[kSearchUnroll];
#pragma unroll
        for (int u = 0; u < kSearchUnroll; ++u) d[u] = block(blk + u, cdown(blk + u));
        // the group's last hit as u * 4 + r (an inline constant, 0 .. 31),
        // turned into a centroid row once per group
        const int before = cnt;
        int loc = 0;
        if constexpr (kSkip) {
            // block minima first; a block is counted only where some lane of
            // the wave has a hit in it, which changes no lane's count or last hit
            float m[kSearchUnroll];
            bool any = false;
#pragma unroll
            for (int u = 0; u < kSearchUnroll; ++u) {
                m[u] = fminf(fminf(d[u][0], d[u][1]), fminf(d[u][2], d[u][3]));
                any |= m[u] <= thr;
            }
            if (__builtin_amdgcn_ballot_w64(any) == 0) continue;
#pragma unroll
            for (int u = 0; u < kSearchUnroll; ++u) {
                if (__builtin_amdgcn_ballot_w64(m[u] <= thr) == 0) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool hit = d[u][r] <= thr;
                    loc = hit ? u * 4 + r : loc;
                    cnt += hit ? 1 : 0;
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSearchUnroll; ++u) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool hit = d[u][r] <= thr;
                    loc = hit ? u * 4 + r : loc;
                    cnt += hit ? 1 : 0;
                }
            }
        }
        cand = cnt != before ? blk * 16 + (loc >> 2) * 16 + (loc & 3) : cand;
    }
}

// pass 3: the lexicographic (fp64 distance, index) minimum over this lane's
// candidates (bd = inf, bi = 0xffffffff when it has none); need as in pass 2
template <typename Block, typename Cop, typename Exact>
__device__ __forceinline__ void search_pass3(Block block, Cop cdown, int b0, int b1, float thr,
                                             int q4, Exact exact, double& bd, uint32_t& bi,
                                             uint32_t need = 0xffffffffu) {
    bd = INFINITY;
    bi = 0xffffffffu;
#pragma nounroll
    for (int blk = b0; blk < b1; blk += kSearchUnroll) {
        if (((need >> ((blk - b0) / kSearchUnroll)) & 1u) == 0) continue;
        f32x4_t d[kSearchUnroll];
#pragma unroll
        for (int u = 0; u < kSearchUnroll; ++u) d[u] = block(blk + u, cdown(blk + u));
        if (__builtin_amdgcn_ballot_w64(group_min(d) <= thr) == 0) continue;
        // the group's hits as bits u * 4 + r, then one fp64 distance per hit
        uint32_t hits = 0;
#pragma unroll
        for (int u = 0; u < kSearchUnroll; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) hits |= (d[u][r] <= thr ? 1u : 0u) << (u * 4 + r);
        while (hits != 0) {
            const int k = __builtin_ctz(hits);
            hits &= hits - 1;
            const uint32_t nc = static_cast<uint32_t>((blk + (k >> 2)) * 16 + q4 + (k & 3));
            const double dd = exact(nc);
            if (nearer(dd, nc, bd, bi)) {
                bd = dd;
                bi = nc;
            }
        }
    }
}

// The lexicographic minimum over the 4 lanes of a sub-vector.
__device__ __forceinline__ void take_lanes16_32(double& bd, uint32_t& bi, int lane) {
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const double d2 = step == 0 ? lane_partner<16>(bd, lane) : lane_partner<32>(bd, lane);
        const uint32_t i2 = step == 0 ? lane_partner<16>(bi, lane) : lane_partner<32>(bi, lane);
        if (nearer(d2, i2, bd, bi)) {
            bd = d2;
            bi = i2;
        }
    }
}

// Sum and maximum over the 4 lanes of a sub-vector.
__device__ __forceinline__ int sum_lanes16_32(int x, int lane) {
    x += static_cast<int>(lane_partner<16>(static_cast<uint32_t>(x), lane));
    return x + static_cast<int>(lane_partner<32>(static_cast<uint32_t>(x), lane));
}
__device__ __forceinline__ int max_lanes16_32(int x, int lane) {
    x = max(x, static_cast<int>(lane_partner<16>(static_cast<uint32_t>(x), lane)));
    return max(x, static_cast<int>(lane_partner<32>(static_cast<uint32_t>(x), lane)));
}

// The runs of the pass-1 minima gmin (search_pass1_runs, search_pass1_groups)
// that may hold a candidate, as the need mask of passes 2 and 3.  A score of pass 3
// differs from the pass-1 score of the same centroid by the difference of
// the norm terms (at most dmax, their largest difference over the table)
// and the rounding of both products; with E's margin over the rounding
// model, 2 dmax + ex bounds the whole, so a run whose pass-1 minimum exceeds
// thr + 2 dmax + ex has no score of pass 3 at or below thr.
template <int N>
__device__ __forceinline__ uint32_t pass3_need(const float (&gmin)[N], float thr, float dmax,
                                               float ex) {
    static_assert(N <= 32, "one bit a run");
    const float lim = thr + 2.f * dmax + ex;
    uint32_t need = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        need |= __builtin_amdgcn_ballot_w64(gmin[i] <= lim) != 0 ? 1u << i : 0u;
    return need;
}

// The whole search over NENT centroids, the norm terms given by cup / cdown
// (dmax: the largest difference cup - cdown of a centroid, read only with
// 1024 or more centroids, where passes 2 and 3 visit only the groups of
// kSearchUnroll blocks that may hold a candidate; pass3_need).
template <int NENT, typename Block, typename Cop, typename Exact>
__device__ __forceinline__ uint32_t nearest16_search(Block block, Cop cup, Cop cdown, float ex,
                                                     float dmax, int lane, Exact exact) {
    static_assert(NENT % (16 * kSearchUnroll) == 0, "whole unrolled groups");
    constexpr int kGroups = NENT / (16 * kSearchUnroll);
    constexpr bool kRuns = NENT >= 1024 && kGroups <= 32;
    const int q4 = 4 * (lane >> 4);   // this lane's first centroid row in a block

    // pass 1: thr = min over c of s(c) + E(c)
    float thr;
    uint32_t need = 0xffffffffu;
    if constexpr (kRuns) {
        float rmin[kGroups];
        search_pass1_runs<kGroups>(block, cup, 0, rmin);
        float smin = rmin[0];
#pragma unroll
        for (int i = 1; i < kGroups; ++i) smin = fminf(smin, rmin[i]);
        smin = fminf(smin, lane_partner<16>(smin, lane));
        thr = fminf(smin, lane_partner<32>(smin, lane)) + ex;
        need = pass3_need(rmin, thr, dmax, ex);
    } else {
        float smin = search_pass1(block, cup, 0, NENT / 16);
        smin = fminf(smin, lane_partner<16>(smin, lane));
        smin = fminf(smin, lane_partner<32>(smin, lane));
        thr = smin + ex;
    }

    // pass 2: each lane counts its candidates and keeps one
    int cnt, cand;
    search_pass2<(NENT >= 1024)>(block, cdown, 0, NENT / 16, thr, cnt, cand, need);
    cnt = sum_lanes16_32(cnt, lane);
    const int best = max_lanes16_32(cand < 0 ? -1 : cand + q4, lane);

    // every sub-vector has exactly one candidate: it is the nearest centroid
    if (__builtin_amdgcn_ballot_w64(cnt != 1) == 0) return static_cast<uint32_t>(best);

    // some sub-vector has several candidates: fp64 distances for all
    // candidates of this block (pass 2 again), lexicographic minimum over
    // the 4 lanes of each sub-vector
    double bd;
    uint32_t bi;
    search_pass3(block, cdown, 0, NENT / 16, thr, q4, exact, bd, bi, need);
    take_lanes16_32(bd, bi, lane);
    return bi;
}

// Norm terms precomputed in LDS: ccu, ccd [NENT] fp32, 16-byte aligned.
template <int NENT, int SUB, typename Block, typename Exact>
__device__ __forceinline__ uint32_t nearest16_core(const float* __restrict__ ccu,
                                                   const float* __restrict__ ccd, Block block,
                                                   float ex, float dmax, int lane, Exact exact) {
    const int q4 = 4 * (lane >> 4);
    const f32x4_t* ucol = reinterpret_cast<const f32x4_t*>(ccu + q4);
    const f32x4_t* dcol = reinterpret_cast<const f32x4_t*>(ccd + q4);
    struct Col {
        const f32x4_t* p;
        __device__ f32x4_t operator()(int blk) const { return p[blk * 4]; }
    };
    return nearest16_search<NENT>(block, Col{ucol}, Col{dcol}, ex, dmax, lane, exact);
}

// One norm table [NENT] (fp32 ||c||^2, 16-byte aligned), scaled by
// (1 +- 2^-16) as it is read.
struct ScaledNorms {
    const f32x4_t* p;
    float scale;
    __device__ f32x4_t operator()(int blk) const { return p[blk * 4] * scale; }
};

// The MFMA score of one block of 16 centroids, d = 8, fp32 centroids laid
// out channel-pair-major: tab [4 pairs][NENT][2] (the 16 lanes of a group
// read 16 consecutive 8-byte pairs: no bank conflicts); b0, b1 = -2x of
// channels 2 (lane / 16) and 2 (lane / 16) + 1 of sub-vector lane % 16.
template <int NENT>
struct BlockF32D8 {
    const float2* acol;
    float b0, b1;
    __device__ BlockF32D8(const float* tab, float b0_, float b1_, int lane)
        : acol(reinterpret_cast<const float2*>(tab) + (lane >> 4) * NENT + (lane & 15)),
          b0(b0_), b1(b1_) {}
    __device__ f32x4_t operator()(int blk, f32x4_t c) const {
        const float2 a = acol[blk * 16];
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b0, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b1, d, 0, 0, 0);
    }
};

// fp16 hi/lo scores (d = 8 first): one v_mfma_f32_16x16x32_f16 per block of 16
// centroids.  The A operand is the fp16 centroid as the codebook stores it
// (lanes 0-15 and 16-31 read the same 16-byte entry, K = 0-7 and 8-15;
// K = 16-31 meet zeros in B).  The B operand of sub-vector l % 16 holds
// X = fl32(-2x) 2^s split into hi = fl16(X) (lane group 0) and
// lo = fl16(X - hi) (group 1), with 2^s putting max |X| in [2^14, 2^15):
// the products are exact in fp32 and X - (hi + lo) is within
// 2^-22 |X| + 2^-25.  The accumulator input is ||c||^2 (1 +- 2^-15) 2^s.
//   Error, in units of 2^s and u = 2^-24, of the score against the exact
//   ||c||^2 - 2 x.c: the matrix cores' sum of 16 products and the input
//   (measured on gfx950: at most 4.2 u of the sum of magnitudes over 65536
//   adversarial cases; modelled here as 2 u per addition, 66 u), plus the
//   split of X (5 u of |x.c| terms) and the fp32 norm (8 u ||c||^2): at
//   most about 140 u ||c||^2 + 70 u ||x||^2 (2 |x||c| <= ||x||^2 + ||c||^2).
//   The bound E = 2^-15 (||x||^2 + ||c||^2) is 512 u of each: 3.6x the
//   modelled error, ~60x the measured one.  (The fp32 search above keeps
//   2^-16.)
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
constexpr float kBoundUpH = 1.0f + 0x1p-15f;
constexpr float kBoundDownH = 1.0f - 0x1p-15f;

// ex of a row (unscaled), for the hi/lo search
__device__ __forceinline__ float row_bound_h(float xx) { return 2.f * (0x1p-15f * xx) + 1e-30f; }

// A scale 2^s shared by a workgroup's sub-vectors (mx = the largest |2x|
// among them): their norm terms can then be scaled once, as the tables are
// built, instead of once per block in every lane.  A sub-vector far below mx
// gets a subnormal lo; its split is then within 2^-25 per channel in units
// of 2^s, so the tables add 2^-24 ||c||_1 to the upper and subtract it from
// the lower norm term (hilo_norm_terms).
__device__ __forceinline__ float hilo_scale(float mx) {
    const int s = mx > 0.f ? min(max(15 - __builtin_amdgcn_frexp_expf(mx), -60), 60) : 0;
    return __builtin_amdgcn_ldexpf(1.f, s);
}
// ||c||^2 (1 +- 2^-15) 2^s +- 2^-24 ||c||_1 (fp32; n = ||c||^2, l1 = ||c||_1)
__device__ __forceinline__ float2 hilo_norm_terms(float n, float l1, float sc) {
    return make_float2(fmaf(n, kBoundUpH * sc, 0x1p-24f * l1),
                       fmaf(n, kBoundDownH * sc, -0x1p-24f * l1));
}
// hi / lo rows of X = fl32(-2x) sc for lane group lane / 16 (0: hi, 1: lo,
// 2 and 3: zeros)
template <int D, typename H>
__device__ __forceinline__ H hilo_rows(const double* x, int lane, float sc) {
    const int g = lane >> 4;
    H b;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const float X = -2.f * static_cast<float>(x[j]) * sc;
        const _Float16 hi = static_cast<_Float16>(X);
        const _Float16 lo = static_cast<_Float16>(X - static_cast<float>(hi));
        b[j] = g == 0 ? hi : (g == 1 ? lo : static_cast<_Float16>(0.f));
    }
    return b;
}
// ||c||_1 of a 4- or 8-dim fp16 centroid (the sum rounded; only a bound term)
__device__ __forceinline__ float l1_4(const uint2 c) {
    return (fabsf(half_bits_to_float(c.x & 0xffffu)) + fabsf(half_bits_to_float(c.x >> 16))) +
           (fabsf(half_bits_to_float(c.y & 0xffffu)) + fabsf(half_bits_to_float(c.y >> 16)));
}

// Per-lane form (one sub-vector's own scale, for the one-token searches): the
// B operand and the scale 2^s of sub-vector lane % 16, x its D values.
struct HiLoD8 {
    h8_t b;
    float scale;
};
__device__ __forceinline__ HiLoD8 hilo_d8(const double* x, int lane) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(-2.f * static_cast<float>(x[j])));
    const float sc = hilo_scale(mx);
    return {hilo_rows<8, h8_t>(x, lane, sc), sc};
}

// 4-dim sub-vectors use v_mfma_f32_16x16x16_f16: lane groups 0 and 1 carry
// hi and lo of the 4 channels, groups 2 and 3 zeros.
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

// Block scores of NC column blocks (16 sub-vectors each) against 4-dim fp16
// centroids as the codebook stores them (8 bytes an entry; arow = the table
// + lane % 16): one A operand and one set of norm terms per centroid block
// feed all NC products.
template <int NC>
struct BlockD4HN {
    const uint2* arow;
    h4_t b[NC];
    __device__ h4_t a(int blk) const { return __builtin_bit_cast(h4_t, arow[blk * 16]); }
    __device__ f32x4_t operator()(h4_t a, int j, f32x4_t c) const {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b[j], c, 0, 0, 0);
    }
};

// The same for 8-dim centroids (16-byte entries, v_mfma_f32_16x16x32_f16).
template <int NC>
struct BlockD8HN {
    const uint4* arow;
    h8_t b[NC];
    __device__ h8_t a(int blk) const { return __builtin_bit_cast(h8_t, arow[blk * 16]); }
    __device__ f32x4_t operator()(h8_t a, int j, f32x4_t c) const {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], c, 0, 0, 0);
    }
};

// The minimum of a group of U blocks' scores in this lane.
template <int U>
__device__ __forceinline__ float group_min_u(const f32x4_t (&d)[U]) {
    float m = INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
        m = fminf(m, fminf(fminf(d[u][0], d[u][1]), fminf(d[u][2], d[u][3])));
    return m;
}

// The scores of U blocks from blk on: every A operand and norm term of the
// group is requested before the first product, so the group waits on LDS
// once rather than once per block.
template <int NC, int U, typename Block, typename Cop>
__device__ __forceinline__ void group_scores(const Block& block, Cop cop, int blk,
                                             f32x4_t (&d)[NC][U]) {
    decltype(block.a(0)) a[U];
    f32x4_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        a[u] = block.a(blk + u);
        c[u] = cop(blk + u);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NC; ++j) d[j][u] = block(a[u], j, c[u]);
}

// Pass 1 for one column block over NG groups of U blocks from b0, unrolled:
// gmin[i] is this lane's minimum of s(c) + E(c) over the run of S blocks
// b0 + S i .. + S - 1 (S divides U or U divides S).  With the threshold
// known, a run whose minimum lies more than the bound's width above it holds
// no candidate (pass3_need).
template <int U, int S, int NG, typename Block, typename Cop>
__device__ __forceinline__ void search_pass1_groups(const Block& block, Cop cup, int b0,
                                                    float (&gmin)[NG * U / S]) {
    static_assert(U % S == 0 || S % U == 0, "whole runs");
#pragma unroll
    for (int i = 0; i < NG * U / S; ++i) gmin[i] = INFINITY;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        f32x4_t d[1][U];
        group_scores<1, U>(block, cup, b0 + q * U, d);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float& m = gmin[(q * U + u) / S];
            m = fminf(m, fminf(fminf(d[0][u][0], d[0][u][1]), fminf(d[0][u][2], d[0][u][3])));
        }
    }
}

// Passes 1 and 3 for NC column blocks sharing the centroid blocks [b0, b1)
// (b1 - b0 a multiple of U): block.a(blk) is the A operand of a block and
// block(a, j, c) the score of column block j.  Per column block they give
// what search_pass1 and search_pass3 give for one; exact(j, c) is the fp64
// distance of the lane's sub-vector in column block j to centroid c.
template <int NC, int U, typename Block, typename Cop>
__device__ __forceinline__ void search_pass1_cols(const Block& block, Cop cup, int b0, int b1,
                                                  float (&smin)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) smin[j] = INFINITY;
#pragma nounroll
    for (int blk = b0; blk < b1; blk += U) {
        f32x4_t d[NC][U];
        group_scores<NC, U>(block, cup, blk, d);
#pragma unroll
        for (int j = 0; j < NC; ++j) smin[j] = fminf(smin[j], group_min_u<U>(d[j]));
    }
}

// need (wave-uniform): bit i set for the runs of S blocks from b0 (a
// multiple of U) that may hold a candidate; the groups of the others are
// skipped without their products.
template <int NC, int U, int S = U, typename Block, typename Cop, typename Exact>
__device__ __forceinline__ void search_pass3_cols(const Block& block, Cop cdown, int b0, int b1,
                                                  const float (&thr)[NC], int q4, Exact exact,
                                                  double (&bd)[NC], uint32_t (&bi)[NC],
                                                  uint32_t need = 0xffffffffu) {
    static_assert(S % U == 0, "whole groups a run");
    static_assert(U * 4 <= 32, "a group's hits fit one 32-bit mask");
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        bd[j] = INFINITY;
        bi[j] = 0xffffffffu;
    }
#pragma nounroll
    for (int blk = b0; blk < b1; blk += U) {
        if (((need >> ((blk - b0) / S)) & 1u) == 0) continue;
        f32x4_t d[NC][U];
        group_scores<NC, U>(block, cdown, blk, d);
        // block minima first: the hit bits of a block are formed only where
        // some lane of the wave has one there (hits are rare)
        float m[NC][U];
        bool any = false;
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                m[j][u] = fminf(fminf(d[j][u][0], d[j][u][1]), fminf(d[j][u][2], d[j][u][3]));
                any |= m[j][u] <= thr[j];
            }
        if (__builtin_amdgcn_ballot_w64(any) == 0) continue;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            uint32_t hits = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (__builtin_amdgcn_ballot_w64(m[j][u] <= thr[j]) != 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        hits |= (d[j][u][r] <= thr[j] ? 1u : 0u) << (u * 4 + r);
                }
            }
            while (hits != 0) {
                const int k = __builtin_ctz(hits);
                hits &= hits - 1;
                const uint32_t nc = static_cast<uint32_t>((blk + (k >> 2)) * 16 + q4 + (k & 3));
                const double dd = exact(j, nc);
                if (nearer(dd, nc, bd[j], bi[j])) {
                    bd[j] = dd;
                    bi[j] = nc;
                }
            }
        }
    }
}

// Pass 2 for NC column blocks (what search_pass2 gives for one, with the
// same skip rule and kSkip meaning); need as in search_pass3_cols.
template <bool kSkip, int NC, int U, int S = U, typename Block, typename Cop>
__device__ __forceinline__ void search_pass2_cols(const Block& block, Cop cdown, int b0, int b1,
                                                  const float (&thr)[NC], int (&cnt)[NC],
                                                  int (&cand)[NC], uint32_t need = 0xffffffffu) {
    static_assert(U * 4 <= 32, "a group's last hit fits an inline constant");
    static_assert(S % U == 0, "whole groups a run");
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        cnt[j] = 0;
        cand[j] = -1;
    }
#pragma nounroll
    for (int blk = b0; blk < b1; blk += U) {
        if (((need >> ((blk - b0) / S)) & 1u) == 0) continue;
        f32x4_t d[NC][U];
        group_scores<NC, U>(block, cdown, blk, d);
        float m[NC][U];
        bool any = false;
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                m[j][u] = fminf(fminf(d[j][u][0], d[j][u][1]), fminf(d[j][u][2], d[j][u][3]));
                any |= m[j][u] <= thr[j];
            }
        if constexpr (kSkip)
            if (__builtin_amdgcn_ballot_w64(any) == 0) continue;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int before = cnt[j];
            int loc = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (kSkip)
                    if (__builtin_amdgcn_ballot_w64(m[j][u] <= thr[j]) == 0) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool hit = d[j][u][r] <= thr[j];
                    loc = hit ? u * 4 + r : loc;
                    cnt[j] += hit ? 1 : 0;
                }
            }
            cand[j] = cnt[j] != before ? blk * 16 + (loc >> 2) * 16 + (loc & 3) : cand[j];
        }
    }
}

// nearest16_core for NC column blocks at once: the block's A operands and
// norm terms are read once for all NC products.  ex[j] is the bound term and
// exact(j, c) the fp64 distance of the lane's sub-vector in column block j;
// out[j] receives its nearest centroid.  U blocks a group (U * NC
// accumulators of 4 registers stay live).
// dmax: the largest ccu[c] - ccd[c] of the table.  With one column block
// and 1024 or more centroids, pass 1 keeps this lane's minimum over each of
// 32 runs of blocks (whole groups of U), and passes 2 and 3 visit only the
// runs where some lane of the wave may have a candidate (pass3_need).
template <int NENT, int NC, int U, typename Block, typename Exact>
__device__ __forceinline__ void nearest16_cols(const float* __restrict__ ccu,
                                               const float* __restrict__ ccd, const Block& block,
                                               const float (&ex)[NC], float dmax, int lane,
                                               Exact exact, uint32_t (&out)[NC]) {
    static_assert(NENT % (16 * U) == 0, "whole groups");
    constexpr bool kRuns = NC == 1 && NENT >= 1024;
    constexpr int kRun = kRuns ? (NENT / 16 / 32 > U ? NENT / 16 / 32 : U) : U;   // blocks a run
    const int q4 = 4 * (lane >> 4);
    struct Col {
        const f32x4_t* p;
        __device__ f32x4_t operator()(int blk) const { return p[blk * 4]; }
    };
    const Col up{reinterpret_cast<const f32x4_t*>(ccu + q4)};
    const Col down{reinterpret_cast<const f32x4_t*>(ccd + q4)};
    float thr[NC];
    uint32_t need = 0xffffffffu;
    if constexpr (kRuns) {
        constexpr int kNr = NENT / (16 * kRun);
        float gmin[kNr];
        search_pass1_groups<U, kRun, NENT / (16 * U)>(block, up, 0, gmin);
        float m = gmin[0];
#pragma unroll
        for (int i = 1; i < kNr; ++i) m = fminf(m, gmin[i]);
        m = fminf(m, lane_partner<16>(m, lane));
        thr[0] = fminf(m, lane_partner<32>(m, lane)) + ex[0];
        need = pass3_need(gmin, thr[0], dmax, ex[0]);
    } else {
        search_pass1_cols<NC, U>(block, up, 0, NENT / 16, thr);
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            thr[j] = fminf(thr[j], lane_partner<16>(thr[j], lane));
            thr[j] = fminf(thr[j], lane_partner<32>(thr[j], lane)) + ex[j];
        }
    }
    int cnt[NC], cand[NC];
    search_pass2_cols<(NENT >= 1024), NC, U, kRun>(block, down, 0, NENT / 16, thr, cnt, cand,
                                                   need);
    bool several = false;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        cnt[j] = sum_lanes16_32(cnt[j], lane);
        out[j] = static_cast<uint32_t>(max_lanes16_32(cand[j] < 0 ? -1 : cand[j] + q4, lane));
        several |= cnt[j] != 1;
    }
    if (__builtin_amdgcn_ballot_w64(several) == 0) return;
    double bd[NC];
    uint32_t bi[NC];
    search_pass3_cols<NC, U, kRun>(block, down, 0, NENT / 16, thr, q4, exact, bd, bi, need);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        take_lanes16_32(bd[j], bi[j], lane);
        out[j] = bi[j];
    }
}

// The block score: ctab [.][8] fp16 centroids (16-byte aligned entries).
struct BlockD8H {
    const uint4* arow;
    h8_t b;
    __device__ BlockD8H(const uint16_t* ctab, h8_t b_, int lane)
        : arow(reinterpret_cast<const uint4*>(ctab) + (lane & 15)), b(b_) {}
    __device__ f32x4_t operator()(int blk, f32x4_t c) const {
        const h8_t a = __builtin_bit_cast(h8_t, arow[blk * 16]);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// d = 4: m2 [4][kSearchStride<NENT>] fp32 -2 fl32(c) by channel; b is this
// lane's B operand, channel lane / 16 of sub-vector lane % 16; dmax the
// largest ccu[c] - ccd[c].
template <int NENT, typename Exact>
__device__ __forceinline__ uint32_t nearest16(const float* __restrict__ m2,
                                              const float* __restrict__ ccu,
                                              const float* __restrict__ ccd, float b, float ex,
                                              float dmax, int lane, Exact exact) {
    const float* acol = m2 + (lane >> 4) * kSearchStride<NENT> + (lane & 15);
    const auto block = [&](int blk, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(acol[blk * 16], b, c, 0, 0, 0);
    };
    return nearest16_core<NENT, 4>(ccu, ccd, block, ex, dmax, lane, exact);
}


// The codes of one token in the d = 8 layout (16 sub-vectors of 8 channels,
// C_k and C_v of 4096 fp16 entries), found by one 1024-thread workgroup: the
// 16 sub-vectors of a tensor are one MFMA column block (per-lane hi/lo
// scale, hilo_d8), and wave w scans centroids 256 w .. 256 w + 255.  Per
// tensor: the waves' pass-1 minima meet in LDS (the threshold), each wave
// keeps its pass-1 minimum per group of 8 blocks for the skip of pass 3, and
// the fp64 minima over the candidates meet in LDS; ties to the lowest index,
// the decisions of the fp64 scan.
//   tab     C_k as stored (16-byte entries), C_v at tab + table_bytes
//   nrm     [4096] fp32 scratch (the current tensor's ||c||^2)
//   xbuf    4 KiB of exchanges
//   xnew    the transformed key and the value (fp64)
//   newc    [2][16] receives the codes
// Every thread of the workgroup calls it; it ends with a barrier.
__device__ __forceinline__ void codes8_one_token(const uint8_t* tab, int table_bytes, float* nrm,
                                                 uint8_t* xbuf, const double (*xnew)[kHeadDim],
                                                 uint32_t (*newc)[kNumSub], int tid, int lane,
                                                 int wave) {
    constexpr int kEnt = 4096, kPos = 16, kThr = 1024, kWv = kThr / 64;
    static_assert(kEnt == kWv * 256, "16 waves of 256 centroids");
    float* wmin = reinterpret_cast<float*>(xbuf);               // [16 waves][16] pass-1 minima
    double* wbd = reinterpret_cast<double*>(xbuf + 1024);       // [16][16] fp64 minima
    uint32_t* wbi = reinterpret_cast<uint32_t*>(xbuf + 3072);   // [16][16] their indices
    const int pos = lane & (kPos - 1), q4 = 4 * (lane >> 4);
    const int b0 = 16 * wave, b1 = b0 + 16;   // this wave's centroid blocks
    for (int t = 0; t < 2; ++t) {
        const uint16_t* table = reinterpret_cast<const uint16_t*>(tab + t * table_bytes);
        for (int i = tid; i < kEnt; i += kThr) {
            const uint4 c = reinterpret_cast<const uint4*>(table)[i];
            const uint32_t w[4] = {c.x, c.y, c.z, c.w};
            float nn = 0.f;   // the squares of fp16 values are exact in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = half_bits_to_float(static_cast<uint16_t>(w[j] & 0xffffu));
                const float hi = half_bits_to_float(static_cast<uint16_t>(w[j] >> 16));
                nn += lo * lo;
                nn += hi * hi;
            }
            nrm[i] = nn;
        }
        __syncthreads();
        double xd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xd[j] = xnew[t][8 * pos + j];
        float xx = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = static_cast<float>(xd[j]);
            xx += v * v;
        }
        // fp16 hi/lo matrix-core scores in units of 2^s (the lane's column)
        const HiLoD8 hl = hilo_d8(xd, lane);
        const BlockD8H block(table, hl.b, lane);
        const f32x4_t* ncol = reinterpret_cast<const f32x4_t*>(nrm + q4);
        const float up = kBoundUpH * hl.scale, down = kBoundDownH * hl.scale;   // exact
        const auto cup = [&](int blk) { return ncol[blk * 4] * up; };
        const auto cdown = [&](int blk) { return ncol[blk * 4] * down; };
        const auto exact = [&](uint32_t nc) {
            return sqdist8_f64(xd, reinterpret_cast<const uint4*>(table)[nc]);
        };
        float rmin[2];   // this lane's minimum over each of the wave's 2 groups of 8 blocks
        static_assert(16 == 2 * kSearchUnroll, "2 groups a wave");
        search_pass1_runs<2>(block, cup, b0, rmin);
        float smin = fminf(rmin[0], rmin[1]);
        smin = fminf(smin, lane_partner<16>(smin, lane));
        smin = fminf(smin, lane_partner<32>(smin, lane));
        if (lane < kPos) wmin[wave * kPos + lane] = smin;
        // the largest norm bounds the difference of the lane's two norm
        // terms: fl(n up) - fl(n down) <= n 2^s (2^-14 + 2^-23 (1 + 2^-14))
        float nmax = 0.f;
        for (int i = lane; i < kEnt / 4; i += 64) {
            const f32x4_t v = reinterpret_cast<const f32x4_t*>(nrm)[i];
            nmax = fmaxf(nmax, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
        }
        const float dmax = wave_max(nmax) * hl.scale * (0x1p-14f + 0x1p-22f);
        __syncthreads();
        float gmin = wmin[pos];
        for (int w = 1; w < kWv; ++w) gmin = fminf(gmin, wmin[w * kPos + pos]);
        const float ex = row_bound_h(xx) * hl.scale;
        const float thr = gmin + ex;
        // fp64 distances of every candidate (about one a sub-vector, so they
        // are evaluated as they are found rather than counted first), in the
        // groups where some lane may have one
        double bd;
        uint32_t bi;
        search_pass3(block, cdown, b0, b1, thr, q4, exact, bd, bi,
                     pass3_need(rmin, thr, dmax, ex));
        take_lanes16_32(bd, bi, lane);
        if (lane < kPos) {
            wbd[wave * kPos + lane] = bd;
            wbi[wave * kPos + lane] = bi;
        }
        __syncthreads();
        if (tid < kPos) {
            double d0 = wbd[tid];
            uint32_t i0 = wbi[tid];
            for (int w = 1; w < kWv; ++w) {
                if (nearer(wbd[w * kPos + tid], wbi[w * kPos + tid], d0, i0)) {
                    d0 = wbd[w * kPos + tid];
                    i0 = wbi[w * kPos + tid];
                }
            }
            newc[t][tid] = i0 & (kEnt - 1);   // (a code always exists for finite inputs)
        }
        __syncthreads();   // the exchange buffers and norms are free for the next tensor
    }
}

}  // namespace vqkv
