// Offline calibration on the GPU: smoothing factors, transformed calibration
// keys and Lloyd K-Means codebooks.
//
// VecInfer page, Method details: the smoothing factors lambda_i =
// sqrt(max_t |K[t, i]|) per channel are precomputed offline from calibration
// keys, and the codebooks are pretrained offline by K-Means, on the
// transformed keys K~ = K diag(lambda)^-1 H_D for C_k and on the values as they
// are for C_v; Experimental setup: at most 30 K-Means iterations.
//
// K-Means is Lloyd's algorithm: every sample goes to its nearest centroid
// (fp64 squared distance with every difference, product and sum rounded
// separately, channels in order, exact ties to the lowest index), then every
// centroid with samples moves to their mean, the samples of a cluster summed
// in sample order from zero and divided once by their count; a centroid
// without samples stays where it is.  Each iteration reproduces that
// definition bit for bit, whatever the launch shape:
//  - assignment: the encoder's certified filter (fp32 scores on the matrix
//    cores, an error bound, fp64 distances for the few centroids under it),
//    here with fp64 centroids whose fp32 roundings feed the matrix cores;
//  - update: a stable counting sort of the samples by cluster, then one
//    sequential fp64 chain per (cluster, channel).
#include "launchers.hpp"
#include "nearest_search.hpp"

namespace vqkv {

namespace {

// ---------------------------------------------------------------------------
// smoothing factors
// ---------------------------------------------------------------------------

constexpr int kLamThreads = 256;
constexpr int kLamRows = 256;   // token rows per workgroup

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v,
                                                       int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Channel maxima of |K| over rows [r0, r0 + kLamRows) of KV head blockIdx.y,
// merged into lam_bits[g][c] as fp32 bit patterns (for non-negative floats the
// patterns order like the values, NaN above infinity).
template <bool F32>
__global__ __launch_bounds__(kLamThreads) void channel_absmax_kernel(
    const void* __restrict__ keys, int num_tokens, uint32_t* __restrict__ lam_bits) {
    constexpr int kPerVec = F32 ? 4 : 8;                  // channels per 16-byte load
    constexpr int kVecPerRow = kHeadDim / kPerVec;        // 32 or 16
    constexpr int kRowStep = kLamThreads / kVecPerRow;    // 8 or 16 rows per sweep
    __shared__ uint32_t red[kRowStep][kHeadDim];
    const int g = blockIdx.y, tid = threadIdx.x;
    const int cv = tid % kVecPerRow, rsub = tid / kVecPerRow;
    const int r0 = blockIdx.x * kLamRows, r1 = min(num_tokens, r0 + kLamRows);
    const uint4* src =
        reinterpret_cast<const uint4*>(keys) + static_cast<size_t>(g) * num_tokens * kVecPerRow;
    // fp16: maxima of the 15-bit magnitude patterns; fp32: of the 31-bit ones
    uint32_t mx[kPerVec];
#pragma unroll
    for (int j = 0; j < kPerVec; ++j) mx[j] = 0;
#pragma unroll 4
    for (int r = r0 + rsub; r < r1; r += kRowStep) {
        const uint4 v = src[static_cast<size_t>(r) * kVecPerRow + cv];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (F32) {
                mx[q] = max(mx[q], w[q] & 0x7fffffffu);
            } else {
                mx[2 * q] = max(mx[2 * q], w[q] & 0x7fffu);
                mx[2 * q + 1] = max(mx[2 * q + 1], (w[q] >> 16) & 0x7fffu);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kPerVec; ++j) {
        uint32_t bits = mx[j];
        if constexpr (!F32)
            bits = __builtin_bit_cast(uint32_t, half_bits_to_float(static_cast<uint16_t>(bits)));
        red[rsub][cv * kPerVec + j] = bits;
    }
    __syncthreads();
    if (tid < kHeadDim) {
        uint32_t m = red[0][tid];
#pragma unroll
        for (int s = 1; s < kRowStep; ++s) m = max(m, red[s][tid]);
        atomicMax(&lam_bits[g * kHeadDim + tid], m);
    }
}

// lambda = sqrt(max |K|): the square root in fp64, rounded once to fp32 (the
// same value as a correctly rounded fp32 square root).
__global__ __launch_bounds__(256) void sqrt_lambda_kernel(uint32_t* __restrict__ lam_bits,
                                                          int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const double m = static_cast<double>(__builtin_bit_cast(float, lam_bits[i]));
        lam_bits[i] = __builtin_bit_cast(uint32_t, static_cast<float>(__dsqrt_rn(m)));
    }
}

// ---------------------------------------------------------------------------
// transformed calibration keys
// ---------------------------------------------------------------------------

// K~ = K diag(lambda)^-1 H_128 for one token row per wave: k / lambda in fp64,
// the +-1 Walsh–Hadamard transform, 1/sqrt(128), rounded once to fp32 (the
// arithmetic of the encoder's key transform).
__global__ __launch_bounds__(256) void transform_keys_kernel(const void* __restrict__ keys,
                                                             int kv_f32,
                                                             const float* __restrict__ lambda,
                                                             int num_tokens,
                                                             float* __restrict__ out) {
    const int g = blockIdx.y, lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= num_tokens) return;   // the whole wave: the transform needs every lane
    const size_t row = static_cast<size_t>(g) * num_tokens + t;
    const float* lam = lambda + g * kHeadDim;
    double k0, k1;
    if (kv_f32) {
        const float2 v = reinterpret_cast<const float2*>(keys)[row * (kHeadDim / 2) + lane];
        k0 = v.x;
        k1 = v.y;
    } else {
        const uint32_t v = reinterpret_cast<const uint32_t*>(keys)[row * (kHeadDim / 2) + lane];
        k0 = half_bits_to_float(static_cast<uint16_t>(v & 0xffffu));
        k1 = half_bits_to_float(static_cast<uint16_t>(v >> 16));
    }
    const float2 l = reinterpret_cast<const float2*>(lam)[lane];
    double x0 = k0 / static_cast<double>(l.x);
    double x1 = k1 / static_cast<double>(l.y);
    fwht128(x0, x1);
    reinterpret_cast<float2*>(out)[row * (kHeadDim / 2) + lane] =
        make_float2(static_cast<float>(x0 * kInvSqrtD64), static_cast<float>(x1 * kInvSqrtD64));
}

// ---------------------------------------------------------------------------
// K-Means
// ---------------------------------------------------------------------------

// Threads of an assignment workgroup: 4096-entry tables fill most of a CU's
// LDS (one workgroup per CU), so those take 16 waves to keep 4 on every SIMD.
template <int NENT>
constexpr int kAssignThreads = NENT >= 4096 ? 1024 : 512;
constexpr int kKmChunk = 8192;                 // samples per assignment workgroup = sort chunk
constexpr int kSortWaves = 4;                  // chunks per scatter workgroup (one per wave)

// fp64 centroids staged in LDS when they fit beside the fp32 tables (8 KiB);
// the 4096-entry case reads its few candidates from global memory (L2).
template <int NENT>
constexpr bool kKmLdsC64 = NENT <= 256;

// fp64 squared distance of fp32 sample x to fp64 centroid c, rounded as the
// definition rounds it (difference, square and running sum separately, in
// channel order, from zero).
__device__ __forceinline__ double sqdist4_c64(const float4 x, const double c[4]) {
    const double e0 = __dadd_rn(static_cast<double>(x.x), -c[0]);
    const double e1 = __dadd_rn(static_cast<double>(x.y), -c[1]);
    const double e2 = __dadd_rn(static_cast<double>(x.z), -c[2]);
    const double e3 = __dadd_rn(static_cast<double>(x.w), -c[3]);
    double d = __dmul_rn(e0, e0);
    d = __dadd_rn(d, __dmul_rn(e1, e1));
    d = __dadd_rn(d, __dmul_rn(e2, e2));
    d = __dadd_rn(d, __dmul_rn(e3, e3));
    return d;
}

// Nearest centroid of every sample of one sort chunk (kKmChunk samples of set
// blockIdx.y): assign[set][i], and, when hist is given, the chunk's cluster
// histogram hist[set][chunk][NENT].  The search is nearest_search.hpp's with
// the fp64 centroids rounded to fp32 for the scores: that rounding adds u
// (||x||^2 + ||c||^2) to the score error, well inside the bound.  Samples
// and centroids must be finite with magnitudes below about 2^60 so that no
// fp32 score overflows.
template <int NENT>
__global__ __launch_bounds__(kAssignThreads<NENT>) void kmeans_assign_kernel(
    const float* __restrict__ samples, int num_samples, const double* __restrict__ centroids,
    int32_t* __restrict__ assign, int32_t* __restrict__ hist) {
    __shared__ float m2[4 * kSearchStride<NENT>];   // -2 fl32(c) by channel
    __shared__ __align__(16) float ccu[NENT];       // fl32(||c||^2) (1 + 2^-16)
    __shared__ __align__(16) float ccd[NENT];       // fl32(||c||^2) (1 - 2^-16)
    __shared__ double c64s[kKmLdsC64<NENT> ? NENT * 4 : 1];
    __shared__ int32_t cnt[NENT];
    __shared__ float wdm[kAssignThreads<NENT> / kWave];

    const int set = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const double* cset = centroids + static_cast<size_t>(set) * NENT * 4;
    const float4* xset = reinterpret_cast<const float4*>(samples) +
                         static_cast<size_t>(set) * num_samples;
    float dm = 0.f;
    for (int i = tid; i < NENT; i += kAssignThreads<NENT>) {
        const double2 lo = reinterpret_cast<const double2*>(cset)[2 * i];
        const double2 hi = reinterpret_cast<const double2*>(cset)[2 * i + 1];
        const double c[4] = {lo.x, lo.y, hi.x, hi.y};
        double nn = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m2[j * kSearchStride<NENT> + i] = -2.f * static_cast<float>(c[j]);
            nn += c[j] * c[j];
            if constexpr (kKmLdsC64<NENT>) c64s[i * 4 + j] = c[j];
        }
        const float nf = static_cast<float>(nn);
        ccu[i] = nf * kBoundUp;
        ccd[i] = nf * kBoundDown;
        dm = fmaxf(dm, nf * kBoundUp - nf * kBoundDown);
        cnt[i] = 0;
    }
    dm = wave_max(dm);
    if (lane == 0) wdm[wave] = dm;
    __syncthreads();
    float dmax = 0.f;   // the largest difference of the two norm terms
#pragma unroll
    for (int w = 0; w < kAssignThreads<NENT> / kWave; ++w) dmax = fmaxf(dmax, wdm[w]);

    const int s0 = chunk * kKmChunk, s1 = min(num_samples, s0 + kKmChunk);
    int32_t* aset = assign + static_cast<size_t>(set) * num_samples;
    for (int base = s0 + wave * 16; base < s1; base += (kAssignThreads<NENT> / kWave) * 16) {
        // this lane's sample base + lane % 16 (zero past the chunk)
        const int r = base + (lane & 15);
        const float4 x = r < s1 ? xset[r] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float xc[4] = {x.x, x.y, x.z, x.w};
        const float bop = xc[lane >> 4];   // B operand: channel lane / 16
        const float ex = row_bound((x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w));
        const auto exact = [&](uint32_t nc) {
            double c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (kKmLdsC64<NENT>)
                    c[j] = c64s[nc * 4 + j];
                else
                    c[j] = cset[nc * 4 + j];
            }
            return sqdist4_c64(x, c);
        };
        const uint32_t code = nearest16<NENT>(m2, ccu, ccd, bop, ex, dmax, lane, exact);
        if (lane < 16 && r < s1) {
            aset[r] = static_cast<int32_t>(code);
            if (hist != nullptr) atomicAdd(&cnt[code & (NENT - 1)], 1);
        }
    }
    if (hist != nullptr) {
        __syncthreads();
        int32_t* h = hist + (static_cast<size_t>(set) * gridDim.x + chunk) * NENT;
        for (int i = tid; i < NENT; i += kAssignThreads<NENT>) h[i] = cnt[i];
    }
}

// The same for 8-dim samples and centroids.
__device__ __forceinline__ double sqdist8_c64(const float x[8], const double c[8]) {
    double d = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double e = __dadd_rn(static_cast<double>(x[j]), -c[j]);
        d = j == 0 ? __dmul_rn(e, e) : __dadd_rn(d, __dmul_rn(e, e));
    }
    return d;
}

// kmeans_assign_kernel for 8-dim samples [S][n][8] and centroids [S][NENT][8]:
// the fp64 centroids rounded to fp32 in a channel-pair-major table (A
// operand), the sample as -2x (B operand), one norm table scaled by
// (1 +- 2^-16) as it is read.  LDS: table 32 NENT bytes, norms and histogram
// 4 NENT bytes each (160 KiB at NENT = 4096), plus the fp64 centroids when
// they fit (NENT <= 256); the 4096-entry case reads its candidates from L2.
template <int NENT>
constexpr int kAssign8Lds = NENT * 40 + (kKmLdsC64<NENT> ? NENT * 64 : 0);

template <int NENT>
__global__ __launch_bounds__(kAssignThreads<NENT>) void kmeans_assign8_kernel(
    const float* __restrict__ samples, int num_samples, const double* __restrict__ centroids,
    int32_t* __restrict__ assign, int32_t* __restrict__ hist) {
    __shared__ __align__(16) uint8_t lds[kAssign8Lds<NENT>];
    float* tab = reinterpret_cast<float*>(lds);                   // [4][NENT][2]
    float* nrm = reinterpret_cast<float*>(lds + NENT * 32);       // [NENT]
    int32_t* cnt = reinterpret_cast<int32_t*>(lds + NENT * 36);   // [NENT]
    double* c64s = reinterpret_cast<double*>(lds + NENT * 40);    // [NENT][8] (small NENT)

    const int set = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const double* cset = centroids + static_cast<size_t>(set) * NENT * 8;
    const float4* xset = reinterpret_cast<const float4*>(samples) +
                         static_cast<size_t>(set) * num_samples * 2;
    for (int i = tid; i < NENT; i += kAssignThreads<NENT>) {
        double c[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double2 v = reinterpret_cast<const double2*>(cset)[4 * i + j];
            c[2 * j] = v.x;
            c[2 * j + 1] = v.y;
        }
        double nn = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            nn += c[j] * c[j];
            if constexpr (kKmLdsC64<NENT>) c64s[i * 8 + j] = c[j];
        }
#pragma unroll
        for (int g2 = 0; g2 < 4; ++g2)
            reinterpret_cast<float2*>(tab)[g2 * NENT + i] =
                make_float2(static_cast<float>(c[2 * g2]), static_cast<float>(c[2 * g2 + 1]));
        nrm[i] = static_cast<float>(nn);
        cnt[i] = 0;
    }
    __syncthreads();
    // a bound on the difference of the two norm terms ScaledNorms forms,
    // fl(n (1 + 2^-16)) - fl(n (1 - 2^-16)) <= n (2^-15 + 2^-23 (1 + 2^-15)),
    // from the largest norm (every wave reads the whole table: the LDS is full)
    float nmax = 0.f;
    for (int i = lane; i < NENT / 4; i += kWave) {
        const f32x4_t v = reinterpret_cast<const f32x4_t*>(nrm)[i];
        nmax = fmaxf(nmax, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
    const float dmax = wave_max(nmax) * (0x1p-15f + 0x1p-22f);

    const int s0 = chunk * kKmChunk, s1 = min(num_samples, s0 + kKmChunk);
    int32_t* aset = assign + static_cast<size_t>(set) * num_samples;
    const int q4 = 4 * (lane >> 4), gq = lane >> 4;
    const ScaledNorms cup{reinterpret_cast<const f32x4_t*>(nrm + q4), kBoundUp};
    const ScaledNorms cdown{reinterpret_cast<const f32x4_t*>(nrm + q4), kBoundDown};
    for (int base = s0 + wave * 16; base < s1; base += (kAssignThreads<NENT> / kWave) * 16) {
        // this lane's sample base + lane % 16 (zero past the chunk)
        const int r = base + (lane & 15);
        const float4 lo = r < s1 ? xset[2 * r] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 hi = r < s1 ? xset[2 * r + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        float xx = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) xx += x[j] * x[j];
        const auto exact = [&](uint32_t nc) {
            double c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if constexpr (kKmLdsC64<NENT>)
                    c[j] = c64s[nc * 8 + j];
                else
                    c[j] = cset[nc * 8 + j];
            }
            return sqdist8_c64(x, c);
        };
        const BlockF32D8<NENT> block(tab, -2.f * x[2 * gq], -2.f * x[2 * gq + 1], lane);
        const uint32_t code =
            nearest16_search<NENT>(block, cup, cdown, row_bound(xx), dmax, lane, exact);
        if (lane < 16 && r < s1) {
            aset[r] = static_cast<int32_t>(code);
            if (hist != nullptr) atomicAdd(&cnt[code & (NENT - 1)], 1);
        }
    }
    if (hist != nullptr) {
        __syncthreads();
        int32_t* h = hist + (static_cast<size_t>(set) * gridDim.x + chunk) * NENT;
        for (int i = tid; i < NENT; i += kAssignThreads<NENT>) h[i] = cnt[i];
    }
}

// Per (set, cluster): the chunk histograms become exclusive prefix sums over
// the chunks (in place), and counts[set][c] the cluster sizes.
__global__ __launch_bounds__(256) void chunk_offsets_kernel(int32_t* __restrict__ hist,
                                                            int nchunks, int nent,
                                                            int32_t* __restrict__ counts) {
    const int set = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (c >= nent) return;
    int32_t* h = hist + static_cast<size_t>(set) * nchunks * nent + c;
    int32_t run = 0;
    int k = 0;
    for (; k + 8 <= nchunks; k += 8) {   // 8 independent loads in flight
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = h[static_cast<size_t>(k + u) * nent];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            h[static_cast<size_t>(k + u) * nent] = run;
            run += v[u];
        }
    }
    for (; k < nchunks; ++k) {
        const int32_t v = h[static_cast<size_t>(k) * nent];
        h[static_cast<size_t>(k) * nent] = run;
        run += v;
    }
    counts[static_cast<size_t>(set) * nent + c] = run;
}

// base[set][c] = exclusive prefix sum of counts[set][.] over the clusters:
// where cluster c starts in the sorted samples.  One 1024-thread workgroup
// per set; nent <= 4096.
__global__ __launch_bounds__(1024) void cluster_base_kernel(const int32_t* __restrict__ counts,
                                                            int nent,
                                                            int32_t* __restrict__ base) {
    __shared__ int32_t wsum[1024 / kWave];
    const int set = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int per = (nent + 1023) / 1024;   // 1 .. 4 consecutive clusters per thread
    const int32_t* cs = counts + static_cast<size_t>(set) * nent;
    int32_t* bs = base + static_cast<size_t>(set) * nent;
    int32_t v[4] = {0, 0, 0, 0};
    int32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid * per + j;
        if (j < per && c < nent) v[j] = cs[c];
        tot += v[j];
    }
    int32_t incl = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int32_t run = incl - tot;
    for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid * per + j;
        if (j < per && c < nent) bs[c] = run;
        run += v[j];
    }
}

// Stable counting sort of the samples by cluster: sample i of chunk k goes to
// base[c] + (samples of c in chunks before k) + (samples of c before i in
// chunk k).  One wave per chunk walks it in order, 64 samples a step; lanes
// with the same cluster are found with one ballot per code bit.  No barrier:
// every wave works alone on its own chunk and its own LDS counters.
template <int BITS, int SUB>
__global__ __launch_bounds__(kSortWaves * kWave) void kmeans_scatter_kernel(
    const float* __restrict__ samples, int num_samples, const int32_t* __restrict__ assign,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ base, int nchunks,
    float* __restrict__ sorted) {
    constexpr int NENT = 1 << BITS;
    __shared__ int32_t cnt[kSortWaves][NENT];
    const int set = blockIdx.y, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int chunk = blockIdx.x * kSortWaves + wave;
    if (chunk >= nchunks) return;
    const int32_t* off = offs + (static_cast<size_t>(set) * nchunks + chunk) * NENT;
    const int32_t* bs = base + static_cast<size_t>(set) * NENT;
    int32_t* my = cnt[wave];
    for (int c = lane; c < NENT; c += kWave) my[c] = bs[c] + off[c];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int s0 = chunk * kKmChunk, s1 = min(num_samples, s0 + kKmChunk);
    const int32_t* aset = assign + static_cast<size_t>(set) * num_samples;
    constexpr int kV = SUB / 4;   // float4 per sample
    const float4* xs = reinterpret_cast<const float4*>(samples) +
                       static_cast<size_t>(set) * num_samples * kV;
    float4* out = reinterpret_cast<float4*>(sorted) + static_cast<size_t>(set) * num_samples * kV;
    const uint64_t below = (1ull << lane) - 1ull;
    // a ring of kAhead steps of 64 samples in flight: each step takes its
    // codes and samples from the ring and requests those kAhead steps later
    // (past the chunk: its last sample, loaded and never placed), so one
    // memory latency is spread over kAhead steps
    constexpr int kAhead = 8;
    static_assert(kV == 1 || kV == 2, "4- or 8-dim samples");
    uint32_t cpre[kAhead];
    float4 xpre0[kAhead], xpre1[kAhead];   // the sample's first and (8-dim) second float4
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
        const size_t i = static_cast<size_t>(min(s0 + k * kWave + lane, s1 - 1));
        cpre[k] = static_cast<uint32_t>(aset[i]);
        xpre0[k] = xs[i * kV];
        if constexpr (kV == 2) xpre1[k] = xs[i * kV + 1];
    }
    for (int j0 = s0; j0 < s1; j0 += kAhead * kWave) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
            const int i = j0 + k * kWave + lane;
            const bool valid = i < s1;
            const uint32_t c = valid ? cpre[k] & (NENT - 1) : 0u;
            const float4 x0 = xpre0[k], x1 = xpre1[k];
            const size_t inext = static_cast<size_t>(min(i + kAhead * kWave, s1 - 1));
            cpre[k] = static_cast<uint32_t>(aset[inext]);
            xpre0[k] = xs[inext * kV];
            if constexpr (kV == 2) xpre1[k] = xs[inext * kV + 1];
            uint64_t same = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
            for (int b = 0; b < BITS; ++b) {
                const bool bit = (c >> b) & 1u;
                const uint64_t set_bits = __builtin_amdgcn_ballot_w64(bit);
                same &= bit ? set_bits : ~set_bits;
            }
            const int rank = __popcll(same & below);
            const int total = __popcll(same);
            int32_t start = 0;
            if (valid) start = my[c];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (valid) my[c] = start + total;   // every lane of the group writes the same value
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int32_t pos = start + rank;
            if (valid && static_cast<uint32_t>(pos) < static_cast<uint32_t>(num_samples)) {
                out[static_cast<size_t>(pos) * kV] = x0;
                if constexpr (kV == 2) out[static_cast<size_t>(pos) * kV + 1] = x1;
            }
        }
    }
}

// New centroids: one wave per (set, cluster).  The 64 lanes stream the
// cluster's sorted samples in tiles of 64 (coalesced 16-byte loads, kPre
// tiles in flight), stage each tile channel-major in LDS, and lanes 0 .. SUB-1
// add channel `lane` of the tile's samples in order onto one fp64 sum each: the
// sum of the cluster's samples in sample order from zero, then one division
// by the count.  A cluster without samples keeps its centroid.
constexpr int kUpdWaves = 4;
constexpr int kPre = 8;   // tiles of 64 samples in flight per wave

template <int SUB>
__global__ __launch_bounds__(kUpdWaves * kWave) void kmeans_update_kernel(
    const float* __restrict__ sorted, int num_samples, const int32_t* __restrict__ base,
    const int32_t* __restrict__ counts, int nent, double* __restrict__ centroids) {
    constexpr int kV = SUB / 4;   // float4 per sample
    __shared__ __align__(16) float stage[kUpdWaves][SUB][kWave];
    const int set = blockIdx.y, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int c = blockIdx.x * kUpdWaves + wave;
    if (c >= nent) return;   // the whole wave; no barrier below
    const int32_t n = counts[static_cast<size_t>(set) * nent + c];
    if (n == 0) return;
    const float4* src = reinterpret_cast<const float4*>(sorted) +
                        (static_cast<size_t>(set) * num_samples +
                         base[static_cast<size_t>(set) * nent + c]) * kV;
    float* st = &stage[wave][0][0];
    const int tiles = (n + kWave - 1) / kWave;
    // loads past the cluster read its last sample (never added): unconditional
    // loads keep the memory counters exact, so the prefetches stay in flight
    float4 pre[kPre][kV];
#pragma unroll
    for (int k = 0; k < kPre; ++k)
#pragma unroll
        for (int v = 0; v < kV; ++v) pre[k][v] = src[min(k * kWave + lane, n - 1) * kV + v];
    double s = 0.0;
    for (int t0 = 0; t0 < tiles; t0 += kPre) {
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int t = t0 + k;   // t >= tiles: a padding tile, loaded and skipped
#pragma unroll
            for (int v = 0; v < kV; ++v) {
                const float4 x = pre[k][v];
                pre[k][v] = src[min((t + kPre) * kWave + lane, n - 1) * kV + v];
                st[(4 * v + 0) * kWave + lane] = x.x;
                st[(4 * v + 1) * kWave + lane] = x.y;
                st[(4 * v + 2) * kWave + lane] = x.z;
                st[(4 * v + 3) * kWave + lane] = x.w;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < SUB && t < tiles) {
                const int m = min(kWave, n - t * kWave);   // samples in this tile
                if (m == kWave) {
                    const float4* row = reinterpret_cast<const float4*>(st + lane * kWave);
#pragma unroll
                    for (int q = 0; q < kWave / 4; ++q) {
                        const float4 v = row[q];
                        s = __dadd_rn(s, static_cast<double>(v.x));
                        s = __dadd_rn(s, static_cast<double>(v.y));
                        s = __dadd_rn(s, static_cast<double>(v.z));
                        s = __dadd_rn(s, static_cast<double>(v.w));
                    }
                } else {
                    for (int q = 0; q < m; ++q)
                        s = __dadd_rn(s, static_cast<double>(st[lane * kWave + q]));
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    if (lane < SUB)
        centroids[(static_cast<size_t>(set) * nent + c) * SUB + lane] =
            __ddiv_rn(s, static_cast<double>(n));
}

// fp64 -> fp16 bit pattern, rounded once to nearest even (subnormal halves,
// overflow to infinity, NaN kept), not through fp32.
__device__ __forceinline__ uint16_t double_to_half_bits(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7fffffffffffffffull;
    if (a >= 0x7ff0000000000000ull)
        return static_cast<uint16_t>(sign | (a > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u));
    const int e = static_cast<int>(a >> 52) - 1023;
    if (e >= 16) return static_cast<uint16_t>(sign | 0x7c00u);
    const uint64_t m = (a & 0x000fffffffffffffull) | (1ull << 52);
    // normal halves keep 11 significant bits (shift 42); subnormal ones count
    // units of 2^-24 (shift 28 - e)
    const int shift = e >= -14 ? 42 : 28 - e;
    if (shift > 53) return static_cast<uint16_t>(sign);   // below half the smallest subnormal
    const uint64_t q = m >> shift, rem = m & ((1ull << shift) - 1ull), half = 1ull << (shift - 1);
    const uint32_t up = (rem > half || (rem == half && (q & 1ull))) ? 1u : 0u;
    const uint32_t mag = e >= -14 ? (static_cast<uint32_t>(e + 15) << 10) +
                                        static_cast<uint32_t>(q - 1024) + up
                                  : static_cast<uint32_t>(q) + up;
    return static_cast<uint16_t>(sign | mag);
}

__global__ __launch_bounds__(256) void centroids_to_half_kernel(const double* __restrict__ c,
                                                                size_t n,
                                                                uint16_t* __restrict__ out) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) out[i] = double_to_half_bits(c[i]);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int kmeans_chunks(int num_samples) { return (num_samples + kKmChunk - 1) / kKmChunk; }

struct KmWorkspace {
    int32_t* assign;   // [sets][n]
    int32_t* hist;     // [sets][chunks][E]
    int32_t* counts;   // [sets][E]
    int32_t* base;     // [sets][E]
    float* sorted;     // [sets][n][d]
};

size_t kmeans_ws_layout(int num_sets, int num_samples, int sub_dim, int code_bits, char* p,
                        KmWorkspace* w) {
    const size_t sets = static_cast<size_t>(num_sets), n = static_cast<size_t>(num_samples);
    const size_t ent = static_cast<size_t>(1) << code_bits;
    const size_t chunks = static_cast<size_t>(kmeans_chunks(num_samples));
    size_t off = 0;
    const auto take = [&](size_t bytes) {
        char* q = p ? p + off : nullptr;
        off += align256(bytes);
        return q;
    };
    char* a = take(sets * n * 4);
    char* h = take(sets * chunks * ent * 4);
    char* c = take(sets * ent * 4);
    char* b = take(sets * ent * 4);
    char* s = take(sets * n * 4 * static_cast<size_t>(sub_dim));
    if (w) {
        w->assign = reinterpret_cast<int32_t*>(a);
        w->hist = reinterpret_cast<int32_t*>(h);
        w->counts = reinterpret_cast<int32_t*>(c);
        w->base = reinterpret_cast<int32_t*>(b);
        w->sorted = reinterpret_cast<float*>(s);
    }
    return off;
}

template <int BITS, int SUB>
hipError_t kmeans_assign(const float* samples, int num_sets, int num_samples,
                         const double* centroids, int32_t* assign, int32_t* hist,
                         hipStream_t stream) {
    const dim3 grid(kmeans_chunks(num_samples), num_sets);
    if constexpr (SUB == 8)
        hipLaunchKernelGGL(kmeans_assign8_kernel<1 << BITS>, grid, dim3(kAssignThreads<1 << BITS>), 0, stream,
                           samples, num_samples, centroids, assign, hist);
    else
        hipLaunchKernelGGL(kmeans_assign_kernel<1 << BITS>, grid, dim3(kAssignThreads<1 << BITS>), 0, stream,
                           samples, num_samples, centroids, assign, hist);
    return hipGetLastError();
}

template <int BITS, int SUB>
hipError_t kmeans_run(const float* samples, int num_sets, int num_samples, const double* init,
                      int iters, double* centroids, uint16_t* codebook, int32_t* assign_out,
                      void* workspace, hipStream_t stream) {
    constexpr int NENT = 1 << BITS;
    KmWorkspace w;
    kmeans_ws_layout(num_sets, num_samples, SUB, BITS, static_cast<char*>(workspace), &w);
    const int nchunks = kmeans_chunks(num_samples);
    const size_t cbytes = static_cast<size_t>(num_sets) * NENT * SUB * sizeof(double);
    hipError_t e = hipSuccess;
    if (init != centroids) {
        e = hipMemcpyAsync(centroids, init, cbytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return e;
    }
    for (int it = 0; it < iters; ++it) {
        if ((e = kmeans_assign<BITS, SUB>(samples, num_sets, num_samples, centroids, w.assign,
                                          w.hist, stream)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3((NENT + 255) / 256, num_sets), dim3(256), 0,
                           stream, w.hist, nchunks, NENT, w.counts);
        hipLaunchKernelGGL(cluster_base_kernel, dim3(num_sets), dim3(1024), 0, stream, w.counts,
                           NENT, w.base);
        hipLaunchKernelGGL((kmeans_scatter_kernel<BITS, SUB>),
                           dim3((nchunks + kSortWaves - 1) / kSortWaves, num_sets),
                           dim3(kSortWaves * kWave), 0, stream, samples, num_samples, w.assign,
                           w.hist, w.base, nchunks, w.sorted);
        hipLaunchKernelGGL(kmeans_update_kernel<SUB>,
                           dim3((NENT + kUpdWaves - 1) / kUpdWaves, num_sets),
                           dim3(kUpdWaves * kWave), 0, stream, w.sorted, num_samples, w.base,
                           w.counts, NENT, centroids);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (assign_out != nullptr &&
        (e = kmeans_assign<BITS, SUB>(samples, num_sets, num_samples, centroids, assign_out,
                                      nullptr, stream)) != hipSuccess)
        return e;
    if (codebook != nullptr) {
        const size_t n = static_cast<size_t>(num_sets) * NENT * SUB;
        hipLaunchKernelGGL(centroids_to_half_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                           dim3(256), 0, stream, centroids, n, codebook);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_calibrate_lambda(const void* keys, bool kv_f32, int num_kv_heads,
                                   int num_tokens, float* lambda, hipStream_t stream) {
    const int n = num_kv_heads * kHeadDim;
    uint32_t* bits = reinterpret_cast<uint32_t*>(lambda);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, bits, 0u, n);
    const dim3 grid((num_tokens + kLamRows - 1) / kLamRows, num_kv_heads);
    if (kv_f32)
        hipLaunchKernelGGL(channel_absmax_kernel<true>, grid, dim3(kLamThreads), 0, stream, keys,
                           num_tokens, bits);
    else
        hipLaunchKernelGGL(channel_absmax_kernel<false>, grid, dim3(kLamThreads), 0, stream, keys,
                           num_tokens, bits);
    hipLaunchKernelGGL(sqrt_lambda_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, bits, n);
    return hipGetLastError();
}

hipError_t launch_transform_keys(const void* keys, bool kv_f32, const float* lambda,
                                 int num_kv_heads, int num_tokens, float* out,
                                 hipStream_t stream) {
    const dim3 grid((num_tokens + 3) / 4, num_kv_heads);
    hipLaunchKernelGGL(transform_keys_kernel, grid, dim3(256), 0, stream, keys, kv_f32 ? 1 : 0,
                       lambda, num_tokens, out);
    return hipGetLastError();
}

size_t kmeans_workspace_bytes(int num_sets, int num_samples, int sub_dim, int code_bits) {
    return kmeans_ws_layout(num_sets, num_samples, sub_dim, code_bits, nullptr, nullptr);
}

hipError_t launch_kmeans(const float* samples, int num_sets, int num_samples, int sub_dim,
                         int code_bits, const double* init, int iters, double* centroids,
                         uint16_t* codebook, int32_t* assign, void* workspace,
                         hipStream_t stream) {
#define VQKV_KM(BITS, SUB)                                                                     \
    return kmeans_run<BITS, SUB>(samples, num_sets, num_samples, init, iters, centroids,        \
                                 codebook, assign, workspace, stream)
    if (sub_dim == 8) {
        if (code_bits == 8) VQKV_KM(8, 8);
        VQKV_KM(12, 8);
    }
    if (code_bits == 8) VQKV_KM(8, 4);
    VQKV_KM(12, 4);
#undef VQKV_KM
}

}  // namespace vqkv
