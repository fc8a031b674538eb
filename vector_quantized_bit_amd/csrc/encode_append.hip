// Nearest-centroid encoder for appended tokens.
//
// VecInfer page, Method details (VQ KV cache in attention): a new key gets
// the online dual transform k~ = k diag(lambda)^-1 H_D and is quantised with
// C_k; its value is quantised untransformed with C_v; the codes are
// concatenated to the cache.  Background (VQ principle): every 4-channel
// sub-vector gets j* = argmin_j ||x_i - C_j||^2.
//
// The transform and the squared distances are evaluated in fp64 (products
// and sums rounded separately, summed over the 4 channels in order), so the
// argmin is decided in the same precision as the fp64 reference; exact ties
// go to the lowest index because the scan is ascending with a strict '<'.
//
// One workgroup encodes 8 tokens of one (sequence, KV head); thread
// (token, position) owns one key and one value sub-vector.
#include "launchers.hpp"

namespace vqkv {

namespace {

constexpr int kEncTok = 8;
constexpr int kEncChunk = 1024;   // codebook entries staged in LDS at a time

__device__ __forceinline__ double load_elem(const void* p, bool f32, size_t i) {
    if (f32) return static_cast<double>(reinterpret_cast<const float*>(p)[i]);
    return static_cast<double>(half_bits_to_float(reinterpret_cast<const uint16_t*>(p)[i]));
}

__device__ __forceinline__ double sqdist4(const double x[4], const float4 c) {
    double d = 0.0;
    const double e0 = __dadd_rn(x[0], -static_cast<double>(c.x));
    const double e1 = __dadd_rn(x[1], -static_cast<double>(c.y));
    const double e2 = __dadd_rn(x[2], -static_cast<double>(c.z));
    const double e3 = __dadd_rn(x[3], -static_cast<double>(c.w));
    d = __dadd_rn(d, __dmul_rn(e0, e0));
    d = __dadd_rn(d, __dmul_rn(e1, e1));
    d = __dadd_rn(d, __dmul_rn(e2, e2));
    d = __dadd_rn(d, __dmul_rn(e3, e3));
    return d;
}

// Scan `entries` fp16 centroids for the nearest one to x; all threads of the
// block call this together (it stages the codebook through LDS).
__device__ __forceinline__ uint32_t nearest(const double x[4], const uint16_t* __restrict__ cb,
                                            int entries, float4* cbuf) {
    double best = INFINITY;
    uint32_t arg = 0;
    const uint2* src = reinterpret_cast<const uint2*>(cb);
    for (int base = 0; base < entries; base += kEncChunk) {
        const int n = min(kEncChunk, entries - base);
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const uint2 raw = src[base + i];
            cbuf[i] = make_float4(half_bits_to_float(raw.x & 0xffffu), half_bits_to_float(raw.x >> 16),
                                  half_bits_to_float(raw.y & 0xffffu), half_bits_to_float(raw.y >> 16));
        }
        __syncthreads();
        for (int j = 0; j < n; ++j) {
            const double d = sqdist4(x, cbuf[j]);
            if (d < best) {
                best = d;
                arg = static_cast<uint32_t>(base + j);
            }
        }
    }
    return arg;
}

}  // namespace

template <int KBITS>
__global__ __launch_bounds__(256) void encode_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    constexpr int KROW = kNumSub * KBITS / 8;
    __shared__ double xk[kEncTok][kHeadDim];
    __shared__ float4 cbuf[kEncChunk];
    __shared__ uint16_t kcode[kEncTok][kNumSub];

    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int tok0 = blockIdx.x * kEncTok;
    const int ntok = min(kEncTok, num_new - tok0);
    const int tid = threadIdx.x;
    const bool f32 = kv_f32 != 0;
    const size_t in_row0 = (static_cast<size_t>(b) * num_kv_heads + g) * num_new + tok0;
    const float* lam = lambda + g * kHeadDim;

    // k / lambda in fp64, then the +-1 Walsh–Hadamard butterflies in LDS
    for (int e = tid; e < kEncTok * kHeadDim; e += 256) {
        const int t = e / kHeadDim, c = e % kHeadDim;
        xk[t][c] = (t < ntok) ? load_elem(k_new, f32, (in_row0 + t) * kHeadDim + c) /
                                    static_cast<double>(lam[c])
                              : 0.0;
    }
    __syncthreads();
    for (int h = 1; h < kHeadDim; h <<= 1) {
        for (int e = tid; e < kEncTok * (kHeadDim / 2); e += 256) {
            const int t = e / (kHeadDim / 2), i = e % (kHeadDim / 2);
            const int lo = (i / h) * 2 * h + (i % h);
            const double a = xk[t][lo], c = xk[t][lo + h];
            xk[t][lo] = a + c;
            xk[t][lo + h] = a - c;
        }
        __syncthreads();
    }

    const int t = tid / kNumSub;
    const int p = tid % kNumSub;
    double x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = xk[t][4 * p + i] * kInvSqrtD64;
    const uint32_t ck = nearest(x, cb_k + static_cast<size_t>(g) * (4u << KBITS), 1 << KBITS, cbuf);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        x[i] = (t < ntok) ? load_elem(v_new, f32, (in_row0 + t) * kHeadDim + 4 * p + i) : 0.0;
    const uint32_t cvc = nearest(x, cb_v + static_cast<size_t>(g) * 1024, 256, cbuf);

    const size_t out_row0 = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + tok0;
    if (t < ntok) codes_v[(out_row0 + t) * kNumSub + p] = static_cast<uint8_t>(cvc);
    if constexpr (KBITS == 8) {
        if (t < ntok) codes_k[(out_row0 + t) * kNumSub + p] = static_cast<uint8_t>(ck);
    } else {
        kcode[t][p] = static_cast<uint16_t>(ck);
        __syncthreads();
        // byte j of a row holds bits [8j, 8j+8) of the little-endian 12-bit stream
        for (int e = tid; e < kEncTok * KROW; e += 256) {
            const int tt = e / KROW, j = e % KROW;
            if (tt >= ntok) continue;
            const int bit = 8 * j;
            const int i0 = bit / 12, sh = bit % 12;
            uint32_t v = static_cast<uint32_t>(kcode[tt][i0]) >> sh;
            if (sh > 4) v |= static_cast<uint32_t>(kcode[tt][i0 + 1]) << (12 - sh);
            codes_k[(out_row0 + tt) * KROW + j] = static_cast<uint8_t>(v & 0xffu);
        }
    }
}

hipError_t launch_encode_append(int k_bits, const void* k_new, const void* v_new, bool kv_f32,
                                const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                                uint8_t* codes_k, uint8_t* codes_v, int batch, int num_kv_heads,
                                int capacity, int cur_len, int num_new, hipStream_t stream) {
    const dim3 grid((num_new + kEncTok - 1) / kEncTok, num_kv_heads, batch);
    if (k_bits == 8)
        hipLaunchKernelGGL(encode_append_kernel<8>, grid, dim3(256), 0, stream, k_new, v_new,
                           kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v, num_kv_heads,
                           capacity, cur_len, num_new);
    else
        hipLaunchKernelGGL(encode_append_kernel<12>, grid, dim3(256), 0, stream, k_new, v_new,
                           kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v, num_kv_heads,
                           capacity, cur_len, num_new);
    return hipGetLastError();
}

}  // namespace vqkv
