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
// argmin is decided in the same precision as the fp64 reference.  Exact ties
// go to the lowest index: every thread scans its centroids in ascending order
// with a strict '<', and the per-thread winners are combined by the
// lexicographic minimum of (distance, index).
//
// One 256-thread workgroup encodes one token of one (sequence, KV head):
// thread (slice s, position p) scans centroids s, s + 8, s + 16, ... of
// sub-vector p, so a single decode-step append (one token per head) is 8x
// shorter than a scan per sub-vector.  Codebooks are staged in LDS (2 KiB,
// or 32 KiB for 12-bit keys); the 8 threads that share a centroid index sit
// in different waves, the 32 threads of a wave read one broadcast address.
#include "launchers.hpp"

namespace vqkv {

namespace {

constexpr int kEncThreads = 256;
constexpr int kEncSlices = kEncThreads / kNumSub;   // 8

__device__ __forceinline__ double load_elem(const void* p, bool f32, size_t i) {
    if (f32) return static_cast<double>(reinterpret_cast<const float*>(p)[i]);
    return static_cast<double>(half_bits_to_float(reinterpret_cast<const uint16_t*>(p)[i]));
}

// Nearest of `entries` LDS centroids to x among indices slice, slice + 8, ...,
// combined across the 8 slices; returns the code for this thread's position.
__device__ __forceinline__ uint32_t nearest(const double x[4], const uint2* cb, int entries,
                                            int slice, int pos, double* bd, uint32_t* bi) {
    double best = INFINITY;
    uint32_t arg = 0;
#pragma unroll 4
    for (int c = slice; c < entries; c += kEncSlices) {
        const double d = sqdist4_f64(x, cb[c]);
        if (d < best) {
            best = d;
            arg = static_cast<uint32_t>(c);
        }
    }
    bd[slice * kNumSub + pos] = best;
    bi[slice * kNumSub + pos] = arg;
    __syncthreads();
    double b0 = bd[pos];
    uint32_t a0 = bi[pos];
#pragma unroll
    for (int s = 1; s < kEncSlices; ++s) {
        const double d = bd[s * kNumSub + pos];
        const uint32_t a = bi[s * kNumSub + pos];
        if (nearer(d, a, b0, a0)) {
            b0 = d;
            a0 = a;
        }
    }
    __syncthreads();   // bd / bi are reused by the next call
    return a0;
}

}  // namespace

template <int KBITS>
__global__ __launch_bounds__(kEncThreads) void encode_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, int kv_f32,
    const float* __restrict__ lambda, const uint16_t* __restrict__ cb_k,
    const uint16_t* __restrict__ cb_v, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, int num_kv_heads, int capacity, int cur_len, int num_new) {
    constexpr int KENT = 1 << KBITS;
    constexpr int KROW = kNumSub * KBITS / 8;
    __shared__ uint2 kcb[KENT];
    __shared__ uint2 vcb[256];
    __shared__ double xk[kHeadDim];
    __shared__ double bd[kEncSlices * kNumSub];
    __shared__ uint32_t bi[kEncSlices * kNumSub];
    __shared__ uint32_t kcode[kNumSub];

    const int tok = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const bool f32 = kv_f32 != 0;
    const size_t in_row = (static_cast<size_t>(b) * num_kv_heads + g) * num_new + tok;

    // this thread's value sub-vector is loaded first so its latency hides
    // behind the codebook staging and the key scan
    const int pos = tid % kNumSub, slice = tid / kNumSub;
    double xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = load_elem(v_new, f32, in_row * kHeadDim + 4 * pos + i);

    const uint2* ksrc = reinterpret_cast<const uint2*>(cb_k) + (static_cast<size_t>(g) << KBITS);
    for (int i = tid; i < KENT; i += kEncThreads) kcb[i] = ksrc[i];
    vcb[tid] = reinterpret_cast<const uint2*>(cb_v)[static_cast<size_t>(g) * 256 + tid];

    // k / lambda in fp64, +-1 Walsh–Hadamard butterflies in one wave, then 1/sqrt(128)
    if (tid < kWave) {
        const float* lam = lambda + g * kHeadDim;
        double x0 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane) /
                    static_cast<double>(lam[2 * lane]);
        double x1 = load_elem(k_new, f32, in_row * kHeadDim + 2 * lane + 1) /
                    static_cast<double>(lam[2 * lane + 1]);
        fwht128(x0, x1);
        xk[2 * lane] = x0 * kInvSqrtD64;
        xk[2 * lane + 1] = x1 * kInvSqrtD64;
    }
    __syncthreads();

    double x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = xk[4 * pos + i];
    const uint32_t ck = nearest(x, kcb, KENT, slice, pos, bd, bi);
    const uint32_t cv = nearest(xv, vcb, 256, slice, pos, bd, bi);

    const size_t out_row = (static_cast<size_t>(b) * num_kv_heads + g) * capacity + cur_len + tok;
    if (tid < kNumSub) codes_v[out_row * kNumSub + pos] = static_cast<uint8_t>(cv);
    if constexpr (KBITS == 8) {
        if (tid < kNumSub) codes_k[out_row * KROW + pos] = static_cast<uint8_t>(ck);
    } else {
        if (tid < kNumSub) kcode[pos] = ck;
        __syncthreads();
        // byte j of the row holds bits [8j, 8j+8) of the little-endian 12-bit stream
        if (tid < KROW) {
            const int bit = 8 * tid;
            const int i0 = bit / 12, sh = bit % 12;
            uint32_t v = kcode[i0] >> sh;
            if (sh > 4) v |= kcode[i0 + 1] << (12 - sh);
            codes_k[out_row * KROW + tid] = static_cast<uint8_t>(v & 0xffu);
        }
    }
}

hipError_t launch_encode_append(int k_bits, const void* k_new, const void* v_new, bool kv_f32,
                                const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                                uint8_t* codes_k, uint8_t* codes_v, int batch, int num_kv_heads,
                                int capacity, int cur_len, int num_new, hipStream_t stream) {
    const dim3 grid(num_new, num_kv_heads, batch);
    if (k_bits == 8)
        hipLaunchKernelGGL(encode_append_kernel<8>, grid, dim3(kEncThreads), 0, stream, k_new,
                           v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,
                           num_kv_heads, capacity, cur_len, num_new);
    else
        hipLaunchKernelGGL(encode_append_kernel<12>, grid, dim3(kEncThreads), 0, stream, k_new,
                           v_new, kv_f32 ? 1 : 0, lambda, cb_k, cb_v, codes_k, codes_v,
                           num_kv_heads, capacity, cur_len, num_new);
    return hipGetLastError();
}

}  // namespace vqkv
