// Cross-split log-sum-exp merge of decode-attention partials.
//
// Every split s of a (sequence, query head) leaves, in base-2 units, the
// running max m_s, the running sum l_s = sum_t 2^(s_t - m_s) and the
// unnormalised output o_s = sum_t 2^(s_t - m_s) v_t.  The softmax over the
// union of the splits is
//     out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// the FlashAttention rescaling step of the VecInfer page's Appendix
// (block recurrence of m, l and O) applied across splits.  A split with no
// tokens has m = -inf and weighs 0.  The sum runs in a fixed order, so the
// result is reproducible bit for bit.
//
// One 256-thread workgroup per (sequence, query head): the split maxima and
// weights go through LDS, then 8 slices of 32 threads each sum every 8th
// split, issuing 8 loads of 16 bytes before using any, so the partials'
// latency (they were just written by other XCDs) overlaps.
#include "launchers.hpp"

namespace vqkv {

namespace {
constexpr int kMergeThreads = 256;
constexpr int kSlices = kMergeThreads / 32;
}  // namespace

__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(int num_splits,
                                                                       Partials part,
                                                                       float* __restrict__ out) {
    __shared__ float wsh[kMaxSplits];
    __shared__ float red[kMergeThreads / 64];
    __shared__ float4 osum[kSlices][32];
    __shared__ float lsum[kSlices];

    const size_t bh = blockIdx.x;
    const size_t base = bh * num_splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    float mx = -INFINITY;
    for (int s = tid; s < num_splits; s += kMergeThreads) {
        const float v = part.m[base + s];
        wsh[s] = v;
        mx = fmaxf(mx, v);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) mx = fmaxf(mx, red[w]);
    for (int s = tid; s < num_splits; s += kMergeThreads) {
        const float v = wsh[s];
        wsh[s] = (v == -INFINITY) ? 0.f : exp2f(v - mx);
    }
    __syncthreads();

    const int j = tid >> 5, c4 = tid & 31;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lacc = 0.f;
    for (int s0 = j; s0 < num_splits; s0 += 8 * kSlices) {
        float4 o[8];
        float l[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + u * kSlices;
            if (s < num_splits) {
                o[u] = reinterpret_cast<const float4*>(part.o + (base + s) * kHeadDim)[c4];
                l[u] = part.l[base + s];
            } else {
                o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                l[u] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + u * kSlices;
            const float w = (s < num_splits) ? wsh[s] : 0.f;
            acc.x += w * o[u].x;
            acc.y += w * o[u].y;
            acc.z += w * o[u].z;
            acc.w += w * o[u].w;
            lacc += w * l[u];
        }
    }
    osum[j][c4] = acc;
    if (c4 == 0) lsum[j] = lacc;
    __syncthreads();
    if (tid < kHeadDim) {
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int jj = 0; jj < kSlices; ++jj) {
            const float4 v = osum[jj][tid >> 2];
            const int e = tid & 3;
            num += e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
            den += lsum[jj];
        }
        out[bh * kHeadDim + tid] = num / den;
    }
}

hipError_t launch_merge_partials(int batch, int num_q_heads, int num_splits, Partials part,
                                 float* out, hipStream_t stream) {
    hipLaunchKernelGGL(merge_partials_kernel, dim3(batch * num_q_heads), dim3(kMergeThreads), 0,
                       stream, num_splits, part, out);
    return hipGetLastError();
}

}  // namespace vqkv
