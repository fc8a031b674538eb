// Cross-split log-sum-exp merge of decode-attention partials.
//
// Every partial s of a (sequence, query head) — a split, or a wave within a
// split — leaves, in base-2 units, the running max m_s, the running sum l_s = sum_t 2^(s_t - m_s) and the
// unnormalised output o_s = sum_t 2^(s_t - m_s) v_t.  The softmax over the
// union of the partials is
//     out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// computed by folding partials pairwise with the FlashAttention rescaling step
// of the VecInfer page's Appendix (block recurrence of m, l and O).  A
// partial with no tokens has m = -inf and weighs 0.  The folds run in a fixed
// order, so the result is reproducible bit for bit.
//
// Four 256-thread workgroups per (sequence, query head), one per 32
// channels; 32 slices of 8 threads each take every 32nd partial.  A thread
// issues the loads of 16 partials (m, l and 16 bytes of o) before using any,
// folds them with the same rescaling step in registers, and the 32 slice
// results are folded once more through LDS: one round trip to memory when
// there are at most 512 partials.
#include "launchers.hpp"

namespace vqkv {

namespace {
constexpr int kMergeThreads = 256;
constexpr int kQuarter = 32;                       // channels per workgroup
constexpr int kCols = kQuarter / 4;                // float4 columns per workgroup
constexpr int kSlices = kMergeThreads / kCols;     // 32
constexpr int kInFlight = 16;

// fold (m2, l2, o2) into the running (m, l, o)
__device__ __forceinline__ void fold(float& m, float& l, float4& o, float m2, float l2,
                                     const float4& o2) {
    if (m2 == -INFINITY) return;   // an empty partial
    const float mn = fmaxf(m, m2);
    const float a = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float b = exp2f(m2 - mn);
    l = a * l + b * l2;
    o.x = a * o.x + b * o2.x;
    o.y = a * o.y + b * o2.y;
    o.z = a * o.z + b * o2.z;
    o.w = a * o.w + b * o2.w;
    m = mn;
}
}  // namespace

__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(int num_partials,
                                                                       Partials part,
                                                                       float* __restrict__ out) {
    __shared__ float msl[kSlices], lsl[kSlices];
    __shared__ float4 osl[kSlices][kCols];

    const size_t bh = blockIdx.x;
    const int quarter = blockIdx.y;
    const size_t base = bh * num_partials;
    const int tid = threadIdx.x;
    const int j = tid / kCols, c4 = tid % kCols;
    const int col = quarter * kCols + c4;

    float m = -INFINITY, l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = j; s0 < num_partials; s0 += kInFlight * kSlices) {
        float mv[kInFlight], lv[kInFlight];
        float4 ov[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int s = s0 + u * kSlices;
            if (s < num_partials) {
                mv[u] = part.m[base + s];
                lv[u] = part.l[base + s];
                ov[u] = reinterpret_cast<const float4*>(part.o + (base + s) * kHeadDim)[col];
            } else {
                mv[u] = -INFINITY;
                lv[u] = 0.f;
                ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) fold(m, l, o, mv[u], lv[u], ov[u]);
    }
    osl[j][c4] = o;
    if (c4 == 0) {
        msl[j] = m;
        lsl[j] = l;
    }
    __syncthreads();
    if (tid < kQuarter) {
        float mm = -INFINITY, ll = 0.f;
        float4 oo = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int jj = 0; jj < kSlices; ++jj) fold(mm, ll, oo, msl[jj], lsl[jj], osl[jj][tid >> 2]);
        const int e = tid & 3;
        const float num = e == 0 ? oo.x : (e == 1 ? oo.y : (e == 2 ? oo.z : oo.w));
        out[bh * kHeadDim + quarter * kQuarter + tid] = num / ll;
    }
}

hipError_t launch_merge_partials(int batch, int num_q_heads, int num_partials, Partials part,
                                 float* out, hipStream_t stream) {
    hipLaunchKernelGGL(merge_partials_kernel, dim3(batch * num_q_heads, kHeadDim / kQuarter),
                       dim3(kMergeThreads), 0, stream, num_partials, part, out);
    return hipGetLastError();
}

}  // namespace vqkv
