// Cross-split log-sum-exp merge of decode-attention partials.
//
// Every split s of a (sequence, query head) leaves, in base-2 units, its
// running max m_s, its running sum l_s = sum_t 2^(x_t - m_s) and its
// unnormalised output o_s = sum_t 2^(x_t - m_s) v_t.  The softmax over the
// union of the splits is
//     out = sum_s w_s o_s / sum_s w_s l_s,   w_s = 2^(m_s - M),  M = max_s m_s,
// the block-merge step of the FlashAttention recurrence (VecInfer page,
// Appendix: m, l and O rescaled by exp(m_old - m_new) across blocks), taken
// here for all splits at once.  A split with no tokens has m = -inf and
// weighs 0.
//
// One 128-thread workgroup per (sequence, query head).  The first 32 o_s
// rows are requested before anything else; meanwhile the threads share the
// m_s, l_s (split s on thread s mod 128), reduce M and the denominator, and
// leave the weights in LDS.  Thread d then accumulates channel d over the
// splits in split order, 32 loads in flight: the result is reproducible.
#include "launchers.hpp"

namespace vqkv {

namespace {
constexpr int kChunk = 32;
constexpr int kPer = kMaxSplits / kHeadDim;   // splits per thread in the weight pass
static_assert(kMaxSplits % kHeadDim == 0 && kMaxSplits % kChunk == 0, "split tiling");
}  // namespace

__global__ __launch_bounds__(kHeadDim) void merge_partials_kernel(int num_partials,
                                                                  Partials part,
                                                                  float* __restrict__ out) {
    __shared__ float wsh[kMaxSplits];   // w_s, zero beyond num_partials
    __shared__ float red[2][2];

    const size_t bh = blockIdx.x;
    const int d = threadIdx.x, lane = d & (kWave - 1), wave = d / kWave;
    const int last = num_partials - 1;
    const float* pm = part.m + bh * num_partials;
    const float* pl = part.l + bh * num_partials;
    const float* po = part.o + bh * num_partials * kHeadDim + d;

    float ov[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) ov[u] = po[static_cast<size_t>(min(u, last)) * kHeadDim];

    float mv[kPer], lv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = d + i * kHeadDim;
        mv[i] = (s < num_partials) ? pm[s] : -INFINITY;
        lv[i] = (s < num_partials) ? pl[s] : 0.f;
    }
    float mx = mv[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) mx = fmaxf(mx, mv[i]);
    mx = wave_max(mx);
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    mx = fmaxf(red[0][0], red[0][1]);
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const float w = (mv[i] == -INFINITY) ? 0.f : exp2f(mv[i] - mx);
        wsh[d + i * kHeadDim] = w;
        den += w * lv[i];
    }
    den = wave_sum(den);
    if (lane == 0) red[1][wave] = den;
    __syncthreads();
    den = red[1][0] + red[1][1];

    float num = 0.f;
    for (int s0 = 0;;) {
#pragma unroll
        for (int u = 0; u < kChunk; ++u) num += wsh[s0 + u] * ov[u];
        s0 += kChunk;
        if (s0 >= num_partials) break;
#pragma unroll
        for (int u = 0; u < kChunk; ++u)
            ov[u] = po[static_cast<size_t>(min(s0 + u, last)) * kHeadDim];
    }
    out[bh * kHeadDim + d] = num / den;
}

hipError_t launch_merge_partials(int batch, int num_q_heads, int num_partials, Partials part,
                                 float* out, hipStream_t stream) {
    if (num_partials < 1 || num_partials > kMaxSplits) return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_partials_kernel, dim3(batch * num_q_heads), dim3(kHeadDim), 0,
                       stream, num_partials, part, out);
    return hipGetLastError();
}

}  // namespace vqkv
