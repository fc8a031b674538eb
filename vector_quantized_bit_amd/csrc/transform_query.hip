// q~ = q diag(lambda) H_128: one wave per (sequence, query head).
// VecInfer page, Method details (smooth factors, Walsh–Hadamard recursion,
// attention-score rewrite).
#include "launchers.hpp"

namespace vqkv {

__global__ __launch_bounds__(256) void transform_query_kernel(
    const void* __restrict__ q, int q_f32, const float* __restrict__ lambda, int num_vec,
    int num_q_heads, int group, float* __restrict__ q_tilde) {
    const int vec = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (vec >= num_vec) return;  // whole wave exits together
    const int lane = threadIdx.x & (kWave - 1);
    const int head = vec % num_q_heads;
    const float* lam = lambda + (head / group) * kHeadDim;
    float x0, x1;
    if (q_f32) {
        const float2 v = reinterpret_cast<const float2*>(q)[vec * (kHeadDim / 2) + lane];
        x0 = v.x;
        x1 = v.y;
    } else {
        const uint32_t w = reinterpret_cast<const uint32_t*>(q)[vec * (kHeadDim / 2) + lane];
        x0 = half_bits_to_float(static_cast<uint16_t>(w & 0xffffu));
        x1 = half_bits_to_float(static_cast<uint16_t>(w >> 16));
    }
    const float2 l = reinterpret_cast<const float2*>(lam)[lane];
    x0 *= l.x;
    x1 *= l.y;
    fwht128(x0, x1);
    reinterpret_cast<float2*>(q_tilde)[vec * (kHeadDim / 2) + lane] =
        make_float2(x0 * kInvSqrtD, x1 * kInvSqrtD);
}

hipError_t launch_transform_query(const void* q, bool q_f32, const float* lambda, int batch,
                                  int num_q_heads, int num_kv_heads, float* q_tilde,
                                  hipStream_t stream) {
    const int num_vec = batch * num_q_heads;
    const int per_block = 256 / kWave;
    const int blocks = (num_vec + per_block - 1) / per_block;
    hipLaunchKernelGGL(transform_query_kernel, dim3(blocks), dim3(256), 0, stream, q,
                       q_f32 ? 1 : 0, lambda, num_vec, num_q_heads,
                       num_q_heads / num_kv_heads, q_tilde);
    return hipGetLastError();
}

}  // namespace vqkv
