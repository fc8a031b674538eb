// Host-side launchers of the libvqkv kernels (internal; called by vqkv_api.hip
// after argument validation).  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.hpp"

namespace vqkv {

struct AttnShape {
    int batch, num_q_heads, num_kv_heads, capacity, context_len;
    int num_splits, tokens_per_split;
};

hipError_t launch_transform_query(const void* q, bool q_f32, const float* lambda, int batch,
                                  int num_q_heads, int num_kv_heads, float* q_tilde,
                                  hipStream_t stream);

// Split-K decode attention over the VQ cache on the matrix cores: one
// partial (m, l, o) per (sequence, query head, split).
hipError_t launch_vq_attention(const AttnShape& s, int k_bits, const void* q, bool q_f32,
                               const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                               const uint8_t* codes_k, const uint8_t* codes_v, Partials part,
                               hipStream_t stream);

// out[bh][:] from the num_partials partials of every (sequence, query head) bh.
hipError_t launch_merge_partials(int batch, int num_q_heads, int num_partials, Partials part,
                                 float* out, hipStream_t stream);

hipError_t launch_encode_append(int k_bits, const void* k_new, const void* v_new, bool kv_f32,
                                const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                                uint8_t* codes_k, uint8_t* codes_v, int batch, int num_kv_heads,
                                int capacity, int cur_len, int num_new, hipStream_t stream);

hipError_t launch_fp16_attention_splits(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, Partials part, hipStream_t stream);

// Tokens one workgroup of the VQ split kernel processes per tile; split
// lengths are multiples of it.
constexpr int kVqWaves = 16;       // waves per workgroup of the VQ kernel; each leaves a partial
constexpr int kVqTile = 512;       // = waves per workgroup x tokens per wave tile
constexpr int kFp16Tile = 128;
constexpr int kMaxSplits = 512;    // bound of the split planner

}  // namespace vqkv
