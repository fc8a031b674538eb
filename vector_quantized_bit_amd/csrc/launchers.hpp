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

// One new token per (sequence, KV head) to encode into slot append_pos
// (k_new == nullptr: none).  k_new, v_new [B][Hkv][128].  The split pass
// then leaves num_splits + 1 partials per (sequence, query head), the last
// one for the new token; AttnShape covers the cached tokens only.
struct AppendArgs {
    const void* k_new = nullptr;
    const void* v_new = nullptr;
    bool kv_f32 = false;
    int append_pos = -1;
    uint8_t* codes_k = nullptr;   // the cache, written at that slot
    uint8_t* codes_v = nullptr;
    // Residual window (win_k != nullptr): the new token goes, as fp16, to slot
    // win_len of win_k / win_v [B][Hkv][win_cap][128] instead of being
    // encoded, and the extra partial covers window slots 0 .. win_len.
    uint16_t* win_k = nullptr;
    uint16_t* win_v = nullptr;
    int win_len = 0;
    int win_cap = 0;
    // No extra workgroup: the last split of every stream encodes the new token
    // (or attends over the window) and leaves that partial before attending
    // over its own tokens.
    bool fold = false;
};

// Split-K decode attention over the VQ cache on the matrix cores: one
// partial (m, l, o) per (sequence, query head, split), plus the new token's
// when appending.
// sub_dim 4 (k_bits 8 or 12, 8-bit values) or 8 (12-bit keys and values).
hipError_t launch_vq_attention(const AttnShape& s, int k_bits, int sub_dim, const void* q,
                               bool q_f32, const float* lambda, const uint16_t* cb_k,
                               const uint16_t* cb_v, const uint8_t* codes_k,
                               const uint8_t* codes_v, Partials part, const AppendArgs& append,
                               hipStream_t stream);

// out[bh][:] from the num_partials partials of every (sequence, query head) bh.
hipError_t launch_merge_partials(int batch, int num_q_heads, int num_partials, Partials part,
                                 float* out, hipStream_t stream);

hipError_t launch_encode_append(int k_bits, int sub_dim, const void* k_new, const void* v_new,
                                bool kv_f32, const float* lambda, const uint16_t* cb_k,
                                const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v,
                                int batch, int num_kv_heads, int capacity, int cur_len,
                                int num_new, hipStream_t stream);

hipError_t launch_fp16_attention_splits(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, Partials part, hipStream_t stream);

// Offline calibration: lambda = sqrt(max |K|) per (KV head, channel) over
// keys [Hkv][T][128]; K~ = K diag(lambda)^-1 H_128 as fp32 [Hkv][T][128];
// Lloyd K-Means over fp32 samples [sets][n][d] with fp64 centroids
// [sets][2^code_bits][d], d = 4 or 8 (init may equal centroids), optional fp16 codebook
// and final assignment outputs, workspace of kmeans_workspace_bytes.
hipError_t launch_calibrate_lambda(const void* keys, bool kv_f32, int num_kv_heads,
                                   int num_tokens, float* lambda, hipStream_t stream);
hipError_t launch_transform_keys(const void* keys, bool kv_f32, const float* lambda,
                                 int num_kv_heads, int num_tokens, float* out,
                                 hipStream_t stream);
size_t kmeans_workspace_bytes(int num_sets, int num_samples, int sub_dim, int code_bits);
hipError_t launch_kmeans(const float* samples, int num_sets, int num_samples, int sub_dim,
                         int code_bits, const double* init, int iters, double* centroids,
                         uint16_t* codebook, int32_t* assign, void* workspace,
                         hipStream_t stream);

// Library-wide deterministic mode (vq_set_deterministic): the split kernel
// hands tiles to waves in a fixed order, so results do not depend on timing.
bool deterministic();
bool set_deterministic(bool on);   // returns the previous setting

// Library-wide score method of the split kernel (vq_set_score_method).
constexpr int kScoresMfma = 0;     // matrix-core products with dequantised keys
constexpr int kScoresLut = 1;      // sums of q~ . C_k lookup-table entries
int score_method();
int set_score_method(int method);   // returns the previous method

// Tokens one workgroup of the VQ split kernel processes per tile; split
// lengths are multiples of it.
constexpr int kVqWaves = 16;       // waves per workgroup of the VQ kernel; each leaves a partial
constexpr int kVqTile = 512;       // shortest split: waves per workgroup x tokens per wave tile
constexpr int kVqTileGrain = 32;   // split lengths are multiples of one wave tile
constexpr int kFp16Tile = 128;
constexpr int kMaxSplits = 512;    // bound of the split planner

}  // namespace vqkv
