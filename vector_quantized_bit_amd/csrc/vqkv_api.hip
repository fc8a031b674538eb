// C ABI of libvqkv (declared in include/vqkv.h): host-side validation, split
// planning, workspace layout and kernel dispatch.  Validation never touches
// the device or dereferences a caller pointer.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "../../include/vqkv.h"
#include "launchers.hpp"

namespace vqkv {

namespace {
std::atomic<bool> g_deterministic{false};
}

bool deterministic() { return g_deterministic.load(std::memory_order_relaxed); }
bool set_deterministic(bool on) { return g_deterministic.exchange(on); }

namespace {
std::atomic<int> g_score_method{kScoresMfma};
}

int score_method() { return g_score_method.load(std::memory_order_relaxed); }
int set_score_method(int method) { return g_score_method.exchange(method); }

}  // namespace vqkv

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return VQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define VQ_REQUIRE_PTR(p)                                                             \
    do {                                                                              \
        if ((p) == nullptr) return fail(VQ_ERR_INVALID_ARG, "%s is NULL", #p);        \
        if (!aligned16(p)) return fail(VQ_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
    } while (0)

// Device-independent plan: the same shape always gets the same split count,
// so results are reproducible across devices and runs.
constexpr int kTargetWorkgroups = 256;       // VQ kernel: one 16-wave workgroup per CU (256 CUs)
constexpr int kTargetWorkgroupsFp16 = 1024;  // fp16 comparator: 4-wave workgroups, 4 per CU
constexpr int kMaxGroup = 8;

int check_layout(const vq_layout* L) {
    if (L == nullptr) return fail(VQ_ERR_INVALID_ARG, "layout is NULL");
    if (L->head_dim != vqkv::kHeadDim)
        return fail(VQ_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", L->head_dim);
    if (L->sub_dim != 4 && L->sub_dim != 8)
        return fail(VQ_ERR_UNSUPPORTED, "sub_dim %d unsupported (4 or 8)", L->sub_dim);
    if (L->sub_dim == 8) {
        if (L->k_code_bits != 12 || L->v_code_bits != 12)
            return fail(VQ_ERR_UNSUPPORTED,
                        "sub_dim 8 takes 12-bit K and V codes (got k_code_bits %d, v_code_bits %d)",
                        L->k_code_bits, L->v_code_bits);
    } else {
        if (L->k_code_bits != 8 && L->k_code_bits != 12)
            return fail(VQ_ERR_UNSUPPORTED, "k_code_bits %d unsupported (8 or 12)",
                        L->k_code_bits);
        if (L->v_code_bits != 8)
            return fail(VQ_ERR_UNSUPPORTED, "v_code_bits %d unsupported with sub_dim 4 (only 8)",
                        L->v_code_bits);
    }
    if (L->num_kv_heads < 1 || L->num_kv_heads > 65535)
        return fail(VQ_ERR_INVALID_ARG, "num_kv_heads %d out of range [1, 65535]", L->num_kv_heads);
    if (L->capacity < 1) return fail(VQ_ERR_INVALID_ARG, "capacity %d < 1", L->capacity);
    return VQ_OK;
}

int check_heads(int batch, int num_q_heads, int num_kv_heads) {
    if (batch < 1 || batch > 65535)
        return fail(VQ_ERR_INVALID_ARG, "batch %d out of range [1, 65535]", batch);
    if (num_q_heads < 1) return fail(VQ_ERR_INVALID_ARG, "num_q_heads %d < 1", num_q_heads);
    if (num_q_heads % num_kv_heads != 0)
        return fail(VQ_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    if (num_q_heads / num_kv_heads > kMaxGroup)
        return fail(VQ_ERR_UNSUPPORTED, "GQA group %d > %d", num_q_heads / num_kv_heads, kMaxGroup);
    return VQ_OK;
}

struct SplitPlan {
    int num_splits;
    int tokens_per_split;
    bool fold = false;   // decode step: the last split encodes the new token
};

// The VQ split kernel addresses one split's code rows through a buffer
// resource whose byte range is a 32-bit count: a split holds fewer than 2^31
// bytes of its widest rows (48 B), rounded down to whole wave tiles.
constexpr int kVqMaxSplitTokens = (0x7fffffff / 48) / 32 * 32;

// Longest split the planner gives while the split count allows (up to
// kMaxSplits): every wave of a split adds its tiles' value products into one
// fp32 accumulator, and once a dominant token sits in it each later tile's
// small contribution is rounded against that large value.  The error grows
// with the tiles a wave takes.  Behind a token 20.5 base-2 units above the
// rest, with value entries of 30: measured 7e-4 to 1.1e-3 on the GPU for one
// 65536-token split; a CPU model of the accumulation gives 1e-4 to 5e-4 there,
// ~2e-3 for one 196608-token split and ~2e-4 at 24576 tokens (48 tiles per
// wave).  24576 also leaves the default plans of the workload shapes as they
// are (up to 21856 tokens per split: a 64-stream window step).  Contexts
// longer than kMaxSplits x 24576 tokens get splits of context / kMaxSplits
// tokens.
constexpr int kVqLongestSplit = 24576;

// Splits hold at least `min_len` tokens (one sweep of the workgroup), at most
// `max_len`, and a multiple of `gran` tokens (one wave tile); the last split
// takes the rest.  A requested count is clamped into that range.
SplitPlan plan_splits(int streams, int context_len, int requested, int min_len,
                      int target = kTargetWorkgroups, int gran = 0,
                      int max_len = kVqMaxSplitTokens) {
    if (gran <= 0) gran = min_len;
    const int64_t n = context_len;   // (64-bit: contexts reach 2^31 - 1 tokens)
    int64_t max_splits = (n + min_len - 1) / min_len;
    if (max_splits > vqkv::kMaxSplits) max_splits = vqkv::kMaxSplits;
    int64_t s = requested > 0 ? requested : (static_cast<int64_t>(target) + streams - 1) / streams;
    const int64_t min_splits = (n + max_len - 1) / max_len;
    if (s < min_splits) s = min_splits;
    if (s < 1) s = 1;
    if (s > max_splits) s = max_splits;
    const int64_t per = (n + s - 1) / s;
    const int64_t tps = ((per + gran - 1) / gran) * gran;
    return {static_cast<int>((n + tps - 1) / tps), static_cast<int>(tps)};
}

// (sequence, KV head) streams of a call, saturated at the int32 limit (the
// launching entry points reject such shapes; the plan queries stay defined).
int streams_of(int32_t batch, int32_t num_kv_heads) {
    const int64_t n = static_cast<int64_t>(batch) * num_kv_heads;
    return n > 0x7fffffff ? 0x7fffffff : static_cast<int>(n);
}

// The VQ kernel's plan for `streams` (sequence, KV head) streams.
SplitPlan plan_vq(int streams, int context_len, int requested) {
    return plan_splits(streams, context_len, requested, vqkv::kVqTile, kTargetWorkgroups,
                       vqkv::kVqTileGrain, kVqLongestSplit);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t partials_bytes(int batch, int num_q_heads, int num_splits) {
    const size_t n = static_cast<size_t>(batch) * num_q_heads * num_splits;
    return 2 * align256(n * sizeof(float)) + align256(n * vqkv::kHeadDim * sizeof(float));
}

vqkv::Partials carve_partials(void* ws, int batch, int num_q_heads, int num_splits) {
    const size_t n = static_cast<size_t>(batch) * num_q_heads * num_splits;
    char* p = static_cast<char*>(ws);
    vqkv::Partials part;
    part.m = reinterpret_cast<float*>(p);
    part.l = reinterpret_cast<float*>(p + align256(n * sizeof(float)));
    part.o = reinterpret_cast<float*>(p + 2 * align256(n * sizeof(float)));
    return part;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(VQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* vq_status_string(int status) {
    switch (status) {
        case VQ_OK: return "ok";
        case VQ_ERR_INVALID_ARG: return "invalid argument";
        case VQ_ERR_UNSUPPORTED: return "unsupported geometry";
        case VQ_ERR_CAPACITY: return "cache capacity exceeded";
        case VQ_ERR_WORKSPACE: return "workspace missing or too small";
        case VQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* vq_last_error(void) { return g_last_error; }

int vq_set_deterministic(int on) { return vqkv::set_deterministic(on != 0) ? 1 : 0; }

int vq_set_score_method(int method) {
    if (method != VQ_SCORES_MFMA && method != VQ_SCORES_LUT) {
        fail(VQ_ERR_INVALID_ARG, "score method %d is not VQ_SCORES_MFMA or VQ_SCORES_LUT", method);
        return -1;
    }
    return vqkv::set_score_method(method);
}


int vq_transform_query(const vq_layout* layout, const void* q, int q_dtype, const float* lambda,
                       int32_t batch, int32_t num_q_heads, float* q_tilde, void* stream) {
    int st = check_layout(layout);
    if (st) return st;
    if ((st = check_heads(batch, num_q_heads, layout->num_kv_heads))) return st;
    if (q_dtype != VQ_F16 && q_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "q_dtype %d is not VQ_F16 or VQ_F32", q_dtype);
    VQ_REQUIRE_PTR(q);
    VQ_REQUIRE_PTR(lambda);
    VQ_REQUIRE_PTR(q_tilde);
    return hip_status(vqkv::launch_transform_query(q, q_dtype == VQ_F32, lambda, batch, num_q_heads,
                                                   layout->num_kv_heads, q_tilde,
                                                   static_cast<hipStream_t>(stream)),
                      "transform_query launch");
}

int vq_encode_append(const vq_layout* layout, const void* k_new, const void* v_new, int kv_dtype,
                     const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                     uint8_t* codes_k, uint8_t* codes_v, int32_t batch, int32_t cur_len,
                     int32_t num_new, void* stream) {
    int st = check_layout(layout);
    if (st) return st;
    if (batch < 1 || batch > 65535)
        return fail(VQ_ERR_INVALID_ARG, "batch %d out of range [1, 65535]", batch);
    if (kv_dtype != VQ_F16 && kv_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "kv_dtype %d is not VQ_F16 or VQ_F32", kv_dtype);
    if (num_new < 0) return fail(VQ_ERR_INVALID_ARG, "num_new %d < 0", num_new);
    if (cur_len < 0) return fail(VQ_ERR_INVALID_ARG, "cur_len %d < 0", cur_len);
    if (static_cast<int64_t>(cur_len) + num_new > layout->capacity)
        return fail(VQ_ERR_CAPACITY, "cur_len %d + num_new %d exceeds capacity %d", cur_len,
                    num_new, layout->capacity);
    VQ_REQUIRE_PTR(k_new);
    VQ_REQUIRE_PTR(v_new);
    VQ_REQUIRE_PTR(lambda);
    VQ_REQUIRE_PTR(cb_k);
    VQ_REQUIRE_PTR(cb_v);
    VQ_REQUIRE_PTR(codes_k);
    VQ_REQUIRE_PTR(codes_v);
    if (num_new == 0) return ok();
    return hip_status(vqkv::launch_encode_append(layout->k_code_bits, layout->sub_dim, k_new, v_new,
                                                 kv_dtype == VQ_F32, lambda, cb_k, cb_v, codes_k,
                                                 codes_v, batch, layout->num_kv_heads,
                                                 layout->capacity, cur_len, num_new,
                                                 static_cast<hipStream_t>(stream)),
                      "encode_append launch");
}

int32_t vq_decode_attention_default_splits(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t context_len) {
    (void)num_q_heads;
    if (layout == nullptr || batch < 1 || context_len < 1 || layout->num_kv_heads < 1) return 0;
    return plan_vq(streams_of(batch, layout->num_kv_heads), context_len, 0).num_splits;
}

size_t vq_decode_attention_workspace_bytes(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t context_len,
                                           int32_t num_splits) {
    if (layout == nullptr || batch < 1 || num_q_heads < 1 || context_len < 1 ||
        layout->num_kv_heads < 1)
        return 0;
    const SplitPlan p =
        plan_vq(streams_of(batch, layout->num_kv_heads), context_len, num_splits);
    return partials_bytes(batch, num_q_heads, p.num_splits);
}

int32_t vq_decode_attention_plan_splits(const vq_layout* layout, int32_t batch,
                                        int32_t num_q_heads, int32_t context_len,
                                        int32_t requested) {
    (void)num_q_heads;
    if (layout == nullptr || batch < 1 || context_len < 1 || layout->num_kv_heads < 1 ||
        requested < 0)
        return 0;
    return plan_vq(streams_of(batch, layout->num_kv_heads), context_len, requested)
        .num_splits;
}

namespace {

// Everything the split pass checks, shared by the partials and the fused entry.
int check_attention_args(const vq_layout* layout, const void* q, int q_dtype, const float* lambda,
                         const uint16_t* cb_k, const uint16_t* cb_v, const uint8_t* codes_k,
                         const uint8_t* codes_v, int32_t batch, int32_t num_q_heads,
                         int32_t context_len, int32_t num_splits) {
    int st = check_layout(layout);
    if (st) return st;
    if ((st = check_heads(batch, num_q_heads, layout->num_kv_heads))) return st;
    if (q_dtype != VQ_F16 && q_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "q_dtype %d is not VQ_F16 or VQ_F32", q_dtype);
    if (context_len < 1)
        return fail(VQ_ERR_INVALID_ARG, "context_len %d < 1 (softmax over no tokens)", context_len);
    if (context_len > layout->capacity)
        return fail(VQ_ERR_CAPACITY, "context_len %d exceeds capacity %d", context_len,
                    layout->capacity);
    if (num_splits < 0) return fail(VQ_ERR_INVALID_ARG, "num_splits %d < 0", num_splits);
    VQ_REQUIRE_PTR(q);
    VQ_REQUIRE_PTR(lambda);
    VQ_REQUIRE_PTR(cb_k);
    VQ_REQUIRE_PTR(cb_v);
    VQ_REQUIRE_PTR(codes_k);
    VQ_REQUIRE_PTR(codes_v);
    return VQ_OK;
}

int check_partials_ptrs(const float* part_m, const float* part_l, const float* part_o) {
    VQ_REQUIRE_PTR(part_m);
    VQ_REQUIRE_PTR(part_l);
    VQ_REQUIRE_PTR(part_o);
    return VQ_OK;
}

}  // namespace

int vq_decode_attention_partials(const vq_layout* layout, const void* q, int q_dtype,
                                 const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                                 const uint8_t* codes_k, const uint8_t* codes_v, int32_t batch,
                                 int32_t num_q_heads, int32_t context_len, int32_t num_splits,
                                 float* part_m, float* part_l, float* part_o, void* stream) {
    int st = check_attention_args(layout, q, q_dtype, lambda, cb_k, cb_v, codes_k, codes_v, batch,
                                  num_q_heads, context_len, num_splits);
    if (st) return st;
    if ((st = check_partials_ptrs(part_m, part_l, part_o))) return st;
    const SplitPlan p =
        plan_vq(streams_of(batch, layout->num_kv_heads), context_len, num_splits);
    if (num_splits != p.num_splits)
        return fail(VQ_ERR_INVALID_ARG,
                    "num_splits %d is not a planned split count for this shape "
                    "(vq_decode_attention_plan_splits gives %d)",
                    num_splits, p.num_splits);
    const vqkv::Partials part{part_m, part_l, part_o};
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity,
                                context_len, p.num_splits, p.tokens_per_split};
    return hip_status(vqkv::launch_vq_attention(shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32,
                                                lambda, cb_k, cb_v, codes_k, codes_v, part,
                                                vqkv::AppendArgs{},
                                                static_cast<hipStream_t>(stream)),
                      "decode_attention_partials launch");
}

int vq_merge_partials(int32_t batch, int32_t num_q_heads, int32_t num_partials,
                      const float* part_m, const float* part_l, const float* part_o, float* out,
                      void* stream) {
    if (batch < 1 || batch > 65535)
        return fail(VQ_ERR_INVALID_ARG, "batch %d out of range [1, 65535]", batch);
    if (num_q_heads < 1) return fail(VQ_ERR_INVALID_ARG, "num_q_heads %d < 1", num_q_heads);
    if (static_cast<int64_t>(batch) * num_q_heads > 0x7fffffff)
        return fail(VQ_ERR_INVALID_ARG, "batch * num_q_heads too large");
    if (num_partials < 1 || num_partials > vqkv::kMaxSplits)
        return fail(VQ_ERR_INVALID_ARG, "num_partials %d out of range [1, %d]", num_partials,
                    vqkv::kMaxSplits);
    int st = check_partials_ptrs(part_m, part_l, part_o);
    if (st) return st;
    VQ_REQUIRE_PTR(out);
    const vqkv::Partials part{const_cast<float*>(part_m), const_cast<float*>(part_l),
                              const_cast<float*>(part_o)};
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, num_partials, part, out,
                                                  static_cast<hipStream_t>(stream)),
                      "merge_partials launch");
}

extern "C++" {  // helpers with C++ return types: not part of the C ABI
namespace {

// Shared by the decode-step entry points: validate the appended rows, then
// the attention over cur_len + 1 tokens.
int check_step_args(const vq_layout* layout, const void* q, int q_dtype, const void* k_new,
                    const void* v_new, int kv_dtype, const float* lambda, const uint16_t* cb_k,
                    const uint16_t* cb_v, const uint8_t* codes_k, const uint8_t* codes_v,
                    int32_t batch, int32_t num_q_heads, int32_t cur_len, int32_t num_splits) {
    int st = check_layout(layout);
    if (st) return st;
    if (cur_len < 0) return fail(VQ_ERR_INVALID_ARG, "cur_len %d < 0", cur_len);
    if (static_cast<int64_t>(cur_len) + 1 > layout->capacity)
        return fail(VQ_ERR_CAPACITY, "cur_len %d + 1 exceeds capacity %d", cur_len,
                    layout->capacity);
    if (kv_dtype != VQ_F16 && kv_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "kv_dtype %d is not VQ_F16 or VQ_F32", kv_dtype);
    VQ_REQUIRE_PTR(k_new);
    VQ_REQUIRE_PTR(v_new);
    return check_attention_args(layout, q, q_dtype, lambda, cb_k, cb_v, codes_k, codes_v, batch,
                                num_q_heads, cur_len + 1, num_splits);
}

// The new token's encode in cached tokens that one split workgroup attends
// over in the same time, rounded up.  The folded split starts on its cached
// tokens about 7-8 us in with 256-entry C_k (encode about 6 us, then the
// one-token partial and the table staging of the token loop) and at most
// about 19 us in with 4096 entries (codes 12.4 us median, 13.3 us max); a
// split takes about 2.35 ns per token with 4 query heads a KV head and
// 3.1 ns with 5 (MI355X, timestamps, the chip loaded by the other splits).
// Too large a value only lengthens the other splits a little; too small a
// one makes the last split the slowest.  0 where the encode is not folded
// (d = 8).
int fold_tokens(const vq_layout* layout) {
    if (layout->sub_dim != 4) return 0;
    return layout->k_code_bits == 8 ? 3072 : 6144;
}

// From this many streams on, a decode step may fold the new token into the
// last split of each stream.  With fewer, the extra workgroups beside the
// splits take at most 1/8 of the CUs, and folding measured slower (8 streams
// of 196608 tokens: split pass 23.2 us folded, 22.3 us with 8 extra
// workgroups), the balance of a folded last split being the harder part.
constexpr int kFoldStreams = 32;

// The split kernel of a decode step.
//  - Many streams with long splits: every stream's splits take all 256 CUs,
//    and the last split of each stream encodes the new token before its
//    tokens; it is shorter than the others by the encode's worth of tokens
//    (splits of (cur_len + fold) / S tokens, the last one taking the rest).
//  - Otherwise one extra workgroup per stream (the new token, or the window)
//    follows the splits, all split workgroups first.  With few streams the
//    extra workgroups get CUs of their own next to the splits (256 - streams
//    split workgroups); from 128 streams on that would give half the chip or
//    more to short workgroups, so the splits fill all 256 CUs and the extra
//    workgroups run after them.
// A window step folds its window the same way from 128 streams on
// (kWindowFoldTokens).
SplitPlan plan_step(int streams, int cur_len, int requested, int fold = 0) {
    const int n = cur_len > 0 ? cur_len : 1;
    if (fold > 0 && streams >= kFoldStreams && n <= 0x7fffffff - fold) {
        const SplitPlan f = plan_splits(streams, n + fold, requested, vqkv::kVqTile,
                                        kTargetWorkgroups, vqkv::kVqTileGrain, kVqLongestSplit);
        // every split keeps tokens, and the encode is a small part of one
        if (static_cast<int64_t>(f.num_splits - 1) * f.tokens_per_split < n &&
            f.tokens_per_split >= 2 * fold)
            return SplitPlan{f.num_splits, f.tokens_per_split, true};
    }
    const int target = kTargetWorkgroups > 2 * static_cast<int64_t>(streams)
                           ? kTargetWorkgroups - streams
                           : kTargetWorkgroups;
    return plan_splits(streams, n, requested, vqkv::kVqTile, target, vqkv::kVqTileGrain,
                       kVqLongestSplit);
}

vqkv::AppendArgs append_args(const void* k_new, const void* v_new, int kv_dtype, int cur_len,
                             uint8_t* codes_k, uint8_t* codes_v, bool fold) {
    vqkv::AppendArgs app;
    app.fold = fold;
    app.k_new = k_new;
    app.v_new = v_new;
    app.kv_f32 = kv_dtype == VQ_F32;
    app.append_pos = cur_len;
    app.codes_k = codes_k;
    app.codes_v = codes_v;
    return app;
}

// A window step splits the num_codes coded tokens like a decode step; with
// no coded tokens there is no code split, only the window workgroup.
// The window's attention in cached tokens, rounded up like fold_tokens.  A
// window step folds from 64 streams on: there, with the window on the matrix
// cores (a 127-token window adds 1.1-2.1 us to the workgroup over an empty
// one), folding measured faster (64 streams of 65536 tokens: window step
// 62.3 us folded, 73.6 us beside the splits; of the fold sizes, 3072 tokens
// beat 2048 by 3% there and 2048 and 1536 by 1% at 128 streams of 32768).
// With fewer streams the window workgroups get CUs of their own beside the
// splits.
constexpr int kWindowFoldTokens = 3072;
constexpr int kWindowFoldStreams = 64;

SplitPlan plan_window_step(int streams, int num_codes, int requested) {
    if (num_codes == 0) return SplitPlan{0, 0};
    return plan_step(streams, num_codes, requested,
                     streams >= kWindowFoldStreams ? kWindowFoldTokens : 0);
}

int check_window_step_args(const vq_layout* layout, const void* q, int q_dtype,
                           const void* k_new, const void* v_new, int kv_dtype,
                           const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                           const uint8_t* codes_k, const uint8_t* codes_v, const uint16_t* win_k,
                           const uint16_t* win_v, int32_t win_cap, int32_t batch,
                           int32_t num_q_heads, int32_t num_codes, int32_t win_len,
                           int32_t num_splits) {
    int st = check_layout(layout);
    if (st) return st;
    if (num_codes < 0) return fail(VQ_ERR_INVALID_ARG, "num_codes %d < 0", num_codes);
    if (num_codes > layout->capacity)
        return fail(VQ_ERR_CAPACITY, "num_codes %d exceeds capacity %d", num_codes,
                    layout->capacity);
    if (win_cap < 1) return fail(VQ_ERR_INVALID_ARG, "window capacity %d < 1", win_cap);
    if (win_len < 0) return fail(VQ_ERR_INVALID_ARG, "win_len %d < 0", win_len);
    if (win_len >= win_cap)
        return fail(VQ_ERR_CAPACITY,
                    "window full: win_len %d, capacity %d (flush it with vq_flush_window)",
                    win_len, win_cap);
    if (kv_dtype != VQ_F16 && kv_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "kv_dtype %d is not VQ_F16 or VQ_F32", kv_dtype);
    VQ_REQUIRE_PTR(k_new);
    VQ_REQUIRE_PTR(v_new);
    VQ_REQUIRE_PTR(win_k);
    VQ_REQUIRE_PTR(win_v);
    // the code-side arguments, for at least one token (none is read when num_codes is 0)
    return check_attention_args(layout, q, q_dtype, lambda, cb_k, cb_v, codes_k, codes_v, batch,
                                num_q_heads, num_codes > 0 ? num_codes : 1, num_splits);
}

vqkv::AppendArgs window_args(const void* k_new, const void* v_new, int kv_dtype, int num_codes,
                             uint16_t* win_k, uint16_t* win_v, int win_len, int win_cap,
                             bool fold) {
    vqkv::AppendArgs app;
    app.fold = fold;
    app.k_new = k_new;
    app.v_new = v_new;
    app.kv_f32 = kv_dtype == VQ_F32;
    app.append_pos = num_codes;   // marks the extra workgroup; no code is written
    app.win_k = win_k;
    app.win_v = win_v;
    app.win_len = win_len;
    app.win_cap = win_cap;
    return app;
}

}  // namespace
}  // extern "C++"

int32_t vq_decode_step_num_partials(const vq_layout* layout, int32_t batch, int32_t num_q_heads,
                                    int32_t cur_len, int32_t requested) {
    (void)num_q_heads;
    if (layout == nullptr || batch < 1 || cur_len < 0 || layout->num_kv_heads < 1 ||
        requested < 0)
        return 0;
    return plan_step(streams_of(batch, layout->num_kv_heads), cur_len, requested, fold_tokens(layout))
               .num_splits + 1;
}

size_t vq_decode_step_workspace_bytes(const vq_layout* layout, int32_t batch,
                                      int32_t num_q_heads, int32_t cur_len, int32_t requested) {
    const int32_t n = vq_decode_step_num_partials(layout, batch, num_q_heads, cur_len, requested);
    if (n < 1 || num_q_heads < 1) return 0;
    return partials_bytes(batch, num_q_heads, n);
}

int vq_decode_step_partials(const vq_layout* layout, const void* q, int q_dtype,
                            const void* k_new, const void* v_new, int kv_dtype,
                            const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                            uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                            int32_t num_q_heads, int32_t cur_len, int32_t num_partials,
                            float* part_m, float* part_l, float* part_o, void* stream) {
    int st = check_step_args(layout, q, q_dtype, k_new, v_new, kv_dtype, lambda, cb_k, cb_v,
                             codes_k, codes_v, batch, num_q_heads, cur_len, 0);
    if (st) return st;
    if ((st = check_partials_ptrs(part_m, part_l, part_o))) return st;
    const SplitPlan p = plan_step(streams_of(batch, layout->num_kv_heads), cur_len,
                                  num_partials > 1 ? num_partials - 1 : 1, fold_tokens(layout));
    if (num_partials != p.num_splits + 1)
        return fail(VQ_ERR_INVALID_ARG,
                    "num_partials %d is not a planned count for this shape "
                    "(vq_decode_step_num_partials gives %d)",
                    num_partials, p.num_splits + 1);
    const vqkv::Partials part{part_m, part_l, part_o};
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity, cur_len,
                                p.num_splits, p.tokens_per_split};
    return hip_status(vqkv::launch_vq_attention(
                          shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32, lambda, cb_k, cb_v,
                          codes_k, codes_v, part,
                          append_args(k_new, v_new, kv_dtype, cur_len, codes_k, codes_v, p.fold),
                          static_cast<hipStream_t>(stream)),
                      "decode_step_partials launch");
}

int vq_decode_step(const vq_layout* layout, const void* q, int q_dtype, const void* k_new,
                   const void* v_new, int kv_dtype, const float* lambda, const uint16_t* cb_k,
                   const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                   int32_t num_q_heads, int32_t cur_len, int32_t num_splits, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_step_args(layout, q, q_dtype, k_new, v_new, kv_dtype, lambda, cb_k, cb_v,
                             codes_k, codes_v, batch, num_q_heads, cur_len, num_splits);
    if (st) return st;
    VQ_REQUIRE_PTR(out);
    const SplitPlan p = plan_step(streams_of(batch, layout->num_kv_heads), cur_len, num_splits,
                                  fold_tokens(layout));
    const int nparts = p.num_splits + 1;
    const size_t need = partials_bytes(batch, num_q_heads, nparts);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (!aligned16(workspace)) return fail(VQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const vqkv::Partials part = carve_partials(workspace, batch, num_q_heads, nparts);
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity, cur_len,
                                p.num_splits, p.tokens_per_split};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(vqkv::launch_vq_attention(
                        shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32, lambda, cb_k, cb_v,
                        codes_k, codes_v, part,
                        append_args(k_new, v_new, kv_dtype, cur_len, codes_k, codes_v, p.fold), s),
                    "decode_step launch");
    if (st) return st;
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, nparts, part, out, s),
                      "decode_step merge launch");
}

// ---- decode step with no allocation ------------------------------------------
// The split partials of vq_decode_step_noalloc live in this file-scope device
// array (one copy per GPU, held until the process ends).  Host code never
// passes its name to a kernel: the array's device address is resolved once
// per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = VQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (resolved on the
// first call there), or VQ_ERR_HIP.
int scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(VQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(VQ_ERR_HIP, "device %d beyond the %d devices this entry point serves", dev,
                    kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr)
                return fail(VQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return VQ_OK;
}

}  // namespace

int vq_decode_step_noalloc(const vq_layout* layout, const void* q, int q_dtype,
                           const void* k_new, const void* v_new, int kv_dtype,
                           const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                           uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                           int32_t num_q_heads, int32_t cur_len, int32_t num_splits, float* out,
                           void* stream) {
    int st = check_step_args(layout, q, q_dtype, k_new, v_new, kv_dtype, lambda, cb_k, cb_v,
                             codes_k, codes_v, batch, num_q_heads, cur_len, num_splits);
    if (st) return st;
    VQ_REQUIRE_PTR(out);
    const SplitPlan p = plan_step(streams_of(batch, layout->num_kv_heads), cur_len, num_splits,
                                  fold_tokens(layout));
    const int nparts = p.num_splits + 1;
    const size_t need = partials_bytes(batch, num_q_heads, nparts);
    if (need > kScratchBytes)
        return fail(VQ_ERR_WORKSPACE,
                    "the step's partials take %zu bytes, above the %zu-byte static buffer of "
                    "vq_decode_step_noalloc (use vq_decode_step with a workspace)",
                    need, kScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_for_current_device(&ws))) return st;
    const vqkv::Partials part = carve_partials(ws, batch, num_q_heads, nparts);
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity, cur_len,
                                p.num_splits, p.tokens_per_split};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(vqkv::launch_vq_attention(
                        shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32, lambda, cb_k, cb_v,
                        codes_k, codes_v, part,
                        append_args(k_new, v_new, kv_dtype, cur_len, codes_k, codes_v, p.fold), s),
                    "decode_step_noalloc launch");
    if (st) return st;
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, nparts, part, out, s),
                      "decode_step_noalloc merge launch");
}

int32_t vq_decode_step_window_num_partials(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t num_codes,
                                           int32_t requested) {
    (void)num_q_heads;
    if (layout == nullptr || batch < 1 || num_codes < 0 || layout->num_kv_heads < 1 ||
        requested < 0)
        return 0;
    return plan_window_step(streams_of(batch, layout->num_kv_heads), num_codes, requested).num_splits + 1;
}

size_t vq_decode_step_window_workspace_bytes(const vq_layout* layout, int32_t batch,
                                             int32_t num_q_heads, int32_t num_codes,
                                             int32_t requested) {
    const int32_t n =
        vq_decode_step_window_num_partials(layout, batch, num_q_heads, num_codes, requested);
    if (n < 1 || num_q_heads < 1) return 0;
    return partials_bytes(batch, num_q_heads, n);
}

int vq_decode_step_window(const vq_layout* layout, const void* q, int q_dtype, const void* k_new,
                          const void* v_new, int kv_dtype, const float* lambda,
                          const uint16_t* cb_k, const uint16_t* cb_v, const uint8_t* codes_k,
                          const uint8_t* codes_v, uint16_t* win_k, uint16_t* win_v,
                          int32_t win_cap, int32_t batch, int32_t num_q_heads, int32_t num_codes,
                          int32_t win_len, int32_t num_splits, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
    int st = check_window_step_args(layout, q, q_dtype, k_new, v_new, kv_dtype, lambda, cb_k, cb_v,
                                    codes_k, codes_v, win_k, win_v, win_cap, batch, num_q_heads,
                                    num_codes, win_len, num_splits);
    if (st) return st;
    VQ_REQUIRE_PTR(out);
    const SplitPlan p = plan_window_step(streams_of(batch, layout->num_kv_heads), num_codes, num_splits);
    const int nparts = p.num_splits + 1;
    const size_t need = partials_bytes(batch, num_q_heads, nparts);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (!aligned16(workspace)) return fail(VQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const vqkv::Partials part = carve_partials(workspace, batch, num_q_heads, nparts);
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity,
                                num_codes, p.num_splits, p.tokens_per_split};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(vqkv::launch_vq_attention(
                        shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32, lambda, cb_k, cb_v,
                        codes_k, codes_v, part,
                        window_args(k_new, v_new, kv_dtype, num_codes, win_k, win_v, win_len,
                                    win_cap, p.fold),
                        s),
                    "decode_step_window launch");
    if (st) return st;
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, nparts, part, out, s),
                      "decode_step_window merge launch");
}

int vq_flush_window(const vq_layout* layout, const uint16_t* win_k, const uint16_t* win_v,
                    const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                    uint8_t* codes_k, uint8_t* codes_v, int32_t win_cap, int32_t batch,
                    int32_t num_codes, void* stream) {
    if (win_cap < 1) return fail(VQ_ERR_INVALID_ARG, "window capacity %d < 1", win_cap);
    return vq_encode_append(layout, win_k, win_v, VQ_F16, lambda, cb_k, cb_v, codes_k, codes_v,
                            batch, num_codes, win_cap, stream);
}

int vq_decode_attention(const vq_layout* layout, const void* q, int q_dtype, const float* lambda,
                        const uint16_t* cb_k, const uint16_t* cb_v, const uint8_t* codes_k,
                        const uint8_t* codes_v, int32_t batch, int32_t num_q_heads,
                        int32_t context_len, int32_t num_splits, float* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
    int st = check_attention_args(layout, q, q_dtype, lambda, cb_k, cb_v, codes_k, codes_v, batch,
                                  num_q_heads, context_len, num_splits);
    if (st) return st;
    VQ_REQUIRE_PTR(out);
    const SplitPlan p =
        plan_vq(streams_of(batch, layout->num_kv_heads), context_len, num_splits);
    const size_t need = partials_bytes(batch, num_q_heads, p.num_splits);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (!aligned16(workspace)) return fail(VQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const vqkv::Partials part = carve_partials(workspace, batch, num_q_heads, p.num_splits);
    const vqkv::AttnShape shape{batch, num_q_heads, layout->num_kv_heads, layout->capacity,
                                context_len, p.num_splits, p.tokens_per_split};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(vqkv::launch_vq_attention(shape, layout->k_code_bits, layout->sub_dim, q, q_dtype == VQ_F32,
                                              lambda, cb_k, cb_v, codes_k, codes_v, part,
                                              vqkv::AppendArgs{}, s),
                    "decode_attention launch");
    if (st) return st;
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, p.num_splits, part, out, s),
                      "decode_attention merge launch");
}

size_t vq_fp16_attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t context_len, int32_t num_splits) {
    if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || context_len < 1) return 0;
    const SplitPlan p = plan_splits(streams_of(batch, num_kv_heads), context_len, num_splits, vqkv::kFp16Tile,
                                      kTargetWorkgroupsFp16);
    return partials_bytes(batch, num_q_heads, p.num_splits);
}

int vq_fp16_decode_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t capacity, int32_t context_len, int32_t num_splits,
                             float* out, void* workspace, size_t workspace_bytes, void* stream) {
    if (num_kv_heads < 1 || num_kv_heads > 65535)
        return fail(VQ_ERR_INVALID_ARG, "num_kv_heads %d out of range [1, 65535]", num_kv_heads);
    int st = check_heads(batch, num_q_heads, num_kv_heads);
    if (st) return st;
    if (capacity < 1) return fail(VQ_ERR_INVALID_ARG, "capacity %d < 1", capacity);
    if (context_len < 1)
        return fail(VQ_ERR_INVALID_ARG, "context_len %d < 1 (softmax over no tokens)", context_len);
    if (context_len > capacity)
        return fail(VQ_ERR_CAPACITY, "context_len %d exceeds capacity %d", context_len, capacity);
    if (num_splits < 0) return fail(VQ_ERR_INVALID_ARG, "num_splits %d < 0", num_splits);
    VQ_REQUIRE_PTR(q);
    VQ_REQUIRE_PTR(k);
    VQ_REQUIRE_PTR(v);
    VQ_REQUIRE_PTR(out);
    const SplitPlan p = plan_splits(streams_of(batch, num_kv_heads), context_len, num_splits, vqkv::kFp16Tile,
                                      kTargetWorkgroupsFp16);
    const size_t need = partials_bytes(batch, num_q_heads, p.num_splits);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (!aligned16(workspace)) return fail(VQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const vqkv::Partials part = carve_partials(workspace, batch, num_q_heads, p.num_splits);
    const vqkv::AttnShape shape{batch, num_q_heads, num_kv_heads, capacity, context_len,
                                p.num_splits, p.tokens_per_split};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(vqkv::launch_fp16_attention_splits(shape, q, k, v, part, s),
                    "fp16 attention split launch");
    if (st) return st;
    return hip_status(vqkv::launch_merge_partials(batch, num_q_heads, p.num_splits, part, out, s),
                      "fp16 attention merge launch");
}

// ---------------------------------------------------------------------------
// offline calibration
// ---------------------------------------------------------------------------

extern "C++" {  // validation helpers: not part of the C ABI
namespace {

int check_calib_keys(const void* keys, int kv_dtype, int32_t num_kv_heads, int32_t num_tokens) {
    if (kv_dtype != VQ_F16 && kv_dtype != VQ_F32)
        return fail(VQ_ERR_INVALID_ARG, "kv_dtype %d is not VQ_F16 or VQ_F32", kv_dtype);
    if (num_kv_heads < 1 || num_kv_heads > 65535)
        return fail(VQ_ERR_INVALID_ARG, "num_kv_heads %d out of range [1, 65535]", num_kv_heads);
    if (num_tokens < 1) return fail(VQ_ERR_INVALID_ARG, "num_tokens %d < 1", num_tokens);
    VQ_REQUIRE_PTR(keys);
    return VQ_OK;
}

constexpr int32_t kMaxKmeansSamples = 1 << 28;
constexpr int32_t kMaxKmeansIters = 10000;

int check_kmeans_shape(int32_t num_sets, int32_t num_samples, int32_t sub_dim, int32_t code_bits) {
    if (num_sets < 1 || num_sets > 65535)
        return fail(VQ_ERR_INVALID_ARG, "num_sets %d out of range [1, 65535]", num_sets);
    if (num_samples < 1 || num_samples > kMaxKmeansSamples)
        return fail(VQ_ERR_INVALID_ARG, "num_samples %d out of range [1, %d]", num_samples,
                    kMaxKmeansSamples);
    if (sub_dim != 4 && sub_dim != 8)
        return fail(VQ_ERR_UNSUPPORTED, "sub_dim %d unsupported (4 or 8)", sub_dim);
    if (code_bits != 8 && code_bits != 12)
        return fail(VQ_ERR_UNSUPPORTED, "code_bits %d unsupported (8 or 12)", code_bits);
    return VQ_OK;
}

}  // namespace
}  // extern "C++"

int vq_calibrate_lambda(const void* keys, int kv_dtype, int32_t num_kv_heads, int32_t num_tokens,
                        float* lambda, void* stream) {
    int st = check_calib_keys(keys, kv_dtype, num_kv_heads, num_tokens);
    if (st) return st;
    VQ_REQUIRE_PTR(lambda);
    return hip_status(vqkv::launch_calibrate_lambda(keys, kv_dtype == VQ_F32, num_kv_heads,
                                                    num_tokens, lambda,
                                                    static_cast<hipStream_t>(stream)),
                      "calibrate_lambda launch");
}

int vq_transform_keys(const void* keys, int kv_dtype, const float* lambda, int32_t num_kv_heads,
                      int32_t num_tokens, float* keys_tilde, void* stream) {
    int st = check_calib_keys(keys, kv_dtype, num_kv_heads, num_tokens);
    if (st) return st;
    VQ_REQUIRE_PTR(lambda);
    VQ_REQUIRE_PTR(keys_tilde);
    return hip_status(vqkv::launch_transform_keys(keys, kv_dtype == VQ_F32, lambda, num_kv_heads,
                                                  num_tokens, keys_tilde,
                                                  static_cast<hipStream_t>(stream)),
                      "transform_keys launch");
}

size_t vq_kmeans_workspace_bytes(int32_t num_sets, int32_t num_samples, int32_t sub_dim,
                                 int32_t code_bits) {
    if (num_sets < 1 || num_sets > 65535 || num_samples < 1 || num_samples > kMaxKmeansSamples ||
        (sub_dim != 4 && sub_dim != 8) || (code_bits != 8 && code_bits != 12))
        return 0;
    return vqkv::kmeans_workspace_bytes(num_sets, num_samples, sub_dim, code_bits);
}

int vq_kmeans(const float* samples, int32_t num_sets, int32_t num_samples, int32_t sub_dim,
              int32_t code_bits, const double* init, int32_t iters, double* centroids,
              uint16_t* codebook, int32_t* assign, void* workspace, size_t workspace_bytes,
              void* stream) {
    int st = check_kmeans_shape(num_sets, num_samples, sub_dim, code_bits);
    if (st) return st;
    if (iters < 0 || iters > kMaxKmeansIters)
        return fail(VQ_ERR_INVALID_ARG, "iters %d out of range [0, %d]", iters, kMaxKmeansIters);
    VQ_REQUIRE_PTR(samples);
    VQ_REQUIRE_PTR(init);
    VQ_REQUIRE_PTR(centroids);
    if (codebook != nullptr && !aligned16(codebook))
        return fail(VQ_ERR_INVALID_ARG, "codebook is not 16-byte aligned");
    if (assign != nullptr && !aligned16(assign))
        return fail(VQ_ERR_INVALID_ARG, "assign is not 16-byte aligned");
    const size_t need = vqkv::kmeans_workspace_bytes(num_sets, num_samples, sub_dim, code_bits);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (!aligned16(workspace)) return fail(VQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    return hip_status(vqkv::launch_kmeans(samples, num_sets, num_samples, sub_dim, code_bits, init, iters,
                                          centroids, codebook, assign, workspace,
                                          static_cast<hipStream_t>(stream)),
                      "kmeans launch");
}

}  // extern "C"
