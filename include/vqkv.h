/*
 * vqkv.h — C ABI of libvqkv.so: single-query decode attention computed
 * directly over a vector-quantised low-bit KV cache on AMD MI355X (gfx950).
 *
 * The method is VecInfer's ("VecInfer: Efficient LLM Inference With Low-Bit
 * KV Cache via Outlier-Suppressed Vector Quantization", notes page):
 *   - keys are smoothed per channel and Walsh–Hadamard transformed,
 *       K~ = K diag(lambda)^-1 H_D            (Method details)
 *     then stored as vector-quantisation codes: every d (4 or 8) consecutive
 *     channels (a sub-vector) is replaced by the index of its nearest
 *     codebook centroid                      (Background, VQ principle);
 *   - values are quantised the same way without any transform;
 *   - the query is transformed as q~ = q diag(lambda) H_D, so that
 *     q~ K~^T = q K^T                        (Method details, score rewrite);
 *   - attention is s = q~ VQ^-1(K~_q)^T / sqrt(D), p = softmax(s),
 *     o = p VQ^-1(V_q)                       (Method details, VQ KV cache in
 *                                             attention)
 *     and the codes are never dequantised to memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers allocated and owned by the
 *    caller.  The library allocates no device memory; split partials live in
 *    a caller-provided workspace or caller-provided arrays, except those of
 *    vq_decode_step_noalloc, which go to one static 4 MiB device array per
 *    GPU inside the library.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream and returns without
 *    synchronising.  Faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; the
 *    validation never dereferences a pointer.  On failure the call returns a
 *    non-zero vq_status, enqueues nothing and leaves a message for
 *    vq_last_error().  No C++ exception crosses this interface.
 *  - D = 128 only.  Two sub-vector layouts (VQ_ERR_UNSUPPORTED otherwise):
 *      d = 4: 32 sub-vectors per vector, k_code_bits 8 or 12, v_code_bits 8
 *             (the VecInfer page's 2-bit choice, 2^8 x 4 x 2 B codebooks);
 *      d = 8: 16 sub-vectors per vector, k_code_bits = v_code_bits = 12 (the
 *             page's 1.5-bit choice, 2^12 x 8 x 2 B codebooks; Results,
 *             codebook-size ablation).
 *  - Layouts (row-major, innermost last; B batch, Hq query heads, Hkv KV
 *    heads, G = Hq / Hkv, P = D / d sub-vectors (32 or 16), cap = capacity):
 *      q        [B][Hq][128]            fp16 or fp32 (q_dtype)
 *      lambda   [Hkv][128]              fp32, finite and > 0 (caller contract)
 *      cb_k     [Hkv][2^k_code_bits][d] fp16 (bit patterns as uint16)
 *      cb_v     [Hkv][2^v_code_bits][d] fp16
 *      codes_k  [B][Hkv][cap][P*k_code_bits/8] uint8 — token-major code rows
 *               (P = 128 / d): 8-bit codes are one byte per sub-vector;
 *               12-bit codes are a little-endian bit stream, code i in bits
 *               [12i, 12i+12) of the row (48 bytes at d = 4, 24 at d = 8).
 *      codes_v  [B][Hkv][cap][P*v_code_bits/8] uint8
 *      out      [B][Hq][128]            fp32
 *    Query head h reads KV head h / G.  One codebook and one lambda per KV
 *    head, shared by every sub-vector position and every sequence.
 *  - Base pointers of codes, codebooks, q, lambda and out must be 16-byte
 *    aligned (VQ_ERR_INVALID_ARG otherwise).
 *  - Numerics of the attention entry points: q~ is formed in fp32 (so q,
 *    lambda and q~ must be finite in fp32; nothing else bounds their
 *    range), then scaled per head by a power of two and split into two
 *    fp16 parts for the matrix cores; dequantised keys and values are the
 *    fp16 codebook entries themselves; scores, the online softmax and every
 *    accumulation are fp32, and the weights 2^(s - m) enter the value
 *    product as two fp16 parts within 2^-20 p + 2^-40 of p (m the running
 *    maximum).  A base-2 score log2(e) s then carries an absolute error of
 *    about 2^-22 times the sum of |q~_i k^_i| / sqrt(128), so weights stay
 *    accurate to ~1e-4 while that sum is below a few hundred units and the
 *    argmax stays exact far beyond (the tests cover scores near +-656 units
 *    and a one-hot softmax at ~1e12 units).
 */
#ifndef VQKV_H
#define VQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VQ_OK = 0,
    VQ_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad alignment, Hq % Hkv != 0 */
    VQ_ERR_UNSUPPORTED = 2,   /* geometry the kernels do not implement */
    VQ_ERR_CAPACITY = 3,      /* tokens beyond the cache capacity */
    VQ_ERR_WORKSPACE = 4,     /* workspace missing or too small */
    VQ_ERR_HIP = 5            /* a HIP runtime or launch error */
} vq_status;

typedef enum { VQ_F16 = 0, VQ_F32 = 1 } vq_dtype;

/*
 * Deterministic mode, for the whole library (all devices and threads):
 * with on != 0 the split kernel hands its 32-token tiles to its 16 waves in
 * a fixed order (wave w takes tiles w, w + 16, ...) instead of as waves
 * become free, so repeated calls with the same inputs and split plan give
 * bit-identical outputs and partials; the encoders, the merge and the
 * calibration kernels are deterministic in either mode.  About 2-3% slower
 * at the 196608-token Llama-3.1-8B layer (measured on MI355X).  Applies to
 * calls made after it returns.  Returns the previous setting (0 or 1).
 */
int vq_set_deterministic(int on);

/*
 * Score method of the attention entry points, for the whole library:
 *   VQ_SCORES_MFMA (default): the query's two fp16 parts times the
 *     dequantised keys on the matrix cores (the key table read as MFMA
 *     operands);
 *   VQ_SCORES_LUT: the VecInfer page's lookup table (Appendix, Algorithm 1:
 *     the table of q~ against C_k, then every score a sum of its entries):
 *     each workgroup first fills LUT[pos][code] = q~[4 pos .. 4 pos + 3] .
 *     C_k[code] for its query heads in fp32, then each score is the sum of
 *     32 entries, one per sub-vector position.  Only 8-bit keys with 4-dim
 *     sub-vectors and G <= 4; other layouts keep the matrix-core scores.
 *     The LUT takes 128 KiB of LDS, so the value table has 4 copies instead
 *     of 32 (bank conflicts in its reads).  Slower on MI355X; it exists to
 *     measure the pages' design against the default.
 * Applies to calls made after it returns.  Returns the previous method, or
 * -1 (VQ_ERR_INVALID_ARG in vq_last_error) for an unknown one.
 */
typedef enum { VQ_SCORES_MFMA = 0, VQ_SCORES_LUT = 1 } vq_score_method;
int vq_set_score_method(int method);

/* Cache geometry, plain data, passed by pointer. */
typedef struct {
    int32_t head_dim;      /* D: must be 128                          */
    int32_t sub_dim;       /* d: 4 or 8                               */
    int32_t k_code_bits;   /* log2 |C_k|: 8 or 12 (d = 4), 12 (d = 8)  */
    int32_t v_code_bits;   /* log2 |C_v|: 8 (d = 4), 12 (d = 8)        */
    int32_t num_kv_heads;  /* Hkv >= 1                                */
    int32_t capacity;      /* token slots per (sequence, KV head) >= 1 */
} vq_layout;

/*
 * q~ = q diag(lambda) H_128 for every (sequence, query head).
 * VecInfer page, Method details: smooth factors and the Walsh–Hadamard
 * recursion H_{2^k} = (1/sqrt 2)[[H, H], [H, -H]]; the query side of the
 * attention-score rewrite.  H is the orthonormal Sylvester matrix in natural
 * order.
 *   q        [B][Hq][128] in q_dtype;   lambda [Hkv][128] fp32
 *   q_tilde  [B][Hq][128] fp32 output
 */
int vq_transform_query(const vq_layout* layout, const void* q, int q_dtype,
                       const float* lambda, int32_t batch, int32_t num_q_heads,
                       float* q_tilde, void* stream);

/*
 * Quantise `num_new` new tokens per (sequence, KV head) and store their codes
 * at token slots [cur_len, cur_len + num_new) of the cache.
 * VecInfer page, Method details (VQ KV cache in attention): each new key gets
 * the online dual transform k~ = k diag(lambda)^-1 H_D and is quantised with
 * C_k; the value is quantised as is with C_v; codes are concatenated to the
 * cache.  Background (VQ principle): j* = argmin_j ||x_i - C_j||^2.
 * The transform and the distances are evaluated in fp64; exact distance ties
 * go to the lowest centroid index.
 *   k_new, v_new [B][Hkv][num_new][128] in kv_dtype (fp16 or fp32)
 *   codes_k / codes_v: written at the slots above, nothing else is touched.
 * Errors: VQ_ERR_CAPACITY if cur_len + num_new > capacity; VQ_ERR_INVALID_ARG
 * if cur_len < 0 or num_new < 0.  num_new = 0 is a no-op that returns VQ_OK.
 * The caller tracks the cache length; the call mutates no length.
 */
int vq_encode_append(const vq_layout* layout, const void* k_new, const void* v_new,
                     int kv_dtype, const float* lambda, const uint16_t* cb_k,
                     const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v,
                     int32_t batch, int32_t cur_len, int32_t num_new, void* stream);

/*
 * Split count vq_decode_attention uses for this shape when num_splits = 0,
 * and the workspace it needs for a given split count (0 = the default).
 */
int32_t vq_decode_attention_default_splits(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t context_len);
size_t vq_decode_attention_workspace_bytes(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t context_len,
                                           int32_t num_splits);

/*
 * Decode attention of one query per (sequence, query head) over the first
 * `context_len` tokens of the VQ cache, without dequantising it to memory.
 * VecInfer page, Method details (VQ KV cache in attention) for what is
 * computed; Appendix (FlashAttention block recurrence and Algorithm 1) for
 * the blockwise online softmax.  The context is split into `num_splits`
 * contiguous ranges processed in parallel, and their partial results are
 * merged by log-sum-exp (0 = library default; larger requests are clamped
 * so that no split is empty, smaller ones raised so that no split holds more
 * than 24576 tokens while 512 splits allow it: fp32 accumulation over longer
 * splits loses accuracy behind a dominant token).
 *   q [B][Hq][128] in q_dtype (raw query: the transform happens inside)
 *   out [B][Hq][128] fp32
 *   workspace: device memory of at least
 *              vq_decode_attention_workspace_bytes(...) bytes, any contents;
 *              it holds the split partials until the merge has read them, so
 *              calls that run concurrently must not share a workspace.
 * Errors: VQ_ERR_CAPACITY if context_len > capacity; VQ_ERR_INVALID_ARG if
 * context_len < 1 (softmax over an empty set) or Hq % Hkv != 0;
 * VQ_ERR_UNSUPPORTED if G > 8; VQ_ERR_WORKSPACE if the workspace is too small.
 * Tiles are scheduled dynamically inside a split, so repeated calls agree to
 * fp32 rounding, not bit for bit, unless deterministic mode is on
 * (vq_set_deterministic).
 */
int vq_decode_attention(const vq_layout* layout, const void* q, int q_dtype,
                        const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                        const uint8_t* codes_k, const uint8_t* codes_v, int32_t batch,
                        int32_t num_q_heads, int32_t context_len, int32_t num_splits,
                        float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of vq_decode_attention, for callers that place the split
 * partials themselves, e.g. to merge partials of context shards held by
 * different devices.
 *
 * vq_decode_attention_plan_splits: the split count the library uses for
 * `requested` splits (0 = its default; clamped as vq_decode_attention
 * clamps it).  Returns 0 for invalid arguments.
 *
 * vq_decode_attention_partials: the split pass alone.  Split s of
 * (sequence b, query head h) covers tokens [s T, min((s + 1) T, context_len))
 * for a T fixed by the plan, and leaves, in base-2 units with
 * x_t = log2(e) (q~ . k^_t) / sqrt(128):
 *     part_m[b][h][s]     a reference value m (>= -inf)
 *     part_l[b][h][s]     l = sum_t 2^(x_t - m)
 *     part_o[b][h][s][:]  o = sum_t 2^(x_t - m) v^_t          (all fp32)
 * i.e. one block of the FlashAttention recurrence (VecInfer page,
 * Appendix).  num_splits must be a value vq_decode_attention_plan_splits
 * returns for this shape (VQ_ERR_INVALID_ARG otherwise).  part_m and
 * part_l hold B * Hq * num_splits floats, part_o 128 times as many.
 * Other arguments and errors as for vq_decode_attention.
 *
 * vq_merge_partials: out[b][h][:] = sum_s w_s o_s / sum_s w_s l_s with
 * w_s = 2^(m_s - max_s m_s), over the num_partials (1 .. 512) partials of
 * each (sequence, query head) laid out as above; a partial with m = -inf
 * weighs 0.  Partials of disjoint token sets may come from different calls
 * or devices: the merge is the softmax over their union.
 */
int32_t vq_decode_attention_plan_splits(const vq_layout* layout, int32_t batch,
                                        int32_t num_q_heads, int32_t context_len,
                                        int32_t requested);
int vq_decode_attention_partials(const vq_layout* layout, const void* q, int q_dtype,
                                 const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                                 const uint8_t* codes_k, const uint8_t* codes_v, int32_t batch,
                                 int32_t num_q_heads, int32_t context_len, int32_t num_splits,
                                 float* part_m, float* part_l, float* part_o, void* stream);
int vq_merge_partials(int32_t batch, int32_t num_q_heads, int32_t num_partials,
                      const float* part_m, const float* part_l, const float* part_o, float* out,
                      void* stream);

/*
 * One decode step: encode the new token of every (sequence, KV head) into
 * slot cur_len of the cache, then decode attention over the first
 * cur_len + 1 tokens — one launch of the split kernel plus the merge.
 * The results equal vq_encode_append(..., cur_len, num_new = 1, ...)
 * followed by vq_decode_attention(..., context_len = cur_len + 1, ...):
 * identical codes, outputs equal to fp32 rounding.
 * VecInfer page, Method details (VQ KV cache in attention): each newly
 * arrived key takes the online dual transform and is quantised with C_k,
 * the value with C_v, both are concatenated to the cache, and the query
 * attends over the updated cache.
 * Inside the launch, the new token of every (sequence, KV head) is encoded
 * (fp64 decisions, ties to the lowest index, as vq_encode_append) and leaves
 * that token's own partial, either in one extra workgroup per (sequence, KV
 * head) or, with many streams and long splits, at the start of each stream's
 * last split; the splits attend over the cur_len cached tokens in num_splits
 * splits (0 = library default).  The library chooses between the two; the
 * results are the same.
 *   k_new, v_new [B][Hkv][128] in kv_dtype (fp16 or fp32)
 *   codes_k / codes_v: read over [0, cur_len), written at slot cur_len only.
 *   workspace: at least vq_decode_step_workspace_bytes(...) bytes, any
 *   contents; not shared by calls that run concurrently.
 * Errors: VQ_ERR_CAPACITY if cur_len + 1 > capacity; VQ_ERR_INVALID_ARG if
 * cur_len < 0; otherwise as for vq_encode_append and vq_decode_attention.
 *
 * vq_decode_step_num_partials: the partial count of a step (attention
 * splits + 1) for `requested` splits (0 = default); 0 for invalid arguments.
 * vq_decode_step_partials: the split pass alone, leaving num_partials
 * partials per (sequence, query head) as vq_decode_attention_partials does
 * (the last one is the new token's); num_partials must be a value
 * vq_decode_step_num_partials returns for this shape.  vq_merge_partials
 * completes it.
 */
int32_t vq_decode_step_num_partials(const vq_layout* layout, int32_t batch, int32_t num_q_heads,
                                    int32_t cur_len, int32_t requested);
size_t vq_decode_step_workspace_bytes(const vq_layout* layout, int32_t batch,
                                      int32_t num_q_heads, int32_t cur_len, int32_t requested);
int vq_decode_step(const vq_layout* layout, const void* q, int q_dtype, const void* k_new,
                   const void* v_new, int kv_dtype, const float* lambda, const uint16_t* cb_k,
                   const uint16_t* cb_v, uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                   int32_t num_q_heads, int32_t cur_len, int32_t num_splits, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);
int vq_decode_step_partials(const vq_layout* layout, const void* q, int q_dtype,
                            const void* k_new, const void* v_new, int kv_dtype,
                            const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                            uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                            int32_t num_q_heads, int32_t cur_len, int32_t num_partials,
                            float* part_m, float* part_l, float* part_o, void* stream);

/*
 * vq_decode_step_noalloc: vq_decode_step for callers that cannot allocate
 * device memory or pass a workspace — code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, codes
 * and results as vq_decode_step minus the workspace: the split partials go
 * to a static device buffer of VQ_NOALLOC_SCRATCH_BYTES (4 MiB) inside the
 * library, one per GPU, held until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *  - Limit: the step's partials, vq_decode_step_workspace_bytes(...) for the
 *    same shape and num_splits, must fit the buffer (VQ_ERR_WORKSPACE
 *    otherwise, before anything is enqueued): e.g. B * Hq * partials up to
 *    about 8000 at the default plans (a 32-query-head layer at B = 16:
 *    0.8 MB).
 *  - The buffer is the current device's: `stream` must belong to it.  The
 *    first call on a device resolves the buffer's address
 *    (hipGetSymbolAddress); make one call before capturing a graph.
 *  - Every call on a GPU shares that GPU's buffer: calls that may overlap on
 *    one GPU (other streams, other threads) race and must be serialised by
 *    the caller.  Each call writes every partial it reads, so the buffer's
 *    contents from an earlier call never matter.
 * Errors as vq_decode_step, plus VQ_ERR_HIP if the buffer's address cannot
 * be resolved.
 */
#define VQ_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int vq_decode_step_noalloc(const vq_layout* layout, const void* q, int q_dtype,
                           const void* k_new, const void* v_new, int kv_dtype,
                           const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                           uint8_t* codes_k, uint8_t* codes_v, int32_t batch,
                           int32_t num_q_heads, int32_t cur_len, int32_t num_splits, float* out,
                           void* stream);

/*
 * Decode step with a full-precision residual window: the most recent tokens
 * of every (sequence, KV head) stay in fp16 beside the VQ cache and enter
 * the same softmax.  VecInfer page, Experiments (every method keeps a
 * residual of 128 full-precision tokens); HACK page (the last, not yet full
 * block stays in fp16 and is multiplied in fp16 within the attention, and
 * is quantised when it fills).
 * The new token of every (sequence, KV head), rounded to fp16 (round to
 * nearest even), is written to window slot win_len; then decode attention
 * runs over the coded tokens [0, num_codes) and the window slots
 * [0, win_len] in one softmax.  Window keys are raw (untransformed): a raw
 * key k scores q . k / sqrt(D), which is q~ . k~ / sqrt(D).  One launch of
 * the split kernel plus the merge; the window is attended over by one extra
 * workgroup per (sequence, KV head) or, from 128 streams with long splits,
 * at the start of each stream's last split (the library chooses; the
 * results are the same).
 *   win_k, win_v [B][Hkv][win_cap][128] fp16, caller-owned; slots
 *   [0, win_len) are read, slot win_len is written.
 *   codes_k / codes_v: read over [0, num_codes) only (num_codes may be 0).
 *   workspace: at least vq_decode_step_window_workspace_bytes(...) bytes.
 * The caller keeps win_len (it grows by one per step).  When the window is
 * full (win_len == win_cap) the next step returns VQ_ERR_CAPACITY: call
 * vq_flush_window first.
 * Errors: VQ_ERR_CAPACITY if num_codes > capacity or win_len >= win_cap;
 * VQ_ERR_INVALID_ARG for negative lengths, win_cap < 1, null or misaligned
 * window pointers; otherwise as for vq_decode_step.
 *
 * vq_flush_window: encode the win_cap window tokens into code slots
 * [num_codes, num_codes + win_cap) — exactly vq_encode_append over the
 * window as fp16 rows (same codes, ties to the lowest index).  Afterwards
 * the caller's num_codes grows by win_cap and win_len restarts at 0.
 * Errors as for vq_encode_append (VQ_ERR_CAPACITY if the codes overflow).
 */
int32_t vq_decode_step_window_num_partials(const vq_layout* layout, int32_t batch,
                                           int32_t num_q_heads, int32_t num_codes,
                                           int32_t requested);
size_t vq_decode_step_window_workspace_bytes(const vq_layout* layout, int32_t batch,
                                             int32_t num_q_heads, int32_t num_codes,
                                             int32_t requested);
int vq_decode_step_window(const vq_layout* layout, const void* q, int q_dtype, const void* k_new,
                          const void* v_new, int kv_dtype, const float* lambda,
                          const uint16_t* cb_k, const uint16_t* cb_v, const uint8_t* codes_k,
                          const uint8_t* codes_v, uint16_t* win_k, uint16_t* win_v,
                          int32_t win_cap, int32_t batch, int32_t num_q_heads, int32_t num_codes,
                          int32_t win_len, int32_t num_splits, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);
int vq_flush_window(const vq_layout* layout, const uint16_t* win_k, const uint16_t* win_v,
                    const float* lambda, const uint16_t* cb_k, const uint16_t* cb_v,
                    uint8_t* codes_k, uint8_t* codes_v, int32_t win_cap, int32_t batch,
                    int32_t num_codes, void* stream);

/*
 * Offline calibration (prefill side)
 * ----------------------------------
 * VecInfer page, Method details: the smoothing factors are precomputed
 * offline from calibration keys, lambda_i = sqrt(max_t |K[t, i]|), and the
 * codebooks are pretrained offline with K-Means, C_k on the transformed keys
 * K~ = K diag(lambda)^-1 H_D and C_v on the values as they are, split into
 * d-channel sub-vectors; Experimental setup: at most 30 K-Means iterations.
 * Calibration keys are [Hkv][T][128] in kv_dtype (one stream of T tokens per
 * KV head; several calibration sequences are concatenated by the caller).
 */

/*
 * lambda[g][i] = sqrt(max_t |keys[g][t][i]|), the square root taken in fp64
 * and rounded once to fp32.  An all-zero channel gives lambda 0, which the
 * attention entry points do not accept: the caller must replace it.
 *   keys    [Hkv][T][128] fp16 or fp32;  lambda [Hkv][128] fp32 output.
 * Errors: VQ_ERR_INVALID_ARG for num_kv_heads outside [1, 65535],
 * num_tokens < 1, a NULL or misaligned pointer.
 */
int vq_calibrate_lambda(const void* keys, int kv_dtype, int32_t num_kv_heads,
                        int32_t num_tokens, float* lambda, void* stream);

/*
 * Transformed calibration keys K~ = K diag(lambda)^-1 H_128 (the key side of
 * the transform), computed in fp64 and rounded once to fp32.  Viewed as
 * [Hkv][T * 32][4], they are the K-Means samples for C_k.
 *   keys [Hkv][T][128] fp16 or fp32; lambda [Hkv][128] fp32 (> 0);
 *   keys_tilde [Hkv][T][128] fp32 output.
 */
int vq_transform_keys(const void* keys, int kv_dtype, const float* lambda,
                      int32_t num_kv_heads, int32_t num_tokens, float* keys_tilde,
                      void* stream);

/*
 * Lloyd K-Means for num_sets independent codebooks of 2^code_bits centroids
 * of dimension d = sub_dim (4 or 8), `iters` iterations from `init`.  One
 * iteration assigns every sample to its nearest centroid, by the fp64 squared
 * distance summed channel by channel (every difference, square and sum
 * rounded once), exact ties to the lowest index; then moves every centroid
 * that received samples to their mean (the samples summed in fp64 in sample
 * order, divided once by their count); a centroid with no samples keeps its
 * place.  The result is identical, bit for bit, to that definition evaluated
 * sequentially.
 *   samples   [num_sets][num_samples][d] fp32, finite, |x| < 2^60
 *   init      [num_sets][2^code_bits][d] fp64, finite, |c| < 2^60
 *   centroids [num_sets][2^code_bits][d] fp64 output (may be init itself)
 *   codebook  [num_sets][2^code_bits][d] fp16 output, or NULL: the
 *             centroids rounded once to nearest even
 *   assign    [num_sets][num_samples] int32 output, or NULL: each sample's
 *             nearest centroid among the returned ones (its code)
 *   workspace vq_kmeans_workspace_bytes(...) bytes, 16-byte aligned; its
 *             contents do not matter.
 * sub_dim 4 or 8 and code_bits 8 or 12 (VQ_ERR_UNSUPPORTED otherwise);
 * num_samples in [1, 2^28]; iters in [0, 10000] (0 copies init and only fills
 * the outputs).  vq_kmeans_workspace_bytes returns 0 for an invalid shape.
 */
size_t vq_kmeans_workspace_bytes(int32_t num_sets, int32_t num_samples, int32_t sub_dim,
                                 int32_t code_bits);
int vq_kmeans(const float* samples, int32_t num_sets, int32_t num_samples, int32_t sub_dim,
              int32_t code_bits, const double* init, int32_t iters, double* centroids,
              uint16_t* codebook, int32_t* assign, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Uncompressed comparator: the same decode attention over an fp16 cache,
 * o = softmax(q K^T / sqrt(128)) V with fp32 accumulation (VecInfer page,
 * Background, KV cache and attention).  No transform, no quantisation.
 *   q [B][Hq][128] fp16; k, v [B][Hkv][capacity][128] fp16; out fp32.
 */
size_t vq_fp16_attention_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t context_len,
                                         int32_t num_splits);
int vq_fp16_decode_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t capacity, int32_t context_len, int32_t num_splits,
                             float* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Static description of a vq_status value. */
const char* vq_status_string(int status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* vq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VQKV_H */
