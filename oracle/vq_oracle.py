"""Plain, slow, fp64 CPU oracle for VQ-KV decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark.  It shares no code, table or helper
with the HIP library and imports nothing from it.

Sources (the pages are cited by title and section):
  [VecInfer]  "VecInfer: Efficient LLM Inference With Low-Bit KV Cache via
              Outlier-Suppressed Vector Quantization" (ACL 2026 notes page).
  [CommVQ]    "CommVQ: Commutative Vector Quantization for KV Cache
              Compression" (ICML 2025 notes page).

What the hot path computes is exact once the codes are fixed: attention
over the dequantised cache.  So this oracle is that definition written
out — dequantise by table lookup, transform the query, textbook softmax
attention in float64 — with no blocking, splitting or fusion.

Readings of points the pages leave open:
  * H_D is the orthonormal Sylvester matrix (1/sqrt(2) per recursion
    level), natural order, no random signs.
  * One lambda in R^128 and one codebook per KV head per tensor, shared by
    every sub-vector position and every sequence.
  * Query head h reads KV head h // G.
  * 12-bit codes are a little-endian bit stream: code i of a token row
    occupies bits [12 i, 12 i + 12).
  * Exact distance ties go to the lowest centroid index.

Pins (tests/test_oracle_pins.py) tie every function here to something
other than itself: closed forms, library routines (scipy's Hadamard and
nearest-code assignment, torch's fp64 scaled-dot-product attention,
scikit-learn's Lloyd), invariants the pages state, hand-worked byte
layouts and the byte counts the pages print.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sylvester_hadamard", "smooth_factors", "transform_keys", "transform_query",
    "vq_assign", "vq_encode", "vq_decode", "pack_codes", "unpack_codes",
    "softmax_attention", "decode_attention", "decode_attention_head",
    "encode_append", "decode_attention_window_head", "decode_attention_window",
    "lloyd_kmeans", "codebook_bytes", "index_bytes",
    "commvq_reduction_ratio",
]


# ---------------------------------------------------------------------------
# transforms — [VecInfer] Method details, "outlier-suppressed vector
# quantisation" (smooth factors, Walsh–Hadamard recursion) and "Hadamard
# lemma and attention-score rewrite".
# ---------------------------------------------------------------------------

def sylvester_hadamard(dim: int) -> np.ndarray:
    """H_D by the recursion H_{2^k} = (1/sqrt 2) [[H, H], [H, -H]], H_1 = [1].

    [VecInfer] Method details: the orthogonal Walsh–Hadamard matrix with
    H_D H_D^T = I; entries are +-1/sqrt(D) (Appendix, proof of the lemma).
    """
    if dim < 1 or dim & (dim - 1):
        raise ValueError("Hadamard size must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < dim:
        h = np.block([[h, h], [h, -h]]) / np.sqrt(2.0)
    return h


def smooth_factors(keys: np.ndarray) -> np.ndarray:
    """lambda_i = sqrt(max_t |K[t, i]|) per channel i.

    [VecInfer] Method details: smoothing factors precomputed offline from
    calibration keys.  ``keys`` is [tokens, D]; returns float64 [D].
    """
    return np.sqrt(np.max(np.abs(np.asarray(keys, dtype=np.float64)), axis=0))


def transform_keys(keys: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """K~ = K diag(lambda)^-1 H_D  (rows are tokens).

    [VecInfer] Method details: smoothing divides the keys by lambda per
    channel, then both sides are multiplied by H_D.
    """
    k = np.asarray(keys, dtype=np.float64)
    h = sylvester_hadamard(k.shape[-1])
    return (k / np.asarray(lam, dtype=np.float64)) @ h


def transform_query(q: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """q~ = q diag(lambda) H_D.

    [VecInfer] Method details, attention-score rewrite:
    s = (q diag(lambda) H_D)(K diag(lambda)^-1 H_D)^T = q K^T.
    """
    x = np.asarray(q, dtype=np.float64)
    h = sylvester_hadamard(x.shape[-1])
    return (x * np.asarray(lam, dtype=np.float64)) @ h


# ---------------------------------------------------------------------------
# vector quantisation — [VecInfer] Background, "vector quantisation
# principle": split x in R^{d_h} into d_h/d sub-vectors and store for each
# the index j* = argmin_j ||x_i - C_j||^2 of its nearest centroid.
# ---------------------------------------------------------------------------

def vq_assign(sub: np.ndarray, codebook: np.ndarray, chunk: int = 4096):
    """Nearest centroid of each row of ``sub`` [n, d] in ``codebook`` [m, d].

    The squared distance is summed dimension by dimension in float64, exactly
    as written on the page.  Exact ties go to the lowest index (np.argmin
    returns the first minimum).  Returns (codes int64 [n], best distance
    [n], runner-up distance minus best distance [n]).
    """
    sub = np.asarray(sub, dtype=np.float64)
    cb = np.asarray(codebook, dtype=np.float64)
    n = sub.shape[0]
    codes = np.empty(n, dtype=np.int64)
    best = np.empty(n, dtype=np.float64)
    gap = np.empty(n, dtype=np.float64)
    for lo in range(0, n, chunk):
        x = sub[lo:lo + chunk]
        dist = np.zeros((x.shape[0], cb.shape[0]), dtype=np.float64)
        for i in range(cb.shape[1]):
            diff = x[:, i:i + 1] - cb[None, :, i]
            dist += diff * diff
        j = np.argmin(dist, axis=1)
        rows = np.arange(x.shape[0])
        codes[lo:lo + chunk] = j
        best[lo:lo + chunk] = dist[rows, j]
        if cb.shape[0] > 1:
            dist[rows, j] = np.inf
            gap[lo:lo + chunk] = dist.min(axis=1) - best[lo:lo + chunk]
        else:
            gap[lo:lo + chunk] = np.inf
    return codes, best, gap


def vq_encode(x: np.ndarray, codebook: np.ndarray, sub_dim: int = 4):
    """VQ(x, C): codes [n, D/d] of the rows of x [n, D]; also the gaps."""
    x = np.asarray(x, dtype=np.float64)
    n, dim = x.shape
    codes, _, gap = vq_assign(x.reshape(n * (dim // sub_dim), sub_dim), codebook)
    return codes.reshape(n, dim // sub_dim), gap.reshape(n, dim // sub_dim)


def vq_decode(codes: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """VQ^-1: replace each index by its centroid; [n, D/d] -> float64 [n, D]."""
    cb = np.asarray(codebook, dtype=np.float64)
    codes = np.asarray(codes, dtype=np.int64)
    return cb[codes].reshape(codes.shape[0], codes.shape[1] * cb.shape[1])


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes [n, P] -> packed bytes [n, P*bits/8] (little-endian bit stream).

    8-bit codes are one byte each.  12-bit codes: code i of a row occupies
    bits [12 i, 12 i + 12) of that row; bit k of the row is bit (k mod 8) of
    byte k // 8.
    """
    codes = np.asarray(codes, dtype=np.int64)
    if bits == 8:
        return codes.astype(np.uint8)
    n, p = codes.shape
    shifts = np.arange(bits)
    bitrows = ((codes[:, :, None] >> shifts) & 1).reshape(n, p * bits).astype(np.uint8)
    return np.packbits(bitrows, axis=1, bitorder="little")


def unpack_codes(packed: np.ndarray, bits: int, num_sub: int) -> np.ndarray:
    """Inverse of pack_codes: packed bytes [n, num_sub*bits/8] -> int64 codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return packed.astype(np.int64)[:, :num_sub]
    n = packed.shape[0]
    bitrows = np.unpackbits(packed, axis=1, bitorder="little")[:, : num_sub * bits]
    bitrows = bitrows.reshape(n, num_sub, bits).astype(np.int64)
    return (bitrows << np.arange(bits)).sum(axis=2)


# ---------------------------------------------------------------------------
# attention — [VecInfer] Background, "KV cache and attention":
# s = q K^T / sqrt(D), p = softmax(s), o = p V; and Method details,
# "VQ KV cache in attention": s = q~ VQ^-1(K~_q, C_k)^T / sqrt(D),
# o = softmax(s) VQ^-1(V_q, C_v).
# ---------------------------------------------------------------------------

def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Textbook single-query attention in float64: q [D] or [h, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    s = (q @ k.T) / np.sqrt(k.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return p @ v


def decode_attention_head(q_heads, lam, cb_k, cb_v, codes_k, codes_v,
                          k_bits: int = 8, v_bits: int = 8) -> np.ndarray:
    """Decode attention of the G query heads that share one KV head.

    q_heads [G, D] as stored (fp16/fp32 values), lam [D] (fp32 values),
    cb_k [2^kb, d], cb_v [2^vb, d] (fp16 values), codes_k / codes_v the
    packed code rows [N, bytes] of that KV head.  Returns float64 [G, D].
    """
    dim = np.asarray(q_heads).shape[-1]
    sub = np.asarray(cb_k).shape[1]
    k_hat = vq_decode(unpack_codes(codes_k, k_bits, dim // sub), cb_k)
    v_hat = vq_decode(unpack_codes(codes_v, v_bits, dim // sub), cb_v)
    q_t = transform_query(q_heads, lam)
    return softmax_attention(q_t, k_hat, v_hat)


def decode_attention(q, lam, cb_k, cb_v, codes_k, codes_v, context_len: int,
                     k_bits: int = 8, v_bits: int = 8) -> np.ndarray:
    """Full layer: q [B, Hq, D]; lam [Hkv, D]; cb_* [Hkv, entries, d];
    codes_* [B, Hkv, >=N, bytes].  Query head h reads KV head h // G.
    Returns float64 [B, Hq, D]."""
    q = np.asarray(q)
    batch, hq, dim = q.shape
    hkv = np.asarray(lam).shape[0]
    group = hq // hkv
    out = np.empty((batch, hq, dim), dtype=np.float64)
    for b in range(batch):
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            out[b, heads] = decode_attention_head(
                q[b, heads], lam[g], cb_k[g], cb_v[g],
                codes_k[b, g, :context_len], codes_v[b, g, :context_len], k_bits, v_bits)
    return out


def decode_attention_window_head(q_heads, lam, cb_k, cb_v, codes_k, codes_v, win_k, win_v,
                                 k_bits: int = 8, v_bits: int = 8) -> np.ndarray:
    """Attention of the G query heads of one KV head over its coded tokens and
    a full-precision residual window, in one softmax.

    [VecInfer] Experiments: every method keeps the most recent tokens (the
    residual, length 128) in full precision; the HACK notes page keeps its
    last, not yet full block in fp16 beside the quantised cache in the same
    attention.  win_k / win_v [n_win, D] are raw (untransformed) rows.  A raw
    key k scores q . k, which equals q~ . k~ with k~ = k diag(lambda)^-1 H_D
    (H_D orthonormal): the window keys are transformed like the cache's,
    appended to the dequantised keys, and one textbook softmax runs over the
    union.  Returns float64 [G, D].
    """
    dim = np.asarray(q_heads).shape[-1]
    sub = np.asarray(cb_k).shape[1]
    k_hat = vq_decode(unpack_codes(codes_k, k_bits, dim // sub), cb_k)
    v_hat = vq_decode(unpack_codes(codes_v, v_bits, dim // sub), cb_v)
    keys = np.concatenate([k_hat, transform_keys(np.asarray(win_k, dtype=np.float64), lam)])
    values = np.concatenate([v_hat, np.asarray(win_v, dtype=np.float64)])
    return softmax_attention(transform_query(q_heads, lam), keys, values)


def decode_attention_window(q, lam, cb_k, cb_v, codes_k, codes_v, num_codes: int, win_k, win_v,
                            win_len: int, k_bits: int = 8, v_bits: int = 8) -> np.ndarray:
    """Full layer with a residual window: q [B, Hq, D]; codes_* [B, Hkv, >=num_codes,
    bytes]; win_* [B, Hkv, >=win_len, D].  Query head h reads KV head h // G.
    Returns float64 [B, Hq, D]."""
    q = np.asarray(q)
    batch, hq, dim = q.shape
    hkv = np.asarray(lam).shape[0]
    group = hq // hkv
    out = np.empty((batch, hq, dim), dtype=np.float64)
    for b in range(batch):
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            out[b, heads] = decode_attention_window_head(
                q[b, heads], lam[g], cb_k[g], cb_v[g], codes_k[b, g, :num_codes],
                codes_v[b, g, :num_codes], win_k[b, g, :win_len], win_v[b, g, :win_len],
                k_bits, v_bits)
    return out


def encode_append(k_new, v_new, lam, cb_k, cb_v, k_bits: int = 8, v_bits: int = 8):
    """Codes of appended tokens for one KV head.

    [VecInfer] Method details: each new key gets the online dual transform
    k~ = k diag(lambda)^-1 H_D and is quantised with C_k; the value is
    quantised untransformed with C_v; both are concatenated to the cache.
    Returns (packed K rows, packed V rows, K gaps, V gaps).
    """
    xk = transform_keys(k_new, lam)
    ck, gk = vq_encode(xk, cb_k, np.asarray(cb_k).shape[1])
    cv, gv = vq_encode(np.asarray(v_new, dtype=np.float64), cb_v, np.asarray(cb_v).shape[1])
    return pack_codes(ck, k_bits), pack_codes(cv, v_bits), gk, gv


# ---------------------------------------------------------------------------
# codebook training (the fixtures' codebooks and the K-Means parity reference)
# — [VecInfer] Method details: codebooks are pretrained offline by K-Means on
# transformed keys (raw values for V); Experimental setup: at most 30
# iterations.  The mean is the in-order fp64 sum (np.add.at adds the samples
# of a cluster one by one, in sample order) divided once by the count.
# ---------------------------------------------------------------------------

def lloyd_kmeans(samples: np.ndarray, init: np.ndarray, iters: int) -> np.ndarray:
    """Lloyd's algorithm: assign every sample to its nearest centroid (ties
    to the lowest index), move each centroid to the mean of its samples; a
    centroid with no samples keeps its place.  float64 [k, d]."""
    x = np.asarray(samples, dtype=np.float64)
    c = np.array(init, dtype=np.float64, copy=True)
    for _ in range(iters):
        assign, _, _ = vq_assign(x, c)
        sums = np.zeros_like(c)
        np.add.at(sums, assign, x)
        counts = np.bincount(assign, minlength=c.shape[0])
        live = counts > 0
        c[live] = sums[live] / counts[live, None]
    return c


# ---------------------------------------------------------------------------
# byte accounting — [VecInfer] Background: a codebook takes 2^b * d * 2
# bytes and each d_h-vector (d_h/d) * (b/8) bytes of indices; [CommVQ]
# Method: reduction ratio RR = 1 - N_c / (16 d) for N_c code bits per
# d-vector.
# ---------------------------------------------------------------------------

def codebook_bytes(bits: int, sub_dim: int, elem_bytes: int = 2) -> int:
    return (1 << bits) * sub_dim * elem_bytes


def index_bytes(head_dim: int, sub_dim: int, bits: int) -> float:
    return head_dim / sub_dim * bits / 8


def commvq_reduction_ratio(code_bits: int, dim: int) -> float:
    return 1.0 - code_bits / (16.0 * dim)
