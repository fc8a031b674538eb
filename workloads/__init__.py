"""Seeded synthetic inputs for VQ-KV decode attention.

This module is shared by the tests, the benchmark and the oracle-side
fixtures.  It holds random-number generation and shape bookkeeping only:
none of the method's arithmetic (no smoothing, no Hadamard transform, no
quantisation, no attention) lives here.

Workload shapes follow the VecInfer page (Experimental setup: Llama-3.1-8B
and Qwen2.5-14B layers; Results: 196K-token latency measurements).  The
pages' real KV caches and calibration data (Pile, Qasper) are not
available, so Gaussian tensors with a few large outlier channels stand in
for them.

Every array is drawn from ``numpy.random.default_rng([config, b, kv_head,
stream])`` so that any (sequence, head) slice can be regenerated alone.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128
SUB_DIM = 4

# stream ids of the per-slice generators
STREAM_Q = 0
STREAM_K = 1
STREAM_V = 2
STREAM_OUTLIERS = 3
STREAM_KMEANS_SAMPLE = 4
STREAM_APPEND_K = 5
STREAM_APPEND_V = 6
STREAM_CODES_K = 7
STREAM_CODES_V = 8
STREAM_CODEBOOK_K = 9
STREAM_CODEBOOK_V = 10
STREAM_LAMBDA = 11
STREAM_CALIB_K = 12
STREAM_CALIB_V = 13
STREAM_CALIB_PICK = 14

# Calibration set size on the VecInfer page (Experimental setup): 256
# sequences of 512 tokens.
CALIB_SEQS = 256
CALIB_SEQ_LEN = 512
CALIB_TOKENS = CALIB_SEQS * CALIB_SEQ_LEN

OUTLIER_CHANNELS = 4
OUTLIER_SCALE = 15.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-attention layer shape."""

    config_id: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    context_len: int
    k_bits: int = 8
    v_bits: int = 8
    qkv_dtype: str = "f16"       # dtype of q, K, V as handed to the library
    kmeans_iters: int = 10
    kmeans_samples: int = 16384
    append_tokens: int = 0       # tokens appended per sequence by the encoder case
    head_dim: int = HEAD_DIM
    sub_dim: int = SUB_DIM

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_sub(self) -> int:
        return self.head_dim // self.sub_dim

    @property
    def k_row_bytes(self) -> int:
        return self.num_sub * self.k_bits // 8

    @property
    def v_row_bytes(self) -> int:
        return self.num_sub * self.v_bits // 8

    @property
    def capacity(self) -> int:
        return self.context_len + self.append_tokens


WORKLOADS = {
    1: Workload(1, "tiny-g4-n1024", batch=1, num_q_heads=4, num_kv_heads=1,
                context_len=1024, qkv_dtype="f32"),
    2: Workload(2, "llama3.1-8b-layer-b1-n32768", batch=1, num_q_heads=32,
                num_kv_heads=8, context_len=32768),
    3: Workload(3, "llama3.1-8b-layer-b16-n32768", batch=16, num_q_heads=32,
                num_kv_heads=8, context_len=32768),
    4: Workload(4, "llama3.1-8b-layer-b1-n196608", batch=1, num_q_heads=32,
                num_kv_heads=8, context_len=196608),
    5: Workload(5, "qwen2.5-14b-layer-b8-n65536-k3bit", batch=8, num_q_heads=40,
                num_kv_heads=8, context_len=65536, k_bits=12, v_bits=8,
                append_tokens=64),
    # the 1.5-bit layout of the VecInfer page (codebook-size ablation:
    # 2^12 x 8 x 2 B): 8-dim sub-vectors, 4096-entry C_k and C_v, 12-bit codes
    6: Workload(6, "llama3.1-8b-layer-b1-n196608-1.5bit", batch=1, num_q_heads=32,
                num_kv_heads=8, context_len=196608, k_bits=12, v_bits=12, sub_dim=8),
    7: Workload(7, "tiny-g4-n1024-1.5bit", batch=1, num_q_heads=4, num_kv_heads=1,
                context_len=1024, k_bits=12, v_bits=12, sub_dim=8, qkv_dtype="f32"),
}


def rng(config_id: int, b: int, kv_head: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(b), int(kv_head), int(stream)])


def outlier_channels(config_id: int, kv_head: int, tensor: str) -> np.ndarray:
    """The 4 distinct channels of one KV head that carry x15 outliers.

    Chosen once per (head, tensor) and shared by every sequence, as a
    model property would be.
    """
    t = {"k": 0, "v": 1}[tensor]
    g = rng(config_id, 0, kv_head, STREAM_OUTLIERS)
    picks = [g.choice(HEAD_DIM, size=OUTLIER_CHANNELS, replace=False) for _ in range(2)]
    return np.sort(picks[t])


def kv_rows(config_id: int, b: int, kv_head: int, tensor: str, n: int,
            append: bool = False) -> np.ndarray:
    """n token rows of K or V for one (sequence, KV head): float64 [n, 128].

    i.i.d. N(0, 1) per element, with OUTLIER_CHANNELS channels scaled by
    OUTLIER_SCALE.  ``append=True`` draws the rows of tokens appended after
    the prompt from their own stream.
    """
    if tensor == "k":
        stream = STREAM_APPEND_K if append else STREAM_K
    else:
        stream = STREAM_APPEND_V if append else STREAM_V
    x = rng(config_id, b, kv_head, stream).standard_normal((n, HEAD_DIM))
    x[:, outlier_channels(config_id, kv_head, tensor)] *= OUTLIER_SCALE
    return x


def queries(config_id: int, b: int, num_q_heads: int) -> np.ndarray:
    """q ~ N(0, 1): float64 [num_q_heads, 128] for one sequence."""
    return rng(config_id, b, 0, STREAM_Q).standard_normal((num_q_heads, HEAD_DIM))


def calibration_rows(config_id: int, kv_head: int, tensor: str, n: int) -> np.ndarray:
    """n calibration token rows of K or V for one KV head: float64 [n, 128].

    The same distribution as ``kv_rows`` (N(0, 1) with the head's x15 outlier
    channels) from streams of their own, standing in for the page's
    calibration text.
    """
    stream = STREAM_CALIB_K if tensor == "k" else STREAM_CALIB_V
    x = rng(config_id, 0, kv_head, stream).standard_normal((n, HEAD_DIM))
    x[:, outlier_channels(config_id, kv_head, tensor)] *= OUTLIER_SCALE
    return x


def calibration_init_rows(config_id: int, kv_head: int, tensor: str, total: int,
                          count: int) -> np.ndarray:
    """Indices of the ``count`` samples (of ``total``) that seed Lloyd: a
    uniform draw without replacement."""
    t = {"k": 0, "v": 1}[tensor]
    g = rng(config_id, t, kv_head, STREAM_CALIB_PICK)
    return np.sort(g.choice(total, size=min(count, total), replace=False))


def kmeans_sample_rows(config_id: int, kv_head: int, tensor: str, total: int,
                       count: int) -> np.ndarray:
    """Indices of the sub-vectors a codebook is trained on (no replacement)."""
    t = {"k": 0, "v": 1}[tensor]
    g = rng(config_id, 0, kv_head, STREAM_KMEANS_SAMPLE)
    perms = [g.permutation(total) for _ in range(2)]
    return perms[t][: min(count, total)]


def kmeans_init_order(config_id: int, kv_head: int, tensor: str, count: int) -> np.ndarray:
    """Permutation of the training samples; its first 2^b entries seed Lloyd."""
    t = {"k": 0, "v": 1}[tensor]
    g = rng(config_id, 1, kv_head, STREAM_KMEANS_SAMPLE)
    perms = [g.permutation(count) for _ in range(2)]
    return perms[t]


# --- directly drawn VQ caches -------------------------------------------------
# For full-size cases the codes themselves are drawn at random: the attention
# kernel's cost and numerics depend on the code values only through which
# codebook entries they select, and a uniformly random choice is the
# high-entropy case a well-trained codebook approaches.

def random_code_rows(config_id: int, b: int, kv_head: int, tensor: str, n: int,
                     row_bytes: int) -> np.ndarray:
    """Packed code rows uint8 [n, row_bytes] of uniformly random codes.

    A stream of independent uniform codes, packed at any bit width, is a
    stream of independent uniform bytes, so the rows are drawn as bytes.
    """
    stream = STREAM_CODES_K if tensor == "k" else STREAM_CODES_V
    return rng(config_id, b, kv_head, stream).integers(0, 256, size=(n, row_bytes),
                                                       dtype=np.uint8)


def random_codebook(config_id: int, kv_head: int, tensor: str, entries: int,
                    scale: float, heavy_fraction: float = 0.0,
                    sub_dim: int = SUB_DIM) -> np.ndarray:
    """fp16-valued codebook [entries, sub_dim] (returned as float16).

    Entries are N(0, scale^2); the last ``heavy_fraction`` of the entries
    are scaled by OUTLIER_SCALE, the way centroids of the sub-vectors that
    hold an outlier channel are.  Values are rounded to fp16, the storage
    type of every codebook.
    """
    stream = STREAM_CODEBOOK_K if tensor == "k" else STREAM_CODEBOOK_V
    c = rng(config_id, 0, kv_head, stream).standard_normal((entries, sub_dim)) * scale
    heavy = int(round(entries * heavy_fraction))
    if heavy:
        c[entries - heavy:] *= OUTLIER_SCALE
    return c.astype(np.float16)


def random_lambda(config_id: int, kv_head: int) -> np.ndarray:
    """Positive per-channel smoothing factors, float32 [128].

    Drawn in the range a square root of a channel maximum takes for the
    Gaussian-with-outliers keys above: about 2 for ordinary channels and
    about 7.7 for the x15 outlier channels.
    """
    g = rng(config_id, 0, kv_head, STREAM_LAMBDA)
    peak = 3.5 + np.abs(g.standard_normal(HEAD_DIM))
    peak[outlier_channels(config_id, kv_head, "k")] *= OUTLIER_SCALE
    return np.sqrt(peak).astype(np.float32)


def as_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 data to the dtype the library receives ('f16'/'f32')."""
    return x.astype(np.float16 if dtype == "f16" else np.float32)
