"""Test inputs and expected values built from the seeded generators and the oracle.

Nothing here comes from the HIP library: every code, codebook, smoothing
factor and expected output is computed on the CPU by ``oracle`` from the
seeded arrays of ``workloads``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import workloads as W


@dataclasses.dataclass
class Cache:
    """A VQ-KV layer in host memory, in the library's storage formats."""

    wl: W.Workload
    q: np.ndarray          # [B, Hq, 128] float16/float32
    lam: np.ndarray        # [Hkv, 128] float32
    cb_k: np.ndarray       # [Hkv, 2^kb, 4] float16
    cb_v: np.ndarray       # [Hkv, 2^vb, 4] float16
    codes_k: np.ndarray    # [B, Hkv, cap, k_row_bytes] uint8
    codes_v: np.ndarray    # [B, Hkv, cap, v_row_bytes] uint8
    context_len: int


def _storage(dtype):
    return np.float16 if dtype == "f16" else np.float32


def chain_cache(wl: W.Workload, seqs=None, heads=None) -> Cache:
    """The full recipe for a workload: Gaussian K/V with outlier channels,
    lambda from sequence 0's keys, Lloyd codebooks on 16384 sampled
    transformed sub-vectors, oracle encoding of every token.

    ``seqs`` / ``heads`` restrict which (sequence, KV head) streams get real
    codes; the other streams get random code rows (their outputs are not
    checked by callers that pass a restriction).
    """
    n, cap = wl.context_len, wl.capacity
    st = _storage(wl.qkv_dtype)
    seqs = range(wl.batch) if seqs is None else seqs
    heads = range(wl.num_kv_heads) if heads is None else heads
    q = np.stack([W.queries(wl.config_id, b, wl.num_q_heads) for b in range(wl.batch)]).astype(st)
    lam = np.empty((wl.num_kv_heads, wl.head_dim), np.float32)
    cb_k = np.empty((wl.num_kv_heads, 1 << wl.k_bits, wl.sub_dim), np.float16)
    cb_v = np.empty((wl.num_kv_heads, 1 << wl.v_bits, wl.sub_dim), np.float16)
    codes_k = np.zeros((wl.batch, wl.num_kv_heads, cap, wl.k_row_bytes), np.uint8)
    codes_v = np.zeros((wl.batch, wl.num_kv_heads, cap, wl.v_row_bytes), np.uint8)
    for g in range(wl.num_kv_heads):
        if g not in heads:
            lam[g] = W.random_lambda(wl.config_id, g)
            cb_k[g] = W.random_codebook(wl.config_id, g, "k", 1 << wl.k_bits, 0.6,
                                        sub_dim=wl.sub_dim)
            cb_v[g] = W.random_codebook(wl.config_id, g, "v", 1 << wl.v_bits, 1.0, 1 / 32,
                                        sub_dim=wl.sub_dim)
            for b in range(wl.batch):
                codes_k[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "k", n, wl.k_row_bytes)
                codes_v[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "v", n, wl.v_row_bytes)
            continue
        k0 = W.kv_rows(wl.config_id, 0, g, "k", n).astype(st)
        v0 = W.kv_rows(wl.config_id, 0, g, "v", n).astype(st)
        lam[g] = oracle.smooth_factors(k0).astype(np.float32)
        kt0 = oracle.transform_keys(k0, lam[g])
        for tensor, x, bits, out in (("k", kt0, wl.k_bits, cb_k), ("v", v0, wl.v_bits, cb_v)):
            subs = np.asarray(x, np.float64).reshape(-1, wl.sub_dim)
            rows = W.kmeans_sample_rows(wl.config_id, g, tensor, subs.shape[0], wl.kmeans_samples)
            train = subs[rows]
            order = W.kmeans_init_order(wl.config_id, g, tensor, train.shape[0])
            init = train[order[: 1 << bits]]
            out[g] = oracle.lloyd_kmeans(train, init, wl.kmeans_iters).astype(np.float16)
        for b in range(wl.batch):
            if b in seqs:
                kb = k0 if b == 0 else W.kv_rows(wl.config_id, b, g, "k", n).astype(st)
                vb = v0 if b == 0 else W.kv_rows(wl.config_id, b, g, "v", n).astype(st)
                pk, pv, _, _ = oracle.encode_append(kb, vb, lam[g], cb_k[g], cb_v[g],
                                                    wl.k_bits, wl.v_bits)
                codes_k[b, g, :n] = pk
                codes_v[b, g, :n] = pv
            else:
                codes_k[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "k", n, wl.k_row_bytes)
                codes_v[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "v", n, wl.v_row_bytes)
    return Cache(wl, q, lam, cb_k, cb_v, codes_k, codes_v, n)


def random_cache(wl: W.Workload, context_len: int | None = None, batch: int | None = None,
                 num_kv_heads: int | None = None) -> Cache:
    """A directly drawn VQ cache of a workload's shape (uniform random codes,
    Gaussian fp16 codebooks, positive lambda, Gaussian q)."""
    n = wl.context_len if context_len is None else context_len
    bsz = wl.batch if batch is None else batch
    hkv = wl.num_kv_heads if num_kv_heads is None else num_kv_heads
    hq = wl.group * hkv
    cap = n + wl.append_tokens
    st = _storage(wl.qkv_dtype)
    q = np.stack([W.queries(wl.config_id, b, hq) for b in range(bsz)]).astype(st)
    lam = np.stack([W.random_lambda(wl.config_id, g) for g in range(hkv)])
    cb_k = np.stack([W.random_codebook(wl.config_id, g, "k", 1 << wl.k_bits, 0.6,
                                       sub_dim=wl.sub_dim) for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(wl.config_id, g, "v", 1 << wl.v_bits, 1.0, 1 / 32,
                                       sub_dim=wl.sub_dim) for g in range(hkv)])
    codes_k = np.zeros((bsz, hkv, cap, wl.k_row_bytes), np.uint8)
    codes_v = np.zeros((bsz, hkv, cap, wl.v_row_bytes), np.uint8)
    for b in range(bsz):
        for g in range(hkv):
            codes_k[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "k", n, wl.k_row_bytes)
            codes_v[b, g, :n] = W.random_code_rows(wl.config_id, b, g, "v", n, wl.v_row_bytes)
    return Cache(wl, q, lam, cb_k, cb_v, codes_k, codes_v, n)


def expected_head(c: Cache, b: int, g: int, context_len: int | None = None) -> np.ndarray:
    """Oracle output [G, 128] of the query heads of KV head g in sequence b."""
    n = c.context_len if context_len is None else context_len
    grp = c.q.shape[1] // c.lam.shape[0]
    return oracle.decode_attention_head(
        c.q[b, g * grp:(g + 1) * grp], c.lam[g], c.cb_k[g], c.cb_v[g],
        c.codes_k[b, g, :n], c.codes_v[b, g, :n], c.wl.k_bits, c.wl.v_bits)


def expected_all(c: Cache, context_len: int | None = None) -> np.ndarray:
    n = c.context_len if context_len is None else context_len
    return oracle.decode_attention(c.q, c.lam, c.cb_k, c.cb_v, c.codes_k, c.codes_v, n,
                                   c.wl.k_bits, c.wl.v_bits)


def attention_errors(got: np.ndarray, ref: np.ndarray):
    """(relative L2 error over the whole output, max absolute error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    return float(rel), float(np.max(np.abs(got - ref)))
