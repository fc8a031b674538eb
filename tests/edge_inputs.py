"""Caches whose softmax is shaped on purpose: a dominant first token, a
steady climb of the scores, scores of large magnitude.

The uniform random caches of the workload shapes give a nearly flat softmax
(score spread of a few base-2 units), which never reaches the online
softmax's corner cases: weights far below the running maximum, repeated
rescaling after a split's first tile, large |s|.  These caches reach them
by construction:

  * q of every head is zero except channel 0, which holds a_h / lambda_0
    (rounded to fp16).  The first row of the orthonormal Sylvester matrix is
    constant, 1/sqrt(128), so q~ = (q . lambda) H_128 is a_h / sqrt(128) in
    every channel (VecInfer page, Method details: the query's smoothing and
    Hadamard rotation).
  * Every key centroid has all its components equal: C_k[j] = lvl(j) (1, .., 1).
    A token's score q~ . K^_t / sqrt(128) is then a_h / 128 times the sum of
    its dequantised key entries: a_h d / 128 times the sum of lvl over its
    codes.  Choosing codes chooses scores.

Nothing here computes an attention output: the expected values of the tests
come from the oracle over these arrays.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W
from fixtures import Cache

LOG2E = 1.4426950408889634
KINDS = ("sink_const", "sink_tail", "climb", "large_pos", "large_neg")


def shaped_cache(kind: str, group: int, k_bits: int, sub_dim: int, n: int, seed: int,
                 hkv: int = 2, batch: int = 1, cap_extra: int = 0, gap: float = 20.5) -> Cache:
    """A VQ cache [batch][hkv][n + cap_extra] of one of KINDS.

    sink_const  token 0's score is `gap` base-2 units above the rest (head h:
                gap (1 + 0.08 h)); every token has the same value codes, so
                the output of any softmax is that value row (entries ~ +-30).
    sink_tail   the same scores; the tail's value entries are all ~ +30, the
                sink's ~ -30 (a same-sign tail behind a sink of the other sign).
    climb       scores rise linearly over the context by 1.5 n / 64 base-2
                units: about 12 per 512 tokens, so every wave's next tile
                exceeds its running maximum by more than the rescale slack.
    large_pos   scores near +640 base-2 units (spread a few units);
    large_neg   the same near -640.
    """
    assert kind in KINDS
    rng = np.random.default_rng([seed, group, k_bits, sub_dim, n, KINDS.index(kind)])
    v_bits = 12 if sub_dim == 8 else 8
    pos = 128 // sub_dim
    ke, ve = 1 << k_bits, 1 << v_bits
    hq = group * hkv
    cap = n + cap_extra
    wl = W.Workload(200 + seed, f"shaped-{kind}", batch=batch, num_q_heads=hq,
                    num_kv_heads=hkv, context_len=n, k_bits=k_bits, v_bits=v_bits,
                    sub_dim=sub_dim, qkv_dtype="f16", append_tokens=cap_extra)
    lam = np.stack([W.random_lambda(wl.config_id, g) for g in range(hkv)])

    # key centroids: lvl(j) in every component
    frac = np.arange(ke) / (ke - 1)
    if kind in ("large_pos", "large_neg"):
        lvl = 7.7 + frac           # sum over a token's codes: pos (7.7 + mean frac)
    else:
        lvl = frac
    cb_k = np.repeat(lvl[:, None], sub_dim, axis=1).astype(np.float16)
    cb_k = np.broadcast_to(cb_k, (hkv, ke, sub_dim)).copy()

    # per-head score scale a_h: base-2 score = a_h log2(e) mean_pos(lvl(code))
    # (d / 128 times the sum over 128 / d positions is the mean)
    if kind.startswith("sink"):
        span = gap / (1.0 - 1.0 / 32.0)          # top code vs the tail's mean
    elif kind == "climb":
        span = 1.5 * n / 64.0
    else:
        span = 78.0                             # 78 (7.7 + u): ~ 640 +- a few
    a = np.array([span / LOG2E * (1.0 + 0.08 * (h % group)) for h in range(hq)])
    if kind == "large_neg":
        a = -a
    q = np.zeros((batch, hq, 128))
    for h in range(hq):
        q[:, h, 0] = a[h] / float(lam[h // group][0])
        # a little of every other channel, so q~ is not exactly constant
        q[:, h, 1:] = 0.01 * rng.standard_normal((batch, 127)) / lam[h // group][1:]
    q = q.astype(np.float16)

    codes_k = np.zeros((batch, hkv, cap, pos), np.int64)
    codes_v = np.zeros((batch, hkv, cap, pos), np.int64)
    cb_v = np.stack([W.random_codebook(wl.config_id, g, "v", ve, 1.0, 1 / 32, sub_dim=sub_dim)
                     for g in range(hkv)])
    for b in range(batch):
        for g in range(hkv):
            if kind.startswith("sink"):
                ck = rng.integers(0, ke // 16, size=(n, pos))
                ck[0] = ke - 1
            elif kind == "climb":
                # code sum rising from 0 to pos (ke - 1): spread evenly over positions
                total = np.round(np.linspace(0, pos * (ke - 1), n)).astype(np.int64)
                total = np.clip(total + rng.integers(-2, 3, size=n), 0, pos * (ke - 1))
                base, rem = total // pos, total % pos
                ck = base[:, None] + (np.arange(pos)[None, :] < rem[:, None])
            else:
                ck = rng.integers(0, ke, size=(n, pos))
            codes_k[b, g, :n] = ck
            if kind == "sink_const":
                codes_v[b, g, :n] = rng.integers(0, ve, size=pos)[None, :]
            elif kind == "sink_tail":
                cv = rng.integers(0, ve // 2, size=(n, pos))
                cv[0] = rng.integers(ve // 2, ve, size=pos)
                codes_v[b, g, :n] = cv
            else:
                codes_v[b, g, :n] = rng.integers(0, ve, size=(n, pos))
    if kind == "sink_const":
        # the selected value entries get magnitudes ~ 30, both signs
        for g in range(hkv):
            used = np.unique(codes_v[:, g, :n])
            sign = np.where(rng.random((used.size, sub_dim)) < 0.5, -1.0, 1.0)
            cb_v[g, used] = (sign * (30.0 + rng.standard_normal((used.size, sub_dim)))
                             ).astype(np.float16)
    elif kind == "sink_tail":
        half = ve // 2
        cb_v[:, :half] = (30.0 + rng.standard_normal((hkv, half, sub_dim))).astype(np.float16)
        cb_v[:, half:] = (-30.0 + rng.standard_normal((hkv, ve - half, sub_dim))
                          ).astype(np.float16)

    pk = np.stack([np.stack([oracle.pack_codes(codes_k[b, g], k_bits) for g in range(hkv)])
                   for b in range(batch)])
    pv = np.stack([np.stack([oracle.pack_codes(codes_v[b, g], v_bits) for g in range(hkv)])
                   for b in range(batch)])
    return Cache(wl, q, lam, cb_k, cb_v, pk, pv, n)


def base2_scores(c: Cache, b: int, h: int, n: int | None = None) -> np.ndarray:
    """Oracle base-2 scores of query head h over the cache's first n tokens
    (log2(e) q~ . K^_t / sqrt(128)), for checking that a case has the shape
    it claims."""
    n = c.context_len if n is None else n
    grp = c.q.shape[1] // c.lam.shape[0]
    g = h // grp
    sub = c.cb_k.shape[2]
    k_hat = oracle.vq_decode(oracle.unpack_codes(c.codes_k[b, g, :n], c.wl.k_bits, 128 // sub),
                             c.cb_k[g])
    qt = oracle.transform_query(c.q[b, h], c.lam[g])
    return (k_hat @ qt) / np.sqrt(128.0) * LOG2E
