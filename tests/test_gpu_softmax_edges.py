"""GPU parity on caches that drive the online softmax into its corners.

The split kernel keeps a running maximum m per (head, wave), raises it only
when a tile's score exceeds m by more than 8 base-2 units, and hands p =
2^(s - m) to the matrix cores as a high and a low fp16 part (VecInfer page,
Appendix: the FlashAttention block recurrence of m, l and O; the rescaled
accumulator of Algorithm 1).  The cases here reach what uniform random
caches never do (tests/edge_inputs.py builds them):

  * a first token 20.5 to 32 base-2 units above every other, so thousands of
    weights sit 2^-20 and further below the running maximum in one split
    (constant values: the output must be that value row; a same-sign tail
    behind a sink of the other sign);
  * scores climbing by about 12 units per 512 tokens, so the rescale fires
    on nearly every tile of every wave;
  * scores near +-640 base-2 units;
  * a query whose transformed entries, scaled to base-2 scores, are far
    beyond the fp16 range.

Each runs for 8- and 12-bit keys over 4-dim sub-vectors and for the 1.5-bit
layout, at G = 4 (the packed softmax) and G = 5, 8, with the fewest splits
the planner allows (a request of one split over 65536 tokens becomes three
of 21856, near the 24576-token cap; one over 16384 tokens stays one) and
with the library's split plan, and through vq_decode_step.  Bounds as everywhere: rel-L2 <=
1e-3 over the output, max-abs <= 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
from edge_inputs import KINDS, shaped_cache
from fixtures import attention_errors, expected_all

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3
ABS_TOL = 2e-3
DEV = "cuda:0"

# (G, key bits, sub-vector size)
LAYOUTS = [(4, 8, 4), (4, 12, 4), (4, 12, 8), (8, 8, 4), (5, 12, 4)]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def context_for(kind):
    return 65536 if kind.startswith("sink") else 16384


_CACHES = {}


def cached(kind, layout):
    key = (kind, layout)
    if key not in _CACHES:
        g, kb, sd = layout
        c = shaped_cache(kind, g, kb, sd, context_for(kind), seed=1)
        _CACHES[key] = (c, expected_all(c))
    return _CACHES[key]


def check(got, ref, what):
    rel, mab = attention_errors(got, ref)
    print(f"{what}: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert rel <= REL_TOL and mab <= ABS_TOL, (what, rel, mab)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"G{l[0]}-k{l[1]}-d{l[2]}")
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("splits", [1, 0], ids=["fewest-splits", "planned"])
def test_shaped_softmax_matches_oracle(kind, layout, splits):
    c, ref = cached(kind, layout)
    n = c.context_len
    print(f"case {kind} {layout} n={n} splits={splits}", flush=True)
    out = vq.decode_attention(dev(c.q), dev(c.lam), dev(c.cb_k), dev(c.cb_v), dev(c.codes_k),
                              dev(c.codes_v), n, num_splits=splits)
    torch.cuda.synchronize()
    check(out.cpu().numpy().astype(np.float64), ref, f"{kind} {layout} splits={splits}")


@pytest.mark.parametrize("layout", [(4, 8, 4), (4, 12, 4), (4, 12, 8), (8, 8, 4)],
                         ids=lambda l: f"G{l[0]}-k{l[1]}-d{l[2]}")
@pytest.mark.parametrize("kind", ["sink_const", "sink_tail", "climb"])
def test_shaped_decode_step(kind, layout):
    """One vq_decode_step over the shaped cache: the new token is encoded into
    the last slot (codes bit-exact with the oracle encoder), then attention
    runs over the whole context, to the usual bound."""
    g, kb, sd = layout
    n = 32768
    c = shaped_cache(kind, g, kb, sd, n, seed=2)
    hkv = c.lam.shape[0]
    rng = np.random.default_rng(7)
    k_new = (rng.standard_normal((1, hkv, 128)) * 2).astype(np.float16)
    v_new = (rng.standard_normal((1, hkv, 128)) * 2).astype(np.float16)
    d_ck, d_cv = dev(c.codes_k), dev(c.codes_v)
    print(f"case step {kind} {layout} n={n}", flush=True)
    out = vq.decode_step(dev(c.q), dev(k_new), dev(v_new), dev(c.lam), dev(c.cb_k), dev(c.cb_v),
                         d_ck, d_cv, n - 1)
    torch.cuda.synchronize()
    got_ck, got_cv = d_ck.cpu().numpy(), d_cv.cpu().numpy()
    for h in range(hkv):
        pk, pv, _, _ = oracle.encode_append(k_new[0, h][None], v_new[0, h][None], c.lam[h],
                                            c.cb_k[h], c.cb_v[h], kb, c.wl.v_bits)
        assert np.array_equal(got_ck[0, h, n - 1], pk[0]), ("key codes", h)
        assert np.array_equal(got_cv[0, h, n - 1], pv[0]), ("value codes", h)
        c.codes_k[0, h, n - 1] = pk[0]
        c.codes_v[0, h, n - 1] = pv[0]
    assert np.array_equal(got_ck[:, :, :n - 1], c.codes_k[:, :, :n - 1])
    check(out.cpu().numpy().astype(np.float64), expected_all(c), f"step {kind} {layout}")


@pytest.mark.parametrize("layout", [(4, 8, 4), (4, 12, 4), (4, 12, 8), (8, 8, 4)],
                         ids=lambda l: f"G{l[0]}-k{l[1]}-d{l[2]}")
@pytest.mark.parametrize("scale", [1e9, 1e-9])
def test_query_scale_far_outside_fp16(layout, scale):
    """fp32 queries whose transformed, base-2-scaled entries are ~1e9 (far
    above the fp16 maximum of 65504) or ~1e-9 (far below its smallest
    normal): the kernel scales q~ per head by a power of two before the fp16
    split, so the output stays finite and equals the oracle's (a one-hot
    softmax for the huge query, a nearly uniform one for the tiny query)."""
    g, kb, sd = layout
    c = shaped_cache("large_pos", g, kb, sd, 4096, seed=3)
    c.q = (c.q.astype(np.float64) * scale).astype(np.float32)
    ref = expected_all(c)
    out = vq.decode_attention(dev(c.q), dev(c.lam), dev(c.cb_k), dev(c.cb_v), dev(c.codes_k),
                              dev(c.codes_v), c.context_len)
    torch.cuda.synchronize()
    check(out.cpu().numpy().astype(np.float64), ref, f"q x {scale:g} {layout}")
