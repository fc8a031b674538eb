"""GPU parity of the lookup-table score path (vq_set_score_method(LUT)).

VecInfer page, Appendix (Algorithm 1): the query is multiplied with the key
codebook once per block, and every score is then a sum of table entries,
one per sub-vector position.  Selected library-wide; it applies to 8-bit
keys over 4-dim sub-vectors with G <= 4 (other layouts keep the matrix-core
scores).  The same bounds as the default path: rel-L2 <= 1e-3, max-abs <=
2e-3 against the fp64 oracle; decode-step codes bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W
from edge_inputs import shaped_cache
from fixtures import attention_errors, chain_cache, expected_all, expected_head, random_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(autouse=True)
def lut_scores():
    prev = vq.set_score_method(vq.SCORES_LUT)
    yield
    vq.set_score_method(prev)


def check(got, ref, what):
    rel, mab = attention_errors(got, ref)
    print(f"{what}: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert np.isfinite(got).all() and rel <= 1e-3 and mab <= 2e-3, (what, rel, mab)


def attend(c, n=None, splits=0):
    n = c.context_len if n is None else n
    out = vq.decode_attention(dev(c.q), dev(c.lam), dev(c.cb_k), dev(c.cb_v), dev(c.codes_k),
                              dev(c.codes_v), n, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_set_score_method_round_trip():
    assert vq.set_score_method(vq.SCORES_MFMA) == vq.SCORES_LUT
    assert vq.set_score_method(vq.SCORES_LUT) == vq.SCORES_MFMA
    with pytest.raises(ValueError):
        vq.set_score_method(7)


def test_lut_tiny_recipe_case():
    c = chain_cache(W.WORKLOADS[1])
    for splits in (0, 1, 2):
        check(attend(c, splits=splits), expected_all(c), f"LUT config1 splits={splits}")


@pytest.mark.parametrize("group,n", [(1, 300), (2, 1000), (3, 777), (4, 2049), (4, 1)])
def test_lut_group_sizes_and_ragged(group, n):
    wl = W.Workload(130 + group, "adhoc", batch=2, num_q_heads=2 * group, num_kv_heads=2,
                    context_len=n, qkv_dtype="f16")
    c = random_cache(wl)
    check(attend(c), expected_all(c), f"LUT G={group} n={n}")


def test_lut_leaves_other_layouts_on_the_matrix_cores():
    # G = 8 and 12-bit keys are outside the LUT path: the default kernel runs
    for kb, g in ((8, 8), (12, 4)):
        wl = W.Workload(140 + g + kb, "adhoc", batch=1, num_q_heads=2 * g, num_kv_heads=2,
                        context_len=700, k_bits=kb, qkv_dtype="f16")
        c = random_cache(wl)
        check(attend(c), expected_all(c), f"LUT-selected G={g} kbits={kb}")


@pytest.mark.parametrize("config,samples", [(2, [(0, 0), (0, 5)]), (4, [(0, 2), (0, 7)])])
def test_lut_full_size_sampled_heads(config, samples):
    wl = W.WORKLOADS[config]
    c = random_cache(wl)
    got = attend(c)
    g = wl.group
    for b, h in samples:
        check(got[b, h * g:(h + 1) * g], expected_head(c, b, h), f"LUT config{config} b={b} kv={h}")


@pytest.mark.parametrize("kind", ["sink_const", "sink_tail", "climb", "large_pos", "large_neg"])
def test_lut_softmax_edges(kind):
    n = 65536 if kind.startswith("sink") else 16384
    c = shaped_cache(kind, 4, 8, 4, n, seed=1)
    ref = expected_all(c)
    for splits in (1, 0):
        check(attend(c, splits=splits), ref, f"LUT {kind} splits={splits}")


@pytest.mark.parametrize("cur", [0, 700, 9000])
def test_lut_decode_step(cur):
    wl = W.Workload(150, "adhoc", batch=4, num_q_heads=32, num_kv_heads=8, context_len=cur,
                    qkv_dtype="f16", append_tokens=1)
    c = random_cache(wl)
    rng = np.random.default_rng(cur)
    k_new = rng.standard_normal((4, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((4, 8, 128)).astype(np.float16)
    d_ck, d_cv = dev(c.codes_k), dev(c.codes_v)
    out = vq.decode_step(dev(c.q), dev(k_new), dev(v_new), dev(c.lam), dev(c.cb_k), dev(c.cb_v),
                         d_ck, d_cv, cur)
    torch.cuda.synchronize()
    got_ck, got_cv = d_ck.cpu().numpy(), d_cv.cpu().numpy()
    for b in range(4):
        for h in range(8):
            pk, pv, _, _ = oracle.encode_append(k_new[b, h][None], v_new[b, h][None], c.lam[h],
                                                c.cb_k[h], c.cb_v[h])
            assert np.array_equal(got_ck[b, h, cur], pk[0]) and np.array_equal(got_cv[b, h, cur], pv[0])
    c.codes_k, c.codes_v = got_ck, got_cv
    check(out.cpu().numpy().astype(np.float64), expected_all(c, cur + 1), f"LUT step cur={cur}")
