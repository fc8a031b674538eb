"""Pins of the CPU oracle to things other than itself.

Each test ties an oracle function to a closed form, a library routine, an
invariant the pages state, a hand-worked layout or a number the pages
print.  A plausible mistake in the oracle (a dropped 1/sqrt(D), an
inverted lambda, a transposed Hadamard, a wrong GQA head map, a swapped
nibble in the 12-bit layout, ties to the wrong index) fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.cluster.vq
import scipy.linalg
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- Walsh–Hadamard matrix -----------------------------------------------------

@pytest.mark.parametrize("dim", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_closed_form(dim):
    h = oracle.sylvester_hadamard(dim)
    i, j = np.meshgrid(np.arange(dim), np.arange(dim), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    np.testing.assert_allclose(h, np.where(parity, -1.0, 1.0) / math.sqrt(dim), rtol=0, atol=1e-15)


@pytest.mark.parametrize("dim", [2, 16, 128])
def test_hadamard_matches_scipy_and_is_orthonormal(dim):
    h = oracle.sylvester_hadamard(dim)
    np.testing.assert_allclose(h, scipy.linalg.hadamard(dim) / math.sqrt(dim), atol=1e-15)
    np.testing.assert_allclose(h @ h.T, np.eye(dim), atol=1e-13)
    hs = h * math.sqrt(dim)                       # the +-1 matrix
    np.testing.assert_allclose(hs @ hs.T, dim * np.eye(dim), atol=1e-10)
    np.testing.assert_array_equal(h, h.T)         # symmetric
    np.testing.assert_allclose(h @ h, np.eye(dim), atol=1e-13)   # involution


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.sylvester_hadamard(96)


# --- smoothing and the transform ------------------------------------------------

def test_smooth_factors_hand_example():
    k = np.array([[1.0, -4.0, 0.25], [-9.0, 2.0, 0.0]])
    np.testing.assert_allclose(oracle.smooth_factors(k), [3.0, 2.0, 0.5])


def test_smoothing_direction_balances_channel_maxima():
    # lambda_i = sqrt(max|K_i|) divides the keys, so every smoothed channel
    # peaks at exactly sqrt(max|K_i|) = lambda_i.  Multiplying instead would
    # give max|K_i|^1.5.
    rng = np.random.default_rng(0)
    k = rng.standard_normal((300, 128))
    k[:, [3, 77]] *= 15
    lam = oracle.smooth_factors(k)
    h = scipy.linalg.hadamard(128) / math.sqrt(128)
    smoothed = oracle.transform_keys(k, lam) @ h.T          # undo H (orthonormal)
    np.testing.assert_allclose(np.abs(smoothed).max(axis=0), lam, rtol=1e-12)
    # the smoothed channel maxima are far closer to each other than the raw ones
    raw = np.abs(k).max(axis=0)
    assert raw.max() / raw.min() > 2 * (lam.max() / lam.min())


def test_transform_preserves_scores_and_attention():
    # s = (q diag(l) H)(K diag(l)^-1 H)^T = q K^T: unquantised transformed
    # attention equals untransformed attention.
    rng = np.random.default_rng(1)
    k = rng.standard_normal((500, 128))
    k[:, [5, 6, 90, 101]] *= 15
    v = rng.standard_normal((500, 128))
    q = rng.standard_normal((4, 128))
    lam = oracle.smooth_factors(k)
    kt = oracle.transform_keys(k, lam)
    qt = oracle.transform_query(q, lam)
    np.testing.assert_allclose(qt @ kt.T, q @ k.T, rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(oracle.softmax_attention(qt, kt, v),
                               oracle.softmax_attention(q, k, v), rtol=1e-11, atol=1e-12)


def test_hadamard_lemma_row_energy_and_outlier_spreading():
    # Rows keep their energy (orthonormal H) while a single-channel spike is
    # spread evenly: |K~_ij| = |K_il| / sqrt(D) for every j.
    k = np.zeros((1, 128))
    k[0, 17] = 12.0
    kt = oracle.transform_keys(k, np.ones(128))
    np.testing.assert_allclose(np.abs(kt), 12.0 / math.sqrt(128), rtol=1e-14)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128))
    x[:, 9] *= 15
    xt = oracle.transform_keys(x, np.ones(128))
    np.testing.assert_allclose((xt ** 2).sum(1), (x ** 2).sum(1), rtol=1e-12)

    def kurt(a):
        a = a - a.mean()
        return (a ** 4).mean() / (a ** 2).mean() ** 2

    assert kurt(xt) < 0.5 * kurt(x)


# --- attention ------------------------------------------------------------------

def test_softmax_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 128))
    k = rng.standard_normal((777, 128)) * 2
    v = rng.standard_normal((777, 128))
    ours = oracle.softmax_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, 5, 777, 128),
        torch.from_numpy(v)[None, None].expand(1, 5, 777, 128))[0, :, 0, :].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


# --- vector quantisation --------------------------------------------------------

def test_vq_assign_matches_scipy_vq():
    rng = np.random.default_rng(4)
    cb = rng.standard_normal((256, 4))
    x = rng.standard_normal((5000, 4)) * 1.3
    codes, best, gap = oracle.vq_assign(x, cb)
    ref_codes, ref_dist = scipy.cluster.vq.vq(x, cb)
    np.testing.assert_array_equal(codes, ref_codes)
    np.testing.assert_allclose(best, ref_dist ** 2, rtol=1e-12, atol=1e-14)
    assert np.all(gap > 0)


def test_vq_assign_bruteforce_tiny():
    rng = np.random.default_rng(5)
    cb = rng.integers(-3, 4, size=(16, 4)).astype(float)
    x = rng.integers(-3, 4, size=(40, 4)).astype(float)
    codes, _, _ = oracle.vq_assign(x, cb)
    for r in range(x.shape[0]):
        dists = [sum((x[r, i] - cb[j, i]) ** 2 for i in range(4)) for j in range(16)]
        first_min = min(range(16), key=lambda j: (dists[j], j))
        assert codes[r] == first_min


def test_vq_ties_go_to_lowest_index():
    cb = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [1.0, 0, 0, 0], [0, 0, 0, 0.0]])
    x = np.array([[0.5, 0.5, 0, 0],     # equidistant to 0, 1, 2 -> 0
                  [1.0, 0, 0, 0],       # exact match of 0 and 2 -> 0
                  [0, 0, 0, 0.5]])      # between 3 and ... 3 is nearest
    codes, _, gap = oracle.vq_assign(x, cb)
    np.testing.assert_array_equal(codes, [0, 0, 3])
    assert gap[0] == 0 and gap[1] == 0


def test_vq_encode_decode_roundtrip_on_centroids():
    rng = np.random.default_rng(6)
    cb = rng.standard_normal((256, 4)).astype(np.float16)
    codes = rng.integers(0, 256, size=(50, 32))
    x = oracle.vq_decode(codes, cb)
    assert x.shape == (50, 128)
    np.testing.assert_array_equal(x[:, 8:12], cb[codes[:, 2]].astype(np.float64))
    back, gap = oracle.vq_encode(x, cb)
    np.testing.assert_array_equal(back, codes)


# --- 12-bit layout -------------------------------------------------------------

def test_pack12_hand_worked_example():
    # code i occupies bits [12 i, 12 i + 12) of the row, little-endian:
    # 0xABC -> byte0 = 0xBC, low nibble of byte1 = 0xA; 0x123 -> high nibble
    # of byte1 = 0x3, byte2 = 0x12; 0xFFF, 0x001 -> 0xFF, 0x1F, 0x00.
    codes = np.array([[0xABC, 0x123, 0xFFF, 0x001]])
    packed = oracle.pack_codes(codes, 12)
    np.testing.assert_array_equal(packed, [[0xBC, 0x3A, 0x12, 0xFF, 0x1F, 0x00]])
    np.testing.assert_array_equal(oracle.unpack_codes(packed, 12, 4), codes)


def test_pack_roundtrip_random():
    rng = np.random.default_rng(7)
    c12 = rng.integers(0, 4096, size=(33, 32))
    p12 = oracle.pack_codes(c12, 12)
    assert p12.shape == (33, 48) and p12.dtype == np.uint8
    np.testing.assert_array_equal(oracle.unpack_codes(p12, 12, 32), c12)
    c8 = rng.integers(0, 256, size=(9, 32))
    np.testing.assert_array_equal(oracle.unpack_codes(oracle.pack_codes(c8, 8), 8, 32), c8)


# --- the dequantise + attention chain -------------------------------------------

def _lossless_layer(rng, hkv, group, n, k_bits, sub=4, v_bits=8):
    """A layer whose keys/values are exactly representable by their codebooks.

    Transformed keys are built from codebook entries, then mapped back to
    raw keys with H^T and lambda; VQ of the transformed keys is lossless, so
    VQ attention must equal textbook attention on the raw (q, K, V)."""
    dim = 128
    h = scipy.linalg.hadamard(dim) / math.sqrt(dim)
    q = rng.standard_normal((hkv * group, dim)).astype(np.float16)
    lam = (1.0 + rng.random((hkv, dim)) * 3).astype(np.float32)
    cb_k = (rng.standard_normal((hkv, 1 << k_bits, sub)) * 0.7).astype(np.float16)
    cb_v = (rng.standard_normal((hkv, 1 << v_bits, sub)) * 2).astype(np.float16)
    ck = rng.integers(0, 1 << k_bits, size=(hkv, n, dim // sub))
    cv = rng.integers(0, 1 << v_bits, size=(hkv, n, dim // sub))
    keys, vals = [], []
    for g in range(hkv):
        kt = cb_k[g].astype(np.float64)[ck[g]].reshape(n, dim)
        keys.append((kt @ h.T) * lam[g].astype(np.float64))
        vals.append(cb_v[g].astype(np.float64)[cv[g]].reshape(n, dim))
    codes_k = np.stack([oracle.pack_codes(ck[g], k_bits) for g in range(hkv)])[None]
    codes_v = np.stack([oracle.pack_codes(cv[g], v_bits) for g in range(hkv)])[None]
    return q, lam, cb_k, cb_v, codes_k, codes_v, keys, vals


@pytest.mark.parametrize("hkv,group,k_bits", [(1, 4, 8), (2, 5, 8), (3, 1, 8), (2, 4, 12)])
def test_lossless_codebook_reduces_to_textbook_attention(hkv, group, k_bits):
    rng = np.random.default_rng(10 + hkv * group + k_bits)
    n = 301
    q, lam, cb_k, cb_v, codes_k, codes_v, keys, vals = _lossless_layer(rng, hkv, group, n, k_bits)
    out = oracle.decode_attention(q[None], lam, cb_k, cb_v, codes_k, codes_v, n, k_bits, 8)[0]
    for hq in range(hkv * group):
        g = hq // group                      # GQA: query head h reads KV head h // G
        ref = oracle.softmax_attention(q[hq].astype(np.float64), keys[g], vals[g])
        np.testing.assert_allclose(out[hq], ref, rtol=1e-10, atol=1e-11)
    # the transformed keys re-encode to the same codes (lossless VQ)
    kt = oracle.transform_keys(keys[0], lam[0])
    codes, _ = oracle.vq_encode(kt, cb_k[0])
    np.testing.assert_array_equal(oracle.pack_codes(codes, k_bits), codes_k[0, 0])


@pytest.mark.parametrize("hkv,group", [(1, 4), (2, 5)])
def test_lossless_codebook_1p5bit_layout(hkv, group):
    """The VecInfer page's 1.5-bit choice (codebook-size ablation: 2^12 x 8 x 2
    bytes): 8-dim sub-vectors, 4096-entry C_k and C_v, 16 codes of 12 bits per
    vector.  With lossless codebooks it reduces to textbook attention, and the
    transformed keys and the values re-encode to their codes."""
    rng = np.random.default_rng(40 + hkv * group)
    n = 257
    q, lam, cb_k, cb_v, codes_k, codes_v, keys, vals = _lossless_layer(rng, hkv, group, n, 12,
                                                                       sub=8, v_bits=12)
    assert codes_k.shape[-1] == 24 and codes_v.shape[-1] == 24
    out = oracle.decode_attention(q[None], lam, cb_k, cb_v, codes_k, codes_v, n, 12, 12)[0]
    for hq in range(hkv * group):
        g = hq // group
        ref = oracle.softmax_attention(q[hq].astype(np.float64), keys[g], vals[g])
        np.testing.assert_allclose(out[hq], ref, rtol=1e-10, atol=1e-11)
    pk, pv, _, _ = oracle.encode_append(keys[0], vals[0], lam[0], cb_k[0], cb_v[0], 12, 12)
    np.testing.assert_array_equal(pk, codes_k[0, 0])
    np.testing.assert_array_equal(pv, codes_v[0, 0])


def test_pack12_sixteen_codes_per_row():
    """16 codes of 12 bits fill 24 bytes; code i occupies bits [12 i, 12 i + 12)
    (hand-checked on the first three codes)."""
    codes = np.array([[0xABC, 0x123, 0xFFF] + [0] * 13])
    packed = oracle.pack_codes(codes, 12)
    assert packed.shape == (1, 24)
    # bits 0-11: ABC, 12-23: 123, 24-35: FFF -> bytes BC, 3A, 12, FF, 0F
    assert list(packed[0, :5]) == [0xBC, 0x3A, 0x12, 0xFF, 0x0F]
    np.testing.assert_array_equal(oracle.unpack_codes(packed, 12, 16), codes)


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(20)
    cb_k = rng.standard_normal((1, 256, 4)).astype(np.float16)
    cb_v = rng.standard_normal((1, 256, 4)).astype(np.float16)
    codes_k = rng.integers(0, 256, size=(1, 1, 1, 32)).astype(np.uint8)
    codes_v = rng.integers(0, 256, size=(1, 1, 1, 32)).astype(np.uint8)
    q = rng.standard_normal((1, 3, 128)).astype(np.float32)
    lam = np.ones((1, 128), np.float32)
    out = oracle.decode_attention(q, lam, cb_k, cb_v, codes_k, codes_v, 1)
    row = cb_v[0].astype(np.float64)[codes_v[0, 0, 0].astype(int)].reshape(128)
    for h in range(3):
        np.testing.assert_array_equal(out[0, h], row)


def test_identical_keys_give_uniform_weights():
    rng = np.random.default_rng(21)
    n = 97
    cb_k = rng.standard_normal((1, 256, 4)).astype(np.float16)
    cb_v = rng.standard_normal((1, 256, 4)).astype(np.float16)
    codes_k = np.tile(rng.integers(0, 256, size=(1, 1, 1, 32)), (1, 1, n, 1)).astype(np.uint8)
    codes_v = rng.integers(0, 256, size=(1, 1, n, 32)).astype(np.uint8)
    q = rng.standard_normal((1, 2, 128)).astype(np.float32)
    lam = (1 + rng.random((1, 128))).astype(np.float32)
    out = oracle.decode_attention(q, lam, cb_k, cb_v, codes_k, codes_v, n)
    vhat = cb_v[0].astype(np.float64)[codes_v[0, 0].astype(int)].reshape(n, 128)
    np.testing.assert_allclose(out[0, 0], vhat.mean(0), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out[0, 1], vhat.mean(0), rtol=1e-12, atol=1e-13)


# --- residual window ------------------------------------------------------------

def test_window_empty_equals_codes_only():
    rng = np.random.default_rng(40)
    q, lam, cb_k, cb_v, codes_k, codes_v, _, _ = _lossless_layer(rng, 2, 4, 77, 8)
    win = np.zeros((1, 2, 5, 128))
    a = oracle.decode_attention_window(q[None], lam, cb_k, cb_v, codes_k, codes_v, 77, win, win, 0)
    b = oracle.decode_attention(q[None], lam, cb_k, cb_v, codes_k, codes_v, 77)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("hkv,group", [(1, 4), (2, 3)])
def test_window_only_is_raw_domain_attention(hkv, group):
    # no codes: the window keys are used untransformed against the raw query
    rng = np.random.default_rng(41 + hkv)
    n = 9
    q = rng.standard_normal((1, hkv * group, 128)).astype(np.float16)
    lam = (1 + 3 * rng.random((hkv, 128))).astype(np.float32)
    cb_k = rng.standard_normal((hkv, 256, 4)).astype(np.float16)
    cb_v = rng.standard_normal((hkv, 256, 4)).astype(np.float16)
    codes = np.zeros((1, hkv, 4, 32), np.uint8)
    wk = rng.standard_normal((1, hkv, n, 128)).astype(np.float16)
    wv = rng.standard_normal((1, hkv, n, 128)).astype(np.float16)
    out = oracle.decode_attention_window(q, lam, cb_k, cb_v, codes, codes, 0, wk, wv, n)
    for h in range(hkv * group):
        ref = oracle.softmax_attention(q[0, h].astype(np.float64), wk[0, h // group], wv[0, h // group])
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("hkv,group,k_bits,moved", [(1, 4, 8, 1), (2, 5, 8, 17), (2, 4, 12, 60)])
def test_window_token_equals_its_coded_twin(hkv, group, k_bits, moved):
    # a coded token and its raw-domain key/value placed in the window instead
    # contribute the same term: moving the last tokens changes nothing
    rng = np.random.default_rng(50 + moved)
    n = 140
    q, lam, cb_k, cb_v, codes_k, codes_v, keys, vals = _lossless_layer(rng, hkv, group, n, k_bits)
    full = oracle.decode_attention(q[None], lam, cb_k, cb_v, codes_k, codes_v, n, k_bits, 8)
    wk = np.stack([keys[g][n - moved:] for g in range(hkv)])[None]
    wv = np.stack([vals[g][n - moved:] for g in range(hkv)])[None]
    split = oracle.decode_attention_window(q[None], lam, cb_k, cb_v, codes_k, codes_v, n - moved,
                                           wk, wv, moved, k_bits, 8)
    np.testing.assert_allclose(split, full, rtol=1e-10, atol=1e-11)


def test_encode_append_lossless_keys():
    rng = np.random.default_rng(22)
    q, lam, cb_k, cb_v, codes_k, codes_v, keys, vals = _lossless_layer(rng, 1, 1, 40, 8)
    pk, pv, gk, gv = oracle.encode_append(keys[0], vals[0], lam[0], cb_k[0], cb_v[0])
    np.testing.assert_array_equal(pk, codes_k[0, 0])
    np.testing.assert_array_equal(pv, codes_v[0, 0])


# --- codebook training (fixture only) -------------------------------------------

def test_lloyd_matches_scikit_learn():
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(30)
    centers = rng.standard_normal((16, 4)) * 4
    x = centers[rng.integers(0, 16, 3000)] + rng.standard_normal((3000, 4))
    init = x[:16].copy()
    ours = oracle.lloyd_kmeans(x, init, 6)
    km = KMeans(n_clusters=16, init=init, n_init=1, max_iter=6, tol=0.0,
                algorithm="lloyd").fit(x)
    # scikit-learn may stop early once labels are stable; more Lloyd steps
    # from a fixed point do not move it.
    np.testing.assert_allclose(ours, km.cluster_centers_, rtol=1e-9, atol=1e-9)


def test_lloyd_objective_never_increases():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4000, 4))
    c = x[:64].copy()
    prev = np.inf
    for _ in range(5):
        _, d, _ = oracle.vq_assign(x, c)
        obj = d.sum()
        assert obj <= prev + 1e-9
        prev = obj
        c = oracle.lloyd_kmeans(x, c, 1)


def test_lloyd_mean_is_the_in_order_sum():
    """One Lloyd step written as plain Python loops (nearest centroid by the
    channel-ordered squared distance, first minimum; each cluster's samples
    added one by one in sample order from 0.0, then one division) equals the
    oracle bit for bit, including an empty cluster that keeps its place."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((300, 4)) * [1.0, 3.0, 0.5, 2.0]).astype(np.float32).astype(np.float64)
    init = x[:6].copy()
    init[5] = [50.0, 50.0, 50.0, 50.0]          # far away: receives no sample
    sums = [[0.0] * 4 for _ in range(6)]
    counts = [0] * 6
    for row in x.tolist():
        best, arg = None, None
        for j, cen in enumerate(init.tolist()):
            d = 0.0
            for a, b in zip(row, cen):
                d = d + (a - b) * (a - b)
            if best is None or d < best:
                best, arg = d, j
        counts[arg] += 1
        for i in range(4):
            sums[arg][i] = sums[arg][i] + row[i]
    want = init.copy()
    for j in range(6):
        if counts[j]:
            want[j] = [v / counts[j] for v in sums[j]]
    got = oracle.lloyd_kmeans(x, init, 1)
    assert counts[5] == 0
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


# --- byte counts the pages print ------------------------------------------------

def test_byte_counts_match_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "byte_counts.json")))
    g = gold["codebook_2bit"]
    assert oracle.codebook_bytes(g["bits"], g["sub_dim"], g["elem_bytes"]) == g["value"]
    g = gold["codebook_1p5bit"]
    assert oracle.codebook_bytes(g["bits"], g["sub_dim"], g["elem_bytes"]) == g["value"]
    for key in ("index_bytes_2bit", "index_bytes_1p5bit"):
        g = gold[key]
        assert oracle.index_bytes(g["head_dim"], g["sub_dim"], g["bits"]) == g["value"]
    g = gold["reduction_2bit"]
    assert oracle.commvq_reduction_ratio(g["code_bits"], g["dim"]) == pytest.approx(g["value"])
    # the stored 8-bit code row of a 128-dim head is the index byte count
    codes = np.zeros((1, 32), dtype=np.int64)
    assert oracle.pack_codes(codes, 8).nbytes == gold["index_bytes_2bit"]["value"]
    assert oracle.pack_codes(codes, 12).nbytes == 48


def test_bruteforce_tiny_decode_attention_loops():
    # pure-Python loops over a tiny cache, independent of numpy broadcasting
    rng = np.random.default_rng(40)
    n = 5
    cb_k = rng.standard_normal((1, 256, 4)).astype(np.float16)
    cb_v = rng.standard_normal((1, 256, 4)).astype(np.float16)
    ck = rng.integers(0, 256, size=(n, 32))
    cv = rng.integers(0, 256, size=(n, 32))
    q = rng.standard_normal(128).astype(np.float32)
    lam = (0.5 + rng.random(128)).astype(np.float32)
    hd = [[(-1) ** bin(i & j).count("1") / math.sqrt(128) for j in range(128)] for i in range(128)]
    qs = [float(q[i]) * float(lam[i]) for i in range(128)]
    qt = [sum(qs[i] * hd[i][j] for i in range(128)) for j in range(128)]
    scores = []
    for t in range(n):
        s = 0.0
        for p, j in itertools.product(range(32), range(4)):
            s += qt[4 * p + j] * float(cb_k[0, ck[t, p], j])
        scores.append(s / math.sqrt(128))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    ref = [sum(w[t] * float(cb_v[0, cv[t, d // 4], d % 4]) for t in range(n)) / tot for d in range(128)]
    out = oracle.decode_attention(q[None, None], lam[None], cb_k, cb_v,
                                  ck[None, None].astype(np.uint8), cv[None, None].astype(np.uint8), n)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-10, atol=1e-12)
