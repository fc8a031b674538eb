"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances on attention outputs are relative L2 <= 1e-3 over the whole
output and max-abs <= 2e-3.  Value codes must be bit-identical.  Key codes
must be bit-identical wherever the fp64 reference has a strict winner
(distance gap above 1e-9 (1 + d)); at a gap below that both indices are
nearest to within fp64 rounding of the key transform and the GPU's pick must
be one of the tied minima.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W
from fixtures import attention_errors, chain_cache, expected_all, expected_head, random_cache

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3
ABS_TOL = 2e-3
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def upload(c):
    return dict(q=dev(c.q), lam=dev(c.lam), cb_k=dev(c.cb_k), cb_v=dev(c.cb_v),
                codes_k=dev(c.codes_k), codes_v=dev(c.codes_v))


def run_attention(d, n, splits=0):
    out = vq.decode_attention(d["q"], d["lam"], d["cb_k"], d["cb_v"], d["codes_k"], d["codes_v"],
                              n, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def assert_close(got, ref, what):
    rel, mab = attention_errors(got, ref)
    print(f"{what}: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert rel <= REL_TOL and mab <= ABS_TOL, (what, rel, mab)


# --- query transform --------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_transform_query_matches_oracle(dtype):
    rng = np.random.default_rng(100)
    q = W.as_storage(rng.standard_normal((3, 8, 128)) * 2, dtype)
    lam = (0.5 + rng.random((2, 128)) * 4).astype(np.float32)
    got = vq.transform_query(dev(q), dev(lam)).cpu().numpy().astype(np.float64)
    ref = np.stack([oracle.transform_query(q[b, h], lam[h // 4]) for b in range(3)
                    for h in range(8)]).reshape(3, 8, 128)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"transform_query {dtype}: max rel {err:.2e}", flush=True)
    assert err < 2e-6


# --- decode attention: the tiny recipe case, in full ----------------------------------

@pytest.fixture(scope="module")
def tiny():
    c = chain_cache(W.WORKLOADS[1])
    return c, upload(c), expected_all(c)


def test_tiny_recipe_case_matches_oracle(tiny):
    c, d, ref = tiny
    assert_close(run_attention(d, c.context_len), ref, "config1 chain")


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 64])
def test_split_count_does_not_change_the_result(tiny, splits):
    c, d, ref = tiny
    assert_close(run_attention(d, c.context_len, splits), ref, f"config1 splits={splits}")


def test_repeated_calls_agree_to_rounding(tiny):
    # tiles are handed to waves dynamically, so summation order may differ
    c, d, _ = tiny
    a = run_attention(d, c.context_len)
    for _ in range(3):
        b = run_attention(d, c.context_len)
        np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-6)


def test_workspace_contents_do_not_matter(tiny):
    c, d, ref = tiny
    n = c.context_len
    args = (d["codes_k"], d["codes_v"], d["cb_k"], d["cb_v"], 1, 4, n)
    ws = torch.full((vq.decode_attention_workspace_bytes(*args, 4),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    outs = []
    for splits in (2, 1, 2):
        o = vq.decode_attention(d["q"], d["lam"], d["cb_k"], d["cb_v"], d["codes_k"],
                                d["codes_v"], n, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy().astype(np.float64))
    for o in outs:
        assert_close(o, ref, "config1 reused workspace")


@pytest.mark.parametrize("n", [1, 2, 7, 255, 256, 257, 511, 700, 1024])
def test_ragged_context_lengths(tiny, n):
    c, d, _ = tiny
    assert_close(run_attention(d, n), expected_all(c, n), f"config1 n={n}")


@pytest.mark.parametrize("group,k_bits,n", [(1, 8, 300), (2, 8, 1000), (3, 12, 777),
                                            (5, 12, 1500), (6, 8, 513), (8, 8, 2049),
                                            (8, 12, 600)])
def test_group_sizes_and_code_widths(group, k_bits, n):
    wl = W.Workload(90 + group, "adhoc", batch=2, num_q_heads=2 * group, num_kv_heads=2,
                    context_len=n, k_bits=k_bits, qkv_dtype="f16")
    c = random_cache(wl)
    d = upload(c)
    assert_close(run_attention(d, n), expected_all(c), f"G={group} kbits={k_bits} n={n}")


# --- decode attention at the full workload sizes (sampled outputs) --------------------

FULL = [(2, [(0, 0), (0, 5)]), (3, [(0, 1), (9, 7), (15, 3)]), (4, [(0, 2), (0, 7)]),
        (5, [(0, 0), (6, 4)])]


@pytest.mark.parametrize("config,samples", FULL)
def test_full_size_sampled_heads(config, samples):
    wl = W.WORKLOADS[config]
    c = random_cache(wl)
    d = upload(c)
    splits = vq.decode_attention_default_splits(d["codes_k"], d["codes_v"], d["cb_k"], d["cb_v"],
                                                wl.batch, wl.num_q_heads, wl.context_len)
    print(f"config{config}: default splits {splits}", flush=True)
    got = run_attention(d, wl.context_len)
    assert np.isfinite(got).all()
    g = wl.group
    for b, h in samples:
        ref = expected_head(c, b, h)
        assert_close(got[b, h * g:(h + 1) * g], ref, f"config{config} b={b} kv={h}")


# --- encoder ------------------------------------------------------------------------

def check_codes(got_rows, ref_rows, gaps, bits, x=None, cb=None, what="", sub=4, values=False):
    """Codes of the GPU encoder against the oracle's.  Value codes must be
    identical: values are not transformed, and the GPU evaluates the fp64
    distances in the oracle's order with every operation rounded as the
    oracle rounds it.  Key codes follow a fp64 transform whose butterfly
    order differs from the oracle's matrix product, so at an fp64 near-tie
    (gap <= 1e-9 (1 + d)) either of the tied minima is accepted."""
    num_sub = 128 // sub
    got = oracle.unpack_codes(got_rows, bits, num_sub)
    ref = oracle.unpack_codes(ref_rows, bits, num_sub)
    gaps = np.asarray(gaps)
    mism = got != ref
    n_mis = int(mism.sum())
    print(f"{what}: {got.size} codes, {n_mis} differ, min gap {gaps.min():.3e}", flush=True)
    if values:
        assert n_mis == 0, what
    if n_mis:
        # every difference must sit at an fp64 near-tie: both picks are nearest
        # centroids to within rounding
        xs = np.asarray(x, np.float64).reshape(-1, num_sub, sub)[mism]
        cbd = np.asarray(cb, np.float64)
        dg = ((xs - cbd[got[mism]]) ** 2).sum(-1)
        dr = ((xs - cbd[ref[mism]]) ** 2).sum(-1)
        assert np.all(gaps[mism] <= 1e-9 * (1 + dr)), what
        assert np.all(np.abs(dg - dr) <= 1e-9 * (1 + dr)), what


def test_encoder_tiny_recipe_case_bit_exact(tiny):
    c, d, _ = tiny
    wl = c.wl
    n = wl.context_len
    k = W.kv_rows(1, 0, 0, "k", n).astype(np.float32)[None, None]
    v = W.kv_rows(1, 0, 0, "v", n).astype(np.float32)[None, None]
    ck = torch.zeros_like(d["codes_k"])
    cv = torch.zeros_like(d["codes_v"])
    vq.encode_append(dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"], ck, cv, 0)
    torch.cuda.synchronize()
    _, _, gk, gv = oracle.encode_append(k[0, 0], v[0, 0], c.lam[0], c.cb_k[0], c.cb_v[0])
    kt = oracle.transform_keys(k[0, 0], c.lam[0])
    check_codes(ck.cpu().numpy()[0, 0, :n], c.codes_k[0, 0, :n], gk, 8, kt, c.cb_k[0], "enc K c1")
    check_codes(cv.cpu().numpy()[0, 0, :n], c.codes_v[0, 0, :n], gv, 8, v[0, 0], c.cb_v[0],
                "enc V c1", values=True)
    # the GPU-encoded cache then decodes to the oracle's attention
    d2 = dict(d, codes_k=ck, codes_v=cv)
    assert_close(run_attention(d2, n), expected_all(c), "config1 encode->attend")


def test_encoder_append_mixed_bits_full_size():
    wl = W.WORKLOADS[5]
    bsz, hkv, t_new, cur = wl.batch, wl.num_kv_heads, wl.append_tokens, wl.context_len
    lam = np.stack([W.random_lambda(5, g) for g in range(hkv)])
    cb_k = np.stack([W.random_codebook(5, g, "k", 4096, 0.6) for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(5, g, "v", 256, 1.0, 1 / 32) for g in range(hkv)])
    k = np.stack([np.stack([W.kv_rows(5, b, g, "k", t_new, append=True) for g in range(hkv)])
                  for b in range(bsz)]).astype(np.float16)
    v = np.stack([np.stack([W.kv_rows(5, b, g, "v", t_new, append=True) for g in range(hkv)])
                  for b in range(bsz)]).astype(np.float16)
    cap = wl.capacity
    ck = torch.full((bsz, hkv, cap, 48), 0xA5, dtype=torch.uint8, device=DEV)
    cv = torch.full((bsz, hkv, cap, 32), 0x5A, dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, cur)
    torch.cuda.synchronize()
    ckh = ck.cpu().numpy()
    cvh = cv.cpu().numpy()
    # nothing outside the appended slots changed
    assert np.all(ckh[:, :, :cur] == 0xA5) and np.all(cvh[:, :, :cur] == 0x5A)
    for b in range(bsz):
        for g in range(hkv):
            pk, pv, gk, gv = oracle.encode_append(k[b, g], v[b, g], lam[g], cb_k[g], cb_v[g], 12, 8)
            kt = oracle.transform_keys(k[b, g], lam[g])
            check_codes(ckh[b, g, cur:cur + t_new], pk, gk, 12, kt, cb_k[g], f"enc K c5 b{b} g{g}")
            check_codes(cvh[b, g, cur:cur + t_new], pv, gv, 8, v[b, g], cb_v[g], f"enc V c5 b{b} g{g}", values=True)


@pytest.mark.parametrize("k_bits,t_new,cur,dtype", [(8, 1, 0, "f16"), (8, 9, 7, "f32"),
                                                     (12, 1, 3, "f16"), (12, 7, 0, "f16"),
                                                     (12, 33, 100, "f32")])
def test_encode_append_ragged(k_bits, t_new, cur, dtype):
    # token counts that leave a workgroup partly empty (4 or 8 tokens per
    # workgroup), into the middle of a cache whose other slots stay untouched
    bsz, hkv = 2, 2
    lam = np.stack([W.random_lambda(150 + k_bits, g) for g in range(hkv)])
    cb_k = np.stack([W.random_codebook(150 + k_bits, g, "k", 1 << k_bits, 0.6)
                     for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(150 + k_bits, g, "v", 256, 1.0, 1 / 32)
                     for g in range(hkv)])
    st = np.float16 if dtype == "f16" else np.float32
    k = np.stack([np.stack([W.kv_rows(150 + k_bits, b, g, "k", t_new, append=True)
                            for g in range(hkv)]) for b in range(bsz)]).astype(st)
    v = np.stack([np.stack([W.kv_rows(150 + k_bits, b, g, "v", t_new, append=True)
                            for g in range(hkv)]) for b in range(bsz)]).astype(st)
    cap, krow = cur + t_new + 3, 32 * k_bits // 8
    ck = torch.full((bsz, hkv, cap, krow), 0xA5, dtype=torch.uint8, device=DEV)
    cv = torch.full((bsz, hkv, cap, 32), 0x5A, dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, cur)
    torch.cuda.synchronize()
    ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
    outside = np.ones(cap, bool)
    outside[cur:cur + t_new] = False
    assert np.all(ckh[:, :, outside] == 0xA5) and np.all(cvh[:, :, outside] == 0x5A)
    for b in range(bsz):
        for g in range(hkv):
            pk, pv, gk, gv = oracle.encode_append(k[b, g], v[b, g], lam[g], cb_k[g], cb_v[g],
                                                  k_bits, 8)
            kt = oracle.transform_keys(k[b, g], lam[g])
            check_codes(ckh[b, g, cur:cur + t_new], pk, gk, k_bits, kt, cb_k[g],
                        f"ragged enc K b{b} g{g}")
            check_codes(cvh[b, g, cur:cur + t_new], pv, gv, 8, v[b, g], cb_v[g],
                        f"ragged enc V b{b} g{g}", values=True)


def test_encoder_exact_ties_go_to_lowest_index():
    rng = np.random.default_rng(200)
    base = rng.standard_normal((128, 4)).astype(np.float16)
    cb_v = np.concatenate([base, base])[None]              # entry j and j+128 identical
    cb_k = cb_v.copy()
    # values equal to centroid entries: both copies tie at distance 0
    codes = rng.integers(0, 128, size=(5, 32))
    v = base.astype(np.float64)[codes].reshape(5, 128).astype(np.float32)[None, None]
    lam = np.ones((1, 128), np.float32)
    ck = torch.zeros((1, 1, 8, 32), dtype=torch.uint8, device=DEV)
    cv = torch.zeros((1, 1, 8, 32), dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(v), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, 2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cv.cpu().numpy()[0, 0, 2:7], codes)
    assert cv.cpu().numpy()[0, 0, 2:7].max() < 128


@pytest.mark.parametrize("t_new", [40, 1030])
def test_encoder12_exact_ties_go_to_lowest_index(t_new):
    # C_k's second half repeats its first (4096 entries): every key sub-vector
    # has two nearest centroids at exactly the same distance, 2048 apart and
    # so in different runs of the search (which skips runs that cannot hold
    # a candidate), and must take the lower index.  40 tokens run 4-token
    # workgroups, 1030 tokens 8-token ones.
    bsz, hkv = 1, 2
    lam = np.stack([W.random_lambda(170, g) for g in range(hkv)])
    half = np.stack([W.random_codebook(170, g, "k", 2048, 0.6) for g in range(hkv)])
    cb_k = np.ascontiguousarray(np.concatenate([half, half], axis=1))
    cb_v = np.stack([W.random_codebook(170, g, "v", 256, 1.0, 1 / 32) for g in range(hkv)])
    k = np.stack([W.kv_rows(170, 0, g, "k", t_new, append=True) for g in range(hkv)])[None]
    v = np.stack([W.kv_rows(170, 0, g, "v", t_new, append=True) for g in range(hkv)])[None]
    k, v = k.astype(np.float16), v.astype(np.float16)
    ck = torch.zeros((bsz, hkv, t_new, 48), dtype=torch.uint8, device=DEV)
    cv = torch.zeros((bsz, hkv, t_new, 32), dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, 0)
    torch.cuda.synchronize()
    ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
    for g in range(hkv):
        assert oracle.unpack_codes(ckh[0, g], 12, 32).max() < 2048
        pk, pv, gk, gv = oracle.encode_append(k[0, g], v[0, g], lam[g], cb_k[g], cb_v[g], 12, 8)
        kt = oracle.transform_keys(k[0, g], lam[g])
        check_codes(ckh[0, g], pk, gk, 12, kt, cb_k[g], f"12-bit ties K g{g} t={t_new}")
        check_codes(cvh[0, g], pv, gv, 8, v[0, g], cb_v[g], f"12-bit ties V g{g} t={t_new}",
                    values=True)


# --- fp16 comparator -----------------------------------------------------------------

@pytest.mark.parametrize("bsz,hq,hkv,n", [(1, 4, 1, 1), (1, 4, 1, 1000), (2, 10, 2, 3001),
                                          (1, 32, 8, 32768)])
def test_fp16_attention_matches_oracle(bsz, hq, hkv, n):
    rng = np.random.default_rng(300 + n)
    q = rng.standard_normal((bsz, hq, 128)).astype(np.float16)
    k = (rng.standard_normal((bsz, hkv, n + 5, 128)) * 1.5).astype(np.float16)
    v = rng.standard_normal((bsz, hkv, n + 5, 128)).astype(np.float16)
    out = vq.fp16_decode_attention(dev(q), dev(k), dev(v), n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    g = hq // hkv
    ref = np.stack([np.stack([oracle.softmax_attention(q[b, h].astype(np.float64),
                                                       k[b, h // g, :n], v[b, h // g, :n])
                              for h in range(hq)]) for b in range(bsz)])
    assert_close(got, ref, f"fp16 b={bsz} hq={hq} hkv={hkv} n={n}")


# --- prepared calls (arguments marshalled once) ----------------------------------------

def test_prepared_calls_match_direct_calls(tiny):
    c, d, ref = tiny
    wl = c.wl
    n = wl.context_len
    k = W.kv_rows(1, 0, 0, "k", n).astype(np.float32)[None, None]
    v = W.kv_rows(1, 0, 0, "v", n).astype(np.float32)[None, None]
    ck, cv = torch.zeros_like(d["codes_k"]), torch.zeros_like(d["codes_v"])
    ck2, cv2 = torch.zeros_like(ck), torch.zeros_like(cv)
    vq.encode_append(dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"], ck, cv, 0)
    enc = vq.prepare_encode_append(dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"], ck2, cv2, 0)
    enc()
    torch.cuda.synchronize()
    assert torch.equal(ck, ck2) and torch.equal(cv, cv2)
    att = vq.prepare_decode_attention(d["q"], d["lam"], d["cb_k"], d["cb_v"], ck2, cv2, n)
    for _ in range(2):
        att()
        torch.cuda.synchronize()
        assert_close(att.out.cpu().numpy().astype(np.float64), expected_all(c), "prepared")


def test_prepared_step_replays_in_a_graph(tiny):
    # append + attention captured once; every replay, with eager work and
    # synchronisations in between, must give the eager result
    c, d, _ = tiny
    wl = c.wl
    n = wl.context_len
    k = dev(W.kv_rows(1, 0, 0, "k", 1, append=True).astype(np.float32)[None, None])
    v = dev(W.kv_rows(1, 0, 0, "v", 1, append=True).astype(np.float32)[None, None])
    ck, cv = d["codes_k"].clone(), d["codes_v"].clone()
    enc = vq.prepare_encode_append(k, v, d["lam"], d["cb_k"], d["cb_v"], ck, cv, n - 1)
    att = vq.prepare_decode_attention(d["q"], d["lam"], d["cb_k"], d["cb_v"], ck, cv, n)
    enc()
    att()
    torch.cuda.synchronize()
    eager = att.out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            enc()
            att()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        att.out.fill_(float("nan"))
        run_attention(d, n)                      # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_allclose(att.out.cpu().numpy(), eager.cpu().numpy(), rtol=1e-5,
                                   atol=1e-6, err_msg=f"replay {rep}")


# --- split pass and merge as separate calls -------------------------------------------

def test_partials_then_merge_equals_decode_attention(tiny):
    c, d, ref = tiny
    n = c.context_len
    args = (d["q"], d["lam"], d["cb_k"], d["cb_v"], d["codes_k"], d["codes_v"], n)
    for splits in (1, 2):
        parts = vq.decode_attention_partials(*args, num_splits=splits)
        assert parts[0].shape[2] == splits
        out = vq.merge_partials(parts)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), ref, f"partials+merge S={splits}")


def test_merging_partials_of_context_shards(tiny):
    # two caches holding disjoint token ranges (as two devices would): their
    # partials, concatenated over the split axis, merge to the full attention
    c, d, ref = tiny
    n = c.context_len
    cut = 700
    shards = [(d["codes_k"][:, :, :cut].contiguous(), d["codes_v"][:, :, :cut].contiguous(), cut),
              (d["codes_k"][:, :, cut:n].contiguous(), d["codes_v"][:, :, cut:n].contiguous(),
               n - cut)]
    parts = [vq.decode_attention_partials(d["q"], d["lam"], d["cb_k"], d["cb_v"], ck, cv, m)
             for ck, cv, m in shards]
    m = torch.cat([p[0] for p in parts], dim=2).contiguous()
    l = torch.cat([p[1] for p in parts], dim=2).contiguous()
    o = torch.cat([p[2] for p in parts], dim=2).contiguous()
    out = vq.merge_partials((m, l, o))
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref, "merged shards")


# --- decode step: append one token, then attend (one split-kernel launch) -------------

def new_rows(wl, bsz, hkv, dtype):
    k = np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "k", 1, append=True)[0]
                            for g in range(hkv)]) for b in range(bsz)]).astype(dtype)
    v = np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "v", 1, append=True)[0]
                            for g in range(hkv)]) for b in range(bsz)]).astype(dtype)
    return k, v


def check_step(c, cur, splits=0, heads=None, what=""):
    """decode_step at slot `cur` of cache `c`: codes at that slot bit-exact to
    the oracle encoder (near-tie rule), nothing else written, output equal to
    the oracle's attention over the cache read back from the device."""
    wl = c.wl
    bsz, hkv = c.codes_k.shape[:2]
    dtype = np.float32 if wl.qkv_dtype == "f32" else np.float16
    k, v = new_rows(wl, bsz, hkv, dtype)
    d = upload(c)
    out = vq.decode_step(d["q"], dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"], d["codes_k"],
                         d["codes_v"], cur, num_splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ck, cv = d["codes_k"].cpu().numpy(), d["codes_v"].cpu().numpy()
    others = np.ones(ck.shape[2], bool)
    others[cur] = False
    assert np.array_equal(ck[:, :, others], c.codes_k[:, :, others]), what
    assert np.array_equal(cv[:, :, others], c.codes_v[:, :, others]), what
    kb, vb, sd = wl.k_bits, wl.v_bits, wl.sub_dim
    for b in range(bsz):
        for g in range(hkv):
            pk, pv, gk, gv = oracle.encode_append(k[b, g][None], v[b, g][None], c.lam[g],
                                                  c.cb_k[g], c.cb_v[g], kb, vb)
            kt = oracle.transform_keys(k[b, g][None], c.lam[g])
            check_codes(ck[b, g, cur:cur + 1], pk, gk, kb, kt, c.cb_k[g], f"{what} K b{b} g{g}",
                        sd)
            check_codes(cv[b, g, cur:cur + 1], pv, gv, vb, v[b, g][None], c.cb_v[g],
                        f"{what} V b{b} g{g}", sd, values=True)
    after = dataclasses.replace(c, codes_k=ck, codes_v=cv, context_len=cur + 1)
    if heads is None:
        assert_close(got, expected_all(after), what)
    else:
        grp = wl.group
        for b, g in heads:
            assert_close(got[b, g * grp:(g + 1) * grp], expected_head(after, b, g),
                         f"{what} b={b} kv={g}")
    return got, ck, cv


@pytest.mark.parametrize("cur,splits", [(0, 0), (1, 0), (31, 0), (32, 0), (33, 2), (511, 0),
                                        (512, 2), (700, 0), (1023, 0), (1023, 2)])
def test_decode_step_slot_positions(cur, splits):
    wl = W.Workload(80, "adhoc", batch=2, num_q_heads=8, num_kv_heads=2, context_len=1024)
    check_step(random_cache(wl), cur, splits, what=f"step cur={cur} S={splits}")


@pytest.mark.parametrize("group,k_bits,cur,splits", [(5, 12, 1499, 0), (5, 12, 700, 2),
                                                     (1, 8, 300, 0), (8, 12, 64, 0)])
def test_decode_step_groups_and_widths(group, k_bits, cur, splits):
    wl = W.Workload(85 + group, "adhoc", batch=2, num_q_heads=2 * group, num_kv_heads=2,
                    context_len=1500, k_bits=k_bits)
    check_step(random_cache(wl), cur, splits, what=f"step G={group} kbits={k_bits} cur={cur}")


def test_decode_step_exact_ties_go_to_lowest_index():
    # C_k's second half repeats its first (4096 entries, 12-bit keys) and C_v's
    # does too (256 entries): every sub-vector of the new token has two
    # nearest centroids at exactly the same distance, in different waves of
    # the key search, and must take the lower index
    wl = W.Workload(95, "adhoc", batch=2, num_q_heads=8, num_kv_heads=2, context_len=600,
                    k_bits=12)
    c = random_cache(wl)
    hk, hv = c.cb_k[:, :2048], c.cb_v[:, :128]
    c = dataclasses.replace(c, cb_k=np.ascontiguousarray(np.concatenate([hk, hk], axis=1)),
                            cb_v=np.ascontiguousarray(np.concatenate([hv, hv], axis=1)))
    _, ck, cv = check_step(c, 599, what="step exact ties")
    assert oracle.unpack_codes(ck[:, :, 599].reshape(-1, 48), 12, 32).max() < 2048
    assert cv[:, :, 599].max() < 128


@pytest.mark.parametrize("k_bits,group,splits", [(8, 4, 2), (8, 4, 1), (12, 5, 2), (12, 1, 1)])
def test_decode_step_folded(k_bits, group, splits):
    # 32 streams with splits long against the new token's encode (20000 or
    # 40000 cached tokens in one or two splits): the last split of each stream
    # encodes the new token before attending over its own, shorter range
    n = 20000 if k_bits == 8 else 40000
    wl = W.Workload(96 + group, "adhoc", batch=8, num_q_heads=4 * group, num_kv_heads=4,
                    context_len=n + 1, k_bits=k_bits)
    c = random_cache(wl)
    check_step(c, n, splits, heads=[(0, 0), (3, 1), (5, 2), (7, 3)],
               what=f"folded step kbits={k_bits} G={group} S={splits}")


def test_decode_step_folded_equals_append_then_attend():
    wl = W.Workload(99, "adhoc", batch=8, num_q_heads=16, num_kv_heads=4, context_len=30001,
                    k_bits=12)
    c = random_cache(wl)
    cur = 30000
    k, v = new_rows(wl, 8, 4, np.float16)
    d1, d2 = upload(c), upload(c)
    out1 = vq.decode_step(d1["q"], dev(k), dev(v), d1["lam"], d1["cb_k"], d1["cb_v"],
                          d1["codes_k"], d1["codes_v"], cur, num_splits=2)   # folded
    vq.encode_append(dev(k[:, :, None]), dev(v[:, :, None]), d2["lam"], d2["cb_k"], d2["cb_v"],
                     d2["codes_k"], d2["codes_v"], cur)
    out2 = vq.decode_attention(d2["q"], d2["lam"], d2["cb_k"], d2["cb_v"], d2["codes_k"],
                               d2["codes_v"], cur + 1)
    torch.cuda.synchronize()
    assert torch.equal(d1["codes_k"], d2["codes_k"]) and torch.equal(d1["codes_v"], d2["codes_v"])
    np.testing.assert_allclose(out1.cpu().numpy(), out2.cpu().numpy(), rtol=1e-5, atol=1e-6)


def test_decode_step_tiny_recipe_case(tiny):
    # the chain's last token appended by the step: the oracle's own codes and
    # attention over the whole chain (fp32 rows)
    c, d, ref = tiny
    n = c.context_len
    k = W.kv_rows(1, 0, 0, "k", n).astype(np.float32)[n - 1][None, None]
    v = W.kv_rows(1, 0, 0, "v", n).astype(np.float32)[n - 1][None, None]
    ck, cv = d["codes_k"].clone(), d["codes_v"].clone()
    ck[:, :, n - 1] = 0
    cv[:, :, n - 1] = 0
    out = vq.decode_step(d["q"], dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"], ck, cv, n - 1)
    torch.cuda.synchronize()
    k1, v1 = k[0, 0][None], v[0, 0][None]
    _, _, gk, gv = oracle.encode_append(k1, v1, c.lam[0], c.cb_k[0], c.cb_v[0])
    check_codes(ck.cpu().numpy()[0, 0, n - 1:n], c.codes_k[0, 0, n - 1:n], gk, 8,
                oracle.transform_keys(k1, c.lam[0]), c.cb_k[0], "step chain K")
    check_codes(cv.cpu().numpy()[0, 0, n - 1:n], c.codes_v[0, 0, n - 1:n], gv, 8, v1,
                c.cb_v[0], "step chain V", values=True)
    assert_close(out.cpu().numpy().astype(np.float64), ref, "step chain")


def test_decode_step_equals_append_then_attend():
    wl = W.Workload(81, "adhoc", batch=2, num_q_heads=8, num_kv_heads=2, context_len=3000)
    c = random_cache(wl)
    cur = 2999
    k, v = new_rows(wl, 2, 2, np.float16)
    d1, d2 = upload(c), upload(c)
    out1 = vq.decode_step(d1["q"], dev(k), dev(v), d1["lam"], d1["cb_k"], d1["cb_v"],
                          d1["codes_k"], d1["codes_v"], cur)
    vq.encode_append(dev(k[:, :, None]), dev(v[:, :, None]), d2["lam"], d2["cb_k"], d2["cb_v"],
                     d2["codes_k"], d2["codes_v"], cur)
    out2 = vq.decode_attention(d2["q"], d2["lam"], d2["cb_k"], d2["cb_v"], d2["codes_k"],
                               d2["codes_v"], cur + 1)
    torch.cuda.synchronize()
    assert torch.equal(d1["codes_k"], d2["codes_k"]) and torch.equal(d1["codes_v"], d2["codes_v"])
    np.testing.assert_allclose(out1.cpu().numpy(), out2.cpu().numpy(), rtol=1e-5, atol=1e-6)


def test_decode_step_partials_then_merge():
    wl = W.Workload(82, "adhoc", batch=1, num_q_heads=4, num_kv_heads=1, context_len=3000)
    c = random_cache(wl)
    k, v = new_rows(wl, 1, 1, np.float16)
    d1, d2 = upload(c), upload(c)
    parts = vq.decode_step_partials(d1["q"], dev(k), dev(v), d1["lam"], d1["cb_k"], d1["cb_v"],
                                    d1["codes_k"], d1["codes_v"], 2999, num_splits=3)
    assert parts[0].shape[2] == 4                  # 3 splits of the cached tokens + the new one
    out1 = vq.merge_partials(parts)
    out2 = vq.decode_step(d2["q"], dev(k), dev(v), d2["lam"], d2["cb_k"], d2["cb_v"],
                          d2["codes_k"], d2["codes_v"], 2999, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(d1["codes_k"], d2["codes_k"]) and torch.equal(d1["codes_v"], d2["codes_v"])
    np.testing.assert_allclose(out1.cpu().numpy(), out2.cpu().numpy(), rtol=1e-5, atol=1e-6)


# full workload sizes, in the configuration bench.py times: the token goes to
# the last slot of the context (or the first free slot with append room)
STEP_FULL = [(4, None, [(0, 2), (0, 7)]), (5, 65536, [(0, 0), (7, 5)])]


@pytest.mark.parametrize("config,cur,samples", STEP_FULL)
def test_decode_step_full_size(config, cur, samples):
    wl = W.WORKLOADS[config]
    c = random_cache(wl)
    cur = wl.context_len - 1 if cur is None else cur
    check_step(c, cur, heads=samples, what=f"step config{config}")


# --- decode step with a full-precision residual window ------------------------------

def window_rows(wl, bsz, hkv, win_cap):
    """Raw fp16 window rows [B][Hkv][win_cap][128] (the same generator as the
    model's keys and values, a stream apart from the step's new token)."""
    wk = np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "k", win_cap + 1, append=True)[1:]
                             for g in range(hkv)]) for b in range(bsz)]).astype(np.float16)
    wv = np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "v", win_cap + 1, append=True)[1:]
                             for g in range(hkv)]) for b in range(bsz)]).astype(np.float16)
    return wk, wv


def check_window_step(c, num_codes, win_len, win_cap=128, splits=0, heads=None, what=""):
    """decode_step_window: window slot win_len holds the new token in fp16
    (bit-exact), nothing else is written, and the output equals the oracle's
    attention over the coded tokens and window slots 0 .. win_len."""
    wl = c.wl
    bsz, hkv = c.codes_k.shape[:2]
    dtype = np.float32 if wl.qkv_dtype == "f32" else np.float16
    k, v = new_rows(wl, bsz, hkv, dtype)
    wk, wv = window_rows(wl, bsz, hkv, win_cap)
    d = upload(c)
    dwk, dwv = dev(wk), dev(wv)
    print(f"{what}: num_codes={num_codes} win_len={win_len} win_cap={win_cap}", flush=True)
    out = vq.decode_step_window(d["q"], dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"],
                                d["codes_k"], d["codes_v"], dwk, dwv, num_codes, win_len,
                                num_splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    exp_wk, exp_wv = wk.copy(), wv.copy()
    exp_wk[:, :, win_len] = k.astype(np.float16)          # round to nearest even, as stored
    exp_wv[:, :, win_len] = v.astype(np.float16)
    assert np.array_equal(dwk.cpu().numpy().view(np.uint16), exp_wk.view(np.uint16)), what
    assert np.array_equal(dwv.cpu().numpy().view(np.uint16), exp_wv.view(np.uint16)), what
    assert np.array_equal(d["codes_k"].cpu().numpy(), c.codes_k), what
    assert np.array_equal(d["codes_v"].cpu().numpy(), c.codes_v), what
    kb, vb = wl.k_bits, wl.v_bits
    if heads is None:
        ref = oracle.decode_attention_window(c.q, c.lam, c.cb_k, c.cb_v, c.codes_k, c.codes_v,
                                             num_codes, exp_wk, exp_wv, win_len + 1, kb, vb)
        assert_close(got, ref, what)
    else:
        grp = wl.group
        for b, g in heads:
            ref = oracle.decode_attention_window_head(
                c.q[b, g * grp:(g + 1) * grp], c.lam[g], c.cb_k[g], c.cb_v[g],
                c.codes_k[b, g, :num_codes], c.codes_v[b, g, :num_codes],
                exp_wk[b, g, :win_len + 1], exp_wv[b, g, :win_len + 1], kb, vb)
            assert_close(got[b, g * grp:(g + 1) * grp], ref, f"{what} b={b} kv={g}")
    return got


@pytest.mark.parametrize("num_codes,win_len,splits", [
    (700, 0, 0), (700, 1, 0), (700, 63, 0), (3000, 127, 0), (3000, 64, 3), (512, 50, 0),
    (1, 17, 0), (0, 0, 0), (0, 5, 0), (0, 127, 0)])
def test_decode_step_window_positions(num_codes, win_len, splits):
    wl = W.Workload(90, "adhoc", batch=2, num_q_heads=8, num_kv_heads=2, context_len=3000)
    check_window_step(random_cache(wl), num_codes, win_len, splits=splits,
                      what=f"window codes={num_codes} win={win_len} S={splits}")


@pytest.mark.parametrize("group,k_bits,dtype,num_codes,win_len", [
    (5, 12, "f16", 1499, 100), (1, 8, "f16", 300, 7), (8, 12, "f16", 64, 127),
    (4, 8, "f32", 1024, 31), (3, 8, "f16", 999, 0)])
def test_decode_step_window_groups_widths_dtypes(group, k_bits, dtype, num_codes, win_len):
    wl = W.Workload(95 + group, "adhoc", batch=2, num_q_heads=2 * group, num_kv_heads=2,
                    context_len=1500, k_bits=k_bits, qkv_dtype=dtype)
    check_window_step(random_cache(wl), num_codes, win_len,
                      what=f"window G={group} kbits={k_bits} {dtype}")


@pytest.mark.parametrize("win_len,splits", [(0, 2), (77, 2), (127, 1)])
def test_decode_step_window_folded(win_len, splits):
    # 128 streams with long splits: the last split of each stream attends over
    # the window before its own coded tokens
    wl = W.Workload(93, "adhoc", batch=32, num_q_heads=16, num_kv_heads=4, context_len=20000)
    check_window_step(random_cache(wl), 20000, win_len, splits=splits,
                      heads=[(0, 0), (9, 3), (22, 1), (31, 2)],
                      what=f"folded window win={win_len} S={splits}")


@pytest.mark.parametrize("group,k_bits", [(5, 12), (8, 8)])
def test_decode_step_window_folded_groups_widths(group, k_bits):
    # the folded window in the 12-bit-key kernel and at the largest group
    wl = W.Workload(94, "adhoc", batch=32, num_q_heads=4 * group, num_kv_heads=4,
                    context_len=20000, k_bits=k_bits)
    check_window_step(random_cache(wl), 20000, 100, splits=2,
                      heads=[(1, 0), (17, 3), (30, 2)],
                      what=f"folded window G={group} kbits={k_bits}")


@pytest.mark.parametrize("win_cap,win_len,num_codes,streams", [
    (16, 15, 700, 4), (16, 0, 0, 4), (256, 200, 3000, 4), (256, 255, 20000, 128),
    (1, 0, 513, 4), (512, 300, 2000, 4), (512, 511, 20000, 128)])
def test_decode_step_window_capacities(win_cap, win_len, num_codes, streams):
    # windows other than 128 slots: the smallest, one slot, and larger ones,
    # beside the splits and folded into them (128 streams); past 256 tokens
    # waves take a second block and the new token is in a later block
    bsz = streams // 2
    wl = W.Workload(92, "adhoc", batch=bsz, num_q_heads=8, num_kv_heads=2,
                    context_len=max(num_codes, 1))
    heads = None if bsz <= 2 else [(0, 0), (bsz // 2, 1), (bsz - 1, 0)]
    check_window_step(random_cache(wl), num_codes, win_len, win_cap=win_cap,
                      splits=2 if streams >= 128 else 0, heads=heads,
                      what=f"window cap={win_cap} len={win_len} codes={num_codes}")


def test_decode_step_window_full_size():
    # the long-context layer: 196608 coded tokens and a nearly full window
    wl = W.WORKLOADS[4]
    check_window_step(random_cache(wl), wl.context_len, 127, heads=[(0, 1), (0, 6)],
                      what="window config4")


def test_window_chain_and_flush():
    # a window of 4 fills over four steps, is flushed into codes, and the next
    # step attends over the longer code prefix and a fresh window
    wl = W.Workload(99, "adhoc", batch=2, num_q_heads=8, num_kv_heads=2, context_len=900)
    c = random_cache(wl)
    bsz, hkv, cap4 = 2, 2, 4
    d = upload(c)
    wk = torch.zeros((bsz, hkv, cap4, 128), dtype=torch.float16, device=DEV)
    wv = torch.zeros_like(wk)
    host_k = np.zeros((bsz, hkv, cap4, 128), np.float16)
    host_v = np.zeros_like(host_k)
    num_codes = 700
    for step in range(cap4 + 1):
        win_len = step % cap4
        if step == cap4:   # full: flush into codes [700, 704)
            vq.flush_window(wk, wv, d["lam"], d["cb_k"], d["cb_v"], d["codes_k"], d["codes_v"],
                            num_codes)
            torch.cuda.synchronize()
            ck, cv = d["codes_k"].cpu().numpy(), d["codes_v"].cpu().numpy()
            for b in range(bsz):
                for g in range(hkv):
                    pk, pv, gk, gv = oracle.encode_append(host_k[b, g], host_v[b, g], c.lam[g],
                                                          c.cb_k[g], c.cb_v[g], 8, 8)
                    kt = oracle.transform_keys(host_k[b, g], c.lam[g])
                    check_codes(ck[b, g, num_codes:num_codes + cap4], pk, gk, 8, kt, c.cb_k[g],
                                f"flush K b{b} g{g}")
                    check_codes(cv[b, g, num_codes:num_codes + cap4], pv, gv, 8, host_v[b, g],
                                c.cb_v[g], f"flush V b{b} g{g}", values=True)
            c = dataclasses.replace(c, codes_k=ck, codes_v=cv)
            num_codes += cap4
        k = np.stack([np.stack([W.kv_rows(wl.config_id + step, b, g, "k", 1, append=True)[0]
                                for g in range(hkv)]) for b in range(bsz)]).astype(np.float16)
        v = np.stack([np.stack([W.kv_rows(wl.config_id + step, b, g, "v", 1, append=True)[0]
                                for g in range(hkv)]) for b in range(bsz)]).astype(np.float16)
        out = vq.decode_step_window(d["q"], dev(k), dev(v), d["lam"], d["cb_k"], d["cb_v"],
                                    d["codes_k"], d["codes_v"], wk, wv, num_codes, win_len)
        torch.cuda.synchronize()
        host_k[:, :, win_len], host_v[:, :, win_len] = k, v
        ref = oracle.decode_attention_window(c.q, c.lam, c.cb_k, c.cb_v, c.codes_k, c.codes_v,
                                             num_codes, host_k, host_v, win_len + 1)
        assert_close(out.cpu().numpy().astype(np.float64), ref, f"chain step {step}")


# --- the 1.5-bit layout: 8-dim sub-vectors, 4096-entry C_k and C_v, 12-bit codes ----

def d8_workload(config_id, batch, group, hkv, n, dtype="f16"):
    return W.Workload(config_id, "adhoc-1.5bit", batch=batch, num_q_heads=group * hkv,
                      num_kv_heads=hkv, context_len=n, k_bits=12, v_bits=12, sub_dim=8,
                      qkv_dtype=dtype)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 511, 512, 513, 1024])
def test_d8_attention_ragged_lengths(n):
    c = random_cache(W.WORKLOADS[7], context_len=n)
    d = upload(c)
    assert_close(run_attention(d, n), expected_all(c), f"1.5bit tiny n={n}")


@pytest.mark.parametrize("group,batch,hkv,n,dtype,splits", [
    (1, 2, 2, 300, "f16", 0), (4, 1, 2, 2049, "f16", 3), (5, 2, 2, 1500, "f16", 0),
    (8, 1, 2, 777, "f32", 0), (3, 3, 1, 4096, "f16", 64)])
def test_d8_attention_groups_and_splits(group, batch, hkv, n, dtype, splits):
    c = random_cache(d8_workload(110 + group, batch, group, hkv, n, dtype))
    d = upload(c)
    assert_close(run_attention(d, n, splits), expected_all(c),
                 f"1.5bit G={group} B={batch} n={n} {dtype} S={splits}")


def test_d8_attention_full_size_sampled_heads():
    wl = W.WORKLOADS[6]
    c = random_cache(wl)
    d = upload(c)
    got = run_attention(d, wl.context_len)
    assert np.isfinite(got).all()
    g = wl.group
    for b, h in [(0, 0), (0, 5)]:
        assert_close(got[b, h * g:(h + 1) * g], expected_head(c, b, h), f"config6 kv={h}")


def test_d8_attention_lossless_codebooks():
    """Keys and values built from codebook entries: the 1.5-bit kernel must
    then equal textbook attention on the raw (q, K, V)."""
    rng = np.random.default_rng(120)
    n, group = 700, 4
    h = oracle.sylvester_hadamard(128)
    cb_k = (rng.standard_normal((1, 4096, 8)) * 0.7).astype(np.float16)
    cb_v = (rng.standard_normal((1, 4096, 8)) * 2).astype(np.float16)
    ck = rng.integers(0, 4096, size=(n, 16))
    cv = rng.integers(0, 4096, size=(n, 16))
    lam = (1.0 + rng.random((1, 128)) * 3).astype(np.float32)
    keys = (cb_k[0].astype(np.float64)[ck].reshape(n, 128) @ h.T) * lam[0].astype(np.float64)
    vals = cb_v[0].astype(np.float64)[cv].reshape(n, 128)
    q = rng.standard_normal((1, group, 128)).astype(np.float16)
    codes_k = oracle.pack_codes(ck, 12)[None, None]
    codes_v = oracle.pack_codes(cv, 12)[None, None]
    d = dict(q=dev(q), lam=dev(lam), cb_k=dev(cb_k), cb_v=dev(cb_v), codes_k=dev(codes_k),
             codes_v=dev(codes_v))
    got = run_attention(d, n)
    ref = np.stack([oracle.softmax_attention(q[0, i].astype(np.float64), keys, vals)
                    for i in range(group)])[None]
    assert_close(got, ref, "1.5bit lossless")


@pytest.mark.parametrize("cur,splits,group", [(0, 0, 4), (31, 0, 4), (511, 2, 4), (1023, 0, 4),
                                              (700, 0, 5), (300, 0, 1)])
def test_d8_decode_step(cur, splits, group):
    wl = d8_workload(130 + group, 2, group, 2, 1024)
    check_step(random_cache(wl), cur, splits, what=f"1.5bit step cur={cur} G={group}")


def test_d8_decode_step_full_size():
    wl = W.WORKLOADS[6]
    check_step(random_cache(wl), wl.context_len - 1, heads=[(0, 2), (0, 7)],
               what="1.5bit step config6")


@pytest.mark.parametrize("t_new,cur,dtype", [(1, 0, "f16"), (13, 5, "f16"), (16, 3, "f16"),
                                             (17, 0, "f16"), (64, 100, "f32"), (200, 0, "f16")])
def test_d8_encode_append(t_new, cur, dtype):
    bsz, hkv = 2, 2
    lam = np.stack([W.random_lambda(140, g) for g in range(hkv)])
    cb_k = np.stack([W.random_codebook(140, g, "k", 4096, 0.6, sub_dim=8) for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(140, g, "v", 4096, 1.0, 1 / 32, sub_dim=8)
                     for g in range(hkv)])
    st = np.float16 if dtype == "f16" else np.float32
    k = np.stack([np.stack([W.kv_rows(140, b, g, "k", t_new, append=True) for g in range(hkv)])
                  for b in range(bsz)]).astype(st)
    v = np.stack([np.stack([W.kv_rows(140, b, g, "v", t_new, append=True) for g in range(hkv)])
                  for b in range(bsz)]).astype(st)
    cap = cur + t_new + 3
    ck = torch.full((bsz, hkv, cap, 24), 0xA5, dtype=torch.uint8, device=DEV)
    cv = torch.full((bsz, hkv, cap, 24), 0x5A, dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, cur)
    torch.cuda.synchronize()
    ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
    outside = np.ones(cap, bool)
    outside[cur:cur + t_new] = False
    assert np.all(ckh[:, :, outside] == 0xA5) and np.all(cvh[:, :, outside] == 0x5A)
    for b in range(bsz):
        for g in range(hkv):
            pk, pv, gk, gv = oracle.encode_append(k[b, g], v[b, g], lam[g], cb_k[g], cb_v[g],
                                                  12, 12)
            kt = oracle.transform_keys(k[b, g], lam[g])
            check_codes(ckh[b, g, cur:cur + t_new], pk, gk, 12, kt, cb_k[g],
                        f"1.5bit enc K b{b} g{g}", 8)
            check_codes(cvh[b, g, cur:cur + t_new], pv, gv, 12, v[b, g], cb_v[g],
                        f"1.5bit enc V b{b} g{g}", 8, values=True)


def test_d8_encode_append_prompt_workgroups():
    # enough tokens for 16-token workgroups on every CU (8 KV heads x 33
    # workgroups, the last one half full); shorter appends take a token a
    # workgroup (the cases above).  Two heads are checked against the oracle.
    hkv, t_new = 8, 520
    lam = np.stack([W.random_lambda(141, g) for g in range(hkv)])
    cb_k = np.stack([W.random_codebook(141, g, "k", 4096, 0.6, sub_dim=8) for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(141, g, "v", 4096, 1.0, 1 / 32, sub_dim=8)
                     for g in range(hkv)])
    k = np.stack([W.kv_rows(141, 0, g, "k", t_new, append=True) for g in range(hkv)])[None]
    v = np.stack([W.kv_rows(141, 0, g, "v", t_new, append=True) for g in range(hkv)])[None]
    k, v = k.astype(np.float16), v.astype(np.float16)
    ck = torch.full((1, hkv, t_new, 24), 0xA5, dtype=torch.uint8, device=DEV)
    cv = torch.full((1, hkv, t_new, 24), 0x5A, dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, 0)
    torch.cuda.synchronize()
    ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
    for g in (0, hkv - 1):
        pk, pv, gk, gv = oracle.encode_append(k[0, g], v[0, g], lam[g], cb_k[g], cb_v[g], 12, 12)
        kt = oracle.transform_keys(k[0, g], lam[g])
        check_codes(ckh[0, g], pk, gk, 12, kt, cb_k[g], f"1.5bit prompt K g{g}", 8)
        check_codes(cvh[0, g], pv, gv, 12, v[0, g], cb_v[g], f"1.5bit prompt V g{g}", 8,
                    values=True)


def test_d8_encoder_exact_ties_go_to_lowest_index():
    rng = np.random.default_rng(150)
    base = rng.standard_normal((2048, 8)).astype(np.float16)
    cb = np.concatenate([base, base])[None]             # entry j and j + 2048 identical
    codes = rng.integers(0, 2048, size=(5, 16))
    v = base.astype(np.float64)[codes].reshape(5, 128).astype(np.float32)[None, None]
    lam = np.ones((1, 128), np.float32)
    ck = torch.zeros((1, 1, 8, 24), dtype=torch.uint8, device=DEV)
    cv = torch.zeros((1, 1, 8, 24), dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(v), dev(v), dev(lam), dev(cb), dev(cb), ck, cv, 2)
    torch.cuda.synchronize()
    got = oracle.unpack_codes(cv.cpu().numpy()[0, 0, 2:7], 12, 16)
    np.testing.assert_array_equal(got, codes)


@pytest.mark.parametrize("num_codes,win_len,group", [(700, 0, 4), (1000, 127, 4), (0, 9, 4),
                                                     (513, 64, 5)])
def test_d8_decode_step_window(num_codes, win_len, group):
    wl = d8_workload(160 + group, 2, group, 2, 1024)
    check_window_step(random_cache(wl), num_codes, win_len,
                      what=f"1.5bit window codes={num_codes} win={win_len} G={group}")


def test_d8_decode_step_window_folded():
    # 128 streams with long splits: the 1.5-bit kernel's last split of each
    # stream attends over the window first
    wl = d8_workload(170, 32, 4, 4, 20000)
    check_window_step(random_cache(wl), 20000, 127, splits=2, heads=[(0, 1), (19, 2), (31, 3)],
                      what="1.5bit folded window")


# --- deterministic mode: a bitwise run-to-run check (race canary) -----------------

@pytest.mark.parametrize("layout", [(4, 8, 4, 5000), (5, 12, 4, 3000), (4, 12, 8, 4000),
                                    (8, 8, 4, 2049)],
                         ids=lambda l: f"G{l[0]}-k{l[1]}-d{l[2]}-n{l[3]}")
def test_deterministic_mode_is_bitwise_reproducible(layout):
    """With a fixed tile order nothing in a call depends on timing, so any
    difference between repeated calls would come from a race (an LDS write
    not ordered before its read, a missing barrier, an uninitialised read).
    Every output and partial must repeat bit for bit: the split pass alone,
    decode attention and a decode step (each on its own copy of the cache),
    over ragged lengths and several split counts."""
    g, kb, sd, n = layout
    wl = W.Workload(120 + g + kb, "adhoc", batch=2, num_q_heads=2 * g, num_kv_heads=2,
                    context_len=n, k_bits=kb, v_bits=12 if sd == 8 else 8, sub_dim=sd,
                    qkv_dtype="f16", append_tokens=1)
    c = random_cache(wl)
    d = upload(c)
    rng = np.random.default_rng(9)
    kn = dev(rng.standard_normal((2, 2, 128)).astype(np.float16))
    prev = vq.set_deterministic(True)
    try:
        for splits in (1, 3, 0):
            runs = []
            for _ in range(3):
                ck, cv = d["codes_k"].clone(), d["codes_v"].clone()
                parts = vq.decode_attention_partials(d["q"], d["lam"], d["cb_k"], d["cb_v"], ck,
                                                     cv, n, num_splits=splits)
                att = vq.decode_attention(d["q"], d["lam"], d["cb_k"], d["cb_v"], ck, cv, n,
                                          num_splits=splits)
                stp = vq.decode_step(d["q"], kn, kn, d["lam"], d["cb_k"], d["cb_v"], ck, cv,
                                     n, num_splits=splits)
                torch.cuda.synchronize()
                runs.append([t.cpu().numpy() for t in (*parts, att, stp, ck, cv)])
            for other in runs[1:]:
                for a, b in zip(runs[0], other):
                    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), splits
        ref = expected_all(c)
        assert_close(runs[0][3].astype(np.float64), ref, f"deterministic G={g} kb={kb} d={sd}")
    finally:
        vq.set_deterministic(prev)
