"""GPU parity of the offline calibration path (through the C ABI) against the
fp64 oracle.

  lambda     bit-identical to the oracle's fp64 square root rounded to fp32.
  K~ (fp32)  within half an fp32 ulp of the oracle's fp64 value, plus 1e-13
             relative for the different fp64 rounding order of the transform.
  K-Means    centroids (fp64), fp16 codebook and final codes bit-identical to
             the oracle's Lloyd iterations on the same fp32 samples and the
             same initial centroids, for every iteration count tested.

Samples are sub-vectors of seeded synthetic calibration keys (transformed by
the oracle, rounded to fp32) and values, in the shapes of the VecInfer page's
calibration set (256 sequences x 512 tokens per KV head).
"""
import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def calib_keys(config_id, hkv, n, dtype, tensor="k"):
    return np.stack([W.as_storage(W.calibration_rows(config_id, g, tensor, n), dtype)
                     for g in range(hkv)])


# --- smoothing factors -----------------------------------------------------------

@pytest.mark.parametrize("dtype,hkv,n", [("f16", 2, 1), ("f16", 3, 1000), ("f32", 2, 257),
                                         ("f32", 1, 4096), ("f16", 8, 2049)])
def test_calibrate_lambda_bit_exact(dtype, hkv, n):
    print(f"lambda {dtype} hkv={hkv} n={n}", flush=True)
    keys = calib_keys(2, hkv, n, dtype)
    got = vq.calibrate_lambda(dev(keys)).cpu().numpy()
    ref = np.stack([oracle.smooth_factors(keys[g]) for g in range(hkv)]).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_calibrate_lambda_special_values(dtype):
    keys = W.as_storage(calib_keys(3, 1, 300, "f32"), dtype).copy()
    keys[0, :, 5] = 0                        # all-zero channel -> lambda 0
    keys[0, 17, 9] = -60000.0                # the peak is negative
    keys[0, :, 11] = 6e-8 if dtype == "f16" else 1e-40   # subnormal magnitudes
    keys[0, 299, 12] = 65504.0               # largest finite half
    keys[0, :, 13] = -0.0
    got = vq.calibrate_lambda(dev(keys)).cpu().numpy()
    ref = oracle.smooth_factors(keys[0]).astype(np.float32)[None]
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert got[0, 5] == 0 and got[0, 13] == 0


def test_calibrate_lambda_full_size():
    """The page's calibration set size: 256 x 512 tokens for each of 8 KV heads."""
    keys = calib_keys(2, 8, W.CALIB_TOKENS, "f16")
    got = vq.calibrate_lambda(dev(keys)).cpu().numpy()
    ref = np.stack([oracle.smooth_factors(keys[g]) for g in range(8)]).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


# --- transformed calibration keys ----------------------------------------------------

def assert_fp32_rounding_of(got, ref, what):
    got = np.asarray(got, np.float64)
    spacing = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref)
    bound = 0.5 * spacing + 1e-13 * np.abs(ref)
    worst = float(np.max(err / bound))
    exact = float(np.mean(got == ref.astype(np.float32)))
    print(f"{what}: worst err/bound {worst:.3f}, equal to fp32(oracle) {exact:.6f}", flush=True)
    assert worst <= 1.0, what
    assert exact >= 1 - 1e-4, what


@pytest.mark.parametrize("dtype,hkv,n", [("f16", 2, 333), ("f32", 3, 64), ("f16", 1, 1)])
def test_transform_keys_matches_oracle(dtype, hkv, n):
    keys = calib_keys(2, hkv, n, dtype)
    lam = np.stack([oracle.smooth_factors(keys[g]) for g in range(hkv)]).astype(np.float32)
    got = vq.transform_keys(dev(keys), dev(lam)).cpu().numpy()
    ref = np.stack([oracle.transform_keys(keys[g], lam[g]) for g in range(hkv)])
    assert_fp32_rounding_of(got, ref, f"transform_keys {dtype} hkv={hkv} n={n}")


# --- K-Means ---------------------------------------------------------------------------

def key_samples(config_id, g, n_tok, sub=4):
    k = W.as_storage(W.calibration_rows(config_id, g, "k", n_tok), "f16")
    lam = oracle.smooth_factors(k).astype(np.float32)
    return oracle.transform_keys(k, lam).astype(np.float32).reshape(-1, sub)


def value_samples(config_id, g, n_tok, sub=4):
    v = W.as_storage(W.calibration_rows(config_id, g, "v", n_tok), "f16")
    return v.astype(np.float32).reshape(-1, sub)


def initial_centroids(samples, bits, config_id, g, tensor):
    """2^bits distinct sample rows; with fewer samples than that, the picks
    repeat cyclically (duplicate centroids: exact distance ties)."""
    ent = 1 << bits
    idx = W.calibration_init_rows(config_id, g, tensor, samples.shape[0], ent)
    return samples[idx[np.arange(ent) % idx.size]].astype(np.float64)


def run_kmeans(samples, init, iters, in_place=False):
    d_init = dev(init)
    cent, cb, asg = vq.kmeans(dev(samples), d_init, iters, codebook=True, assign=True,
                              centroids=d_init if in_place else None)
    torch.cuda.synchronize()
    return cent.cpu().numpy(), cb.cpu().numpy(), asg.cpu().numpy()


def check_set(samples, init, iters, cent, cb, asg, what):
    x = samples.astype(np.float64)
    ref = oracle.lloyd_kmeans(x, init, iters)
    codes, _, _ = oracle.vq_assign(x, ref)
    same_c = np.array_equal(cent.view(np.uint64), ref.view(np.uint64))
    diff = np.abs(cent - ref).max()
    print(f"{what}: centroids bit-exact {same_c} (max diff {diff:.3e}), codes equal "
          f"{np.mean(asg == codes):.6f}", flush=True)
    assert same_c, what
    np.testing.assert_array_equal(cb.view(np.uint16), ref.astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(asg, codes)


@pytest.mark.parametrize("tensor,bits,sets,n_tok,iters", [
    ("k", 8, 2, 640, 0),     # 20480 samples: two full sort chunks and a ragged third
    ("k", 8, 2, 640, 1),
    ("k", 8, 2, 640, 4),
    ("v", 8, 2, 640, 3),
    ("k", 12, 1, 300, 2),    # 4096 centroids over 9600 samples
    ("v", 8, 3, 1, 2),       # 32 samples, 256 centroids: most clusters empty, duplicates
])
def test_kmeans_bit_exact(tensor, bits, sets, n_tok, iters):
    print(f"kmeans {tensor} bits={bits} sets={sets} tokens={n_tok} iters={iters}", flush=True)
    make = key_samples if tensor == "k" else value_samples
    samples = np.stack([make(2, g, n_tok) for g in range(sets)])
    init = np.stack([initial_centroids(samples[g], bits, 2, g, tensor) for g in range(sets)])
    cent, cb, asg = run_kmeans(samples, init, iters)
    for g in range(sets):
        check_set(samples[g], init[g], iters, cent[g], cb[g], asg[g], f"set {g}")


@pytest.mark.parametrize("tensor,bits,sets,n_tok,iters", [
    ("k", 12, 2, 600, 1),    # the 1.5-bit C_k: 4096 centroids of 8 dims, 9600 samples
    ("k", 12, 1, 300, 0),
    ("v", 12, 1, 300, 2),
    ("v", 8, 2, 1100, 3),    # 17600 samples: three sort chunks
    ("k", 8, 1, 2, 2),       # 32 samples, 256 centroids: duplicates, empty clusters
])
def test_kmeans_bit_exact_8dim(tensor, bits, sets, n_tok, iters):
    print(f"kmeans d=8 {tensor} bits={bits} sets={sets} tokens={n_tok} iters={iters}", flush=True)
    make = key_samples if tensor == "k" else value_samples
    samples = np.stack([make(2, g, n_tok, 8) for g in range(sets)])
    init = np.stack([initial_centroids(samples[g], bits, 2, g, tensor) for g in range(sets)])
    cent, cb, asg = run_kmeans(samples, init, iters)
    assert cent.shape[-1] == 8 and cb.shape[-1] == 8
    for g in range(sets):
        check_set(samples[g], init[g], iters, cent[g], cb[g], asg[g], f"d8 set {g}")


def test_kmeans_8dim_full_calibration_set_sampled():
    """The 1.5-bit C_k at the calibration-set size: 131072 tokens per KV head
    as 2,097,152 8-dim sub-vectors, 4096 centroids, one Lloyd iteration (two
    heads).  Checked on sampled rows: each code is the nearest returned
    centroid by the fp64 distance (ties to the lowest index)."""
    n_tok, sets = W.CALIB_TOKENS, 2
    samples = np.stack([key_samples(2, g, n_tok, 8) for g in range(sets)])
    init = np.stack([initial_centroids(samples[g], 12, 2, g, "k") for g in range(sets)])
    cent, cb, asg = run_kmeans(samples, init, 1)
    rows = np.random.default_rng(42).choice(samples.shape[1], 2048, replace=False)
    for g in range(sets):
        codes, _, _ = oracle.vq_assign(samples[g, rows].astype(np.float64), cent[g])
        np.testing.assert_array_equal(asg[g, rows], codes)
        np.testing.assert_array_equal(cb[g].view(np.uint16), cent[g].astype(np.float16).view(np.uint16))


def test_kmeans_exact_ties_and_degenerate_sets():
    """Half-integer samples against integer centroids (many exact distance
    ties between distinct centroids), one sample, all samples identical."""
    rng = np.random.default_rng(40)
    n = 5000
    lattice = (rng.integers(-6, 7, size=(n, 4)) * 0.5).astype(np.float32)
    grid = np.array(np.meshgrid(*[np.arange(-2, 2)] * 4, indexing="ij")).reshape(4, -1).T
    init_a = grid.astype(np.float64)          # 256 integer points
    same = np.tile(np.float32([[0.25, -1.5, 3.0, 0.0]]), (n, 1))
    for what, samples, init, iters in (("lattice", lattice, init_a, 3),
                                       ("identical", same, init_a, 2)):
        cent, cb, asg = run_kmeans(samples[None], init[None], iters)
        check_set(samples, init, iters, cent[0], cb[0], asg[0], what)
    # a single sample
    cent, cb, asg = run_kmeans(lattice[None, :1], init_a[None], 2)
    check_set(lattice[:1], init_a, 2, cent[0], cb[0], asg[0], "one sample")


def test_kmeans_in_place_matches_separate_output():
    samples = np.stack([value_samples(2, 0, 200)])
    init = initial_centroids(samples[0], 8, 2, 0, "v")[None]
    a = run_kmeans(samples, init, 3)
    b = run_kmeans(samples, init, 3, in_place=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_kmeans_full_size_calibration_set():
    """8 KV heads x 256 x 512 calibration tokens = 4,194,304 key sub-vectors per
    head, one Lloyd iteration on the GPU at that shape; head 3 is checked in
    full against the oracle, the final codes of every head on sampled rows
    (nearest fp64 centroid among the returned ones, ties to the lowest)."""
    n_tok = W.CALIB_TOKENS
    samples = np.stack([key_samples(2, g, n_tok) for g in range(8)])
    init = np.stack([initial_centroids(samples[g], 8, 2, g, "k") for g in range(8)])
    cent, cb, asg = run_kmeans(samples, init, 1)
    x = samples[3].astype(np.float64)
    ref = oracle.lloyd_kmeans(x, init[3], 1)
    assert np.array_equal(cent[3].view(np.uint64), ref.view(np.uint64))
    np.testing.assert_array_equal(cb[3].view(np.uint16), ref.astype(np.float16).view(np.uint16))
    rows = np.random.default_rng(41).choice(x.shape[0], 65536, replace=False)
    codes, _, _ = oracle.vq_assign(x[rows], ref)
    np.testing.assert_array_equal(asg[3, rows], codes)
    for g in range(8):
        xs = samples[g, rows].astype(np.float64)
        dist = np.zeros((rows.size, 256))
        for j in range(4):
            e = xs[:, j:j + 1] - cent[g][None, :, j]
            dist += e * e
        np.testing.assert_array_equal(asg[g, rows], np.argmin(dist, axis=1))


def test_calibration_pipeline_end_to_end():
    """keys -> lambda -> K~ -> K-Means on the GPU, against the same chain on
    the oracle.  The chain is exact wherever the GPU's fp32 K~ equals the
    oracle's rounded to fp32 (checked: it does for these inputs)."""
    n_tok, hkv, it = 600, 2, 3
    keys = calib_keys(2, hkv, n_tok, "f16")
    d_keys = dev(keys)
    lam = vq.calibrate_lambda(d_keys)
    kt = vq.transform_keys(d_keys, lam)
    kt_host = kt.cpu().numpy()
    samples_ref = []
    for g in range(hkv):
        lam_ref = oracle.smooth_factors(keys[g]).astype(np.float32)
        samples_ref.append(oracle.transform_keys(keys[g], lam_ref).astype(np.float32))
    samples_ref = np.stack(samples_ref)
    assert np.array_equal(kt_host.view(np.uint32), samples_ref.view(np.uint32))
    samples_ref = samples_ref.reshape(hkv, -1, 4)
    init = np.stack([initial_centroids(samples_ref[g], 8, 2, g, "k") for g in range(hkv)])
    cent, cb, asg = vq.kmeans(kt.view(hkv, -1, 4), dev(init), it, assign=True)
    torch.cuda.synchronize()
    for g in range(hkv):
        check_set(samples_ref[g], init[g], it, cent[g].cpu().numpy(), cb[g].cpu().numpy(),
                  asg[g].cpu().numpy(), f"pipeline head {g}")
