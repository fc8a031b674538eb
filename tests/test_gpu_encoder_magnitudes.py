"""Codes at extreme input magnitudes, bit-exact against the oracle: the
scale and bound paths of the fp16 hi/lo nearest-centroid search (one scale
per workgroup and tensor in vq_encode_append, one per sub-vector for the
decode step's new token).  Rows span 2^-30 .. 2^12 inside one workgroup,
with zero rows and rows of one large channel among tiny ones; codebook
entries span 2^-20 .. 2^5 (fp16 subnormals included).  Value codes must be
identical; key codes follow the near-tie rule of check_codes."""
import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W
from test_gpu_parity import DEV, check_codes, dev

pytestmark = pytest.mark.gpu


def extreme_rows(rng, t):
    x = rng.standard_normal((t, 128)) * np.exp2(rng.integers(-30, 13, (t, 1)))
    x[3] = 0.0                                   # a zero row
    x[4] = rng.standard_normal(128) * 2.0 ** -28
    x[4, 7] = 2.0 ** 10                          # one large channel among tiny ones
    x[5] = 2.0 ** -60                            # far below every centroid
    x[6, :64] *= 2.0 ** -40                      # half the row tiny, half not
    return x.astype(np.float32)


def extreme_codebook(rng, n, sub_dim):
    cb = rng.standard_normal((n, sub_dim)) * np.exp2(rng.integers(-20, 6, (n, 1)))
    cb[0] = 0.0
    return cb.astype(np.float16)


@pytest.mark.parametrize("k_bits,sub_dim", [(8, 4), (12, 4), (12, 8)])
def test_encoder_codes_at_extreme_magnitudes(k_bits, sub_dim):
    rng = np.random.default_rng(300 + k_bits + sub_dim)
    hkv, t = 2, 40                               # several workgroups, a ragged last one
    v_bits = 12 if sub_dim == 8 else 8
    lam = np.stack([W.random_lambda(300, g) for g in range(hkv)])
    cb_k = np.stack([extreme_codebook(rng, 1 << k_bits, sub_dim) for _ in range(hkv)])
    cb_v = np.stack([extreme_codebook(rng, 1 << v_bits, sub_dim) for _ in range(hkv)])
    k = np.stack([extreme_rows(rng, t) for _ in range(hkv)])[None]
    v = np.stack([extreme_rows(rng, t) for _ in range(hkv)])[None]
    num_sub = 128 // sub_dim
    ck = torch.zeros((1, hkv, t, num_sub * k_bits // 8), dtype=torch.uint8, device=DEV)
    cv = torch.zeros((1, hkv, t, num_sub * v_bits // 8), dtype=torch.uint8, device=DEV)
    vq.encode_append(dev(k), dev(v), dev(lam), dev(cb_k), dev(cb_v), ck, cv, 0)
    torch.cuda.synchronize()
    ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
    for g in range(hkv):
        pk, pv, gk, gv = oracle.encode_append(k[0, g], v[0, g], lam[g], cb_k[g], cb_v[g],
                                              k_bits, v_bits)
        kt = oracle.transform_keys(k[0, g], lam[g])
        what = f"extreme enc kb={k_bits} d={sub_dim} g{g}"
        check_codes(ckh[0, g], pk, gk, k_bits, kt, cb_k[g], what + " K", sub_dim)
        check_codes(cvh[0, g], pv, gv, v_bits, v[0, g], cb_v[g], what + " V", sub_dim,
                    values=True)


@pytest.mark.parametrize("k_bits,sub_dim", [(12, 4), (12, 8), (8, 4)])
def test_decode_step_new_token_codes_at_extreme_magnitudes(k_bits, sub_dim):
    """The decode step's in-kernel encode of the new token (12-bit keys and
    the 1.5-bit layout take the hi/lo search with a scale per sub-vector)."""
    rng = np.random.default_rng(400 + k_bits + sub_dim)
    bsz, hkv, g_q, n = 1, 2, 4, 96
    v_bits = 12 if sub_dim == 8 else 8
    num_sub = 128 // sub_dim
    lam = np.stack([W.random_lambda(400, g) for g in range(hkv)])
    cb_k = np.stack([extreme_codebook(rng, 1 << k_bits, sub_dim) for _ in range(hkv)])
    cb_v = np.stack([extreme_codebook(rng, 1 << v_bits, sub_dim) for _ in range(hkv)])
    krow, vrow = num_sub * k_bits // 8, num_sub * v_bits // 8
    codes_k = rng.integers(0, 256, (bsz, hkv, n, krow), dtype=np.uint8)
    codes_v = rng.integers(0, 256, (bsz, hkv, n, vrow), dtype=np.uint8)
    q = rng.standard_normal((bsz, hkv * g_q, 128)).astype(np.float32)
    rows = extreme_rows(rng, 8)
    for i in range(rows.shape[0]):               # one step per kind of row
        kn = np.stack([rows[i], rows[(i + 3) % 8]])[None].astype(np.float32)
        vn = np.stack([rows[(i + 5) % 8], rows[i]])[None].astype(np.float32)
        ck, cv = dev(codes_k.copy()), dev(codes_v.copy())
        out = vq.decode_step(dev(q), dev(kn), dev(vn), dev(lam), dev(cb_k), dev(cb_v), ck, cv,
                             n - 1)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        ckh, cvh = ck.cpu().numpy(), cv.cpu().numpy()
        assert np.array_equal(ckh[:, :, : n - 1], codes_k[:, :, : n - 1])
        for g in range(hkv):
            pk, pv, gk, gv = oracle.encode_append(kn[0, g][None], vn[0, g][None], lam[g],
                                                  cb_k[g], cb_v[g], k_bits, v_bits)
            kt = oracle.transform_keys(kn[0, g][None], lam[g])
            what = f"extreme step row{i} kb={k_bits} d={sub_dim} g{g}"
            check_codes(ckh[0, g, n - 1:n], pk, gk, k_bits, kt, cb_k[g], what + " K", sub_dim)
            check_codes(cvh[0, g, n - 1:n], pv, gv, v_bits, vn[0, g][None], cb_v[g],
                        what + " V", sub_dim, values=True)
