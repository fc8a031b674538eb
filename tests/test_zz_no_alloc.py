"""vq_decode_step_noalloc (partials in the library's static device buffer)
against vq_decode_step (partials in a caller workspace) through the C ABI:
the same appended codes bit for bit and outputs within rel-L2 1e-3 /
max-abs 2e-3 of each other and of the fp64 oracle, on two calls in a row,
the second on a smaller shape (so its partials overwrite only part of what
the first left in the buffer)."""
import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W
from fixtures import attention_errors, random_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def one_case(cid, batch, hkv, group, n, k_bits, sub_dim=4):
    wl = W.Workload(cid, "noalloc", batch=batch, num_q_heads=group * hkv, num_kv_heads=hkv,
                    context_len=n, k_bits=k_bits, v_bits=12 if sub_dim == 8 else 8,
                    sub_dim=sub_dim, qkv_dtype="f16", append_tokens=1)
    c = random_cache(wl)
    rng = np.random.default_rng(cid)
    k_new = rng.standard_normal((batch, hkv, 128)).astype(np.float16)
    v_new = rng.standard_normal((batch, hkv, 128)).astype(np.float16)
    args = [dev(c.q), dev(k_new), dev(v_new), dev(c.lam), dev(c.cb_k), dev(c.cb_v)]
    ck_a, cv_a = dev(c.codes_k), dev(c.codes_v)
    ck_b, cv_b = dev(c.codes_k), dev(c.codes_v)
    print(f"noalloc case B={batch} Hkv={hkv} G={group} n={n} k_bits={k_bits} d={sub_dim}",
          flush=True)
    out_a = vq.decode_step(*args, ck_a, cv_a, n)
    out_b = vq.decode_step_noalloc(*args, ck_b, cv_b, n)
    torch.cuda.synchronize()
    assert torch.equal(ck_a, ck_b) and torch.equal(cv_a, cv_b)
    a = out_a.cpu().numpy().astype(np.float64)
    b = out_b.cpu().numpy().astype(np.float64)
    rel, mab = attention_errors(b, a)
    print(f"  noalloc vs workspace: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert rel <= 1e-3 and mab <= 2e-3
    c.codes_k, c.codes_v = ck_b.cpu().numpy(), cv_b.cpu().numpy()
    ref = oracle.decode_attention(c.q, c.lam, c.cb_k, c.cb_v, c.codes_k, c.codes_v, n + 1,
                                  k_bits, wl.v_bits)
    rel, mab = attention_errors(b, ref)
    print(f"  noalloc vs oracle: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert rel <= 1e-3 and mab <= 2e-3


def test_noalloc_step_matches_the_workspace_step_twice_then_smaller():
    one_case(301, batch=4, hkv=8, group=4, n=33000, k_bits=8)     # 32 streams: folded plan
    one_case(302, batch=1, hkv=2, group=5, n=700, k_bits=12)      # smaller, extra workgroups


def test_noalloc_step_other_layouts():
    one_case(303, batch=2, hkv=2, group=8, n=3000, k_bits=8)
    one_case(304, batch=1, hkv=2, group=4, n=2000, k_bits=12, sub_dim=8)
