"""The C ABI from a plain C++ program (tests/c_abi_decode_step.cpp, built by
__graft_entry__.build()): device memory from the HIP runtime, no Python and no
torch in the caller.  One decode step on the small recipe workload; its codes
must be the oracle encoder's, and its output equal to the Python binding's
call on the same inputs (to fp32 rounding) and to the oracle's attention (to
the parity bound)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import vector_quantized_bit_amd as vq
import workloads as W
from fixtures import attention_errors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_decode_step")
DEV = "cuda:0"


@pytest.mark.gpu
def test_plain_cpp_caller_decode_step(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("tests/c_abi_decode_step is not built (run __graft_entry__.build())")
    bsz, hq, hkv, cap, cur = 2, 8, 2, 700, 650
    wl = W.Workload(1, "c-abi", batch=bsz, num_q_heads=hq, num_kv_heads=hkv, context_len=cap)
    q = np.stack([W.queries(1, b, hq) for b in range(bsz)]).astype(np.float16)
    lam = np.stack([W.random_lambda(1, g) for g in range(hkv)]).astype(np.float32)
    cb_k = np.stack([W.random_codebook(1, g, "k", 256, 0.6) for g in range(hkv)])
    cb_v = np.stack([W.random_codebook(1, g, "v", 256, 1.0, 1 / 32) for g in range(hkv)])
    ck = np.stack([np.stack([W.random_code_rows(1, b, g, "k", cap, 32) for g in range(hkv)])
                   for b in range(bsz)])
    cv = np.stack([np.stack([W.random_code_rows(1, b, g, "v", cap, 32) for g in range(hkv)])
                   for b in range(bsz)])
    kn = np.stack([np.stack([W.kv_rows(1, b, g, "k", 1, append=True)[0] for g in range(hkv)])
                   for b in range(bsz)]).astype(np.float16)
    vn = np.stack([np.stack([W.kv_rows(1, b, g, "v", 1, append=True)[0] for g in range(hkv)])
                   for b in range(bsz)]).astype(np.float16)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.array([bsz, hq, hkv, cap, cur], np.int32).tobytes())
        for a in (q, kn, vn, lam, cb_k.astype(np.float16), cb_v.astype(np.float16), ck, cv):
            f.write(np.ascontiguousarray(a).tobytes())
    print(f"c-abi caller: B={bsz} Hq={hq} Hkv={hkv} cap={cap} cur={cur}", flush=True)
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(fout, np.uint8)
    nout = bsz * hq * 128 * 4
    got = raw[:nout].view(np.float32).reshape(bsz, hq, 128).astype(np.float64)
    new_k = raw[nout:nout + bsz * hkv * 32].reshape(bsz, hkv, 32)
    new_v = raw[nout + bsz * hkv * 32:].reshape(bsz, hkv, 32)

    # the codes: the oracle encoder's (these inputs have no near-ties)
    for b in range(bsz):
        for g in range(hkv):
            pk, pv, _, _ = oracle.encode_append(kn[b, g][None], vn[b, g][None], lam[g], cb_k[g],
                                                cb_v[g])
            np.testing.assert_array_equal(new_k[b, g], pk[0])
            np.testing.assert_array_equal(new_v[b, g], pv[0])
    # the same step through the Python binding
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    dck, dcv = dev(ck), dev(cv)
    ref_bind = vq.decode_step(dev(q), dev(kn), dev(vn), dev(lam), dev(cb_k), dev(cb_v), dck, dcv,
                              cur)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dck.cpu().numpy()[:, :, cur], new_k)
    np.testing.assert_allclose(got, ref_bind.cpu().numpy(), rtol=1e-5, atol=1e-6)
    # the oracle's attention over the cache with the appended token
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, :, cur], cv2[:, :, cur] = new_k, new_v
    g_ = hq // hkv
    ref = np.stack([np.concatenate([
        oracle.decode_attention_head(q[b, g * g_:(g + 1) * g_], lam[g], cb_k[g], cb_v[g],
                                     ck2[b, g, :cur + 1], cv2[b, g, :cur + 1])
        for g in range(hkv)]) for b in range(bsz)])
    rel, mab = attention_errors(got, ref)
    print(f"c-abi decode step: rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
    assert rel <= 1e-3 and mab <= 2e-3, (rel, mab)
