"""The Python binding refuses tensors whose shapes disagree with the cache
before anything reaches the C ABI: the ABI takes raw pointers, so a short
tensor would be read or written past its end on the device.  Every call here
raises ValueError and launches nothing."""
import numpy as np
import pytest
import torch

import vector_quantized_bit_amd as vq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cache():
    b, hkv, g, cap = 2, 2, 4, 600
    t = dict(
        q=torch.zeros((b, hkv * g, 128), dtype=torch.float16, device=DEV),
        lam=torch.ones((hkv, 128), dtype=torch.float32, device=DEV),
        cb_k=torch.zeros((hkv, 256, 4), dtype=torch.float16, device=DEV),
        cb_v=torch.zeros((hkv, 256, 4), dtype=torch.float16, device=DEV),
        codes_k=torch.zeros((b, hkv, cap, 32), dtype=torch.uint8, device=DEV),
        codes_v=torch.zeros((b, hkv, cap, 32), dtype=torch.uint8, device=DEV),
    )
    return t


def attend(t, **over):
    a = dict(t, **over)
    return vq.decode_attention(a["q"], a["lam"], a["cb_k"], a["cb_v"], a["codes_k"],
                               a["codes_v"], 500, out=a.get("out"), workspace=a.get("ws"))


def step(t, fn=vq.decode_step, **over):
    a = dict(t, **over)
    b, hkv = a["codes_k"].shape[:2]
    kn = a.get("kn", torch.zeros((b, hkv, 128), dtype=torch.float16, device=DEV))
    return fn(a["q"], kn, kn, a["lam"], a["cb_k"], a["cb_v"], a["codes_k"], a["codes_v"], 500,
              out=a.get("out"))


BAD = [
    ("q with more sequences than the cache",
     lambda t: dict(q=torch.zeros((3, 8, 128), dtype=torch.float16, device=DEV)), "sequences"),
    ("q rows of 64", lambda t: dict(q=torch.zeros((2, 8, 64), dtype=torch.float16, device=DEV)),
     "[B][Hq][128]"),
    ("lambda for one KV head",
     lambda t: dict(lam=torch.ones((1, 128), dtype=torch.float32, device=DEV)), "lambda"),
    ("cb_k for one KV head",
     lambda t: dict(cb_k=torch.zeros((1, 256, 4), dtype=torch.float16, device=DEV)), "cb_k"),
    ("cb_v of 200 entries",
     lambda t: dict(cb_v=torch.zeros((2, 200, 4), dtype=torch.float16, device=DEV)), "cb_v"),
    ("31-byte key rows",
     lambda t: dict(codes_k=torch.zeros((2, 2, 600, 31), dtype=torch.uint8, device=DEV),
                    codes_v=torch.zeros((2, 2, 600, 31), dtype=torch.uint8, device=DEV)),
     "codes_k rows"),
    ("12-bit key codebook with 32-byte rows",
     lambda t: dict(cb_k=torch.zeros((2, 4096, 4), dtype=torch.float16, device=DEV)),
     "codes_k rows"),
    ("out with one query head too few",
     lambda t: dict(out=torch.empty((2, 7, 128), dtype=torch.float32, device=DEV)), "out"),
    ("out in fp16", lambda t: dict(out=torch.empty((2, 8, 128), dtype=torch.float16, device=DEV)),
     "out"),
    ("non-contiguous out",
     lambda t: dict(out=torch.empty((2, 128, 8), dtype=torch.float32, device=DEV).transpose(1, 2)),
     "out"),
]


@pytest.mark.parametrize("name,make,needle", BAD, ids=[b[0] for b in BAD])
def test_decode_attention_refuses(cache, name, make, needle):
    with pytest.raises(ValueError, match=None) as e:
        attend(cache, **make(cache))
    assert needle in str(e.value), str(e.value)


@pytest.mark.parametrize("fn", [vq.decode_step, vq.decode_step_noalloc],
                         ids=["decode_step", "decode_step_noalloc"])
@pytest.mark.parametrize("name,make,needle", BAD, ids=[b[0] for b in BAD])
def test_decode_step_refuses(cache, fn, name, make, needle):
    with pytest.raises(ValueError) as e:
        step(cache, fn, **make(cache))
    assert needle in str(e.value), str(e.value)


def test_workspace_of_the_wrong_dtype(cache):
    with pytest.raises(ValueError, match="workspace"):
        attend(cache, ws=torch.empty(1 << 20, dtype=torch.float32, device=DEV))


def test_new_rows_of_the_wrong_width(cache):
    with pytest.raises(ValueError, match="k_new"):
        step(cache, kn=torch.zeros((2, 2, 64), dtype=torch.float16, device=DEV))


def test_the_good_shapes_pass(cache):
    out = attend(cache)
    torch.cuda.synchronize()
    assert out.shape == (2, 8, 128) and bool(torch.isfinite(out).all())
