"""The benchmark's byte accounting, pinned to the byte counts the pages print."""
import json
import os

import pytest

import bench
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "byte_counts.json")


@pytest.fixture(scope="module")
def gold():
    return json.load(open(GOLDEN))


def test_code_bytes_per_token_head(gold):
    wl = W.WORKLOADS[4]
    ab = bench.algorithmic_bytes(wl, wl.context_len)
    assert ab["per_unit"] == 2 * gold["index_bytes_2bit"]["value"]        # K and V codes
    assert ab["units"] == wl.batch * wl.num_kv_heads * wl.context_len
    cb = 2 * gold["codebook_2bit"]["value"] * wl.num_kv_heads             # C_k and C_v
    fixed = cb + 32 * 128 * 2 + 8 * 128 * 4 + 32 * 128 * 4
    assert ab["total"] == ab["per_unit"] * ab["units"] + fixed


def test_mixed_bit_code_bytes():
    wl = W.WORKLOADS[5]
    assert bench.algorithmic_bytes(wl, 10)["per_unit"] == 48 + 32


def test_fp16_bytes_match_the_blog_example(gold):
    # a 4096-wide MHA layer: 32 KV heads of 128 -> 16 KB of K+V per token
    g = gold["fp16_kv_bytes_per_token_layer"]
    wl = W.Workload(0, "mha", batch=1, num_q_heads=32, num_kv_heads=32, context_len=1)
    per_token = bench.fp16_bytes(wl, 1000) - bench.fp16_bytes(wl, 999)
    assert per_token == g["value"]
    assert per_token // 32 == 2 * gold["fp16_vector_bytes"]["value"]


def test_multi_gpu_request_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
