"""Benchmark: one decode step over a VQ-KV cache layer on one MI355X.

A step is the whole hot path over one batch: append one new token per
(sequence, KV head) into the last slot of the cache and run decode attention
of every query head over the full context — one vq_decode_step call, whose
split kernel encodes the token before attending.  The default workload is the
Llama-3.1-8B-shaped layer at 196608 tokens (batch 1, 32 query heads over 8 KV
heads, D = 128, 2-bit K and V: 8-bit codes over 4-dim sub-vectors, 256-entry
fp16 codebooks).

Inputs are seeded synthetic tensors (see ``workloads``); the cache is drawn
directly as uniform codes.  Timing keeps every input resident in HBM and
rotates over enough independent copies of the cache (>= 1 GiB in total) that
the 256 MB Infinity Cache cannot hold the codes between steps.

Prints one JSON line (rank 0).  Only N = 1 GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "VQ-KV decode attn: KV tokens/s per layer + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
COLD_BYTES = 1 << 30


def algorithmic_bytes(wl: W.Workload, context_len: int, append: bool = False) -> dict:
    """Bytes one decode-attention launch must move at minimum.

    Per KV token per KV head: (D/d) (bk + bv) / 8 bytes of codes (VecInfer
    page, Background: (d_h/d)(b/8) index bytes per vector), i.e. 64 B for 8-bit
    K and V codes; plus once per launch the fp16 codebooks (2^b x d x 2 bytes
    each), q, lambda and the fp32 output.  With `append`, the launch also reads
    the new token's k and v rows (fp16) and writes its codes (its read of the
    codes is already counted in the context)."""
    units = wl.batch * wl.num_kv_heads * context_len
    per_unit = wl.num_sub * (wl.k_bits + wl.v_bits) // 8
    fixed = (wl.num_kv_heads * ((1 << wl.k_bits) + (1 << wl.v_bits)) * wl.sub_dim * 2
             + wl.batch * wl.num_q_heads * wl.head_dim * 2
             + wl.num_kv_heads * wl.head_dim * 4
             + wl.batch * wl.num_q_heads * wl.head_dim * 4)
    if append:
        fixed += wl.batch * wl.num_kv_heads * (2 * wl.head_dim * 2 + per_unit)
    return {"per_unit": per_unit, "units": units, "total": per_unit * units + fixed}


def fp16_bytes(wl: W.Workload, context_len: int) -> int:
    """K and V in fp16: 2 x D x 2 bytes per KV token per KV head (VecInfer page,
    Background: an uncompressed d_h-vector takes d_h x 2 bytes), plus q/out."""
    return (wl.batch * wl.num_kv_heads * context_len * 2 * wl.head_dim * 2
            + wl.batch * wl.num_q_heads * wl.head_dim * (2 + 4))


def cpu_baseline(wl: W.Workload, seconds: float) -> dict:
    """The fp64 oracle, as is, timed on the host: whole KV heads of sequence 0
    at the full context, cycling over the layer's KV heads until `seconds`
    have passed, scaled to KV tokens/s per layer.  Inputs are drawn before
    the clock starts."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    n, g = wl.context_len, wl.group
    q = W.queries(wl.config_id, 0, wl.num_q_heads).astype(np.float16)
    heads = []
    for h in range(wl.num_kv_heads):
        heads.append((q[h * g:(h + 1) * g], W.random_lambda(wl.config_id, h),
                      W.random_codebook(wl.config_id, h, "k", 1 << wl.k_bits, 0.6,
                                        sub_dim=wl.sub_dim),
                      W.random_codebook(wl.config_id, h, "v", 1 << wl.v_bits, 1.0, 1 / 32,
                                        sub_dim=wl.sub_dim),
                      W.random_code_rows(wl.config_id, 0, h, "k", n, wl.k_row_bytes),
                      W.random_code_rows(wl.config_id, 0, h, "v", n, wl.v_row_bytes)))
    def run(limit_s: float) -> tuple[int, float]:
        done = 0
        t0 = time.perf_counter()
        while True:
            oracle.decode_attention_head(*heads[done % len(heads)], wl.k_bits, wl.v_bits)
            done += 1
            dt = time.perf_counter() - t0
            if dt >= limit_s:
                return done, dt

    done, dt = run(seconds)
    per_layer = dt / done * wl.num_kv_heads
    threads = max([1] + [p.get("num_threads", 1) for p in threadpool_info()])
    # the same oracle with its thread pools held to one thread, a shorter sample
    with threadpool_limits(limits=1):
        done1, dt1 = run(seconds / 4)
    value = n / per_layer
    value1 = n / (dt1 / done1 * wl.num_kv_heads)
    return {"value": value, "unit": "KV tokens/s per layer",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} KV-head passes (of {wl.num_kv_heads} per layer) of sequence 0 at "
                      f"N={n} in {dt:.1f} s, scaled to one layer of one sequence",
            "host": host_info(),
            "thread_scaling": value / value1,
            "note": "cores is the BLAS thread pool the oracle ran with; only its two matrix "
                    "products use it, and its table-lookup dequantisation (most of the time) "
                    "runs on one core, so the rate barely scales with threads "
                    "(thread_scaling = rate / single-thread rate)",
            "single_thread": {"value": value1, "cores": 1,
                              "sample": f"{done1} KV-head passes in {dt1:.1f} s"}}


def host_info() -> dict:
    """The host CPU the oracle ran on: model name, logical CPUs, the CPUs this
    process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0))}


# Sources that determine the attention kernel's code: a counter record taken
# from other sources no longer describes it.
KERNEL_SOURCES = ["vector_quantized_bit_amd/csrc/vq_attention_mfma.hip",
                  "vector_quantized_bit_amd/csrc/launchers.hpp",
                  "vector_quantized_bit_amd/csrc/device_common.hpp",
                  "vector_quantized_bit_amd/csrc/nearest_search.hpp",
                  "vector_quantized_bit_amd/build.py"]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters(workload: str, score_method: str) -> dict | None:
    """Per-dispatch shader counters of the split kernel (waves, instructions,
    LDS activity) from the committed counter record of this workload, or None
    when there is no record, it was taken with another score method, or the
    kernel sources have changed since."""
    suffix = "" if score_method == "mfma" else f".{score_method}"
    path = os.path.join(ROOT, "profiles", f"counters_{workload}{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    if rec.get("score_method", "mfma") != score_method:
        return None
    return dict(rec["per_dispatch"], source=os.path.relpath(path, ROOT))


def sampled_parity(oracle, wl: W.Workload, q, lam, cb_k, cb_v, codes_k, codes_v, out,
                   heads) -> dict:
    """The GPU output of sequence 0 against the fp64 oracle for the given KV
    heads, over the codes as they are on the device (the timed steps have
    appended tokens to them): rel-L2 and max-abs over those query heads."""
    g = wl.group
    got, ref = [], []
    for h in heads:
        ref.append(oracle.decode_attention_head(
            q[0, h * g:(h + 1) * g], lam[h], cb_k[h], cb_v[h], codes_k[h], codes_v[h],
            wl.k_bits, wl.v_bits))
        got.append(out[0, h * g:(h + 1) * g].astype(np.float64))
    got, ref = np.concatenate(got), np.concatenate(ref)
    return {"kv_heads": list(heads), "sequence": 0, "context_len": wl.context_len,
            "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
            "max_abs": float(np.abs(got - ref).max()),
            "bound": {"rel_l2": 1e-3, "max_abs": 2e-3}}


def percentiles(us: np.ndarray) -> dict:
    return {"median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90)), "calls": int(us.size)}


def measured_traffic(workload: str, score_method: str) -> dict | None:
    """HBM bytes per attention launch from the committed counter record of
    this workload (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what
    the same counter read for a plain copy of known size), or None when there
    is no record, it was taken with another score method, or the kernel
    sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    if rec.get("score_method", "mfma") != score_method:
        return None
    fetch = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"]
    write = rec["write_kib_per_dispatch"] * 1024 * rec["write_scale"]
    return {"bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "source": os.path.relpath(path, ROOT)}


def copy_calibration(torch, dev, mib: int = 256, reps: int = 3) -> None:
    """Plain device copies of known size (`mib` MiB read, `mib` MiB written)
    for scaling the HBM byte counters; each copy is its own dispatch."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def copy_bandwidth(torch, dev, head_start, mib: int = 512, reps: int = 20) -> float:
    """GB/s of a plain device copy (`mib` MiB read and written per copy, far
    above the 256 MB Infinity Cache), back to back between one event pair:
    the streaming rate this chip reaches in practice."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    head_start()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2 * (mib << 20) * reps / (a.elapsed_time(b) * 1e-3) / 1e9


MFMA_F32_PEAK_TFLOPS = 157.3
PREFILL_TOKENS = 32768


def synthetic_rows(torch, wl, dev, shape, tensor, seed):
    """N(0, 1) rows [..., Hkv, T, 128] in fp16 with each head's x15 outlier
    channels (the distribution of the test inputs), drawn on the GPU."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.empty(shape, dtype=torch.float32, device=dev).normal_(generator=g)
    for h in range(shape[-3]):
        ch = torch.from_numpy(W.outlier_channels(wl.config_id, h, tensor)).to(dev)
        x[..., h, :, ch] *= W.OUTLIER_SCALE
    return x.to(torch.float16)


def time_calls(torch, fn, reps, head_start, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    head_start()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def distance_flops(pairs: int, sub_dim: int = 4) -> int:
    """One dense pass of the nearest-centroid search as a contraction:
    ||c||^2 - 2 x.c for every (sub-vector, centroid) pair, d multiply-adds."""
    return 2 * sub_dim * pairs


def prefill_encode(torch, vq, wl, dev, lam, cb_k, cb_v, head_start) -> dict:
    """A prompt of PREFILL_TOKENS tokens per sequence encoded by one
    vq_encode_append call (every KV head of the layer)."""
    bsz, hkv = wl.batch, wl.num_kv_heads
    p = min(PREFILL_TOKENS, wl.context_len)
    kp = synthetic_rows(torch, wl, dev, (bsz, hkv, p, 128), "k", 1000 + wl.config_id)
    vp = synthetic_rows(torch, wl, dev, (bsz, hkv, p, 128), "v", 2000 + wl.config_id)
    ck = torch.empty((bsz, hkv, p, wl.k_row_bytes), dtype=torch.uint8, device=dev)
    cv = torch.empty((bsz, hkv, p, wl.v_row_bytes), dtype=torch.uint8, device=dev)
    enc = vq.prepare_encode_append(kp, vp, lam, cb_k, cb_v, ck, cv, 0)
    us = time_calls(torch, enc, 5, head_start)
    pairs = bsz * hkv * p * wl.num_sub * ((1 << wl.k_bits) + (1 << wl.v_bits))
    flops = distance_flops(pairs, wl.sub_dim)
    tflops = flops / (us * 1e-6) / 1e12
    hbm = bsz * hkv * p * (2 * 128 * 2 + wl.k_row_bytes + wl.v_row_bytes)
    return {"workload": f"{wl.name}-prompt-{p}", "tokens": bsz * p, "avg_launch_us": us,
            "tokens_per_s": bsz * p / (us * 1e-6), "hbm_gbps": hbm / (us * 1e-6) / 1e9,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / MFMA_F32_PEAK_TFLOPS,
                         "kernel": "encode_append8_kernel" if wl.sub_dim == 8
                         else "encode_append_kernel",
                         "flops_per_launch": flops}}


APPEND_TOKENS = 64


def append_encode(torch, vq, wl, dev, lam, cb_k, cb_v, codes_k, codes_v, head_start) -> dict:
    """A chunk of APPEND_TOKENS new tokens per sequence encoded into the
    cache's last slots by one vq_encode_append call (every KV head)."""
    bsz, hkv, n = wl.batch, wl.num_kv_heads, wl.context_len
    t = min(APPEND_TOKENS, n)
    kp = synthetic_rows(torch, wl, dev, (bsz, hkv, t, 128), "k", 5000 + wl.config_id)
    vp = synthetic_rows(torch, wl, dev, (bsz, hkv, t, 128), "v", 6000 + wl.config_id)
    enc = vq.prepare_encode_append(kp, vp, lam, cb_k, cb_v, codes_k, codes_v, n - t)
    us = time_calls(torch, enc, 10, head_start)
    pairs = bsz * hkv * t * wl.num_sub * ((1 << wl.k_bits) + (1 << wl.v_bits))
    tflops = distance_flops(pairs, wl.sub_dim) / (us * 1e-6) / 1e12
    return {"tokens_per_sequence": t, "cur_len": n - t, "avg_launch_us": us,
            "token_heads_per_s": bsz * hkv * t / (us * 1e-6),
            "dense_pass_tflops": tflops, "frac_of_mfma_f32_peak": tflops / MFMA_F32_PEAK_TFLOPS}


def calibration(torch, vq, wl, dev, head_start, iters: int) -> dict:
    """The offline calibration path at the page's calibration-set size (256
    sequences x 512 tokens per KV head): lambda, K~, and Lloyd K-Means for
    C_k and C_v (and a 4096-entry C_k)."""
    hkv, t = wl.num_kv_heads, W.CALIB_TOKENS
    keys = synthetic_rows(torch, wl, dev, (hkv, t, 128), "k", 3000)
    vals = synthetic_rows(torch, wl, dev, (hkv, t, 128), "v", 4000)
    lam = torch.empty((hkv, 128), dtype=torch.float32, device=dev)
    kt = torch.empty((hkv, t, 128), dtype=torch.float32, device=dev)
    lam_us = time_calls(torch, lambda: vq.calibrate_lambda(keys, out=lam), 10, head_start)
    tk_us = time_calls(torch, lambda: vq.transform_keys(keys, lam, out=kt), 10, head_start)
    out = {"workload": f"{hkv} KV heads x {W.CALIB_SEQS} x {W.CALIB_SEQ_LEN} calibration tokens",
           "lambda_us": lam_us, "lambda_gbps": keys.numel() * 2 / (lam_us * 1e-6) / 1e9,
           "transform_keys_us": tk_us,
           "transform_keys_gbps": keys.numel() * 6 / (tk_us * 1e-6) / 1e9}
    n = t * 32
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5)
    km = {}
    for name, samples, bits, its in (("k8", kt.view(hkv, n, 4), 8, iters),
                                     ("v8", vals.float().view(hkv, n, 4), 8, iters),
                                     ("k12", kt.view(hkv, n, 4), 12, max(1, iters // 2)),
                                     ("k12_d8", kt.view(hkv, n // 2, 8), 12, max(1, iters // 2))):
        ent = 1 << bits
        rows = samples.shape[1]
        idx = torch.randperm(rows, generator=gen)[:ent].to(dev)
        init = samples[:, idx].double().contiguous()
        cent = torch.empty_like(init)
        sub = samples.shape[2]
        ws = torch.empty(vq.kmeans_workspace_bytes(hkv, rows, bits, sub), dtype=torch.uint8,
                         device=dev)
        us = time_calls(torch, lambda: vq.kmeans(samples, init, its, centroids=cent, workspace=ws),
                        1, head_start, warm=1)
        per_it = us / its
        tflops = distance_flops(hkv * rows * ent, sub) / (per_it * 1e-6) / 1e12
        km[name] = {"sets": hkv, "samples_per_set": rows, "sub_dim": sub, "entries": ent,
                    "iters": its,
                    "us_per_iter": per_it, "dense_pass_tflops": tflops,
                    "frac_of_mfma_f32_peak": tflops / MFMA_F32_PEAK_TFLOPS}
    out["kmeans"] = km
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="workload id (see workloads)")
    ap.add_argument("--splits", type=int, default=0, help="split count (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="host time spent timing the oracle")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain copies of known size (for byte-counter runs)")
    ap.add_argument("--no-fp16", action="store_true", help="skip the fp16 comparator")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill encode timing")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration timings (lambda, K~, K-Means)")
    ap.add_argument("--kmeans-iters", type=int, default=3,
                    help="Lloyd iterations per timed K-Means call")
    ap.add_argument("--score-method", choices=["mfma", "lut"], default="mfma",
                    help="split-kernel scores: matrix cores (default) or the q~ . C_k lookup "
                         "table (8-bit keys, G <= 4)")
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed tile order in the split kernel (bit-reproducible results)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration",
              file=sys.stderr)
        return 2

    import torch

    import vector_quantized_bit_amd as vq

    wl = W.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    vq.set_score_method(vq.SCORES_LUT if args.score_method == "lut" else vq.SCORES_MFMA)
    vq.set_deterministic(args.deterministic)
    torch.cuda.set_device(dev)
    n, cap, bsz, hkv, hq = wl.context_len, wl.context_len, wl.batch, wl.num_kv_heads, wl.num_q_heads
    st = np.float16 if wl.qkv_dtype == "f16" else np.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- inputs (resident in HBM before timing) ---------------------------
    q = t(np.stack([W.queries(wl.config_id, b, hq) for b in range(bsz)]).astype(st))
    lam = t(np.stack([W.random_lambda(wl.config_id, g) for g in range(hkv)]))
    cb_k = t(np.stack([W.random_codebook(wl.config_id, g, "k", 1 << wl.k_bits, 0.6,
                                         sub_dim=wl.sub_dim) for g in range(hkv)]))
    cb_v = t(np.stack([W.random_codebook(wl.config_id, g, "v", 1 << wl.v_bits, 1.0, 1 / 32,
                                         sub_dim=wl.sub_dim) for g in range(hkv)]))
    ck0 = torch.empty((bsz, hkv, cap, wl.k_row_bytes), dtype=torch.uint8, device=dev)
    cv0 = torch.empty((bsz, hkv, cap, wl.v_row_bytes), dtype=torch.uint8, device=dev)
    for b in range(bsz):
        for g in range(hkv):
            ck0[b, g] = t(W.random_code_rows(wl.config_id, b, g, "k", cap, wl.k_row_bytes))
            cv0[b, g] = t(W.random_code_rows(wl.config_id, b, g, "v", cap, wl.v_row_bytes))
    k_new = t(np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "k", 1, append=True)
                                  for g in range(hkv)]) for b in range(bsz)]).astype(st))
    v_new = t(np.stack([np.stack([W.kv_rows(wl.config_id, b, g, "v", 1, append=True)
                                  for g in range(hkv)]) for b in range(bsz)]).astype(st))
    cache_bytes = ck0.numel() + cv0.numel()
    copies = max(1, -(-COLD_BYTES // cache_bytes))
    caches = [(ck0, cv0)] + [(ck0.clone(), cv0.clone()) for _ in range(copies - 1)]
    out = torch.empty((bsz, hq, 128), dtype=torch.float32, device=dev)
    splits = args.splits or vq.decode_attention_default_splits(ck0, cv0, cb_k, cb_v, bsz, hq, n)

    # Arguments are marshalled once per cache copy, so the host stays ahead
    # of the GPU.  A step appends one token per (sequence, KV head) at slot
    # n - 1 and attends over all n tokens: vq_decode_step, i.e. one launch of
    # the split kernel (which encodes the token) and the merge.
    k_new2, v_new2 = k_new[:, :, 0].contiguous(), v_new[:, :, 0].contiguous()
    step_parts = vq.decode_step_num_partials(ck0, cv0, cb_k, cb_v, bsz, hq, n - 1, args.splits)
    ws_step = torch.empty(vq.decode_step_workspace_bytes(ck0, cv0, cb_k, cb_v, bsz, hq, n - 1,
                                                         args.splits),
                          dtype=torch.uint8, device=dev)
    steps_fused = [vq.prepare_decode_step(q, k_new2, v_new2, lam, cb_k, cb_v, ck, cv, n - 1,
                                          args.splits, out, ws_step) for ck, cv in caches]
    parts = vq.decode_step_partials(q, k_new2, v_new2, lam, cb_k, cb_v, ck0, cv0, n - 1,
                                    args.splits)
    split_pass = [vq.prepare_decode_step_partials(q, k_new2, v_new2, lam, cb_k, cb_v, ck, cv,
                                                  n - 1, args.splits, partials=parts)
                  for ck, cv in caches]
    merge = vq.prepare_merge_partials(parts, out)
    ws = torch.empty(vq.decode_attention_workspace_bytes(ck0, cv0, cb_k, cb_v, bsz, hq, n, splits),
                     dtype=torch.uint8, device=dev)
    attends = [vq.prepare_decode_attention(q, lam, cb_k, cb_v, ck, cv, n, splits, out, ws)
               for ck, cv in caches]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def head_start():
        # a spin kernel (a few ms) ahead of a timed loop: the host enqueues the
        # whole loop meanwhile, so no timed interval contains host gaps
        torch.cuda._sleep(10_000_000)
    steps, warm = args.steps, args.warmup

    for i in range(warm):
        steps_fused[i % copies](stream)
    torch.cuda.synchronize()

    # 1. whole steps back to back: the throughput (no events inside, since
    #    every event costs the stream a few microseconds)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    head_start()
    start.record()
    for i in range(steps):
        steps_fused[i % copies](stream)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps

    # 2. the split kernel alone: the steps' split passes back to back between
    #    one event pair, averaged over the launches
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    head_start()
    ev0.record()
    for i in range(steps):
        split_pass[i % copies](stream)
    ev1.record()
    torch.cuda.synchronize()
    split_us = ev0.elapsed_time(ev1) * 1e3 / steps
    merge(stream)

    # 3. decode attention alone (no append): vq_decode_attention calls (split
    #    pass and merge) back to back between one event pair
    head_start()
    ev0.record()
    for i in range(steps):
        attends[i % copies](stream)
    ev1.record()
    torch.cuda.synchronize()
    call_us = ev0.elapsed_time(ev1) * 1e3 / steps

    # 3b. the same calls and the steps one by one, each between its own event
    #     pair (an event costs the stream a few microseconds, so these read
    #     higher than the back-to-back averages): the spread of a call
    def per_call(calls):
        ea = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        head_start()
        for i in range(steps):
            ea[i].record()
            calls[i % copies](stream)
            eb[i].record()
        torch.cuda.synchronize()
        return percentiles(np.array([ea[i].elapsed_time(eb[i]) * 1e3 for i in range(steps)]))
    call_pct = per_call(attends)
    step_pct = per_call(steps_fused)

    # 4. decode steps with a full-precision residual window of 128 tokens at
    #    the same total length: n - 128 coded tokens, window slots 0..127
    #    (slot 127 takes the new token), and the flush that encodes a full
    #    window into codes
    win = 128
    win_k = torch.empty((bsz, hkv, win, 128), dtype=torch.float16, device=dev)
    win_v = torch.empty_like(win_k)
    win_k.normal_()
    win_v.normal_()
    steps_win = [vq.prepare_decode_step_window(q, k_new2, v_new2, lam, cb_k, cb_v, ck, cv, win_k,
                                               win_v, n - win, win - 1, args.splits)
                 for ck, cv in caches]
    for i in range(3):
        steps_win[i % copies](stream)
    torch.cuda.synchronize()
    head_start()
    ev0.record()
    for i in range(steps):
        steps_win[i % copies](stream)
    ev1.record()
    torch.cuda.synchronize()
    win_step_us = ev0.elapsed_time(ev1) * 1e3 / steps
    flushes = max(10, steps // 5)
    head_start()
    ev0.record()
    for i in range(flushes):
        ck, cv = caches[i % copies]
        vq.flush_window(win_k, win_v, lam, cb_k, cb_v, ck, cv, n - win)
    ev1.record()
    torch.cuda.synchronize()
    flush_us = ev0.elapsed_time(ev1) * 1e3 / flushes

    attn_us = float(split_us)
    assert torch.isfinite(out).all().item()

    if args.copy_calibration:
        copy_calibration(torch, dev)

    ab = algorithmic_bytes(wl, n, append=True)
    ab_attn = algorithmic_bytes(wl, n)
    achieved = ab["total"] / (attn_us * 1e-6) / 1e9
    traffic = measured_traffic(wl.name, args.score_method)
    tokens = bsz * n
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "KV tokens/s per layer",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands (q~ and p split into hi/lo fp16 parts), f32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": bsz, "context_len": n, "q_heads": hq,
                   "kv_heads": hkv, "head_dim": 128, "k_code_bits": wl.k_bits,
                   "v_code_bits": wl.v_bits, "sub_dim": wl.sub_dim, "append_tokens_per_step": 1,
                   "step_partials": step_parts, "attention_splits": splits,
                   "cold_cache_copies": copies, "score_method": args.score_method,
                   "deterministic": args.deterministic},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic["bytes"],
                     "kernel": "vq_attention_mfma_kernel (vq_decode_step_partials: append + split pass)",
                     "bytes_per_launch": ab["total"], "bytes_per_unit": ab["per_unit"],
                     "units_per_launch": ab["units"], "avg_launch_us": attn_us,
                     "timing": "one HIP event pair around the back-to-back split passes, per launch",
                     "traffic_record": None if traffic is None else traffic["source"]},
        "step_hbm_gbps": ab["total"] / (ms_step * 1e-3) / 1e9,
        "decode_step_window": {"avg_us": win_step_us, "coded_tokens": n - win,
                               "window_tokens": win,
                               "tokens_per_s": tokens / (win_step_us * 1e-6),
                               "flush_us": flush_us, "flush_tokens_per_stream": win},
        "decode_attention": {"avg_us": call_us,
                             "gbps": ab_attn["total"] / (call_us * 1e-6) / 1e9,
                             "kernels": "vq_attention_mfma_kernel + merge_partials_kernel",
                             "per_call_us": call_pct},
        "decode_step_per_call_us": step_pct,
    }
    counters = measured_counters(wl.name, args.score_method)
    if counters is not None:
        result["roofline"]["counters"] = counters
    copy_gbps = copy_bandwidth(torch, dev, head_start)
    result["roofline"]["copy_gbps"] = copy_gbps
    result["roofline"]["frac_of_copy"] = achieved / copy_gbps

    if not args.no_fp16:
        fk = torch.empty((bsz, hkv, cap, 128), dtype=torch.float16, device=dev)
        fv = torch.empty_like(fk)
        g16 = torch.Generator(device=dev)
        g16.manual_seed(wl.config_id)
        fk.normal_(generator=g16)
        fv.normal_(generator=g16)
        fcopies = max(1, -(-COLD_BYTES // (2 * fk.numel() * 2)))
        fcaches = [(fk, fv)] + [(fk.clone(), fv.clone()) for _ in range(fcopies - 1)]
        q16 = q.to(torch.float16)
        fws = torch.empty(vq.fp16_attention_workspace_bytes(bsz, hq, hkv, n), dtype=torch.uint8,
                          device=dev)
        fout = torch.empty_like(out)
        reps = max(10, steps // 2)
        fa = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        fb = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(3):
            vq.fp16_decode_attention(q16, *fcaches[i % fcopies], n, out=fout, workspace=fws)
        torch.cuda.synchronize()
        head_start()
        for i in range(reps):
            fa[i].record()
            vq.fp16_decode_attention(q16, *fcaches[i % fcopies], n, out=fout, workspace=fws)
            fb[i].record()
        torch.cuda.synchronize()
        f_us = float(np.mean([fa[i].elapsed_time(fb[i]) for i in range(reps)]) * 1e3)
        result["fp16_comparator"] = {
            "avg_launch_us": f_us, "gbps": fp16_bytes(wl, n) / (f_us * 1e-6) / 1e9,
            "vq_decode_attention_speedup": f_us / call_us, "cold_cache_copies": fcopies}
        del fcaches, fk, fv

    if not args.no_prefill:
        result["prefill_encode"] = prefill_encode(torch, vq, wl, dev, lam, cb_k, cb_v, head_start)
        result["append_encode"] = append_encode(torch, vq, wl, dev, lam, cb_k, cb_v, ck0, cv0,
                                                head_start)
    if not args.no_calibration:
        result["calibration"] = calibration(torch, vq, wl, dev, head_start, args.kmeans_iters)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        # the same leg checks the output of one more call against the oracle
        import oracle
        ck, cv = caches[0]
        attends[0](stream)
        torch.cuda.synchronize()
        heads = sorted({0, hkv - 1})
        result["cpu_baseline"]["parity"] = sampled_parity(
            oracle, wl, q.cpu().numpy(), lam.cpu().numpy(), cb_k.cpu().numpy(),
            cb_v.cpu().numpy(), {h: ck[0, h].cpu().numpy() for h in heads},
            {h: cv[0, h].cpu().numpy() for h in heads}, out.cpu().numpy(), heads)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
