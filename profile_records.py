"""Reduce rocprofv3 output of bench.py runs to the short text records kept
under profiles/.

Three reductions, each reading the CSV files that rocprofv3 wrote with
``--output-format csv -d DIR -o PREFIX``:

  trace     ``--kernel-trace --stats`` of a bench.py run -> a Markdown summary:
            per-kernel statistics, and the split kernel's durations per timed
            loop of bench.py (each loop starts behind one spin kernel), with the
            idle gaps between launches.
  traffic   two ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE) of
            ``bench.py --copy-calibration`` -> HBM bytes per split-kernel
            dispatch, each counter scaled by what it read for the plain 256 MiB
            copy of the same run; JSON (read by bench.py) plus a Markdown copy.
  counters  one or more ``--pmc`` runs of shader counters -> per-dispatch means
            for the split kernel, as JSON (read by bench.py).
  compare   two counter records side by side -> a Markdown table.
  encoder, calibration
            the prefill encoder's or the K-Means assignment's launches of a
            ``--kernel-trace`` run, by grid, with the same run's bench.py
            figures -> a Markdown summary.

Each record stores the commands given here and a sha256 of the kernel's
sources; bench.py ignores a record whose hash no longer matches.

Usage, from the repository root, for example:

  python profile_records.py trace --dir <rocprofv3 output dir> --prefix trace \\
      --command "rocprofv3 ... -- python -u bench.py ..." \\
      --out profiles/vq_attention_mfma_kernel.<workload>.kernel_trace.md
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics as st
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

SPLIT = "vq_attention_mfma_kernel"
MERGE = "merge_partials_kernel"
SPIN = "spin_kernel"
COPY = "MulFunctor"   # torch.mul(src, 1.0, out=dst) of --copy-calibration

# The timed loops of bench.py in the order they run; each follows one spin
# kernel (its head start).
BENCH_LOOPS = [
    "decode steps back to back (split pass + merge)",
    "split passes back to back (the event-timed loop: roofline.avg_launch_us)",
    "vq_decode_attention calls back to back (split pass + merge, no append)",
    "vq_decode_attention calls, one event pair each",
    "decode steps, one event pair each",
    "decode steps with a 128-token residual window",
    "window flushes",
]


def _csv(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(directory: str, suffix: str) -> str:
    for dirpath, _, files in os.walk(directory):
        for name in sorted(files):
            if name.endswith(suffix):
                return os.path.join(dirpath, name)
    raise SystemExit(f"no *{suffix} under {directory}")


def short_name(name: str) -> str:
    """Kernel name without the argument list and the namespace of torch's
    templated elementwise kernels."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    if base.startswith("void "):
        base = base[5:]
    if "at::native" in base or "at::cuda" in base:
        tail = base.split("::")[-1] or base
        return "torch " + tail[-40:]
    return base


def kernel_loops(trace_rows: list[dict]) -> list[list[tuple[str, float, float]]]:
    """Dispatches grouped into the loops that follow each spin kernel:
    [(short name, start ns, end ns)] per loop, in start order."""
    rows = sorted(trace_rows, key=lambda r: int(r["Start_Timestamp"]))
    loops, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        if SPIN in name:
            cur = []
            loops.append(cur)
            continue
        if cur is not None:
            cur.append((name, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    return loops


def loop_table(loops) -> list[str]:
    lines = ["| loop | split launches | split avg us | min | max | merge avg us "
             "| gap before a split, avg us |",
             "|---|---|---|---|---|---|---|"]
    for i, lp in enumerate(loops):
        sp = [(e - s) / 1e3 for n, s, e in lp if SPLIT in n]
        if not sp:
            continue
        mg = [(e - s) / 1e3 for n, s, e in lp if MERGE in n]
        gaps = [(lp[j][1] - lp[j - 1][2]) / 1e3 for j in range(1, len(lp)) if SPLIT in lp[j][0]]
        label = f"{i + 1}: {BENCH_LOOPS[i]}" if i < len(BENCH_LOOPS) else f"{i + 1}"
        merge_avg = f"{st.mean(mg):.2f}" if mg else "-"
        gap_avg = f"{st.mean(gaps):.2f}" if gaps else "-"
        lines.append(f"| {label} | {len(sp)} | {st.mean(sp):.2f} | {min(sp):.2f} | "
                     f"{max(sp):.2f} | {merge_avg} | {gap_avg} |")
    return lines


def grid_groups(trace: list[dict], sub: str) -> list:
    """Launch durations (us) of the kernels whose name contains `sub`, by
    (short name, grid in workgroups), longest average first."""
    groups: dict = collections.defaultdict(list)
    for r in trace:
        if sub in r["Kernel_Name"]:
            grid = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                    int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
            groups[(short_name(r["Kernel_Name"]), grid)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return sorted(groups.items(), key=lambda kv: -st.mean(kv[1]))


def bench_line(path: str) -> dict:
    """The JSON line bench.py printed into a log."""
    with open(path) as f:
        lines = [ln for ln in f if ln.startswith('{"metric"')]
    if not lines:
        raise SystemExit(f"no bench.py line in {path}")
    return json.loads(lines[-1])


def _header(title: str, command: str, reduced: str) -> list[str]:
    return [f"# Kernel trace summary: {title}", "",
            "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`; the",
            "library built in-tree):", "", f"    {command}", "",
            "Reduced by:", "", f"    {reduced}", ""]


def cmd_encoder(a) -> None:
    """The prefill encoder's launches in a bench.py run (by grid), with the
    same run's bench.py figures, and the other layouts' prefill launches."""
    trace = _csv(os.path.join(a.dir, f"{a.prefix}_kernel_trace.csv"))
    line = bench_line(a.log)
    pe, ae = line["prefill_encode"], line["append_encode"]
    out = _header(a.title, a.command,
                  f"python profile_records.py encoder --dir {a.dir} --log {a.log} "
                  f"--others ... --out {a.out} --command '...'")
    out += ["bench.py's `prefill_encode` section times one `vq_encode_append` call over a",
            f"{pe['tokens']}-token prompt for every KV head of the layer (fp16 K and V, "
            f"`{pe['roofline']['kernel']}`): warm-up and timed launches back to back. The",
            "64-token append and the residual-window flushes launch the same kernel.", "",
            "| kernel | grid (workgroups) | launches | avg us | min us | max us |",
            "|---|---|---|---|---|---|"]
    for (name, grid), d in grid_groups(trace, "encode_append"):
        out.append(f"| {name} | {grid[0]} x {grid[1]} x {grid[2]} | {len(d)} | "
                   f"{st.mean(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    r = pe["roofline"]
    out += ["", "The same run's bench.py line (HIP events around the back-to-back launches):",
            f"{pe['avg_launch_us']:.1f} us per prefill launch, {pe['tokens_per_s']:.3g} prompt "
            f"tokens/s, {r['achieved']:.1f} TFLOP/s of one dense distance pass (8 flops per",
            f"sub-vector/centroid pair at d = 4) = {100 * r['frac']:.1f}% of the "
            f"{r['peak']} TFLOP/s fp32 matrix peak; 64-token append {ae['avg_launch_us']:.1f} us."]
    if a.others:
        out += ["", "The other layouts' prefill launches, from their own runs under the same "
                "profiler:", "", "| run | kernel | grid (workgroups) | launches | avg us |",
                "|---|---|---|---|---|"]
        for d in a.others:
            t = _csv(os.path.join(d, f"{a.prefix}_kernel_trace.csv"))
            groups = grid_groups(t, "encode_append")
            if groups:
                (name, grid), dur = groups[0]   # the longest: the prefill
                out.append(f"| {d} | {name} | {grid[0]} x {grid[1]} x {grid[2]} | {len(dur)} | "
                           f"{st.mean(dur):.1f} |")
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print(a.out)


def cmd_calibration(a) -> None:
    """The K-Means assignment launches of a bench.py run (by grid) with the
    same run's calibration figures."""
    trace = _csv(os.path.join(a.dir, f"{a.prefix}_kernel_trace.csv"))
    cal = bench_line(a.log)["calibration"]
    out = _header(a.title, a.command,
                  f"python profile_records.py calibration --dir {a.dir} --log {a.log} "
                  f"--out {a.out} --command '...'")
    out += ["bench.py's `calibration` section: lambda and K~ over the calibration tokens, then "
            "Lloyd K-Means iterations on every codebook's sub-vectors (every KV head a set).", "",
            "| kernel | grid (workgroups) | launches | avg us | min us | max us |",
            "|---|---|---|---|---|---|"]
    for (name, grid), d in grid_groups(trace, "kmeans_assign"):
        out.append(f"| {name} | {grid[0]} x {grid[1]} x {grid[2]} | {len(d)} | "
                   f"{st.mean(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    out += ["", "The same run's bench.py line (HIP events around whole calls):", "",
            f"- lambda: {cal['lambda_us']:.1f} us ({cal['lambda_gbps']:.0f} GB/s); K~: "
            f"{cal['transform_keys_us']:.1f} us ({cal['transform_keys_gbps']:.0f} GB/s)."]
    for name, k in cal["kmeans"].items():
        out.append(f"- K-Means {name}: {k['us_per_iter']:.0f} us per Lloyd iteration over "
                   f"{k['sets']} x {k['samples_per_set']} samples (d = {k['sub_dim']}), "
                   f"{k['entries']} centroids; one dense distance pass per iteration = "
                   f"{k['dense_pass_tflops']:.1f} TFLOP/s "
                   f"({100 * k['frac_of_mfma_f32_peak']:.1f}% of the fp32 matrix peak).")
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print(a.out)


def cmd_trace(a) -> None:
    stats = _csv(os.path.join(a.dir, f"{a.prefix}_kernel_stats.csv"))
    trace = _csv(os.path.join(a.dir, f"{a.prefix}_kernel_trace.csv"))
    title = a.title or f"split kernel in bench.py on {a.workload}"
    out = [f"# Kernel trace summary: {title}", "",
           "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`; the",
           "library built in-tree):", "", f"    {a.command}", "",
           "Reduced by:", "",
           f"    python profile_records.py trace --dir {a.dir} --prefix {a.prefix} "
           f"--workload {a.workload} --out {a.out} --command '...'", "",
           "Per-kernel statistics (rocprofv3 --stats):", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} |")
    out += ["", "The split kernel per timed loop of bench.py (rocprofv3 per-launch "
            "durations; the gap is the idle time between the previous kernel's end and "
            "the split kernel's start):", ""]
    out += loop_table(kernel_loops(trace))
    for sub in a.breakdown or []:
        out += ["", f"Launches of kernels matching `{sub}` by grid size (workgroups):", "",
                "| kernel | grid | launches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for (name, grid), d in grid_groups(trace, sub):
            out.append(f"| {name} | {grid[0]} x {grid[1]} x {grid[2]} | {len(d)} | "
                       f"{st.mean(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    if a.note:
        out += ["", a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print(a.out)


def _per_dispatch(rows: list[dict]) -> tuple[dict, dict]:
    """{dispatch: {counter: value summed over the chip}}, {dispatch: (name, ns)}."""
    vals: dict = collections.defaultdict(dict)
    meta = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        c = r["Counter_Name"]
        vals[d][c] = vals[d].get(c, 0.0) + float(r["Counter_Value"])
        meta[d] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return vals, meta


def _split_means(directory: str, match: str = SPLIT) -> tuple[dict, int, float]:
    """Per-dispatch means of every counter over the dispatches whose kernel
    name contains `match`; their count; their mean duration in us."""
    vals, meta = _per_dispatch(_csv(_find(directory, "counter_collection.csv")))
    ds = [d for d in vals if match in meta[d][0]]
    if not ds:
        raise SystemExit(f"no {match} dispatches in {directory}")
    keys = sorted(vals[ds[0]])
    means = {k: st.mean(vals[d][k] for d in ds) for k in keys}
    return means, len(ds), st.mean(meta[d][1] for d in ds) / 1e3


def _copy_reading(directory: str, counter: str) -> float:
    """Mean reading of the calibration copies: the multiply dispatches within
    10% of the largest reading (other, small multiplies of the run are not
    the 256 MiB copy)."""
    vals, meta = _per_dispatch(_csv(_find(directory, "counter_collection.csv")))
    ds = [d for d in vals if COPY in meta[d][0]]
    if not ds:
        raise SystemExit(f"no copy-calibration dispatches in {directory} "
                         "(run bench.py with --copy-calibration)")
    top = max(vals[d][counter] for d in ds)
    return st.mean(vals[d][counter] for d in ds if vals[d][counter] >= 0.9 * top)


def _source_record() -> dict:
    return {"kernel_source_sha256": bench.kernel_source_digest(),
            "kernel_sources": list(bench.KERNEL_SOURCES)}


def cmd_traffic(a) -> None:
    wl = next((w for w in W.WORKLOADS.values() if w.name == a.workload), None)
    if wl is None:
        raise SystemExit(f"unknown workload {a.workload}")
    copy_kib = 256 * 1024
    fetch, n_f, _ = _split_means(a.fetch_dir)
    write, n_w, _ = _split_means(a.write_dir)
    f_copy = _copy_reading(a.fetch_dir, "FETCH_SIZE")
    w_copy = _copy_reading(a.write_dir, "WRITE_SIZE")
    rec = {"kernel": a.kernel, "workload": a.workload, "score_method": a.score_method,
           **_source_record(),
           "fetch_kib_per_dispatch": fetch["FETCH_SIZE"],
           "write_kib_per_dispatch": write["WRITE_SIZE"],
           "dispatches": min(n_f, n_w),
           "fetch_scale": copy_kib / f_copy, "write_scale": copy_kib / w_copy,
           "calibration": "torch.mul(src, 1.0, out=dst) on 256 MiB float32 tensors: "
                          f"{copy_kib} KiB read and {copy_kib} KiB written per dispatch; "
                          f"FETCH_SIZE read {f_copy:.1f} KiB, WRITE_SIZE {w_copy:.1f} KiB",
           "commands": a.commands}
    base = a.out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(base, f"traffic_{a.workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    fb = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"]
    wb = rec["write_kib_per_dispatch"] * 1024 * rec["write_scale"]
    alg = bench.algorithmic_bytes(wl, wl.context_len, append=True)["total"]
    md = [f"# HBM bytes of {SPLIT} on {a.workload}", "",
          "Two counter runs (one counter each), from the repository root:", ""]
    md += [f"    {c}" for c in a.commands]
    md += ["", "Reduced by `python profile_records.py traffic` into "
           f"`profiles/traffic_{a.workload}.json`.", "",
           f"Per dispatch (mean of {rec['dispatches']} dispatches of the split kernel):", "",
           "| counter | raw KiB | scale | bytes |", "|---|---|---|---|",
           f"| FETCH_SIZE | {rec['fetch_kib_per_dispatch']:.1f} | {rec['fetch_scale']:.4f} "
           f"| {fb / 1e6:.2f} MB |",
           f"| WRITE_SIZE | {rec['write_kib_per_dispatch']:.1f} | {rec['write_scale']:.4f} "
           f"| {wb / 1e6:.3f} MB |", "",
           "Scale: what the same counter read for a plain copy of known size in the",
           f"same run (`--copy-calibration`: {rec['calibration']}).", "",
           f"Algorithmic bytes per split pass of a decode step: {alg / 1e6:.2f} MB (the codes "
           "of every KV token, the codebooks, q, lambda, the new token's rows and codes, the "
           "output).",
           f"Measured HBM traffic: {(fb + wb) / 1e6:.2f} MB, i.e. {(fb + wb) / alg:.3f} x the "
           "algorithmic bytes (the writes are the split partials).", "",
           f"Kernel sources hashed (sha256 {rec['kernel_source_sha256'][:16]}...): "
           + ", ".join(rec["kernel_sources"])]
    with open(os.path.join(base, f"{SPLIT}.{a.workload}.hbm_bytes.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps({"fetch_mb": fb / 1e6, "write_mb": wb / 1e6, "alg_mb": alg / 1e6}))


def cmd_counters(a) -> None:
    per, n, durs = {}, [], []
    for d in a.dir:
        means, nd, dur = _split_means(d, a.match)
        per.update(means)
        n.append(nd)
        durs.append(dur)
    derived = {}
    if "SQ_INSTS_VALU" in per and "SQ_INSTS_MFMA" in per:
        derived["valu_per_mfma"] = per["SQ_INSTS_VALU"] / per["SQ_INSTS_MFMA"]
    if "SQ_LDS_BANK_CONFLICT" in per and "SQ_LDS_IDX_ACTIVE" in per:
        derived["lds_bank_conflict_per_lds_active"] = (per["SQ_LDS_BANK_CONFLICT"]
                                                       / per["SQ_LDS_IDX_ACTIVE"])
    if "SQ_BUSY_CYCLES" in per:
        # SQ_BUSY_CYCLES counts per shader engine (32 of them): cycles of one
        # engine over the serialized dispatch time give its clock
        derived["sq_busy_ghz"] = per["SQ_BUSY_CYCLES"] / 32 / (st.mean(durs) * 1e3)
    rec = {"kernel": a.kernel, "workload": a.workload, "score_method": a.score_method,
           **_source_record(), "dispatches": min(n),
           "serialized_duration_us": st.mean(durs), "per_dispatch": per, "derived": derived,
           "note": "rocprofv3 counter values per dispatch of the split kernel, averaged over "
                   "the dispatches of the run; counters serialise dispatches",
           "commands": a.commands}
    name = f"counters_{a.workload}.json" if a.score_method == "mfma" else \
        f"counters_{a.workload}.{a.score_method}.json"
    path = a.out or os.path.join(ROOT, "profiles", name)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(path)


# Rows of a counter comparison, in this order (where both records hold them).
COMPARE_ROWS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES"]


def cmd_compare(a) -> None:
    """Two counter records of the same loops side by side (the first is the
    reference of the ratio column) as a Markdown table."""
    recs = [json.load(open(path)) for path in a.records]
    md = [f"# {a.title}", "",
          "Counter runs, one per variant (from the repository root, after "
          "`cd /tmp && export TMPDIR=/tmp`):", ""]
    for r in recs:
        md += [f"    {c}" for c in r["commands"]]
    md += ["", "Reduced by `python profile_records.py counters` into "
           + " and ".join(f"`{os.path.relpath(p, ROOT)}`" for p in a.records)
           + ", compared by `python profile_records.py compare`. Per dispatch of the split "
           "kernel (means over the run's dispatches; counters serialise dispatches):", "",
           f"| counter | {a.labels[0]} | {a.labels[1]} | ratio |", "|---|---|---|---|"]
    p0, p1 = recs[0]["per_dispatch"], recs[1]["per_dispatch"]
    for k in COMPARE_ROWS:
        if k in p0 and k in p1:
            md.append(f"| {k} | {p0[k]:,.0f} | {p1[k]:,.0f} | {p1[k] / p0[k]:.2f} |")
    d0, d1 = recs[0]["derived"], recs[1]["derived"]
    if "lds_bank_conflict_per_lds_active" in d0 and "lds_bank_conflict_per_lds_active" in d1:
        md.append("| LDS bank conflicts / LDS-active cycles | "
                  f"{d0['lds_bank_conflict_per_lds_active']:.3f} | "
                  f"{d1['lds_bank_conflict_per_lds_active']:.3f} | |")
    t0, t1 = recs[0]["serialized_duration_us"], recs[1]["serialized_duration_us"]
    md.append(f"| serialized dispatch duration (us) | {t0:.2f} | {t1:.2f} | {t1 / t0:.2f} |")
    if "sq_busy_ghz" in d0 and "sq_busy_ghz" in d1:
        md.append(f"| SQ_BUSY_CYCLES / 32 engines / duration (GHz) | {d0['sq_busy_ghz']:.2f} "
                  f"| {d1['sq_busy_ghz']:.2f} | |")
    if a.note:
        md += ["", a.note]
    md += ["", "Kernel sources hashed (sha256 "
           f"{recs[0]['kernel_source_sha256'][:16]}...): " + ", ".join(recs[0]["kernel_sources"])]
    with open(a.out, "w") as f:
        f.write("\n".join(md) + "\n")
    print(a.out)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--prefix", default="trace")
    t.add_argument("--workload", default="llama3.1-8b-layer-b1-n196608")
    t.add_argument("--command", required=True)
    t.add_argument("--title")
    t.add_argument("--note")
    t.add_argument("--breakdown", action="append",
                   help="also list the launches of kernels whose name contains this, by grid size")
    t.add_argument("--out", required=True)
    for name in ("traffic", "counters"):
        p = sub.add_parser(name)
        p.add_argument("--workload", default="llama3.1-8b-layer-b1-n196608")
        p.add_argument("--kernel", default=f"{SPLIT}<4, 8, 4>")
        p.add_argument("--score-method", default="mfma", choices=["mfma", "lut"])
        p.add_argument("--commands", nargs="+", required=True)
    sub.choices["traffic"].add_argument("--fetch-dir", required=True)
    sub.choices["traffic"].add_argument("--write-dir", required=True)
    sub.choices["traffic"].add_argument("--out-dir", help="default: profiles/")
    sub.choices["counters"].add_argument("--dir", action="append", required=True)
    sub.choices["counters"].add_argument("--out")
    sub.choices["counters"].add_argument(
        "--match", default=SPLIT,
        help="substring of the kernel name selecting the dispatches (default: the split kernel)")
    for name in ("encoder", "calibration"):
        e = sub.add_parser(name)
        e.add_argument("--dir", required=True, help="rocprofv3 --kernel-trace output")
        e.add_argument("--prefix", default="trace")
        e.add_argument("--log", required=True, help="the same run's bench.py output")
        e.add_argument("--command", required=True)
        e.add_argument("--title", required=True)
        e.add_argument("--out", required=True)
    sub.choices["encoder"].add_argument("--others", nargs="*",
                                        help="trace directories of the other layouts' runs")
    c = sub.add_parser("compare")
    c.add_argument("--records", nargs=2, required=True, help="two counter records (JSON)")
    c.add_argument("--labels", nargs=2, required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--note")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters,
     "compare": cmd_compare, "encoder": cmd_encoder, "calibration": cmd_calibration}[a.what](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
