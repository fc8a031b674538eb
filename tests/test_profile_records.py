"""The reduction of rocprofv3 CSV output into profiles/ records, on small
hand-made CSV files (no GPU)."""
import csv
import json
import os

import pytest

import profile_records as P

SPLIT = "void vqkv::vq_attention_mfma_kernel<4, 8, 4, false>(int) [clone .kd]"
MERGE = "vqkv::merge_partials_kernel(int)"
SPIN = "at::cuda::(anonymous namespace)::spin_kernel(long)"
COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, "
        "float, float, at::native::binary_internal::MulFunctor<float> > >")


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_trace_loops_and_gaps(tmp_path):
    # spin, then split/merge pairs; spin, then splits alone with a 5 us gap
    seq = [(SPIN, 0, 1000), (SPLIT, 1000, 22000), (MERGE, 22000, 26000),
           (SPLIT, 26000, 54000), (MERGE, 54000, 58000),
           (SPIN, 60000, 70000), (SPLIT, 75000, 96000), (SPLIT, 101000, 121000)]
    _write(tmp_path / "t_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[n, s, e] for n, s, e in seq])
    _write(tmp_path / "t_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
           [[SPLIT, 4, 90000, 22500, 20000, 28000], [MERGE, 2, 8000, 4000, 4000, 4000]])
    out = tmp_path / "trace.md"
    P.main(["trace", "--dir", str(tmp_path), "--prefix", "t", "--command", "cmd",
            "--out", str(out)])
    text = out.read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| 1:") or ln.startswith("| 2:")]
    # loop 1: splits of 21 and 28 us, merges of 4 us, no gap before either split
    assert "| 2 | 24.50 | 21.00 | 28.00 | 4.00 | 0.00 |" in lines[0]
    # loop 2: 21 and 20 us, gaps of 5 us (after the spin and between the splits)
    assert "| 2 | 20.50 | 20.00 | 21.00 | - | 5.00 |" in lines[1]
    assert "vqkv::vq_attention_mfma_kernel<4, 8, 4, false>" in text


def _pmc(path, entries):
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    _write(path, header, entries)


def test_counters_and_traffic(tmp_path):
    d1, d2 = tmp_path / "f", tmp_path / "w"
    d1.mkdir()
    d2.mkdir()
    # two split dispatches whose counters arrive as two partial rows each
    # (summed per dispatch), plus one copy dispatch
    _pmc(d1 / "pmc_counter_collection.csv", [
        [1, SPLIT, "FETCH_SIZE", 100.0, 0, 20000], [1, SPLIT, "FETCH_SIZE", 50.0, 0, 20000],
        [2, SPLIT, "FETCH_SIZE", 200.0, 0, 30000], [2, SPLIT, "FETCH_SIZE", 50.0, 0, 30000],
        [3, COPY, "FETCH_SIZE", 131072.0, 0, 90000],
        [4, COPY, "FETCH_SIZE", 3.0, 0, 2000]])   # a small multiply elsewhere in the run
    _pmc(d2 / "pmc_counter_collection.csv", [
        [1, SPLIT, "WRITE_SIZE", 10.0, 0, 20000], [2, SPLIT, "WRITE_SIZE", 30.0, 0, 20000],
        [3, COPY, "WRITE_SIZE", 262144.0, 0, 90000]])
    P.main(["traffic", "--fetch-dir", str(d1), "--write-dir", str(d2), "--commands", "a", "b",
            "--out-dir", str(tmp_path)])
    rec = json.loads((tmp_path / "traffic_llama3.1-8b-layer-b1-n196608.json").read_text())
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(200.0)
    assert rec["write_kib_per_dispatch"] == pytest.approx(20.0)
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["score_method"] == "mfma" and rec["commands"] == ["a", "b"]

    d3 = tmp_path / "s"
    d3.mkdir()
    _pmc(d3 / "pmc_counter_collection.csv", [
        [1, SPLIT, "SQ_INSTS_VALU", 800.0, 0, 20000], [1, SPLIT, "SQ_INSTS_MFMA", 100.0, 0, 20000],
        [1, SPLIT, "SQ_BUSY_CYCLES", 32 * 40000.0, 0, 20000],
        [2, MERGE, "SQ_INSTS_VALU", 5.0, 0, 4000]])
    out = tmp_path / "c.json"
    P.main(["counters", "--dir", str(d3), "--commands", "c", "--out", str(out)])
    rec = json.loads(out.read_text())
    assert rec["dispatches"] == 1
    assert rec["per_dispatch"]["SQ_INSTS_VALU"] == 800.0
    assert rec["derived"]["valu_per_mfma"] == pytest.approx(8.0)
    # 40000 cycles per engine over 20 us: 2 GHz
    assert rec["derived"]["sq_busy_ghz"] == pytest.approx(2.0)
    assert rec["serialized_duration_us"] == pytest.approx(20.0)


def test_records_follow_kernel_sources():
    import bench
    assert os.path.basename(bench.KERNEL_SOURCES[0]) == "vq_attention_mfma.hip"
    assert len(bench.kernel_source_digest()) == 64


def test_compare_two_counter_records(tmp_path):
    def rec(path, valu, conflicts, dur, cmd):
        r = {"kernel": "k", "workload": "w", "score_method": "mfma",
             "kernel_source_sha256": "ab" * 32, "kernel_sources": ["a.hip"],
             "dispatches": 3, "serialized_duration_us": dur,
             "per_dispatch": {"SQ_INSTS_VALU": valu, "SQ_LDS_BANK_CONFLICT": conflicts,
                              "SQ_LDS_IDX_ACTIVE": 4 * conflicts},
             "derived": {"lds_bank_conflict_per_lds_active": 0.25}, "commands": [cmd]}
        path.write_text(json.dumps(r))
        return str(path)

    a = rec(tmp_path / "a.json", 1000.0, 10.0, 20.0, "run-a")
    b = rec(tmp_path / "b.json", 3000.0, 50.0, 30.0, "run-b")
    out = tmp_path / "cmp.md"
    P.main(["compare", "--records", a, b, "--labels", "A", "B", "--title", "T",
            "--out", str(out)])
    text = out.read_text()
    assert "    run-a" in text and "    run-b" in text
    assert "| SQ_INSTS_VALU | 1,000 | 3,000 | 3.00 |" in text
    assert "| SQ_LDS_BANK_CONFLICT | 10 | 50 | 5.00 |" in text
    assert "| serialized dispatch duration (us) | 20.00 | 30.00 | 1.50 |" in text
    # counters absent from either record are left out
    assert "SQ_WAVES" not in text


def test_encoder_and_calibration_records(tmp_path):
    enc = "void vqkv::encode_append_kernel<8>(int) [clone .kd]"
    asg = "void vqkv::kmeans_assign_kernel<256>(int) [clone .kd]"
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
           "Grid_Size_Z", "Workgroup_Size_X"]
    # prefill launches (4096 workgroups of 512 threads) and short appends (8)
    rows = [[enc, 0, 1000000, 4096 * 512, 8, 1, 512], [enc, 2000000, 3100000, 4096 * 512, 8, 1, 512],
            [enc, 4000000, 4015000, 8 * 512, 8, 1, 512],
            [asg, 5000000, 7000000, 512 * 256, 8, 1, 256]]
    _write(tmp_path / "t_kernel_trace.csv", hdr, rows)
    line = {"metric": "m",
            "prefill_encode": {"tokens": 32768, "avg_launch_us": 1050.0, "tokens_per_s": 3.1e7,
                               "roofline": {"kernel": "encode_append_kernel", "achieved": 32.7,
                                            "peak": 157.3, "frac": 0.208}},
            "append_encode": {"avg_launch_us": 15.0},
            "calibration": {"lambda_us": 50.0, "lambda_gbps": 5000.0, "transform_keys_us": 360.0,
                            "transform_keys_gbps": 2200.0,
                            "kmeans": {"k8": {"us_per_iter": 3200.0, "sets": 8,
                                              "samples_per_set": 4194304, "sub_dim": 4,
                                              "entries": 256, "dense_pass_tflops": 21.5,
                                              "frac_of_mfma_f32_peak": 0.137}}}}
    log = tmp_path / "bench.log"
    log.write_text("noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "enc.md"
    P.main(["encoder", "--dir", str(tmp_path), "--prefix", "t", "--log", str(log),
            "--command", "cmd", "--title", "T", "--out", str(out)])
    text = out.read_text()
    # the two prefill launches (1000 and 1100 us) group by grid; the append separately
    assert "| vqkv::encode_append_kernel<8> | 4096 x 8 x 1 | 2 | 1050.0 | 1000.0 | 1100.0 |" in text
    assert "| vqkv::encode_append_kernel<8> | 8 x 8 x 1 | 1 | 15.0 |" in text
    assert "1050.0 us per prefill launch" in text and "20.8% of the 157.3" in text
    out = tmp_path / "cal.md"
    P.main(["calibration", "--dir", str(tmp_path), "--prefix", "t", "--log", str(log),
            "--command", "cmd", "--title", "T", "--out", str(out)])
    text = out.read_text()
    assert "| vqkv::kmeans_assign_kernel<256> | 512 x 8 x 1 | 1 | 2000.0 |" in text
    assert "- K-Means k8: 3200 us per Lloyd iteration" in text
