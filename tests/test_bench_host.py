"""Host logic of bench.py (CPU): the steady-state flush schedule of the timed steps and
the rocprofv3 counter summaries (HBM traffic, instruction issue) that the bench line
reports beside its event timings."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import kvq_workloads as wl  # noqa: E402
from oracle.kvq_oracle import quantized_count  # noqa: E402


@pytest.mark.parametrize("name", ["gqa_128k_2bit", "million_1m", "gqa_128k_2bit_rope", "llama2_7b_b8_32k"])
def test_will_flush_follows_the_residual_rule(name):
    """A step flushes exactly when the quantized count of the residual rule grows."""
    w = wl.WORKLOADS[name]
    T0 = int(w.context_lengths()[0])
    for T in range(T0 - 70, T0 + 70):
        grows = quantized_count(T + 1, w.residual, w.group, w.sink) != quantized_count(T, w.residual, w.group,
                                                                                        w.sink)
        assert bench.will_flush(T, w) == grows, T


@pytest.mark.parametrize("name", ["gqa_128k_2bit", "million_1m", "gqa_128k_2bit_rope"])
@pytest.mark.parametrize("copies,warmup", [(8, 16), (8, 5), (4, 3), (1, 0)])
@pytest.mark.parametrize("steps", [1, 7, 20, 64, 256])
def test_timed_steps_hold_the_steady_flush_share(name, copies, warmup, steps):
    """Replaying the bench's round-robin schedule: with the extra prefill tokens of
    steady_offsets, the timed steps hold steps / 32 group flushes (rounded either
    way), at any step count, warmup and number of copies."""
    w = wl.WORKLOADS[name]
    extra = bench.steady_offsets(w, copies, warmup)
    assert all(0 <= e < 32 for e in extra)
    T = [int(w.context_lengths()[0]) + e for e in extra]
    flushes = 0
    for s in range(warmup + steps):
        c = s % copies
        if s >= warmup and bench.will_flush(T[c], w):
            flushes += 1
        T[c] += 1
    assert abs(flushes - steps / 32) < 1, (flushes, steps)


def _write_counters(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_summarize_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    k = "void kvq::decode_split_kernel<2, 4, false>(DecodeArgs)"
    # the decode's FETCH_SIZE comes in two samples per dispatch (summed), two dispatches
    _write_counters(tmp_path / "df", [(1, k, "FETCH_SIZE", 30000), (1, k, "FETCH_SIZE", 20000),
                                      (2, k, "FETCH_SIZE", 26000), (2, k, "FETCH_SIZE", 26000),
                                      (2, "other_kernel", "FETCH_SIZE", 99999)])
    _write_counters(tmp_path / "dw", [(1, k, "WRITE_SIZE", 1000), (2, k, "WRITE_SIZE", 1100)])
    copy = "__amd_rocclr_copyBuffer"
    cb = bench.COPY_BYTES
    _write_counters(tmp_path / "cf", [(7, copy, "FETCH_SIZE", cb / 2048)])   # counts half the bytes
    _write_counters(tmp_path / "cw", [(7, copy, "WRITE_SIZE", cb / 1024)])
    out = tmp_path / "traffic.json"
    bench.summarize_traffic(str(tmp_path / "df"), str(tmp_path / "dw"), str(tmp_path / "cf"),
                            str(tmp_path / "cw"), "wk", str(out))
    d = json.load(open(out))
    assert d["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["calibration"]["write_scale"] == pytest.approx(1.0)
    r = d["workloads"]["wk"]
    assert r["fetch_kib_per_dispatch"] == pytest.approx(51000)
    assert r["write_kib_per_dispatch"] == pytest.approx(1050)
    assert r["bytes_per_launch"] == int(51000 * 1024 * 2.0 + 1050 * 1024 * 1.0)
    assert r["dispatches"] == [2, 2] and r["kernel_source_sha256"] == "h"
    # a second workload reuses the stored calibration
    bench.summarize_traffic(str(tmp_path / "df"), str(tmp_path / "dw"), "-", "-", "wk2", str(out))
    d = json.load(open(out))
    assert set(d["workloads"]) == {"wk", "wk2"}
    assert d["workloads"]["wk2"]["bytes_per_launch"] == r["bytes_per_launch"]


def test_summarize_issue_fractions(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    k = "void kvq::decode_split_kernel<2, 4, false>(DecodeArgs)"
    groups = 1000
    _write_counters(tmp_path / "s1", [(1, k, "SQ_WAVE_CYCLES", 600000), (1, k, "SQ_WAVE_CYCLES", 400000),
                                      (1, k, "SQ_INSTS_VALU", 232000), (1, k, "SQ_INSTS_MFMA", 16000),
                                      (1, k, "SQ_ACTIVE_INST_VALU", 280000), (1, k, "SQ_WAIT_INST_ANY", 250000)])
    _write_counters(tmp_path / "s2", [(1, k, "SQ_ACTIVE_INST_ANY", 400000), (1, k, "SQ_INSTS_LDS", 21000),
                                      (1, k, "SQ_INSTS_VMEM_RD", 6500)])
    out = tmp_path / "issue.json"
    bench.summarize_issue(str(tmp_path / "s1"), str(tmp_path / "s2"), "wk", str(groups), "2", str(out))
    r = json.load(open(out))["workloads"]["wk"]
    assert r["valu_instructions_per_group"] == 232.0 and r["mfma_per_group"] == 16.0
    assert r["lds_per_group"] == 21.0 and r["vmem_reads_per_group"] == 6.5
    assert r["valu_active_per_wave_cycle"] == pytest.approx(0.28)
    assert r["simd_valu_busy_frac"] == pytest.approx(0.56)
    assert r["simd_any_active_per_cycle"] == pytest.approx(0.8)
    assert r["wait_per_wave_cycle"] == pytest.approx(0.25)
    assert r["kernel_source_sha256"] == "h"


def test_summarize_issue_needs_its_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    k = "decode_split_kernel<2, 4, false>"
    _write_counters(tmp_path / "s1", [(1, k, "SQ_WAVE_CYCLES", 1000)])
    _write_counters(tmp_path / "s2", [(1, k, "SQ_INSTS_LDS", 10)])
    with pytest.raises(SystemExit):
        bench.summarize_issue(str(tmp_path / "s1"), str(tmp_path / "s2"), "wk", "10", "2",
                              str(tmp_path / "issue.json"))


def test_summarize_trace_averages_the_split_kernel(tmp_path, monkeypatch):
    """The traced average is total duration over calls of the split kernel rows only,
    stored beside the workload's counter figures without disturbing them."""
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    d = tmp_path / "tr" / "host" / "123"
    os.makedirs(d)
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow(["void kvq::decode_split_kernel<2, 4, false>(DecodeArgs)", 200, 5_400_000, 27000, 50, 1, 1, 1])
        wr.writerow(["void kvq::combine_kernel(float const*)", 200, 840_000, 4200, 10, 1, 1, 1])
    out = tmp_path / "traffic.json"
    json.dump({"calibration": None, "workloads": {"wk": {"bytes_per_launch": 5, "kernel_source_sha256": "h"}}},
              open(out, "w"))
    bench.summarize_trace(str(tmp_path / "tr"), "wk", str(out))
    r = json.load(open(out))["workloads"]["wk"]
    assert r["bytes_per_launch"] == 5
    assert r["trace"] == {"avg_us": 27.0, "dispatches": 200, "kernel_source_sha256": "h"}


def test_committed_counter_summaries_describe_the_committed_kernel():
    """profiles/traffic.json and profiles/issue.json: the bench only reports figures
    whose kernel source hash is the current one, so the committed files carry it."""
    h = bench.kernel_source_hash()
    for name in ("traffic.json", "issue.json"):
        d = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert d["workloads"], name
        for wname, r in d["workloads"].items():
            assert wname in wl.WORKLOADS, (name, wname)
            assert r["kernel_source_sha256"] == h, (name, wname)
            if name == "traffic.json":
                assert r["trace"]["kernel_source_sha256"] == h, wname
