"""The measurement plumbing of bench.py that runs without a GPU: the one-GPU
contract, the kernel-source hash that ties recorded HBM counters to the code
they were taken on, and the recorded counter summaries themselves."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOADS = ["mha7b_fp16", "gqa70b_bf16", "prefix_share_fp16", "long_splitk_bf16"]


def test_more_than_one_gpu_is_refused_with_a_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def test_kernel_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SOURCE, encoding="utf-8").read()
    base = bench.kernel_source_hash()
    edited = tmp_path / "commented.h"
    edited.write_text("// a new comment line\n\n" + src.replace("\n", "   // trailing note\n", 3), encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(edited))
    assert bench.kernel_source_hash() == base
    changed = tmp_path / "changed.h"
    changed.write_text(src + "\nconstexpr int kUnused = 1;\n", encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(changed))
    assert bench.kernel_source_hash() != base


@pytest.mark.parametrize("workload", WORKLOADS)
def test_recorded_traffic_summaries_are_consistent(workload):
    """Each summary ends with the record bench.py reads: HBM bytes from the
    two counters scaled by the copy-kernel calibration, close to (and not
    below) the algorithmic bytes of the counted run."""
    path = os.path.join(bench.PROFILES, f"decode_{workload}_traffic.txt")
    text = open(path, encoding="utf-8").read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    rec = json.loads([line for line in text.splitlines() if line.startswith("{")][-1])
    for key in ("kernel_source_sha256", "decode", "hbm_bytes_per_call", "algorithmic_bytes_per_call",
                "fetch_factor", "write_factor"):
        assert key in rec, key
    assert rec["decode"] in ("pa_decode", "pa_decode_shared_prefix", "pa_decode_append")
    assert abs(rec["fetch_factor"] - 2.0) < 0.05 and abs(rec["write_factor"] - 1.0) < 0.05
    ratio = rec["hbm_bytes_per_call"] / rec["algorithmic_bytes_per_call"]
    assert 1.0 <= ratio <= 1.1, ratio
    # bench.py uses the record only for the code it was taken on
    got = bench.recorded_traffic(workload, rec["decode"])
    if rec["kernel_source_sha256"] == bench.kernel_source_hash():
        assert got == (rec["hbm_bytes_per_call"], round(ratio, 4))
    else:
        assert got == (None, None)


def test_span_timing_brackets_at_least_one_step_of_any_run():
    """Span timing takes every n-th step counted from the run's first, so a
    short run (a 3-step counter pass) still records one span; steps with other
    kernels between the layers' calls fall back to one rotating layer."""
    import bench
    span = {"mode": "span", "every": 4}
    for steps in (1, 3, 4, 5, 50):
        modes = [bench.step_timing(span, True, 0, i) for i in range(steps)]
        assert modes.count("span") == -(-steps // 4) and modes[0] == "span"
        assert set(modes) <= {"span", None}
    assert bench.step_timing(span, False, 0, 0) == "one"          # pa_write_kv between the calls
    assert bench.step_timing(span, True, 3, 0) == "one"           # copy-on-write copies first
    assert bench.step_timing({"mode": "all", "every": 4}, True, 0, 1) == "all"
    assert bench.step_timing({"mode": "one", "every": 4}, True, 0, 1) == "one"
    assert bench.step_timing(None, True, 0, 0) is None
