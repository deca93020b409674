"""Host logic of bench.py (no GPU): counter ingestion, the source-hash check
that retires stale counter records, the one-GPU guard and the host record.

Counter CSVs here are synthetic, in the column layout rocprofv3 writes.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def records(tmp_path, monkeypatch):
    path = tmp_path / "counters.json"
    path.write_text(json.dumps({"other": {"kernels": {}}}))
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(path))
    return path


def test_ingest_scales_by_the_calibration_copy(tmp_path, records):
    fwd = "void attn::(anonymous namespace)::attn_fwd_kernel<128, 128, 8, 2, true, false, 0>(...)"
    grads = "void attn::(anonymous namespace)::bwd_grads_kernel<128, 4, 128, 8, 2, true, false>(...)"
    copy = bench.COPY_KERNEL
    # the copy kernel also moved two small input uploads; the largest dispatch is the calibration
    write_csv(tmp_path / "f.csv", [(copy, "FETCH_SIZE", 16), (copy, "FETCH_SIZE", 524288), (copy, "FETCH_SIZE", 8),
                                   (fwd, "FETCH_SIZE", 1000), (fwd, "FETCH_SIZE", 3000),
                                   (grads, "FETCH_SIZE", 5000), ("other_kernel", "FETCH_SIZE", 7)])
    write_csv(tmp_path / "w.csv", [(copy, "WRITE_SIZE", 1048576), (fwd, "WRITE_SIZE", 100),
                                   (fwd, "WRITE_SIZE", 300), (grads, "WRITE_SIZE", 600)])
    rec = bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1024, "wl")
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    e = rec["kernels"]["attn_fwd_kernel"]
    assert e["fetch_kib"] == 2000 and e["write_kib"] == 200        # mean per dispatch
    assert e["hbm_bytes"] == pytest.approx((2000 * 2.0 + 200 * 1.0) * 1024)
    assert rec["kernels"]["bwd_grads_kernel"]["hbm_bytes"] == pytest.approx((5000 * 2.0 + 600) * 1024)
    assert set(rec["kernels"]) == {"attn_fwd_kernel", "bwd_grads_kernel"}
    saved = json.loads(records.read_text())
    assert set(saved) == {"other", "wl"}                            # other workloads kept


def test_recorded_traffic_retires_stale_records(tmp_path, records, monkeypatch):
    fwd = "void attn::(anonymous namespace)::attn_fwd_kernel<128, 128, 8, 2, true, false, 0>(...)"
    write_csv(tmp_path / "f.csv", [(bench.COPY_KERNEL, "FETCH_SIZE", 524288), (fwd, "FETCH_SIZE", 10)])
    write_csv(tmp_path / "w.csv", [(bench.COPY_KERNEL, "WRITE_SIZE", 1048576), (fwd, "WRITE_SIZE", 5)])
    bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1024, "wl")
    assert bench.recorded_traffic("attn_fwd_kernel", "wl") == pytest.approx((10 * 2.0 + 5) * 1024)
    assert bench.recorded_traffic("attn_fwd_kernel", "missing") is None
    assert bench.recorded_traffic("bwd_grads_kernel", "wl") is None
    monkeypatch.setattr(bench, "source_sha", lambda k: "changed")
    assert bench.recorded_traffic("attn_fwd_kernel", "wl") is None


def test_source_hash_covers_the_kernel_sources():
    for k, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(bench.CSRC, f)), (k, f)
        assert len(bench.source_sha(k)) == 16
    assert bench.source_sha("attn_fwd_kernel") != bench.source_sha("bwd_grads_kernel")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_host_record():
    h = bench.host_info()
    assert set(h) == {"cpu_model", "affinity_cpus", "torch_threads", "numpy_blas"}
    assert h["affinity_cpus"] >= 1 and h["torch_threads"] >= 1
