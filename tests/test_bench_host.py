"""Host-side parts of bench.py (no GPU): the one-GPU guard, the HBM-traffic
summary from counter CSVs (scaled by a copy of known size), and the
kernel-source check that voids stale traffic figures."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _counter_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch, capsys):
    pytest.importorskip("ctypes")
    from block_quantized_matvec_gguf_amd import binding as qb
    try:
        qb.load()
    except Exception as e:  # the library must be built for kernel names
        pytest.skip("libqmv.so not built: %s" % e)
    monkeypatch.setattr(bench, "traffic_path",
                        lambda w, op="fwd": str(tmp_path / ("traffic_%s.json" % w)))
    gemv = "void qmv::qmv_gemv_staged<qmv::UQ6_K, 1, 1, 1, 4, true>(...)"
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>(...)"
    calib = 512 * 1024 * 1024
    # counters: FETCH reads half the copy's bytes (factor 2), WRITE all of them
    _counter_csv(tmp_path / "fetch.csv",
                 [(1, gemv, "FETCH_SIZE", 270000.0), (2, gemv, "FETCH_SIZE", 271000.0),
                  (3, copy, "FETCH_SIZE", calib / 2048.0)])
    _counter_csv(tmp_path / "write.csv",
                 [(1, gemv, "WRITE_SIZE", 1024.0), (2, gemv, "WRITE_SIZE", 1024.0),
                  (3, copy, "WRITE_SIZE", calib / 1024.0)])

    class A:
        workload = "q6_k_vocab_outproj"
        op = "fwd"
        algo = "auto"
        calib_bytes = calib
        summarize_pmc = [str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv")]

    bench.summarize_pmc(A)
    out = json.load(open(tmp_path / "traffic_q6_k_vocab_outproj.json"))
    assert out["kernel_family"] == "gemv"
    assert out["fetch_factor"] == pytest.approx(2.0)
    assert out["write_factor"] == pytest.approx(1.0)
    assert out["fetch_bytes_per_launch"] == pytest.approx(270500.0 * 1024 * 2.0)
    assert out["write_bytes_per_launch"] == pytest.approx(1024.0 * 1024)
    assert out["bytes_per_launch"] == pytest.approx(270500.0 * 2048 + 1024.0 * 1024)
    assert out["kernel_source_sha256"] == bench.kernel_source_hash("gemv")


def test_stale_traffic_is_ignored(tmp_path, monkeypatch):
    p = tmp_path / "traffic_w.json"
    monkeypatch.setattr(bench, "traffic_path", lambda w, op="fwd": str(p))
    p.write_text(json.dumps({"kernel_source_sha256": "0" * 64, "bytes_per_launch": 1.0}))
    assert bench.load_traffic("w", "gemv") is None
    p.write_text(json.dumps({"kernel_source_sha256": bench.kernel_source_hash("gemv"),
                             "bytes_per_launch": 1.0}))
    assert bench.load_traffic("w", "gemv")["bytes_per_launch"] == 1.0


def test_cpu_baseline_threads(monkeypatch):
    """The oracle baseline uses every CPU in the process's affinity mask,
    capped by OMP_NUM_THREADS when set, and reports what it used and why."""
    import bench
    avail = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.host_threads() == (avail, avail, None)
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_threads() == (1, avail, "1")
    monkeypatch.setenv("OMP_NUM_THREADS", str(avail + 5))
    assert bench.host_threads()[0] == avail
    e = bench.cpu_baseline_entry(1.5, 1, avail, "1", "sample text")
    for key in ("value", "unit", "cores", "kind", "sample", "nproc", "cpus_in_affinity",
                "omp_num_threads", "cpu_model"):
        assert key in e
    assert e["kind"] == "oracle" and e["cores"] == 1 and e["cpu_model"]
