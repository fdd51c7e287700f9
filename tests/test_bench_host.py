"""Host-side logic of bench.py (no GPU): the HBM-counter ingest and its copy
calibration, the source-hash gate on recorded traffic, the prefill's
algorithmic work per launch, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_ingest_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    kname = "_ZN3kla12_GLOBAL__N_1" + bench.KERNEL_MATCH[bench.PREFILL_KERNEL] + "EEvPKDF16b"
    fetch, write, cf, cw = (tmp_path / n for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _write_csv(fetch, [{"Kernel_Name": kname, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
                       for v in (100.0, 300.0)])
    _write_csv(write, [{"Kernel_Name": kname, "Counter_Name": "WRITE_SIZE", "Counter_Value": 50.0}])
    # the 1 GiB calibration copy: FETCH_SIZE counts half the bytes it reads, WRITE_SIZE all
    _write_csv(cf, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                     "Counter_Value": 524288.0}])
    _write_csv(cw, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                     "Counter_Value": 1048576.0}])
    bench.ingest_counters(str(fetch), str(write), str(cf), str(cw))
    recs = json.load(open(out))
    rec = recs[bench.PREFILL_KERNEL]
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes"] == 200 * 2 * 1024  # the mean of the dispatches, in KiB, scaled
    assert rec["write_bytes"] == 50 * 1024
    assert rec["bytes_per_launch"] == rec["read_bytes"] + rec["write_bytes"]
    assert rec["source_sha256"] == bench.source_hash(bench.PREFILL_KERNEL)
    # kernels absent from the runs get no record (the states-only instance of
    # the same kernel template is another instantiation)
    assert set(recs) == {bench.PREFILL_KERNEL}


def test_recorded_traffic_needs_the_current_source(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    good = {"source_sha256": bench.source_hash(bench.DECODE_KERNEL), "bytes_per_launch": 123}
    json.dump({bench.DECODE_KERNEL: good}, open(out, "w"))
    assert bench.measured_traffic(bench.DECODE_KERNEL) == 123
    assert bench.measured_traffic(bench.PREFILL_KERNEL) is None  # no record
    json.dump({bench.DECODE_KERNEL: dict(good, source_sha256="0" * 64)}, open(out, "w"))
    assert bench.measured_traffic(bench.DECODE_KERNEL) is None   # the kernel changed since


def test_prefill_work_per_launch():
    """1288 B per token-head plus the final state per (sequence, head);
    180,224 full-tile flops per token-head in the W/U form and 163,840 in
    the kernel's regrouped form: the layer workload's figures."""
    n, T, H, d = 8, 2048, 16, 128
    th = n * T * H
    b, f, fi = bench.prefill_work(th, n, H, d)
    assert b == th * (3 * 256 + 8 + 512) + n * H * d * d * 4 == 346_030_080
    assert f == th * 180_224 == 47_244_640_256
    assert fi == th * (8 * 64 * d + 6 * d * d) == 42_949_672_960


def test_settle_runs_for_the_requested_time(monkeypatch):
    """The clock-settle phase keeps launching until the wall time is spent."""
    import types
    calls = []
    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None))
    monkeypatch.setitem(sys.modules, "torch", fake)
    import time as _t
    ms = bench.settle(lambda: (calls.append(1), _t.sleep(0.001)), 30.0)
    assert ms >= 30.0 and len(calls) % 16 == 0 and len(calls) >= 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
