"""Host-side logic of bench.py that needs no GPU: turning two rocprofv3 counter
collections (FETCH_SIZE, WRITE_SIZE) into HBM bytes per decode launch.

The counts are calibrated against the plain copy kernel of known size, and only the
dispatches with the per-layer step's grid are averaged -- a run also holds the
layer-batched capability launches, whose much larger grid must not enter the mean."""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
          "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
          "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
DECODE = "void kvq::decode_mfma_kernel<3, 12>(unsigned short const*, unsigned char*, long const*)"
COPY = "__amd_rocclr_copyBuffer"


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, value) in enumerate(rows):
            r = {k: "0" for k in FIELDS}
            r.update({"Correlation_Id": str(i + 1), "Dispatch_Id": str(i + 1), "Grid_Size": str(grid),
                      "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": "%.6f" % value})
            w.writerow(r)


def test_traffic_from_averages_the_step_grid_and_scales_by_the_copy(tmp_path, monkeypatch, capsys):
    b = _bench()
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_mib = 256
    copy_bytes = copy_mib << 20
    # the copy probe reads its bytes as FETCH_SIZE/2 KiB units and writes them 1:1 (the ratio the
    # counters showed on the device); three copy dispatches close the run
    fetch = [(COPY, 512, 3.0)] + [(DECODE, 131584, 13500.0 + d) for d in (-20, 0, 20)] * 10 + \
        [(DECODE, 184320, 480000.0)] * 2 + [(COPY, 131072, copy_bytes / 2048.0)] * 3
    write = [(COPY, 512, 1.0)] + [(DECODE, 131584, 2190.0)] * 30 + [(DECODE, 184320, 99999.0)] * 2 + \
        [(COPY, 131072, copy_bytes / 1024.0)] * 3
    _write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write(tmp_path / "w.csv", "WRITE_SIZE", write)
    b.traffic_from(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy_mib, "wl")
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert out["launches"] == [30, 30]                      # the two layer-batched dispatches left out
    assert out["fetch_kib_per_launch"] == pytest.approx(13500.0)
    assert out["write_kib_per_launch"] == pytest.approx(2190.0)
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    assert out["hbm_bytes_per_launch"] == int(13500.0 * 1024 * 2.0 + 2190.0 * 1024 * 1.0)
    saved = json.load(open(tmp_path / "traffic.json"))
    assert saved["wl"]["source_sha256_16"] == b.kernel_source_hash("mfma")


def test_kernel_source_hash_tracks_the_decode_sources():
    b = _bench()
    h = b.kernel_source_hash("mfma")
    assert len(h) == 16 and h == b.kernel_source_hash("mfma")
    assert h != b.kernel_source_hash("generic")
