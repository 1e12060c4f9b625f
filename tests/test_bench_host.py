"""Host-side logic of bench.py, on the CPU: the one-GPU rule, the counter
summary (rocprofv3 FETCH_SIZE / WRITE_SIZE readings scaled by a plain copy of
known size) and the rule that a summary only counts for the kernel source it
was taken on."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MR = "hyena_fwd_kernel<false, 4, 2, 8, false, false>(Params)"
SE = "hyena_fwd_kernel<false, 1, 1, 8, false, false, 16>(Params)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(d, counter, rows):
    """A rocprofv3-style counter_collection.csv: one row per (dispatch, kernel)."""
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write('%d,"%s",%s,%r\n' % (i, name, counter, value))
    return d


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    path = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    return path


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_counter_summary_scales_by_the_copy(tmp_path, traffic_file, capsys):
    # per dispatch, in KiB; the copy moved 1 GiB each way
    fetch = _counters(str(tmp_path / "f"), "FETCH_SIZE", [(MR, 100000.0), (MR, 110000.0), (SE, 98000.0)])
    write = _counters(str(tmp_path / "w"), "WRITE_SIZE", [(MR, 65536.0), (MR, 65538.0), (SE, 65536.0)])
    cf = _counters(str(tmp_path / "cf"), "FETCH_SIZE", [(COPY, 524288.0)])
    cw = _counters(str(tmp_path / "cw"), "WRITE_SIZE", [(COPY, 1048576.0)])
    bench.summarize_counters(fetch, write, cf, cw)
    capsys.readouterr()
    t = json.load(open(traffic_file))
    assert t["kernel_source_sha256"] == bench.source_digest()
    assert t["scale"] == {"fetch": 2.0, "write": 1.0, "copy_bytes": 1 << 30}
    mr = t["layers"]["mr"]
    assert mr["fetch_bytes"] == 105000 * 1024 * 2
    assert mr["write_bytes"] == 65537 * 1024
    assert mr["hbm_bytes_per_launch"] == mr["fetch_bytes"] + mr["write_bytes"]
    se = t["layers"]["se"]
    assert se["hbm_bytes_per_launch"] == 98000 * 1024 * 2 + 65536 * 1024
    # what the bench line reports while the source is unchanged
    assert bench.measured_traffic("mr") == mr["hbm_bytes_per_launch"]
    assert bench.measured_traffic("se") == se["hbm_bytes_per_launch"]


def test_a_summary_of_another_source_is_not_reported(traffic_file):
    entry = {"hbm_bytes_per_launch": 123}
    with open(traffic_file, "w") as f:
        json.dump({"kernel_source_sha256": "0" * 64, "layers": {"mr": entry}}, f)
    assert bench.measured_traffic("mr") is None
    with open(traffic_file, "w") as f:
        json.dump({"kernel_source_sha256": bench.source_digest(), "layers": {"mr": entry}}, f)
    assert bench.measured_traffic("mr") == 123
    assert bench.measured_traffic("se") is None
    os.remove(traffic_file)
    assert bench.measured_traffic("mr") is None
