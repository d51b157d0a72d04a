"""Host-side pieces of bench.py on a machine without a GPU: the algorithmic byte counts behind
the roofline (against the workload figures, worked out by hand from the packed format), the
percentile helper, the amd-smi parser of the device monitor, the traffic-counter source hash and
the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_of_the_workloads():
    # 2048 x 2048 at M = 1: 2 MiB of nibbles + 256 KiB of fp16 scales (64 blocks x 2048 columns x 2 B)
    # + 4 KiB in + 8 KiB out
    assert bench.algorithmic_bytes(1, 2048, 2048) == 2 * 2**20 + 2**18 + 2**12 + 2**13 == 2371584
    # the gate_up launch the roofline is quoted on
    assert bench.algorithmic_bytes(1, 2048, 16384) == 18944000
    layer = sum(bench.algorithmic_bytes(1, k, n) for k, n in [(2048, 2560), (2048, 2048), (2048, 16384),
                                                               (8192, 2048)])
    assert layer == 33740800


def test_percentile_nearest_rank():
    vals = sorted([5.0, 1.0, 3.0, 2.0, 4.0, 9.0, 7.0, 8.0, 6.0])
    assert bench.percentile(vals, 50) == 5.0
    assert bench.percentile(vals, 10) == 2.0
    assert bench.percentile(vals, 90) == 8.0
    assert bench.percentile([4.0], 90) == 4.0


AMD_SMI_SAMPLE = {
    "gpu_data": [{
        "gpu": 0,
        "power": {"socket_power": {"value": 305, "unit": "W"}},
        "clock": {
            "gfx_0": {"clk": {"value": 2400, "unit": "MHz"}},
            "gfx_1": {"clk": {"value": 2398, "unit": "MHz"}},
            "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
        },
        "temperature": {"edge": "N/A", "hotspot": {"value": 48, "unit": "C"}, "mem": {"value": 40, "unit": "C"}},
    }]
}


def test_device_monitor_parses_amd_smi(monkeypatch):
    class Res:
        stdout = "WARNING: something\n" + json.dumps(AMD_SMI_SAMPLE)

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Res())
    s = bench.DeviceMonitor()._sample()
    assert s == {"gfx_clk_MHz": 2399.0, "mem_clk_MHz": 2000.0, "power_W": 305.0, "hotspot_C": 48.0}


def test_device_monitor_summary_keeps_busy_samples():
    mon = bench.DeviceMonitor()
    mon.samples = [{"gfx_clk_MHz": 150.0, "mem_clk_MHz": 2000.0, "power_W": 200.0, "hotspot_C": 40.0},
                   {"gfx_clk_MHz": 2400.0, "mem_clk_MHz": 2000.0, "power_W": 310.0, "hotspot_C": 48.0},
                   {"gfx_clk_MHz": 2390.0, "mem_clk_MHz": 2000.0, "power_W": 300.0, "hotspot_C": 47.0}]
    out = mon.summary()
    assert out["samples"] == 3 and out["busy_samples"] == 2
    assert out["gfx_clk_MHz"] == {"min": 2390.0, "median": 2400.0, "max": 2400.0}
    assert out["power_W"]["min"] == 300.0


def test_traffic_summary_matches_the_sources():
    """The committed HBM counter summary is only reported while its source hash matches the GEMV
    sources it was taken on; the hash is a function of those files alone."""
    h = bench.gemv_source_hash()
    assert h == bench.gemv_source_hash() and len(h) == 16
    with open(os.path.join(ROOT, bench.TRAFFIC_FILE)) as f:
        t = json.load(f)
    assert bench.measured_traffic() in (None, t["bytes_per_launch"])
    assert t["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(1, 2048, 16384)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
