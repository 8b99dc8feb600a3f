"""Host-side logic of bench.py (CPU): the one-GPU guard and the amd-smi reading.

The benchmark itself needs an MI355X; these check the parts that decide what it
reports without touching a GPU.
"""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration that was not measured


def _fake_run(payload, returncode=0):
    def run(cmd, capture_output, text, timeout):
        assert cmd[:2] == ["amd-smi", "metric"]
        return types.SimpleNamespace(returncode=returncode, stdout=payload, stderr="")
    return run


def test_smi_sample_reads_socket_power_and_mean_gfx_clock(monkeypatch):
    clocks = {f"gfx_{i}": {"clk": {"value": 1800 + 10 * i, "unit": "MHz"}, "min_clk": {"value": 500}}
              for i in range(8)}
    clocks["socclk_0"] = {"clk": {"value": 38, "unit": "MHz"}}  # not a shader clock
    payload = json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1288, "unit": "W"}},
                                        "clock": clocks}]})
    monkeypatch.setattr(subprocess, "run", _fake_run(payload))
    watts, mhz = bench._smi_sample()
    assert watts == 1288.0
    assert mhz == pytest.approx(1835.0)  # mean of 1800 .. 1870 over the 8 XCDs


def test_smi_sample_is_none_without_a_reading(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run("", returncode=1))
    assert bench._smi_sample() is None
    monkeypatch.setattr(subprocess, "run", _fake_run(json.dumps({"gpu_data": [{"power": {}}]})))
    assert bench._smi_sample() is None

    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench._smi_sample() is None
