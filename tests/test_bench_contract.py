"""bench.py's output contract: one JSON line with the metric, the roofline
object and the oracle baseline (the run itself needs a GPU); a request for
more than one GPU is refused before anything runs."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_one_json_line_with_roofline_and_cpu_baseline():
    r = _bench("--steps", "3", "--warmup", "1", "--flush-mib", "64", "--cpu-seconds", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "bf16_causal_n8192_d128"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value = FLOPs x steps / wall time of the timed steps
    assert abs(d["value"] - d["config"]["flops_per_step"] / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == pytest.approx(2516.6, abs=0.1)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert "rows of bf16_causal_n8192_d128" in cb["sample"]
    assert d["settle"]["steps"] >= 1 and d["settle"]["ms"] <= 3500
    assert d["clock"]["counter_ghz"] is None or 0.5 <= d["clock"]["counter_ghz"] <= 2.5
    smu = d["clock"]["smu"]
    if smu is not None:  # read under load: the settle phase runs until the SMU table refreshed twice
        assert 100 <= smu["median_mhz"] <= 2500
        assert smu["median_socket_w"] is None or 100 <= smu["median_socket_w"] <= 2000
        assert smu["power_cap_w"] is None or smu["power_cap_w"] > 0


@pytest.mark.gpu
def test_key_padded_roofline_credits_allowed_pairs_only():
    r = _bench("--workload", "f16_keypad_n4096_d64", "--steps", "3", "--warmup", "1", "--flush-mib", "0",
               "--settle-ms", "0", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    rf, eff = d["roofline"], d["effective"]
    assert rf["achieved"] == pytest.approx(eff["tflops"], rel=1e-3)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    assert rf["nominal_frac"] > rf["frac"] and 0 < eff["fraction_of_nominal"] < 1


def test_cpu_baseline_sample_stays_near_its_time_target(monkeypatch):
    """The oracle baseline's sample sizing, with the oracle replaced by a
    stand-in whose cost per row rises 16-fold past 20000 rows (a host whose
    CPU share shrinks under load): the reported sample must still take about
    the target time, never more than the 1.5x cap plus one head."""
    import time
    import types

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import bench
    from online_softmax_03_amd import workloads as W

    done = {"rows": 0}

    def fake_attention(q, k, v, scale, causal, mask, rows=None, nthreads=1):
        done["rows"] += len(rows)
        per_row = 2e-6 if done["rows"] < 20000 else 3.2e-5
        time.sleep(per_row * len(rows))

    fake = types.SimpleNamespace(attention=fake_attention, max_threads=lambda: 4)
    monkeypatch.setitem(sys.modules, "oracle", fake)
    w = {x.name: x for x in W.WORKLOADS}["bf16_causal_n8192_d128"]
    x = {n: torch.zeros(1, dtype=torch.bfloat16) for n in ("q", "k", "v")}
    x.update(mask=None, scale=0.0884, causal=True)

    class _Arr:
        def __init__(self):
            self.shape = (w.B, w.H, w.N, w.d)

        def __getitem__(self, key):
            return self

    monkeypatch.setattr(torch.Tensor, "float", lambda self: types.SimpleNamespace(numpy=lambda: _Arr()))
    target = 0.4
    r = bench.cpu_baseline(w, x, target)
    seconds = float(r["sample"].rsplit(", ", 1)[1].rstrip(" s"))
    nrows = int(r["sample"].split(" ", 1)[0])
    assert 0 < nrows < w.B * w.H * w.N
    assert 0.7 * target <= seconds <= 1.5 * target + 0.05, r["sample"]
    assert np.isfinite(r["value"]) and r["value"] > 0
