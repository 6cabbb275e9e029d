"""Host-side checks of bench.py: the one-GPU guard and the helpers that turn
measurements into the roofline fields.  Nothing here touches a GPU."""
from __future__ import annotations

import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line for a run that measured nothing


def test_at_clock_scales_peak_with_the_measured_clock():
    b = _bench()
    assert b.at_clock(None, 800.0, 1000.0, 700.0) is None
    got = b.at_clock({"mean_mhz": 1920.0}, 800.0, 1000.0, 700.0)
    peak = 2500.0 * 1920.0 / 2400.0
    assert got["peak_tflops"] == pytest.approx(peak, abs=0.05)
    assert got["frac_of_peak"] == pytest.approx(800.0 / peak, abs=1e-4)
    assert got["fwd_frac_of_peak"] == pytest.approx(1000.0 / peak, abs=1e-4)
    assert got["bwd_frac_of_peak"] == pytest.approx(700.0 / peak, abs=1e-4)
    # at the nominal 2.4 GHz the figure is the published peak itself
    assert b.at_clock({"mean_mhz": 2400.0}, 1250.0, 0.0, 0.0)["frac_of_peak"] == pytest.approx(0.5)


def _records(path):
    out = {}
    for ln in open(path).read().splitlines():
        if ln.startswith("traffic-record: "):
            rec = json.loads(ln[len("traffic-record: "):])
            out[rec["phase"]] = rec
    return out


def test_recorded_traffic_reads_the_committed_records():
    b = _bench()
    recs = _records(b.TRAFFIC_PROFILE)
    assert {"fwd", "bwd_main", "bwd_post"} <= set(recs)
    assert b.recorded_traffic("no_such_phase") is None
    for phase, rec in recs.items():
        got = b.recorded_traffic(phase)
        # a record is used only while the kernel's sources hash the same as when
        # the counters were taken; otherwise the field is null
        if got is not None:
            assert got == int(rec["read_bytes"]) + int(rec["write_bytes"])


def test_recorded_traffic_is_null_once_sources_change(tmp_path, monkeypatch):
    b = _bench()
    rec = _records(b.TRAFFIC_PROFILE)["fwd"]
    good = dict(rec)
    stale = dict(rec, phase="fwd_stale", source_sha256="0" * 64)
    p = tmp_path / "traffic.md"
    p.write_text("# test records\n" + "".join(f"traffic-record: {json.dumps(r)}\n" for r in (good, stale)))
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(p))
    assert b.recorded_traffic("fwd_stale") is None
    expect = int(rec["read_bytes"]) + int(rec["write_bytes"])
    assert b.recorded_traffic("fwd") in (None, expect)
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert b.recorded_traffic("fwd") is None
