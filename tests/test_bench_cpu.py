"""Host logic of bench.py that needs no GPU: it refuses more than one GPU
before touching one, and the HBM traffic it reports from the counter passes
is voided once the kernel sources they were taken with change."""
import copy
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_void_when_sources_change():
    bench = _bench()
    entry = {"fetch_kib": 100.0, "fetch_scale": 2.0, "write_kib": 50.0, "write_scale": 1.0,
             "sources": ["include/orbit.h"]}
    entry["source_digest"] = bench.source_digest(entry["sources"])
    assert bench.measured_traffic(entry) == int(100.0 * 1024 * 2.0 + 50.0 * 1024)
    stale = copy.deepcopy(entry)
    stale["source_digest"] = "0" * 16
    assert bench.measured_traffic(stale) is None
    assert bench.measured_traffic(None) is None


def test_recorded_traffic_entries_are_well_formed():
    bench = _bench()
    tr = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for name in ("qlinear_gemm", "quant_act"):
        e = tr[name]
        for f in e["sources"]:
            assert os.path.exists(os.path.join(ROOT, f)), f
        assert e["algorithmic_bytes"] > 0
        got = bench.measured_traffic(e)
        if got is not None:  # the sources are the ones the counters were taken with
            assert got == e["hbm_bytes"]
