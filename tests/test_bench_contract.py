"""bench.py measures one GPU: asked for more it exits with status 2 and says so,
before touching the GPU.  It reports the committed HBM traffic counters only
for the configuration they were taken on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_counters_only_for_the_plain_step(monkeypatch):
    spec = importlib.util.spec_from_file_location("bench_contract_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "8", "--warmup", "2", "--no-graph"])
    assert b.counters_apply(b.parse())
    for extra in (["--budget", "4096"], ["--gates", "0.5"], ["--tier", "host"],
                  ["--query-corr", "0.9"], ["--svd", "randomized"], ["--zoom-frac", "0.1"],
                  ["--batch", "4"], ["--residency-gb", "4"], ["--n-tokens", "9000"]):
        monkeypatch.setattr(sys, "argv", ["bench.py", *extra])
        assert not b.counters_apply(b.parse()), extra
