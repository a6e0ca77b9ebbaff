"""bench.py measures one GPU: asked for more it exits with status 2 and says so,
before touching the GPU.  It reports the committed HBM traffic counters only
for the configuration they were taken on, and it turns counter files into
those figures by the copy probe's scale; its trace reader gives the per-kernel
figures of the profiles."""
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


def test_write_traffic_scales_counters_by_the_probes(tmp_path, monkeypatch):
    """roofline.traffic: each layer kernel's FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, the mean over its dispatches) scaled by what the counter reads
    for the 2 GiB device-copy probe; the read-only probe's fetch scale is
    recorded beside it.  Synthetic counter files with known values."""
    import csv
    import json
    spec = importlib.util.spec_from_file_location("bench_traffic_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = b.kernel_source_hash()   # of the sources under the real root
    monkeypatch.setattr(b, "kernel_source_hash", lambda: h)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))   # the summary goes to a scratch profiles/
    (tmp_path / "profiles").mkdir()
    gib_kib = 2 * 1024 * 1024
    reduce_name = ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float, "
                   "at::native::func_wrapper_t<float, at::native::sum_functor<float, float, "
                   "float>::operator()>(at::TensorIterator&)::{lambda(float, float)#1}>, "
                   "unsigned int, float, 4, 4> >(at::native::ReduceOp<...>)")
    kernels = {   # name: (FETCH_SIZE per dispatch, WRITE_SIZE per dispatch), in KiB
        "__amd_rocclr_copyBuffer": (gib_kib / 2, gib_kib),          # fetch counts half
        reduce_name: (gib_kib / 2 * 1.001, 2048.0),
        "void sekv::route_kernel<unsigned short, 4, 2>(sekv::LayerGeom, sekv::LayerArgs)": (100.0, 10.0),
        "void sekv::attend_kernel<unsigned short, 4>(sekv::LayerGeom, sekv::LayerArgs, int)":
            (1000.0, 50.0),
        "void sekv::layer_tail_kernel<4>(sekv::LayerGeom, sekv::LayerArgs, int)": (20.0, 2.0),
    }
    paths = {}
    for ci, counter in enumerate(("FETCH_SIZE", "WRITE_SIZE")):
        path = tmp_path / f"{counter}.csv"
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                              "Counter_Value"])
            w.writeheader()
            did = 0
            for name, vals in kernels.items():
                for rep in range(6):   # the same value on every dispatch but one
                    did += 1
                    v = vals[ci] * (0.5 if rep == 0 and "sekv" in name else 1.0)
                    w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                                "Counter_Value": v})
        paths[counter] = str(path)
    b.write_traffic("synthetic", paths["FETCH_SIZE"], paths["WRITE_SIZE"], "1000000")
    out = json.loads((tmp_path / "profiles" / "traffic_layer_kernel_synthetic.json").read_text())
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert abs(out["read_probe_fetch_scale"] - 2.0 / 1.001) < 1e-12
    mean = lambda v: (0.5 * v + 5 * v) / 6   # noqa: E731  (the half-valued dispatch included)
    fetch_kib = mean(100.0) + mean(1000.0) + mean(20.0)
    write_kib = mean(10.0) + mean(50.0) + mean(2.0)
    assert abs(out["fetch_bytes"] - fetch_kib * 1024 * 2.0) < 1e-6
    assert abs(out["write_bytes"] - write_kib * 1024 * 1.0) < 1e-6
    assert abs(out["bytes_per_launch"] - (out["fetch_bytes"] + out["write_bytes"])) < 1e-6
    assert out["kernel_source_hash"] == h


def test_trace_summary_means_gaps_and_fetch_overlap(tmp_path, capsys):
    """The kernel-trace reader behind the profiles: per-kernel means over the
    last launches, the median gap between consecutive decode launches, and a
    host-tier fetch's overlap with the layer launch beside it.  A synthetic
    trace with known timestamps (nanoseconds)."""
    import csv
    import json
    spec = importlib.util.spec_from_file_location("bench_trace_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    rows, t = [], 0
    route = "void sekv::route_kernel<unsigned short, 4, 2>(sekv::LayerGeom, sekv::LayerArgs)"
    attend = "void sekv::attend_kernel<unsigned short, 4>(sekv::LayerGeom, sekv::LayerArgs, int)"
    for i, dur in enumerate((7000, 8000, 9000)):   # three layers: route, 1 us gap, attend
        rows.append((route, t, t + dur))
        t += dur + 1000
        rows.append((attend, t, t + 2 * dur))
        t += 2 * dur + 1000
    fetch = "void sekv::fetch_gather_kernel(int, int)"
    layer = "void sekv::layer_kernel<unsigned short, 4>(sekv::LayerGeom, sekv::LayerArgs, int)"
    rows.append((layer, t, t + 10000))               # a host-tier pair: the fetch runs
    rows.append((fetch, t + 6000, t + 14000))        # 4 of its 8 us beside the layer launch
    path = tmp_path / "run_kernel_trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, a, e in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a, "End_Timestamp": e})
    b.trace_summary(str(path), last=2)
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    k = out["kernels"]["sekv::route_kernel<unsigned short, 4, 2>"]
    assert k["launches"] == 3 and k["mean_us"] == 8.0 and k["last_mean_us"] == 8.5
    assert k["last_min_us"] == 8.0 and k["last_max_us"] == 9.0
    a = out["kernels"]["sekv::attend_kernel<unsigned short, 4>"]
    assert a["last_mean_us"] == 17.0 and a["total_us"] == 48.0
    assert out["decode_gap_us_median"] == 1.0
    ov = out["fetch_overlap"]
    assert ov["fetches"] == 1 and ov["of_fetch_time_mean"] == 0.5
    assert ov["of_shorter_launch_mean"] == 0.5
    # the window before the last launch: the first two routes
    b.trace_summary(str(path), last=2, skip=1)
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    k = out["kernels"]["sekv::route_kernel<unsigned short, 4, 2>"]
    assert k["skipped"] == 1 and k["last"] == 2 and k["last_mean_us"] == 7.5
