"""Decode-step benchmark of the SeKV HIP library on one MI355X.

One step = for every layer, in order: route (gate + zoom lists) and the
mixed-resolution attention over anchors, window, zoomed spans (factored) and
coarse entries.  Inputs are seeded synthetic tensors with the shapes of the
Llama-3-8B workload at 128K context (32 layers, 32 query / 8 KV heads, d 128,
bf16 K/V, spans of ~80 tokens, rank cap 32, window 512, 10% of heads zoom ~20%
of spans and the rest ~1%), resident in HBM before timing starts.

Prints ONE JSON line (one per share with --zoom-sweep).  ``value`` is decode
steps/s of the whole job.  ``roofline`` covers a layer, the step's only work:
the layer kernel (routing, full-resolution rows, coarse entries), the zoom
kernel (zoomed spans) and the tail launch (merge and lists); algorithmic bytes
per layer / average layer time from HIP events recorded on the launch stream.
``cpu_baseline`` times the CPU oracle, pinned to one core, on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn steps/s at 128K ctx (Llama-3-8B shape); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
PCIE_GBS = 64.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_128k")
    ap.add_argument("--tier", choices=["device", "host"], default="device")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=1,
                    help="layers the CPU oracle decodes for cpu_baseline: 1 = the middle layer, "
                         "3 = first, middle and last")
    ap.add_argument("--cpu-configs", nargs="?", const="all", default=None,
                    help="only time the CPU oracle (one pinned core) on the decode workloads "
                         "(comma-separated names, default all) and print one JSON line; uses no "
                         "GPU")
    ap.add_argument("--n-layers", type=int, default=None, help="override layer count (testing)")
    ap.add_argument("--n-tokens", type=int, default=None, help="override context (testing)")
    ap.add_argument("--batch", type=int, default=None,
                    help="sequences per step (default: the workload's); above 1 each layer runs "
                         "through the batched calls, one layer launch and one tail launch for "
                         "all sequences")
    ap.add_argument("--budget", type=int, default=None,
                    help="matched-budget cap in tokens per KV head and layer (or per layer, "
                         "with --budget-scope layer): each layer runs sekv_route (gate values "
                         "kept), sekv_cap_budget, sekv_decode_attn")
    ap.add_argument("--budget-scope", choices=["kv_head", "layer"], default="kv_head",
                    help="the budget covers each KV head of a layer, or the whole layer")
    ap.add_argument("--residency-gb", type=float, default=0.0,
                    help="host tier: HBM residency cache of factor blocks, in GB (0 = none)")
    ap.add_argument("--slot-kb", type=int, default=64, help="residency cache slot size, KiB")
    ap.add_argument("--fetch", choices=["gather", "memcpy"], default="gather",
                    help="host tier: factor fetch by the gather kernel, or one hipMemcpyAsync per "
                         "run of union spans (the host waits for each layer's route)")
    ap.add_argument("--write-traffic", nargs=3, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "ALG_BYTES"),
                    help="from the counter CSVs of a FETCH_SIZE and a WRITE_SIZE rocprofv3 pass "
                         "over the default step and its algorithmic bytes per layer, write the "
                         "traffic file roofline.traffic reads; uses no GPU")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup time stamps of each layer's route, attend and tail "
                         "launches (one sequence, device tier; needs the diagnostic library: "
                         "python -m compressed_kv_attention_sekv_amd.build --timeline, loaded "
                         "with SEKV_LIBRARY=compressed_kv_attention_sekv_amd/libsekv_timeline.so); "
                         "prints a JSON summary instead of the bench line")
    ap.add_argument("--trace-last", type=int, default=640,
                    help="with --trace-summary: the per-kernel statistics of each kernel's last "
                         "this many launches (default 640: 20 steps x 32 layers)")
    ap.add_argument("--trace-skip", type=int, default=0,
                    help="with --trace-summary: leave out each kernel's last this many launches "
                         "before taking the last --trace-last (640 with the defaults: the timed, "
                         "graph-replayed steps instead of the byte count's launches after them)")
    ap.add_argument("--trace-summary", default=None,
                    help="summarise a rocprofv3 kernel trace CSV (per-kernel launches and mean "
                         "duration; host tier: how much of each layer's factor fetch overlaps "
                         "its full-resolution launch) and exit; uses no GPU")
    ap.add_argument("--query-corr", type=float, default=0.0,
                    help="AR(1) correlation of consecutive step queries (0 = independent)")
    ap.add_argument("--svd", choices=["exact", "randomized"], default="exact",
                    help="per-span truncated SVD of the build")
    ap.add_argument("--gates", type=float, default=None,
                    help="soft-gate the factors after the build (Eq. 8) with synthetic gates, "
                         "dropping components whose gate is below this value")
    ap.add_argument("--zoom-sweep", default=None,
                    help="comma-separated zoom shares: one build, one JSON line per share")
    ap.add_argument("--full-rank", action="store_true",
                    help="build every span at full rank (rank cap d, every component kept); with "
                         "--zoom-frac 1 the step is the dense-attention check")
    ap.add_argument("--zoom-frac", type=float, default=None,
                    help="share of spans every query head zooms, replacing the workload's own "
                         "shares (0 zooms nothing, 1 zooms every span)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the sources the layer kernels are compiled from."""
    h = hashlib.sha256()
    for f in ("sekv_decode.hip", "sekv_internal.h"):
        with open(os.path.join(ROOT, "compressed_kv_attention_sekv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters_apply(args) -> bool:
    """The committed counter summaries are of the plain step (device tier, every
    option at its default); a run with any other option moves other bytes."""
    return (args.tier == "device" and args.budget is None and args.gates is None
            and args.query_corr == 0.0 and args.svd == "exact" and args.zoom_frac is None
            and args.batch is None and args.n_layers is None and args.n_tokens is None
            and args.residency_gb == 0.0 and not args.zoom_sweep and not args.full_rank)


LAYER_KERNELS = ("route_kernel", "attend_kernel", "layer_tail_kernel")   # a device-tier layer


def counter_means(path: str, last: int = 64) -> dict:
    """Mean of each counter per kernel over its last `last` dispatches, from a
    rocprofv3 --pmc counter collection CSV: {kernel: {counter: mean}}."""
    import csv
    import statistics
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = (r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                 .replace("void ", "").strip())
            did = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per.setdefault(k, {}).setdefault(r["Counter_Name"], {})[did] = float(r["Counter_Value"])
    out = {}
    for k, cs in per.items():
        out[k] = {}
        for c, byd in cs.items():
            vals = [byd[i] for i in sorted(byd)[-last:]]
            out[k][c] = statistics.mean(vals)
            out[k]["dispatches"] = len(vals)
    return out


def write_traffic(workload: str, fetch_csv: str, write_csv: str, alg_bytes: str) -> None:
    """HBM bytes per layer (its layer, zoom and tail launches) from FETCH_SIZE
    and WRITE_SIZE in KiB per dispatch, each scaled by what it reads for the
    device-copy probe of this script (a 2 GiB torch copy_, dispatched as
    __amd_rocclr_copyBuffer), into profiles/traffic_layer_kernel_<workload>.json
    with the hash of the kernel sources it was taken on."""
    import statistics
    fm, wm = counter_means(fetch_csv, last=1 << 30), counter_means(write_csv, last=1 << 30)

    def per_layer(m, counter):
        return sum(v[counter] for k, v in m.items() if any(n in k for n in LAYER_KERNELS)
                   and counter in v)

    def probe_kib(path, counter, names, top):
        import csv
        with open(path) as f:
            vals = [float(r["Counter_Value"]) for r in csv.DictReader(f)
                    if all(n in r["Kernel_Name"] for n in names) and r["Counter_Name"] == counter]
        return statistics.median(sorted(vals)[-top:]) if vals else None

    def copy_kib(path, counter):
        return probe_kib(path, counter, ("copyBuffer",), 6)

    fm64, wm64 = counter_means(fetch_csv), counter_means(write_csv)
    fetch_raw, write_raw = per_layer(fm64, "FETCH_SIZE"), per_layer(wm64, "WRITE_SIZE")
    moved_kib = 2 * 1024 * 1024   # the probe copies 2 GiB each way
    cf, cw = copy_kib(fetch_csv, "FETCH_SIZE"), copy_kib(write_csv, "WRITE_SIZE")
    fs, ws = moved_kib / cf, moved_kib / cw
    rf = probe_kib(fetch_csv, "FETCH_SIZE", ("reduce_kernel", "ReduceOp<float",
                                             "sum_functor<float, float, float>"), 5)
    fb, wb = fetch_raw * 1024 * fs, write_raw * 1024 * ws
    out = {"workload": workload,
           "kernel": "sekv::route_kernel + sekv::attend_kernel + sekv::layer_tail_kernel (one layer)",
           "kernel_source_hash": kernel_source_hash(), "bytes_per_launch": fb + wb,
           "fetch_bytes": fb, "write_bytes": wb, "fetch_KiB_raw": fetch_raw,
           "write_KiB_raw": write_raw, "fetch_scale": fs, "write_scale": ws,
           "copy_probe_fetch_KiB": cf, "copy_probe_write_KiB": cw,
           # a second point for the fetch scale: the read-only probe's row sums
           # over the same 2 GiB (a float sum reduction that reads 2 GiB, writes 2 MiB)
           "read_probe_fetch_KiB": rf,
           "read_probe_fetch_scale": moved_kib / rf if rf else None,
           "algorithmic_bytes_per_launch_same_steps": float(alg_bytes),
           "per_kernel_KiB": {k: {"FETCH_SIZE": fm64[k].get("FETCH_SIZE"),
                                  "WRITE_SIZE": wm64.get(k, {}).get("WRITE_SIZE")}
                              for k in fm64 if any(n in k for n in LAYER_KERNELS)},
           "launches_averaged": 64}
    path = os.path.join(ROOT, "profiles", f"traffic_layer_kernel_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def read_traffic(workload: str):
    """HBM traffic per attention launch from committed rocprofv3 --pmc
    summaries, only if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_layer_kernel_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_last, args.trace_skip)
        return
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic)
        return
    if args.cpu_configs:
        cpu_configs(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path runs on a "
              "single MI355X; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import compressed_kv_attention_sekv_amd as S
    import synth

    S.lib()
    dev = "cuda"
    over = {}
    if args.n_layers:
        over["n_layers"] = args.n_layers
    if args.n_tokens:
        over["n_tokens"] = args.n_tokens
    if args.batch is not None:
        over["batch"] = args.batch
    wl = synth.workload(args.workload, **over)
    B = wl.batch
    if not 1 <= B <= S.SEKV_MAX_BATCH:
        print(f"--batch must be in [1, {S.SEKV_MAX_BATCH}]", file=sys.stderr)
        sys.exit(2)
    if B > 1 and args.tier != "device":
        print("batched steps run with device-tier factors only", file=sys.stderr)
        sys.exit(2)
    if args.residency_gb > 0 and args.tier != "host":
        print("--residency-gb applies to host-tier factors (--tier host)", file=sys.stderr)
        sys.exit(2)
    if args.budget is not None and (B > 1 or args.budget < 0):
        print("--budget takes a count >= 0 and one sequence", file=sys.stderr)
        sys.exit(2)
    seed = synth.default_seed(wl)
    L, Hq, Hkv, d, G = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.group

    # ---- inputs, resident in HBM, and one cache per sequence ---------------------
    w, p = synth.route_weights(wl, seed, device=dev)
    if args.full_rank:
        wl = wl.with_(max_rank=d)
    cfg = S.make_config(L, Hq, Hkv, head_dim=d, route_dim=wl.route_dim, window=wl.window,
                        max_rank=wl.max_rank, min_span_len=wl.min_span_len, alpha=wl.alpha,
                        gamma=wl.gamma, kv_dtype=wl.kv_dtype, factor_tier=args.tier,
                        svd=args.svd)
    caches, build_s = [], 0.0
    for b in range(B):
        t0 = time.time()
        s_b, spike_b = synth.surprisal(wl, seed, seq=b, device=dev)
        k, v, ranks_b = synth.kv_cache(wl, seed, spike_b, seq=b, device=dev)
        if args.full_rank:
            ranks_b = torch.full_like(ranks_b, d)
        torch.cuda.synchronize()
        log(f"sequence {b}: inputs drawn in {time.time() - t0:.1f}s: K/V "
            f"{2 * k.numel() * k.element_size() / 1e9:.1f} GB")
        t0 = time.time()
        c = S.sekv_build_spans(cfg, s_b, k, v, w, ranks_b)
        torch.cuda.synchronize()
        dt = time.time() - t0
        build_s += dt
        i_ = c.info
        log(f"sequence {b}: build {dt:.2f}s: spans {i_.n_spans} compressed {i_.n_compressed} "
            f"anchors {i_.n_anchors} dense {i_.n_dense} factor pool "
            f"{i_.factor_pool_bytes / 1e9:.2f} GB")
        if args.gates is not None:
            if args.tier != "device":
                print("--gates needs device-tier factors", file=sys.stderr)
                sys.exit(2)
            fb = c.info.factor_bytes
            t0 = time.time()
            S.sekv_apply_gates(c, synth.span_gates(wl, seed, c.info.n_compressed, "k", device=dev),
                               synth.span_gates(wl, seed, c.info.n_compressed, "v", device=dev),
                               args.gates)
            log(f"sequence {b}: gates applied in {time.time() - t0:.2f}s, factor bytes "
                f"{fb / 1e9:.2f} -> {c.info.factor_bytes / 1e9:.2f} GB")
        if args.tier == "host" and args.fetch != "gather":
            c.set_fetch_mode(args.fetch)
        caches.append(c)
        if b == 0:
            s, spike, ranks = s_b, spike_b, ranks_b   # the CPU baseline's sample
        # the K/V inputs are not needed by the decode step
        del k, v
        torch.cuda.empty_cache()
    cache = caches[0]
    info = cache.info
    sc = info.n_compressed

    def measure(zoom_arg):
        """Calibrate the thresholds for a zoom share (None: the workload's own
        shares), time the steps and account their bytes; returns the JSON line."""
        # ---- thresholds: calibrated on the library's own gate values (sequence 0;
        # thresholds belong to the model, so every sequence uses them) -------------
        if zoom_arg is not None:
            # one share for every (layer, head), whatever the workload's own mode
            targets = torch.full((L, Hq), float(zoom_arg), dtype=torch.float64)
        elif wl.tau_mode == "uniform":
            targets = None
        else:
            targets = synth.zoom_targets(wl, seed)
        if targets is None:
            tau = synth.tau_uniform(wl, seed, device=dev)
        else:
            cq = synth.calibration_queries(wl, seed, 16, device=dev)
            tau = torch.empty(L, Hq, dtype=torch.float32, device=dev)
            rb = S.RouteBuffers.allocate(cache, with_prob=True)
            big = torch.full((Hq,), 2.0, device=dev)
            for layer in range(L):
                probs = []
                for i in range(cq.shape[0]):
                    S.sekv_route(cache, layer, cq[i, layer].contiguous(), p[layer].contiguous(), big, rb)
                    probs.append(rb.prob.clone())
                allp = torch.cat(probs, dim=1)
                # a share of 0 zooms nothing (p <= 1 is never above 1), 1 zooms all
                tau[layer] = torch.stack([
                    torch.tensor(1.0, device=dev) if float(targets[layer, h]) <= 0.0 else
                    torch.tensor(-1.0, device=dev) if float(targets[layer, h]) >= 1.0 else
                    torch.quantile(allp[h], 1.0 - float(targets[layer, h])).float()
                    for h in range(Hq)]).float()
            torch.cuda.synchronize()

        if args.timeline:
            return timeline_summary(S, cache, wl, seed, p, tau, dev)

        # ---- per-step buffers ----------------------------------------------------------
        n_q = args.steps + args.warmup
        if args.query_corr:
            qs = torch.stack([synth.correlated_queries(wl, seed, n_q, args.query_corr, seq=b,
                                                       device=dev) for b in range(B)], dim=1)
        else:
            qs = torch.stack([torch.stack([synth.queries(wl, seed, i, seq=b, device=dev)
                                           for b in range(B)]) for i in range(n_q)])
        # qs: [T][B][L][Hq][d]
        if args.residency_gb > 0:
            cache.set_residency(int(args.residency_gb * 1e9), args.slot_kb * 1024)
        q_cur = torch.empty(B, L, Hq, d, device=dev)
        p_c = [p[l].contiguous() for l in range(L)]
        tau_c = [tau[l].contiguous() for l in range(L)]
        capped = args.budget is not None
        routes = [[S.RouteBuffers.allocate(c, with_prob=capped) for _ in range(L)]
                  for c in caches]   # [B][L]
        outs = torch.zeros(B, L, Hq, d, device=dev)
        wss = [torch.empty(c.workspace_bytes(), dtype=torch.uint8, device=dev) for c in caches]
        side = torch.cuda.Stream() if args.tier == "host" else None

        def layer_call(layer):
            if capped:
                S.sekv_route(cache, layer, q_cur[0, layer], p_c[layer], tau_c[layer], routes[0][layer])
                S.sekv_cap_budget(cache, routes[0][layer], args.budget, scope=args.budget_scope)
                S.sekv_decode_attn(cache, layer, q_cur[0, layer], routes[0][layer], outs[0, layer],
                                   wss[0], fetch_stream=side)
            elif B == 1:
                S.sekv_route_attn(cache, layer, q_cur[0, layer], p_c[layer], tau_c[layer],
                                  routes[0][layer], outs[0, layer], wss[0], fetch_stream=side)
            else:
                S.sekv_route_attn_batch(caches, layer, [q_cur[b, layer] for b in range(B)],
                                        p_c[layer], tau_c[layer], [r[layer] for r in routes],
                                        [outs[b, layer] for b in range(B)], wss)

        def step():
            for layer in range(L):
                layer_call(layer)

        graph = None
        if not args.no_graph and args.tier == "device":
            q_cur.copy_(qs[0])
            step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()

        def run(i):
            q_cur.copy_(qs[i])
            if graph is not None:
                graph.replay()
            else:
                step()

        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()

        # ---- timed region ----------------------------------------------------------
        if args.residency_gb > 0:
            cache.residency_stats(reset=True)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.time()
        ev0.record()
        for i in range(args.warmup, n_q):
            run(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.time() - wall0
        total_ms = ev0.elapsed_time(ev1)
        ms_per_step = total_ms / args.steps
        log(f"{args.steps} steps in {total_ms:.1f} ms (wall {wall * 1e3:.1f} ms): {ms_per_step:.4f} ms/step")
        res_stats = cache.residency_stats(reset=True) if args.residency_gb > 0 else None
        if res_stats:
            log(f"residency: {res_stats['hit_blocks']} blocks from HBM, {res_stats['fetched_blocks']} "
                f"over the host link ({res_stats['fetched_bytes'] / args.steps / 1e9:.3f} GB/step)")

        # ---- algorithmic bytes of the timed steps ----------------------------------
        # per sequence: the resident bytes every layer launch reads, and the factor
        # bytes 4 (rK + rV) (n + d + 1) of each (layer, KV head, span) for the zoom part
        eb = 2 if wl.kv_dtype == "bf16" else 4
        span_bytes, resident_layer = [], 0
        for c in caches:
            sp = c.spans()
            clen = sp["span_len"][sp["cspan"].long()].to(torch.float64)
            rank_tab = torch.stack([torch.stack([sum(c.group_data(l, g)[3:5]) for g in range(Hkv)])
                                    for l in range(L)]).to(torch.float64)  # [L][Hkv][Sc] rK + rV
            span_bytes.append((4.0 * rank_tab * (clen + d + 1)).to(dev))
            D_b, sc_b = c.info.n_dense, c.info.n_compressed
            resident_layer += (Hkv * (2 * d * eb * D_b + 2 * d * eb * sc_b) +
                               Hq * wl.route_dim * eb * sc_b + Hq * (wl.route_dim * d + d + 1) * 4 +
                               Hq * d * 4 + 4 * sc_b)

        # the zoomed spans' bytes, from the union lists of the timed steps' queries
        # (the first 128 of them: the union fractions vary little between steps,
        # and re-running every step of a long batched run layer by layer would
        # take minutes)
        acct = min(args.steps, 128)
        zoom_bytes = torch.zeros(acct, L, dtype=torch.float64, device=dev)
        zoom_frac = torch.zeros(L, Hq, dtype=torch.float64, device=dev)
        union_frac = torch.zeros(L, Hkv, dtype=torch.float64, device=dev)
        for si, i in enumerate(range(args.warmup, args.warmup + acct)):
            q_cur.copy_(qs[i])
            for layer in range(L):
                layer_call(layer)
                for b, c in enumerate(caches):
                    rb = routes[b][layer]
                    sc_b = c.info.n_compressed
                    if sc_b == 0:
                        continue
                    ar = torch.arange(sc_b, device=dev)
                    valid = ar.unsqueeze(0) < rb.union_count.unsqueeze(1)           # [Hkv][Sc]
                    ids = torch.where(valid, rb.union_list.long(),
                                      torch.zeros_like(rb.union_list.long()))
                    zb = torch.gather(span_bytes[b][layer], 1, ids) * valid
                    zoom_bytes[si, layer] += zb.sum()
                    zoom_frac[layer] += rb.count.double() / (sc_b * B)
                    union_frac[layer] += rb.union_count.double() / (sc_b * B)
        torch.cuda.synchronize()
        zoom_frac /= acct
        union_frac /= acct
        zb_step = zoom_bytes.sum(1)                       # [steps]
        bytes_step = float(zb_step.mean()) + L * resident_layer
        step_gbs = bytes_step / (ms_per_step * 1e-3) / 1e9
        log(f"bytes/step {bytes_step / 1e9:.3f} GB (zoom {float(zb_step.mean()) / 1e9:.3f} GB): "
            f"{step_gbs:.0f} GB/s = {step_gbs / HBM_PEAK_GBS:.3f} of peak")

        # ---- mean launch of the layer kernel, live, from the timed region ----------
        # The graph replays launch the 32 layer kernels back to back on one stream
        # (no host gaps: in a kernel trace the step's span equals the sum of its
        # launches), so the HIP events around the timed region over its steps x L
        # launches give the kernel's mean duration (plus one small query copy per
        # step).  Algorithmic bytes: the timed steps' zoomed-span factors per launch
        # plus the resident bytes every launch reads.
        attn_us_mean = total_ms * 1e3 / (args.steps * L)   # with --budget: the layer's 3 launches
        attn_bytes_meas = float(zoom_bytes.mean()) + resident_layer
        attn_gbs = attn_bytes_meas / (attn_us_mean * 1e-6) / 1e9
        log(f"layer launch: {attn_us_mean:.2f} us avg, {attn_bytes_meas / 1e6:.2f} MB algorithmic "
            f"-> {attn_gbs:.0f} GB/s")

        # ---- reference probes: device copy and pinned host->device copy ------------
        x = torch.empty(512 * 1024 * 1024, dtype=torch.float32, device=dev)   # 2 GiB
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 5 * 2 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        # read-only stream: row sums over the same 2 GiB (4096-float rows; writes
        # 0.02% of what it reads), the fastest read-only torch op on this GPU
        acc = x.view(-1, 4096).sum(dim=1)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            acc = x.view(-1, 4096).sum(dim=1)
        e1.record()
        torch.cuda.synchronize()
        read_gbs = 5 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del x, y, acc
        hpin = torch.empty(64 * 1024 * 1024, dtype=torch.float32, pin_memory=True)   # 256 MiB
        hd = torch.empty(hpin.shape, dtype=torch.float32, device=dev)
        hd.copy_(hpin, non_blocking=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(4):
            hd.copy_(hpin, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        h2d_gbs = 4 * hpin.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del hpin, hd
        log(f"probes: device copy {copy_gbs:.0f} GB/s (read+write), read-only {read_gbs:.0f} GB/s, "
            f"pinned H2D {h2d_gbs:.1f} GB/s")

        host_link = None
        if args.tier == "host":
            # bytes that crossed the link: every union block, or with the residency
            # cache only the blocks it did not hold
            link_bytes = (res_stats["fetched_bytes"] / args.steps if res_stats
                          else float(zb_step.mean()))
            link_gbs = link_bytes / (ms_per_step * 1e-3) / 1e9
            host_link = {"gbs": link_gbs, "bytes_per_step": link_bytes,
                         "frac_of_measured_h2d": link_gbs / h2d_gbs,
                         "frac_of_pcie5_x16": link_gbs / PCIE_GBS}
            if res_stats:
                tot = res_stats["hit_blocks"] + res_stats["fetched_blocks"]
                host_link["residency"] = {
                    "capacity_gb": args.residency_gb, "slot_bytes": res_stats["slot_bytes"],
                    "sets": res_stats["sets"],
                    "hit_rate_blocks": res_stats["hit_blocks"] / tot if tot else None,
                    "hit_bytes_per_step": res_stats["hit_bytes"] / args.steps}

        # ---- CPU oracle baseline on a bounded sample --------------------------------
        cpu = None
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(wl, seed, s, spike, w, p, tau, qs[:, 0], args, ranks, B)

        traffic = read_traffic(wl.name) if counters_apply(args) else None
        result = {
            "metric": METRIC,
            "value": 1e3 / ms_per_step,
            "unit": "steps/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": wl.kv_dtype,
            "data": "synthetic",
            "config": {
                "workload": wl.name, "n_layers": L, "n_q_heads": Hq, "n_kv_heads": Hkv,
                "head_dim": d, "context": wl.n_tokens, "batch": B, "kv_dtype": wl.kv_dtype,
                "factor_dtype": "f32", "factor_tier": args.tier, "window": wl.window,
                "max_rank": wl.max_rank, "route_dim": wl.route_dim, "graph": graph is not None,
                "budget_tokens": args.budget,
                "budget_scope": args.budget_scope if args.budget is not None else None,
                "query_corr": args.query_corr,
                "gate_eps": args.gates, "svd": args.svd,
                "fetch": args.fetch if args.tier == "host" else None,
                "zoom": ("skewed" if wl.tau_mode == "skewed" and zoom_arg is None else
                         (f"{float(targets[0, 0]):g} per head" if targets is not None
                          else "uniform tau")),
            },
            "roofline": {
                "bound": "hbm",
                "achieved": attn_gbs,
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": attn_gbs / HBM_PEAK_GBS,
                "traffic": traffic,
                "kernel": ("sekv_route (sekv::route_kernel + sekv::layer_tail_kernel), "
                           "sekv_cap_budget (sekv::cap_budget_kernel), sekv_decode_attn "
                           "(sekv::layer_kernel for the chunk masks + sekv::attend_kernel + "
                           "sekv::layer_tail_kernel): one layer, capped" if capped else
                           "host tier: sekv::route_kernel + sekv::layer_tail_kernel (route, lists), "
                           "the factor fetch (fetch_gather_kernel, one hipMemcpyAsync per run of "
                           "union spans, or res_claim_kernel + res_fetch_kernel with a residency "
                           "cache), sekv::layer_kernel (rows and coarse entries), sekv::zoom_kernel "
                           "(zoomed spans) and sekv::layer_tail_kernel (merge)"
                           if args.tier == "host" else
                           "sekv::route_kernel + sekv::attend_kernel + sekv::layer_tail_kernel "
                           "(sekv_route_attn, one layer: the route, then the zoomed spans beside "
                           "the full-resolution rows, coarse entries and lists, then the merge)"
                           if B == 1 else
                           f"sekv::route_batch_kernel + sekv::attend_batch_kernel + "
                           f"sekv::layer_tail_batch_kernel (sekv_route_attn_batch, one layer of "
                           f"{B} sequences)"),
                "algorithmic_bytes_per_launch": attn_bytes_meas,
                "avg_launch_us": attn_us_mean,
                "avg_launch_from": "HIP events around the timed region / (steps x layers); "
                                   "a layer is every launch named under kernel",
                "frac_of_measured_read": attn_gbs / read_gbs,
            },
            "cpu_baseline": cpu,
            "step_hbm": {"bytes_per_step": bytes_step, "gbs": step_gbs, "frac": step_gbs / HBM_PEAK_GBS,
                         "measured_copy_gbs": copy_gbs, "measured_read_gbs": read_gbs},
            "host_link": host_link,
            "measured_h2d_gbs": h2d_gbs,
            "cache": {"n_spans": info.n_spans, "n_compressed": sc, "n_anchors": info.n_anchors,
                      "n_dense": info.n_dense, "factor_pool_gb": info.factor_pool_bytes / 1e9,
                      "resident_gb": info.resident_bytes / 1e9, "build_s": build_s,
                      "zoom_frac_per_head_mean": float(zoom_frac.mean()),
                      "union_frac_per_group_mean": float(union_frac.mean()),
                      "zoom_bytes_per_step_gb": float(zb_step.mean()) / 1e9,
                      # the GPU KV budget of a step: what is resident plus the factors
                      # of the spans zoomed in it, against the full-resolution K/V
                      "kv_budget_frac": (sum(c.info.resident_bytes for c in caches) +
                                         float(zb_step.mean())) /
                                        (B * L * Hkv * wl.n_tokens * d * 2 * eb),
                      "tokens_per_s": B * 1e3 / ms_per_step},
        }
        return result

    if args.zoom_sweep:
        for zf in [float(x) for x in args.zoom_sweep.split(",")]:
            print(json.dumps(measure(zf)), flush=True)
    else:
        print(json.dumps(measure(args.zoom_frac)), flush=True)


def timeline_summary(S, cache, wl, seed, p, tau, dev) -> dict:
    """Time stamps of one step: for each layer, sekv_route_attn runs twice and
    the second run's stamps are read (route, attend and tail workgroups, in
    microseconds from the route's first workgroup).  Returns the means over
    the layers of each phase; `layers` holds each layer's figures."""
    import ctypes

    import numpy as np
    import torch

    import synth

    lib = S.lib()
    if not hasattr(lib, "sekv_timeline_read"):
        print("--timeline needs the time-stamped library: build it with python -m "
              "compressed_kv_attention_sekv_amd.build --timeline and load it with "
              "SEKV_LIBRARY=compressed_kv_attention_sekv_amd/libsekv_timeline.so", file=sys.stderr)
        sys.exit(2)
    lib.sekv_timeline_read.restype = ctypes.c_int
    lib.sekv_timeline_read.argtypes = [ctypes.c_void_p] * 3
    lib.sekv_timeline_clear.restype = ctypes.c_int
    if wl.batch != 1 or cache.cfg.factor_tier != S.SEKV_TIER_DEVICE:
        print("--timeline takes one sequence with device-tier factors", file=sys.stderr)
        sys.exit(2)
    slots = 16
    tr, ta, tt = (np.zeros(4096 * slots, dtype=np.uint64) for _ in range(3))
    L, Hq, d = wl.n_layers, wl.n_q_heads, wl.head_dim
    q = synth.queries(wl, seed, 3, device=dev)
    o = torch.zeros(Hq, d, device=dev)
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device=dev)
    layers = []
    for layer in range(L):
        rb = S.RouteBuffers.allocate(cache)
        call = (cache, layer, q[layer].contiguous(), p[layer].contiguous(),
                tau[layer].contiguous(), rb, o, ws)
        S.sekv_route_attn(*call)
        torch.cuda.synchronize()
        if lib.sekv_timeline_clear() != 0:
            raise RuntimeError("sekv_timeline_clear failed")
        S.sekv_route_attn(*call)
        torch.cuda.synchronize()
        if lib.sekv_timeline_read(tr.ctypes.data, ta.ctypes.data, tt.ctypes.data) != 0:
            raise RuntimeError("sekv_timeline_read failed")
        r, a, t = (x.reshape(-1, slots).astype(np.int64) for x in (tr, ta, tt))
        r, a, t = r[r[:, 0] > 0], a[a[:, 0] > 0], t[t[:, 0] > 0]
        base = r[:, 0].min()

        def us(x):
            return (x - base) / 100.0   # the stamps count a 100 MHz clock

        z, rows = a[a[:, 1] == 0], a[a[:, 1] == 1]
        zw = z[z[:, 10] > 0]   # zoom workgroups that got a share
        wave_end = us(zw[:, 6:10]).max(axis=1)
        first = us(a[:, 0]).min()
        rec = {
            "route_end": float(us(r[:, 1]).max()),
            "route_query": float((us(r[:, 4]) - us(r[:, 0])).mean()),
            "route_projection": float((us(r[:, 2]) - us(r[:, 4])).mean()),
            "route_first_chunk_gates": float((us(r[:, 3]) - us(r[:, 2])).mean()),
            "route_rest": float((us(r[:, 1]) - us(r[:, 3])).mean()),
            "attend_start": first,
            "zoom_allocation": float((us(zw[:, 3]) - us(zw[:, 0])).mean()),
            "zoom_lookup": float((us(zw[:, 4]) - us(zw[:, 3])).mean()),
            "zoom_metadata": float((us(zw[:, 5]) - us(zw[:, 4])).mean()),
            "zoom_pipeline_mean": float((wave_end - us(zw[:, 5])).mean()),
            "zoom_pipeline_max": float((wave_end - us(zw[:, 5])).max()),
            "zoom_wave_spread": float((us(zw[:, 6:10]).max(axis=1) -
                                       us(zw[:, 6:10]).min(axis=1)).mean()),
            "zoom_merge": float((us(zw[:, 2]) - wave_end).mean()),
            "zoom_end_max": float(us(zw[:, 2]).max()),
            "rows_prologue": float((us(rows[:, 3]) - us(rows[:, 0])).mean()),
            "rows_compute": float((us(rows[:, 4]) - us(rows[:, 3])).mean()),
            "rows_write": float((us(rows[:, 2]) - us(rows[:, 4])).mean()),
            "rows_late": int((us(rows[:, 0]) > first + 2.0).sum()),
            "rows_end_max": float(us(rows[:, 2]).max()),
            "attend_end": float(us(a[:, 2]).max()),
            "zoom_last": bool(us(zw[:, 2]).max() >= us(a[:, 2]).max()),
            "tail_start": float(us(t[:, 0]).min()),
            "tail_end": float(us(t[:, 1]).max()),
            "tail_workgroup": float((us(t[:, 1]) - us(t[:, 0])).mean()),
        }
        layers.append(rec)
        log(f"timeline layer {layer}: route ends {rec['route_end']:.2f}, attend "
            f"{rec['attend_start']:.2f}-{rec['attend_end']:.2f}, tail ends {rec['tail_end']:.2f} us")
    summary = {k: float(np.mean([x[k] for x in layers])) for k in layers[0]}
    return {"timeline": "microseconds from the route launch's first workgroup, means over the "
                        f"{L} layers of one step (second of two runs of each layer)",
            "workload": wl.name, "summary": summary, "layers": layers}


def trace_summary(path: str, last: int = 640, skip: int = 0) -> None:
    """Per-kernel launches and mean duration of a rocprofv3 kernel trace CSV,
    the gaps between consecutive decode launches, and for host-tier traces
    the overlap of each layer's factor fetch (fetch_gather_kernel) with the
    full-resolution launch that runs beside it on the other stream: the time
    both run, over the fetch's own time and over the shorter of the two (1 =
    the shorter one hides entirely under the other).  Prints one JSON line."""
    import csv
    import statistics
    with open(path) as f:
        head = f.readline()
    if "Counter_Name" in head:   # a counter collection: per-kernel means instead
        print(json.dumps({"counters": counter_means(path)}), flush=True)
        return
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))

    def span(r):
        return int(r["Start_Timestamp"]), int(r["End_Timestamp"])

    def short(name):
        name = name.replace("(anonymous namespace)::", "")
        return name.split("(")[0].replace("void ", "").strip()

    per = {}
    for r in rows:
        a, b = span(r)
        per.setdefault(short(r["Kernel_Name"]), []).append((b - a) / 1e3)
    # the last `last` launches of a kernel before its final `skip` (640 and 0
    # in a default run: the byte-count pass over 20 steps x 32 layers, the
    # timed steps' work launched one layer at a time; 640 and 640: the timed
    # steps themselves, graph-replayed; both free of the calibration's
    # route-only launches)
    def kept(v):
        return skip if 0 < skip < len(v) else 0

    def window(v):
        return v[:len(v) - kept(v)][-last:]

    kernels = {k: {"launches": len(v), "mean_us": statistics.mean(v),
                   "median_us": statistics.median(v), "total_us": sum(v),
                   "last": len(window(v)), "skipped": kept(v),
                   "last_mean_us": statistics.mean(window(v)),
                   "last_median_us": statistics.median(window(v)),
                   "last_min_us": min(window(v)), "last_max_us": max(window(v))}
               for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))}
    decode = [r for r in rows if any(k in r["Kernel_Name"] for k in
                                     ("route_kernel", "attend_kernel", "layer_kernel", "zoom_kernel",
                                      "layer_tail", "fetch_gather"))]
    gaps = [(span(b)[0] - span(a)[1]) / 1e3 for a, b in zip(decode, decode[1:])
            if span(b)[0] >= span(a)[1]]
    out = {"trace": os.path.basename(path), "kernels": kernels,
           "decode_gap_us_median": statistics.median(gaps) if gaps else None}
    # host tier: each fetch against the layer launch that starts closest to it
    fetch = [r for r in rows if "fetch_gather_kernel" in r["Kernel_Name"]]
    layer = [r for r in rows if "layer_kernel" in r["Kernel_Name"]]
    if fetch and layer:
        fracs = []
        for fr in fetch:
            f0, f1 = span(fr)
            lr = min(layer, key=lambda r: abs(span(r)[0] - f0))
            l0, l1 = span(lr)
            both = max(0, min(f1, l1) - max(f0, l0))
            fracs.append((both / max(f1 - f0, 1), both / max(min(f1 - f0, l1 - l0), 1)))
        out["fetch_overlap"] = {
            "fetches": len(fracs),
            "of_fetch_time_mean": statistics.mean(f for f, _ in fracs),
            "of_shorter_launch_mean": statistics.mean(g for _, g in fracs)}
    print(json.dumps(out), flush=True)


def host_info() -> dict:
    """CPU model and thread counts of the host the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": model, "nproc": os.cpu_count(), "threads_allowed": aff}


class one_core:
    """Pin this process to one core (the first it may run on) and every thread
    pool to one thread; restore both on exit."""

    def __enter__(self):
        import torch
        from threadpoolctl import threadpool_limits
        self.aff = os.sched_getaffinity(0)
        self.core = min(self.aff)
        os.sched_setaffinity(0, {self.core})
        self.torch_threads = torch.get_num_threads()
        torch.set_num_threads(1)
        self.tp = threadpool_limits(limits=1)
        return self

    def __exit__(self, *exc):
        import torch
        self.tp.unregister()
        torch.set_num_threads(self.torch_threads)
        os.sched_setaffinity(0, self.aff)
        return False


def oracle_cache(wl, seg, sv, seed, spike, w, layers, device):
    """The oracle's cache of the given layers (all KV heads), untimed."""
    import oracle as O
    import synth
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    g = wl.group
    groups = {}
    for layer in layers:
        kk, vv, rk = synth.kv_cache(wl, seed, spike, device=device, layers=[layer])
        wl_ = f64(w[layer])
        groups[layer] = {kh: O.build_group(seg, sv, f64(kk[0, kh]), f64(vv[0, kh]),
                                           {h: wl_[h] for h in range(kh * g, kh * g + g)},
                                           rk[0, kh].cpu().numpy(), wl.kv_dtype, wl.max_rank)
                         for kh in range(wl.n_kv_heads)}
        del kk, vv
    return groups


def time_oracle_decode(wl, seg, groups, p, tau, qs, layers, budget_s=12.0, max_steps=200):
    """Route + attention of the given layers, every query head, over fresh step
    queries until about ``budget_s`` of work; returns (seconds per layer, steps)."""
    import oracle as O
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    g = wl.group
    pr = {layer: f64(p[layer]) for layer in layers}
    ta = {layer: f64(tau[layer]) for layer in layers}
    summ = {layer: {h: groups[layer][h // g].summary[h] for h in range(wl.n_q_heads)}
            for layer in layers}
    n_steps, dt = 0, 0.0
    while dt < budget_s and n_steps < min(max_steps, qs.shape[0]):
        q = f64(qs[n_steps])
        t0 = time.time()
        for layer in layers:
            route = O.route_layer(q[layer], pr[layer], ta[layer], summ[layer], seg, wl.gamma,
                                  wl.n_kv_heads)
            O.decode_layer(q[layer], route, groups[layer], seg, n_kv_heads=wl.n_kv_heads)
        dt += time.time() - t0
        n_steps += 1
    return dt / (n_steps * len(layers)), n_steps, dt


def cpu_baseline(wl, seed, s, spike, w, p, tau, qs, args, ranks, batch=1):
    """The oracle as it stands, pinned to one core with one thread: build the
    oracle's cache for a few layers spread over the depth (untimed), then time
    its decode (route + attention, every query head) of those layers over
    fresh step queries until about 10 s of CPU work, and scale to a full step
    (of sequence 0; a step of a batch is ``batch`` such sequences)."""
    import oracle as O

    L = wl.n_layers
    layers = sorted({0, L // 2, L - 1}) if args.cpu_layers >= 3 else [L // 2]
    with one_core() as pin:
        t0 = time.time()
        sv = s.detach().cpu().double().numpy()
        seg = O.segment(sv, wl.window, wl.alpha, wl.min_span_len)
        groups = oracle_cache(wl, seg, sv, seed, spike, w, layers, s.device)
        build_s = time.time() - t0
        per_layer, n_steps, dt = time_oracle_decode(wl, seg, groups, p, tau, qs, layers)
        core = pin.core
    per_step = per_layer * L * batch
    log(f"cpu oracle (core {core}): layers {layers} x {n_steps} steps decoded in {dt:.2f}s "
        f"(build {build_s:.1f}s) -> {per_step:.2f} s/step")
    out = {"value": 1.0 / per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_steps} decode steps of layers {layers} ({len(layers)} of {L}), all "
                     f"{wl.n_q_heads} query heads, route + attention, float64 numpy pinned to "
                     f"core {core} with one thread ({dt:.1f} s); time per layer scaled by {L}" +
                     (f" and by {batch} sequences" if batch > 1 else ""),
           "pinned_core": core}
    out.update(host_info())
    return out


def cpu_configs(args):
    """The oracle on one pinned core for every decode workload (no GPU): the
    tiny single-layer reference whole, and sampled layers of the 32K, 128K and
    batch-4 128K shapes, each scaled to a full step.  Inputs are drawn on the
    CPU; thresholds are calibrated on the oracle's own gate values as the
    workloads state (the batch-4 shape at its 10% share per head)."""
    import numpy as np
    import torch

    import oracle as O
    import synth

    results = []
    names = ["tiny", "llama32_3b_32k", "llama3_8b_128k", "qwen25_14b_128k_b4"]
    if args.cpu_configs != "all":
        names = [n for n in args.cpu_configs.split(",") if n]
    for name in names:
        wl = synth.workload(name)
        seed = synth.default_seed(wl)
        L = wl.n_layers
        layers = [L // 2]   # one layer's oracle cache keeps the untimed setup to minutes
        t0 = time.time()
        s, spike = synth.surprisal(wl, seed)
        w, p = synth.route_weights(wl, seed)
        sv = s.double().numpy()
        seg = O.segment(sv, wl.window, wl.alpha, wl.min_span_len)
        groups = oracle_cache(wl, seg, sv, seed, spike, w, layers, "cpu")
        g = wl.group
        if wl.tau_mode == "uniform":
            tau = synth.tau_uniform(wl, seed)
        else:
            targets = synth.zoom_targets(wl, seed)
            cq = synth.calibration_queries(wl, seed, 16)
            tau = torch.ones(L, wl.n_q_heads)
            for layer in layers:
                summ = {h: groups[layer][h // g].summary[h] for h in range(wl.n_q_heads)}
                probs = np.concatenate([O.route_layer(
                    cq[i, layer].double().numpy(), p[layer].double().numpy(),
                    np.full(wl.n_q_heads, 2.0), summ, seg, wl.gamma, wl.n_kv_heads).prob
                    for i in range(cq.shape[0])], axis=1)
                for h in range(wl.n_q_heads):
                    f = float(targets[layer, h])
                    tau[layer, h] = float(np.quantile(probs[h], 1.0 - f)) if f > 0 else 1.0
        qs = torch.stack([synth.queries(wl, seed, i) for i in range(400)])
        setup_s = time.time() - t0
        with one_core() as pin:
            per_layer, n_steps, dt = time_oracle_decode(wl, seg, groups, p, tau, qs, layers)
            core = pin.core
        per_step = per_layer * L * wl.batch
        log(f"cpu oracle {name}: {n_steps} steps of layers {layers} in {dt:.1f}s "
            f"(setup {setup_s:.0f}s) -> {per_step:.3f} s/step")
        results.append({"workload": name, "value": 1.0 / per_step, "unit": "steps/s",
                        "cores": 1, "pinned_core": core, "kind": "oracle",
                        "sample": f"{n_steps} decode steps of layers {layers} ({len(layers)} of "
                                  f"{L}), route + attention of all {wl.n_q_heads} query heads "
                                  f"({dt:.1f} s); scaled by {L} layers"
                                  + (f" and {wl.batch} sequences" if wl.batch > 1 else ""),
                        "context": wl.n_tokens, "n_compressed": seg.n_compressed})
    out = {"cpu_oracle_configs": results}
    out.update(host_info())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
