"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs: span table bit-exact, means and summaries bit-exact up to
float64 rounding-order ties at the storage rounding point, factors by
reconstruction and singular values, zoom masks and lists bit-exact outside the
|p - tau| < 1e-5 band, attention within 1e-5 (float32 K/V) or 2e-3 (bf16 K/V)
norm-wise relative error."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import (Inputs, OracleSide, attn_err, calibrate_tau, compare_group,
                          compare_route, compare_spans, log, make_cfg, rel_err,
                          route_from_gpu, to64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def run_gpu_layer(S, cache, layer, q, p, tau, with_prob=True, fused=False):
    """One layer through the C ABI: sekv_route + sekv_decode_attn, or the
    single-launch sekv_route_attn."""
    rb = S.RouteBuffers.allocate(cache, with_prob=with_prob)
    o = torch.zeros(cache.cfg.n_q_heads, cache.cfg.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    if fused:
        S.sekv_route_attn(cache, layer, q.contiguous(), p.contiguous(), tau.contiguous(), rb, o, ws)
    else:
        S.sekv_route(cache, layer, q.contiguous(), p.contiguous(), tau.contiguous(), rb)
        S.sekv_decode_attn(cache, layer, q.contiguous(), rb, o, ws)
    torch.cuda.synchronize()
    return rb, o


def assert_same_route(a, b):
    assert torch.equal(a.mask, b.mask)
    assert torch.equal(a.count, b.count) and torch.equal(a.union_count, b.union_count)
    for h in range(a.count.numel()):
        n = int(a.count[h])
        assert torch.equal(a.list[h, :n], b.list[h, :n])
    for g in range(a.union_count.numel()):
        n = int(a.union_count[g])
        assert torch.equal(a.union_list[g, :n], b.union_list[g, :n])
    if a.prob is not None and b.prob is not None:
        assert torch.equal(a.prob, b.prob)


def check_layer(S, cache, orc, inp, layer, q, tau, gamma, tol):
    """Both call paths against the oracle; the single-launch path must give
    bit-identical routes and outputs to the two-call path.  Masks and lists
    are compared outside the tie band; the attention of every head is
    compared with the oracle's over the GPU's own zoom mask (which equals the
    oracle's whenever the band is empty)."""
    p = inp.p[layer]
    rb, o = run_gpu_layer(S, cache, layer, q, p, tau)
    rbf, of = run_gpu_layer(S, cache, layer, q, p, tau, fused=True)
    assert_same_route(rb, rbf)
    assert torch.equal(o, of)
    route = orc.route(layer, to64(q), to64(p), to64(tau), gamma)
    n_tie = compare_route(rb, route, to64(tau), inp.wl)
    ref = orc.decode(layer, to64(q), route_from_gpu(rb, route.prob, inp.wl.n_kv_heads))
    og = to64(o)
    worst = max(attn_err(og[h], ref[h]) for h in range(inp.wl.n_q_heads))
    assert worst <= tol, f"attention error {worst} > {tol}"
    return n_tie, worst, route


@pytest.mark.parametrize("seed", list(range(1, 17)))
def test_tiny_workload_full_parity(S, seed):
    wl = synth.workload("tiny")
    log(f"[parity] tiny seed={seed} N={wl.n_tokens}")
    inp = Inputs(wl, seed)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    compare_spans(cache, orc)
    compare_group(cache, orc, 0, 0, n_factor_checks=1000)
    tau = synth.tau_uniform(wl, seed, device="cuda")
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, inp.query(0)[0], tau[0], wl.gamma,
                                      TOL["f32"])
    log(f"[parity] tiny seed={seed} spans={cache.info.n_compressed} zoomed={int(route.mask.sum())} "
        f"ties={n_tie} err={worst:.2e}")


def _reduced(name, **kw):
    return synth.workload(name, **kw)


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_128k", dict(n_layers=2, n_tokens=16384 + 77)),
    ("llama32_3b_32k", dict(n_layers=1, n_tokens=8192 + 5)),
    ("qwen25_14b_128k_b4", dict(n_layers=1, n_tokens=6000, batch=1)),
])
def test_bf16_reduced_shapes(S, name, kw):
    wl = _reduced(name, **kw)
    seed = synth.default_seed(wl)
    log(f"[parity] {name} {kw}")
    inp = Inputs(wl, seed)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    layers = list(range(wl.n_layers))
    orc = OracleSide(inp, layers, wl.max_rank)
    compare_spans(cache, orc)
    for layer in layers:
        for kh in range(wl.n_kv_heads):
            compare_group(cache, orc, layer, kh, n_factor_checks=6)
    tau = calibrate_tau(orc, inp, layers, synth.zoom_targets(wl, seed), wl.gamma).cuda()
    for step in range(2):
        q = inp.query(step)
        for layer in layers:
            n_tie, worst, route = check_layer(S, cache, orc, inp, layer, q[layer], tau[layer],
                                              wl.gamma, TOL["bf16"])
            log(f"[parity] {name} step={step} layer={layer} zoom={route.mask.mean():.3f} "
                f"ties={n_tie} err={worst:.2e}")


def _sdpa(q, k, v):
    hq, hkv = q.shape[0], k.shape[0]
    kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=0))
    vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=0))
    o = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], kt, vt)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict()),
    ("llama3_8b_128k", dict(n_layers=1, n_tokens=6000, n_q_heads=8, n_kv_heads=2)),
])
def test_all_zoomed_full_rank_is_dense_attention(S, name, kw):
    """Every span zoomed with every component kept: textbook attention over
    all N rows (torch SDPA on the CPU in float64), any gamma."""
    wl = synth.workload(name, **kw)
    log(f"[parity] dense check {name} {kw}")
    inp = Inputs(wl, 5)
    cache = S.sekv_build_spans(make_cfg(S, wl, max_rank=128), inp.s, inp.k, inp.v, inp.w,
                               torch.full_like(inp.ranks, 128))
    q = inp.query(0)[0]
    tau = torch.full((wl.n_q_heads,), -1.0, device="cuda")
    rb, o = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    rbf, of = run_gpu_layer(S, cache, 0, q, inp.p[0], tau, fused=True)
    assert torch.equal(o, of)
    assert int(rb.mask.sum()) == wl.n_q_heads * cache.info.n_compressed
    ref = _sdpa(to64(q), to64(inp.k[0]), to64(inp.v[0]))
    err = max(attn_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads))
    log(f"[parity] dense check err={err:.2e}")
    assert err <= TOL[wl.kv_dtype]


@pytest.mark.parametrize("case", ["none_zoomed", "short_context", "constant_surprisal",
                                  "ragged_small"])
def test_edge_cases(S, case):
    wl = synth.workload("tiny")
    tau_val = None
    surprisal = None
    if case == "none_zoomed":
        tau_val = 1.0
    elif case == "short_context":
        wl = wl.with_(n_tokens=300)
    elif case == "constant_surprisal":
        surprisal = torch.full((wl.n_tokens,), 0.75)
    elif case == "ragged_small":
        wl = wl.with_(n_tokens=777, window=100, min_span_len=3)
    log(f"[parity] edge case {case} N={wl.n_tokens}")
    inp = Inputs(wl, 11, surprisal=surprisal)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    compare_spans(cache, orc)
    if cache.info.n_compressed:
        compare_group(cache, orc, 0, 0, n_factor_checks=50)
    tau = synth.tau_uniform(wl, 11, device="cuda")[0]
    if tau_val is not None:
        tau = torch.full_like(tau, tau_val)
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, inp.query(0)[0], tau, wl.gamma,
                                      TOL["f32"])
    if case == "none_zoomed":
        assert not route.mask.any()
    if case == "constant_surprisal":
        assert cache.info.n_anchors == 0 and cache.info.n_compressed == 1
    log(f"[parity] edge case {case} spans={cache.info.n_compressed} err={worst:.2e}")


def test_repeat_runs_are_bit_identical(S):
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=9000)
    log("[parity] determinism")
    inp = Inputs(wl, 3)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    q = inp.query(0)[0]
    tau = torch.full((wl.n_q_heads,), 0.6, device="cuda")
    rb1, o1 = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    rb2, o2 = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    assert torch.equal(o1, o2)
    for _ in range(3):
        rbf, of = run_gpu_layer(S, cache, 0, q, inp.p[0], tau, fused=True)
        assert torch.equal(o1, of)
        assert_same_route(rb1, rbf)
    assert torch.equal(rb1.mask, rb2.mask) and torch.equal(rb1.union_list, rb2.union_list)
    assert torch.equal(rb1.list, rb2.list) and torch.equal(rb1.count, rb2.count)
    cache2 = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    _, o3 = run_gpu_layer(S, cache2, 0, q, inp.p[0], tau)
    assert torch.equal(o1, o3)


def test_uneven_zoom_parity_and_repeat(S):
    """Zoom concentrated on a few KV heads (three zoom ~75% of their spans,
    two have one head at ~40%, three zoom nothing), so a few workgroups attend
    many spans while most attend none: against the oracle, and bit-identical
    over repeated launches of both call paths."""
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=20000)
    log("[parity] uneven zoom")
    inp = Inputs(wl, 6)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    q = inp.query(0)[0]
    q64, p64 = to64(q), to64(inp.p[0])
    prob = orc.route(0, q64, p64, np.full(wl.n_q_heads, 2.0), wl.gamma).prob
    frac = np.zeros(wl.n_q_heads)
    for h in range(wl.n_q_heads):
        kh, i = divmod(h, wl.group)
        frac[h] = 0.75 if kh < 3 else (0.4 if kh < 5 and i == 0 else 0.0)
    tau = torch.tensor([float(np.quantile(prob[h], 1.0 - frac[h])) if frac[h] > 0 else 1.0
                        for h in range(wl.n_q_heads)], dtype=torch.float32).cuda()
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, q, tau, wl.gamma, TOL["bf16"])
    heavy = 0   # 32-span chunks with more than 8 zoomed spans (two per wave)
    for kh in range(wl.n_kv_heads):
        ids = np.asarray(route.unions[kh])
        if ids.size:
            heavy += int((np.bincount(ids // 32) > 8).sum())
    log(f"[parity] uneven zoom: chunks with >8 zoomed {heavy} ties={n_tie} err={worst:.2e}")
    assert heavy >= 10
    assert all(len(route.unions[kh]) == 0 for kh in range(5, wl.n_kv_heads))
    rb0, o0 = run_gpu_layer(S, cache, 0, q, inp.p[0], tau, fused=True)
    for _ in range(4):
        rb1, o1 = run_gpu_layer(S, cache, 0, q, inp.p[0], tau, fused=True)
        assert torch.equal(o0, o1)
        assert_same_route(rb0, rb1)
        rb2, o2 = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
        assert torch.equal(o0, o2)


@pytest.mark.parametrize("name,kw,lens", [
    ("qwen25_14b_128k_b4", dict(), [6000, 4096, 300, 9000]),
    ("tiny", dict(n_q_heads=4, n_kv_heads=1), [3000, 200, 5000])], ids=["bf16_G5", "f32_G4"])
def test_batched_layer_matches_single_calls(S, name, kw, lens):
    """Sequences of one model shape (Qwen2.5-14B heads, G = 5, bf16 K/V; and
    float32 K/V at G = 4), each with its own cache and context length, one of
    them shorter than the window (no compressed span), through the batched
    calls (one launch for the rest): routes and outputs bit-identical to the
    single-sequence calls, and the first sequence against the oracle."""
    base = synth.workload(name, n_layers=1, n_tokens=4096, **kw)
    seed = synth.default_seed(base)
    log(f"[parity] batched layer {name} {kw}, contexts {lens}")
    inps, caches = [], []
    for i, n in enumerate(lens):
        wl = base.with_(n_tokens=n)
        inp = Inputs(wl, seed, seq=i)
        inps.append(inp)
        caches.append(S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks))
    assert min(c.info.n_compressed for c in caches) == 0 and caches[0].info.n_compressed > 0
    Hq, d = base.n_q_heads, base.head_dim
    p = inps[0].p[0].contiguous()   # one model layer's projections, shared by the batch
    qs = [inp.query(i)[0].contiguous() for i, inp in enumerate(inps)]
    orc = OracleSide(inps[0], [0], base.max_rank)
    prob = orc.route(0, to64(qs[0]), to64(p), np.full(Hq, 2.0), base.gamma).prob
    tau = torch.tensor([float(np.quantile(prob[h], 0.9)) for h in range(Hq)],
                       dtype=torch.float32).cuda()   # ~10% zoom per head

    def fresh():
        return ([S.RouteBuffers.allocate(c, with_prob=True) for c in caches],
                [torch.zeros(Hq, d, device="cuda") for _ in caches],
                [torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda") for c in caches])
    rbs, outs, wss = fresh()
    S.sekv_route_attn_batch(caches, 0, qs, p, tau, rbs, outs, wss)
    torch.cuda.synchronize()
    assert sum(int(r.union_count.sum()) for r in rbs) > 0
    for i, c in enumerate(caches):
        rb, o = run_gpu_layer(S, c, 0, qs[i], p, tau, fused=True)
        assert_same_route(rb, rbs[i])
        assert torch.equal(o, outs[i]), f"sequence {i}"
    _, outs_d, wss_d = fresh()
    S.sekv_decode_attn_batch(caches, 0, qs, rbs, outs_d, wss_d)
    torch.cuda.synchronize()
    for i, c in enumerate(caches):
        _, o = run_gpu_layer(S, c, 0, qs[i], p, tau)
        assert torch.equal(o, outs_d[i]), f"sequence {i}"
    route = orc.route(0, to64(qs[0]), to64(p), to64(tau), base.gamma)
    n_tie = compare_route(rbs[0], route, to64(tau), inps[0].wl)
    ref = orc.decode(0, to64(qs[0]), route_from_gpu(rbs[0], route.prob, base.n_kv_heads))
    worst = max(attn_err(to64(outs[0])[h], ref[h]) for h in range(Hq))
    log(f"[parity] batched layer: ties={n_tie} err={worst:.2e}")
    assert worst <= TOL[base.kv_dtype]


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_128k", dict(n_tokens=9000)),
    ("tiny", dict(n_q_heads=4, n_kv_heads=1))], ids=["bf16_G4", "f32_G4"])
def test_host_tier_matches_oracle_and_device_tier(S, name, kw):
    """Factors in pinned host memory, fetched per layer for the union of the
    zoomed spans (the SeKV page, Sec. 3.2: bases kept on the CPU and fetched
    for the selected spans): routes against the oracle, outputs against the
    oracle over the same mask, with and without a separate fetch stream, and
    equal to the device tier's up to the order of the float32 merge (the
    zoomed spans form their own partials)."""
    wl = synth.workload(name, n_layers=2, **kw)
    log(f"[parity] host tier {name} {kw}")
    inp = Inputs(wl, 4)
    dev = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    assert host.info.factor_pool_bytes == dev.info.factor_pool_bytes
    orc = OracleSide(inp, [0, 1], wl.max_rank)
    compare_spans(host, orc)
    for layer in range(2):
        for kh in range(wl.n_kv_heads):
            compare_group(host, orc, layer, kh, n_factor_checks=4)
    if name == "tiny":   # about a quarter of the spans zoomed per head
        prob = orc.route(0, to64(inp.query(1)[0]), to64(inp.p[0]), np.full(wl.n_q_heads, 2.0),
                         wl.gamma).prob
        tau = torch.tensor([float(np.quantile(prob[h], 0.75)) for h in range(wl.n_q_heads)],
                           dtype=torch.float32, device="cuda")
    else:
        tau = torch.full((wl.n_q_heads,), 0.7, device="cuda")
    side = torch.cuda.Stream()
    for layer in range(2):
        q = inp.query(1)[layer]
        rbd, od = run_gpu_layer(S, dev, layer, q, inp.p[layer], tau)
        route = orc.route(layer, to64(q), to64(inp.p[layer]), to64(tau), wl.gamma)
        for fused, fst in ((False, side), (True, side), (True, None), (False, None)):
            rb = S.RouteBuffers.allocate(host, with_prob=True)
            oh = torch.zeros_like(od)
            ws = torch.empty(host.workspace_bytes(), dtype=torch.uint8, device="cuda")
            if fused:
                S.sekv_route_attn(host, layer, q, inp.p[layer].contiguous(), tau, rb, oh, ws,
                                  fetch_stream=fst)
            else:
                S.sekv_route(host, layer, q, inp.p[layer].contiguous(), tau, rb)
                S.sekv_decode_attn(host, layer, q, rb, oh, ws, fetch_stream=fst)
            torch.cuda.synchronize()
            assert int(rb.union_count.sum()) > 0
            n_tie = compare_route(rb, route, to64(tau), wl)
            ref = orc.decode(layer, to64(q), route_from_gpu(rb, route.prob, wl.n_kv_heads))
            err_o = max(attn_err(to64(oh)[h], ref[h]) for h in range(wl.n_q_heads))
            assert torch.equal(rb.mask, rbd.mask) and torch.equal(rb.union_count, rbd.union_count)
            err = float((oh - od).abs().max() / od.abs().max())
            log(f"[parity] host tier layer={layer} fused={fused} side stream={fst is not None} "
                f"ties={n_tie} err vs oracle={err_o:.2e} rel diff vs device={err:.2e}")
            assert err_o <= TOL[wl.kv_dtype]
            assert err <= 1e-6


def test_host_tier_fetch_failure_leaves_cache_usable(S):
    """A failing host-tier fetch (forced by the library's test hook) makes the
    call fail with the HIP status before anything of its attention is queued;
    the next calls on the same cache give the outputs of a call that never
    failed, bit for bit."""
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=6000)
    log("[parity] host tier fetch failure")
    inp = Inputs(wl, 5)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    tau = torch.full((wl.n_q_heads,), 0.6, device="cuda")
    q = inp.query(0)[0]
    p = inp.p[0].contiguous()
    ws = torch.empty(host.workspace_bytes(), dtype=torch.uint8, device="cuda")

    def call(fused):
        rb = S.RouteBuffers.allocate(host)
        o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
        if fused:
            S.sekv_route_attn(host, 0, q, p, tau, rb, o, ws)
        else:
            S.sekv_route(host, 0, q, p, tau, rb)
            S.sekv_decode_attn(host, 0, q, rb, o, ws)
        torch.cuda.synchronize()
        return rb, o

    rb0, o0 = call(True)
    assert int(rb0.union_count.sum()) > 0
    for fused in (True, False):
        S.sekv_test_fail_fetch(1)
        with pytest.raises(S.SekvError, match="injected"):
            call(fused)
        rb, o = call(fused)
        assert torch.equal(rb.mask, rb0.mask) and torch.equal(o, o0)
    S.sekv_test_fail_fetch(0)


def test_host_tier_memcpy_fetch_equals_gather(S):
    """The hipMemcpyAsync-per-run fetch moves the same blocks as the gather
    kernel: routes and outputs bit-identical, with and without a fetch stream,
    over both call paths; device-tier caches refuse the setting."""
    wl = synth.workload("llama3_8b_128k", n_layers=2, n_tokens=7000)
    log("[parity] host tier memcpy fetch")
    inp = Inputs(wl, 6)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    tau = torch.full((wl.n_q_heads,), 0.65, device="cuda")
    side = torch.cuda.Stream()
    ws = torch.empty(host.workspace_bytes(), dtype=torch.uint8, device="cuda")

    def call(layer, fused, fst):
        q = inp.query(2)[layer]
        p = inp.p[layer].contiguous()
        rb = S.RouteBuffers.allocate(host)
        o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
        if fused:
            S.sekv_route_attn(host, layer, q, p, tau, rb, o, ws, fetch_stream=fst)
        else:
            S.sekv_route(host, layer, q, p, tau, rb)
            S.sekv_decode_attn(host, layer, q, rb, o, ws, fetch_stream=fst)
        torch.cuda.synchronize()
        return rb, o

    for layer in range(2):
        for fused, fst in ((True, side), (False, None)):
            host.set_fetch_mode("gather")
            rb0, o0 = call(layer, fused, fst)
            host.set_fetch_mode("memcpy")
            rb1, o1 = call(layer, fused, fst)
            assert int(rb0.union_count.sum()) > 0
            assert torch.equal(rb0.union_list, rb1.union_list)
            assert torch.equal(o0, o1)
    host.set_fetch_mode("gather")
    dev = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    with pytest.raises(S.SekvError, match="host-tier"):
        dev.set_fetch_mode("memcpy")


def test_many_chunks_merge_parity(S):
    """Thousands of short spans, so a KV head has more than 128 chunks and the
    tail's merge runs more than one round of slot loads per thread (three with
    the host tier's separate zoom slots): routes and outputs against the
    oracle, and the host tier against the device tier."""
    wl = synth.workload("tiny", n_tokens=40000, min_span_len=1)
    log("[parity] many chunks: tiny N=40000, min span 1")
    inp = Inputs(wl, 4)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    assert cache.info.n_compressed > 128 * 32
    orc = OracleSide(inp, [0], wl.max_rank)
    tau = synth.tau_uniform(wl, 4, device="cuda")[0].contiguous()
    q = inp.query(0)[0]
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, q, tau, wl.gamma, TOL["f32"])
    log(f"[parity] many chunks: spans={cache.info.n_compressed} zoomed={int(route.mask.sum())} "
        f"ties={n_tie} err={worst:.2e}")
    assert int(route.mask.sum()) > 0
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    rbd, od = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    rb = S.RouteBuffers.allocate(host)
    oh = torch.zeros_like(od)
    ws = torch.empty(host.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(host, 0, q, inp.p[0].contiguous(), tau, rb, oh, ws,
                      fetch_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(rb.mask, rbd.mask) and torch.equal(rb.union_count, rbd.union_count)
    ref = orc.decode(0, to64(q), route_from_gpu(rb, route.prob, wl.n_kv_heads))
    err_o = max(attn_err(to64(oh)[h], ref[h]) for h in range(wl.n_q_heads))
    err = float((oh - od).abs().max() / od.abs().max())
    log(f"[parity] many chunks: host tier err vs oracle={err_o:.2e} rel diff vs device={err:.2e}")
    assert err_o <= TOL["f32"]
    assert err <= 1e-6


@pytest.mark.parametrize("n_tokens,chunks_per_wg", [(20000, 2), (40000, 4)])
def test_route_chunks_per_workgroup(S, n_tokens, chunks_per_wg):
    """The route launch gates 1, 2 or 4 chunks of 32 spans per workgroup as
    Hkv x chunks grows past one and two workgroups per CU: 4 KV heads of
    short spans reach the 2- and 4-chunk launches.  Routes and outputs of
    every head against the oracle; the batched call (whose route launch
    counts the chunks of all its sequences) bit-identical to single calls."""
    wl = synth.workload("tiny", n_tokens=n_tokens, min_span_len=1, n_q_heads=8, n_kv_heads=4)
    log(f"[parity] route chunks per workgroup: N={n_tokens}, 4 KV heads")
    inp = Inputs(wl, 7)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    wgs1 = wl.n_kv_heads * -(-cache.info.n_compressed // 32)
    assert (wgs1 > 512) == (chunks_per_wg == 4) and (256 < wgs1 <= 512) == (chunks_per_wg == 2)
    orc = OracleSide(inp, [0], wl.max_rank)
    tau = synth.tau_uniform(wl, 7, device="cuda")[0].contiguous()
    q = inp.query(0)[0]
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, q, tau, wl.gamma, TOL["f32"])
    log(f"[parity] route chunks: spans={cache.info.n_compressed} chunk workgroups={wgs1} "
        f"zoomed={int(route.mask.sum())} ties={n_tie} err={worst:.2e}")
    assert int(route.mask.sum()) > 0
    # two sequences through the batched call: its route launch sees both
    inp2 = Inputs(wl, 8)
    cache2 = S.sekv_build_spans(make_cfg(S, wl), inp2.s, inp2.k, inp2.v, inp2.w, inp2.ranks)
    q2 = inp2.query(0)[0]
    p = inp.p[0].contiguous()
    single = [run_gpu_layer(S, c, 0, qq, p, tau) for c, qq in ((cache, q), (cache2, q2))]
    rbs = [S.RouteBuffers.allocate(c, with_prob=True) for c in (cache, cache2)]
    outs = [torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda") for _ in range(2)]
    wss = [torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda") for c in (cache, cache2)]
    S.sekv_route_attn_batch([cache, cache2], 0, [q.contiguous(), q2.contiguous()], p, tau, rbs,
                            outs, wss)
    torch.cuda.synchronize()
    for (rb, o), rbb, ob in zip(single, rbs, outs):
        assert torch.equal(rb.mask, rbb.mask) and torch.equal(rb.prob, rbb.prob)
        assert torch.equal(rb.list, rbb.list) and torch.equal(o, ob)


@pytest.fixture(scope="module")
def full_c3(S):
    """The Llama-3-8B-shape workload at full size (32 layers, 131072 tokens,
    bf16), built once for the sampled-group checks."""
    wl = synth.workload("llama3_8b_128k")
    seed = synth.default_seed(wl)
    log("[parity] full size: drawing inputs and building the 128K cache")
    inp = Inputs(wl, seed)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    s64 = to64(inp.s)
    seg = O.segment(s64, wl.window, wl.alpha, wl.min_span_len)
    return wl, inp, cache, s64, seg


def sampled_group_parity(S, wl, inp, cache, s64, seg, layer, kv_head, step, tag):
    """One (layer, KV head) of a full-size cache: the oracle rebuilds that group
    from the same inputs and checks its means, summaries, sampled factors, the
    zoom masks and lists of its query heads (the first zooming ~20% of spans,
    the others ~1%, every other head of the layer at 0.5), and their outputs,
    through the single-launch call the bench times."""
    class One:  # the oracle side for a single group
        pass
    orc = One()
    orc.wl, orc.seg = wl, seg
    g = wl.group
    w = to64(inp.w[layer])
    gc = O.build_group(seg, s64, to64(inp.k[layer, kv_head]), to64(inp.v[layer, kv_head]),
                       {h: w[h] for h in range(kv_head * g, kv_head * g + g)},
                       inp.ranks[layer, kv_head].cpu().numpy(), wl.kv_dtype, wl.max_rank)
    orc.groups = {layer: {kv_head: gc}}
    compare_spans(cache, orc)
    nmis, worst = compare_group(cache, orc, layer, kv_head, n_factor_checks=12)
    q = inp.query(step)[layer]
    heads = list(range(kv_head * g, kv_head * g + g))
    pr = to64(inp.p[layer])
    ll = O.span_log_len(seg)
    tau = torch.full((wl.n_q_heads,), 0.5)
    for i, h in enumerate(heads):
        p, _ = O.route_head(to64(q[h]), pr[h], gc.summary[h], ll, wl.gamma, 2.0)
        tau[h] = float(np.quantile(p, 0.8 if i == 0 else 0.99))
    tau = tau.cuda()
    rb, o = run_gpu_layer(S, cache, layer, q, inp.p[layer], tau, fused=True)
    qn, tn = to64(q), to64(tau)
    h0, h1 = heads[0], heads[-1] + 1
    route = O.route_layer(qn[h0:h1], pr[h0:h1], tn[h0:h1],
                          {i: gc.summary[h] for i, h in enumerate(heads)}, seg, wl.gamma, 1)
    mask = rb.mask.cpu().numpy().astype(bool)[h0:h1, :seg.n_compressed]
    tie = np.abs(route.prob - tn[h0:h1, None]) < 1e-5
    assert np.array_equal(mask[~tie], route.mask[~tie])
    if not tie.any():
        cnt, lst = rb.count.cpu().numpy(), rb.list.cpu().numpy()
        for i, h in enumerate(heads):
            assert lst[h, :cnt[h]].tolist() == route.lists[i].tolist()
        uc, ul = rb.union_count.cpu().numpy(), rb.union_list.cpu().numpy()
        assert ul[kv_head, :uc[kv_head]].tolist() == route.unions[0].tolist()
    # every head's output over the GPU's own mask (the oracle's outside the band)
    og = to64(o)
    err = max(attn_err(og[h], O.mixed_attention(qn[h], gc, seg, mask[i]))
              for i, h in enumerate(heads))
    log(f"[parity] {tag} layer={layer} kv_head={kv_head}: storage mismatches {nmis}, factor "
        f"rel err {worst:.2e}, zoom {route.mask.mean(axis=1).round(3).tolist()} ties "
        f"{int(tie.sum())} attention err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.fixture(scope="module")
def full_c2(S):
    """The Llama-3.2-3B-shape workload at full size (28 layers, 24 query / 8 KV
    heads, 32768 tokens, bf16), built once."""
    wl = synth.workload("llama32_3b_32k")
    seed = synth.default_seed(wl)
    log("[parity] full size: drawing inputs and building the 32K cache")
    inp = Inputs(wl, seed)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    s64 = to64(inp.s)
    seg = O.segment(s64, wl.window, wl.alpha, wl.min_span_len)
    return wl, inp, cache, s64, seg


@pytest.mark.parametrize("layer,kv_head", [(0, 0), (13, 4), (27, 7), (20, 2)])
def test_full_size_32k_sampled_parity(S, full_c2, layer, kv_head):
    """Full-size Llama-3.2-3B shape (32K): sampled (layer, KV head) groups
    against the oracle through the single-launch call."""
    wl, inp, cache, s64, seg = full_c2
    sampled_group_parity(S, wl, inp, cache, s64, seg, layer, kv_head, 3 + layer, "full size 32K")


@pytest.mark.parametrize("layer,kv_head", [(0, 3), (31, 6), (12, 0), (20, 7), (7, 5), (27, 2)])
def test_full_size_sampled_parity(S, full_c3, layer, kv_head):
    """Full-size Llama-3-8B shape (the bench's cache): the whole span table
    bit-exact, and sampled (layer, KV head) groups against the oracle."""
    wl, inp, cache, s64, seg = full_c3
    sampled_group_parity(S, wl, inp, cache, s64, seg, layer, kv_head, 7 + layer,
                         "full size 128K")


@pytest.mark.parametrize("name,hq,hkv", [
    ("llama3_8b_128k", 4, 4), ("llama3_8b_128k", 8, 4), ("llama3_8b_128k", 6, 2),
    ("llama3_8b_128k", 12, 2), ("llama3_8b_128k", 16, 2),
    ("tiny", 2, 2), ("tiny", 4, 2), ("tiny", 8, 1), ("tiny", 256, 128)])
def test_group_sizes(S, name, hq, hkv):
    """Query heads per KV head G = 1, 2, 3, 6 and 8 with bf16 K/V and G = 1, 2
    and 8 with float32 K/V (the kernels are instantiated for every G up to 8
    and both storage types), and 128 KV heads (the zoom workgroups' shares
    are taken 64 KV heads at a time): route and attention against the oracle,
    both call paths bit-identical, and the budget cap in both scopes on the
    same route."""
    kw = dict(n_layers=1, n_tokens=5000) if name != "tiny" else {}
    wl = synth.workload(name, n_q_heads=hq, n_kv_heads=hkv, **kw)
    log(f"[parity] group size G={hq // hkv} ({hq}/{hkv} heads)")
    inp = Inputs(wl, 12)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    compare_spans(cache, orc)
    q = inp.query(0)[0]
    prob = orc.route(0, to64(q), to64(inp.p[0]), np.full(hq, 2.0), wl.gamma).prob
    tau = torch.tensor([float(np.quantile(prob[h], 0.75)) for h in range(hq)],
                       dtype=torch.float32).cuda()
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, q, tau, wl.gamma, TOL[wl.kv_dtype])
    # the budget cap on the GPU's own route, against the oracle's cap
    rb, _ = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    gp = rb.prob.cpu().numpy()[:, :cache.info.n_compressed]
    gm = rb.mask.cpu().numpy().astype(bool)[:, :cache.info.n_compressed]
    g = hq // hkv
    uncapped = O.LayerRoute(prob=gp, mask=gm, lists=[O.compact(gm[h]) for h in range(hq)],
                            unions=[O.union_lists(list(gm[k * g:(k + 1) * g])) for k in range(hkv)])
    n = orc.seg.span_len[orc.seg.cspan].astype(np.int64)
    budget = int(np.median([n[u].sum() for u in uncapped.unions]) // 2)
    S.sekv_cap_budget(cache, rb, budget)
    torch.cuda.synchronize()
    ref = O.cap_budget(uncapped, orc.seg, hkv, budget)
    assert np.array_equal(rb.mask.cpu().numpy().astype(bool)[:, :cache.info.n_compressed], ref.mask)
    for k in range(hkv):
        assert rb.union_list[k, :int(rb.union_count[k])].cpu().tolist() == ref.unions[k].tolist()
    for h in range(hq):
        assert rb.list[h, :int(rb.count[h])].cpu().tolist() == ref.lists[h].tolist()
    # one budget for the layer: half of every KV head's union tokens together
    lbudget = sum(int(n[u].sum()) for u in uncapped.unions) // 2
    rl, _ = run_gpu_layer(S, cache, 0, q, inp.p[0], tau)
    S.sekv_cap_budget(cache, rl, lbudget, scope="layer")
    torch.cuda.synchronize()
    lref = O.cap_budget(uncapped, orc.seg, hkv, lbudget, scope="layer")
    assert np.array_equal(rl.mask.cpu().numpy().astype(bool)[:, :cache.info.n_compressed],
                          lref.mask)
    for k in range(hkv):
        assert rl.union_list[k, :int(rl.union_count[k])].cpu().tolist() == lref.unions[k].tolist()
    for h in range(hq):
        assert rl.list[h, :int(rl.count[h])].cpu().tolist() == lref.lists[h].tolist()
    log(f"[parity] G={g}: zoom={route.mask.mean():.3f} ties={n_tie} err={worst:.2e} "
        f"budget={budget} capped pairs={int(ref.mask.sum())}, layer budget={lbudget} "
        f"capped pairs={int(lref.mask.sum())}")


@pytest.mark.parametrize("case", ["route_dim_7", "route_dim_64_bf16", "no_window_unit_spans",
                                  "one_past_window", "rank_one"])
def test_config_edges(S, case):
    """Configurations off the common path: routing dimensions that take the
    general summary loads (7 floats, 64 bf16), no local window with every
    non-anchor run compressed down to one-token spans, a context one token past
    the window, and rank-1 factors; all against the oracle."""
    wl = synth.workload("tiny")
    max_rank = None
    if case == "route_dim_7":
        wl = wl.with_(route_dim=7)
    elif case == "route_dim_64_bf16":
        wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=4000, route_dim=64)
    elif case == "no_window_unit_spans":
        wl = wl.with_(n_tokens=1500, window=0, min_span_len=1)
    elif case == "one_past_window":
        wl = wl.with_(n_tokens=wl.window + 1)
    elif case == "rank_one":
        max_rank = 1
    log(f"[parity] config edge {case}")
    inp = Inputs(wl, 21)
    cache = S.sekv_build_spans(make_cfg(S, wl, max_rank=max_rank), inp.s, inp.k, inp.v, inp.w,
                               inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank if max_rank is None else max_rank)
    compare_spans(cache, orc)
    if cache.info.n_compressed:
        for kh in range(wl.n_kv_heads):
            compare_group(cache, orc, 0, kh, n_factor_checks=20)
    q = inp.query(0)[0]
    if cache.info.n_compressed:
        prob = orc.route(0, to64(q), to64(inp.p[0]), np.full(wl.n_q_heads, 2.0), wl.gamma).prob
        tau = torch.tensor([float(np.quantile(prob[h], 0.7)) for h in range(wl.n_q_heads)],
                           dtype=torch.float32).cuda()
    else:
        tau = torch.full((wl.n_q_heads,), 0.5, device="cuda")
    n_tie, worst, route = check_layer(S, cache, orc, inp, 0, q, tau, wl.gamma, TOL[wl.kv_dtype])
    log(f"[parity] config edge {case}: spans={cache.info.n_compressed} dense={cache.info.n_dense} "
        f"zoomed pairs={int(route.mask.sum())} ties={n_tie} err={worst:.2e}")
