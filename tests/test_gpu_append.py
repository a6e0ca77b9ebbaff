"""Window append and retire (sekv_append_tokens) through the C ABI, against
the oracle's segment_appended + build_group on the whole token history: the
span table, anchors, open run and full-resolution positions bit-exact; the
appended spans' means and summaries within a storage ulp and their factors by
reconstruction; routing and attention of every head after the appends; every
span zoomed at full rank after appends is dense attention over all tokens;
capacity and argument errors change nothing."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import (Inputs, attn_err, compare_group, compare_route, log, make_cfg,
                          route_from_gpu, to64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N0, N1 = 6000, 6400


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def workload(**kw):
    # spans of ~20 tokens, so the 400 appended tokens close a dozen spans
    base = dict(n_layers=2, n_tokens=N1, n_q_heads=8, n_kv_heads=2, spike_frac=1.0 / 21)
    base.update(kw)
    return synth.workload("llama3_8b_128k", **base)


def build_and_append(S, wl, inp, capacity, max_rank=None, ranks=None, steps=(1,) * 100 + (300,)):
    ranks = inp.ranks if ranks is None else ranks
    cfg = make_cfg(S, wl, max_rank=max_rank)
    cfg.append_capacity = capacity
    cache = S.sekv_build_spans(cfg, inp.s[:N0].contiguous(), inp.k[:, :, :N0].contiguous(),
                               inp.v[:, :, :N0].contiguous(), inp.w, ranks[:, :, :N0].contiguous())
    t = N0
    for n in steps:
        S.sekv_append_tokens(cache, inp.s[t:t + n].contiguous(), inp.k[:, :, t:t + n].contiguous(),
                             inp.v[:, :, t:t + n].contiguous(), inp.w,
                             ranks[:, :, t:t + n].contiguous())
        t += n
    torch.cuda.synchronize()
    assert t == N1 and cache.info.n_tokens == N1 and cache.info.n_appended == N1 - N0
    return cache


def oracle_after_appends(inp, wl, layers, rank_cap):
    s64 = to64(inp.s)
    build = O.segment(s64[:N0], wl.window, wl.alpha, wl.min_span_len)
    seg = O.segment_appended(s64, N0, build, wl.min_span_len)

    class Side:
        pass
    orc = Side()
    orc.wl, orc.seg, orc.groups = wl, seg, {}
    g = wl.group
    for layer in layers:
        w = to64(inp.w[layer])
        orc.groups[layer] = {
            kh: O.build_group(seg, s64, to64(inp.k[layer, kh]), to64(inp.v[layer, kh]),
                              {h: w[h] for h in range(kh * g, kh * g + g)},
                              inp.ranks[layer, kh].cpu().numpy(), wl.kv_dtype, rank_cap)
            for kh in range(wl.n_kv_heads)}
    return build, seg, orc


@pytest.mark.parametrize("kw", [dict(), dict(kv_dtype="f32", n_q_heads=4, n_kv_heads=4)],
                         ids=["bf16_G4", "f32_G1"])
def test_append_matches_oracle(S, kw):
    wl = workload(**kw)
    log(f"[append] {kw} build {N0} tokens, append {N1 - N0} (100 single tokens, then 300)")
    inp = Inputs(wl, 31)
    cache = build_and_append(S, wl, inp, capacity=512)
    build, seg, orc = oracle_after_appends(inp, wl, [0, 1], wl.max_rank)
    assert seg.n_compressed > build.n_compressed + 5, "the appends should close several spans"
    sp = cache.spans()
    for key in ("anchors", "span_start", "span_len", "kind", "cspan", "dense_pos"):
        assert sp[key].numpy().astype(np.int64).tolist() == getattr(seg, key).tolist(), key
    assert (cache.info.open_start, cache.info.open_len) == (
        (seg.open_start, seg.open_len) if seg.open_len else (cache.info.open_start, 0))
    for layer in (0, 1):
        for kh in range(wl.n_kv_heads):
            nmis, rec = compare_group(cache, orc, layer, kh, n_factor_checks=400)
    # routing and attention after the appends, about a quarter of spans zoomed
    for layer in (0, 1):
        q = inp.query(0)[layer].contiguous()
        p = inp.p[layer].contiguous()
        g = wl.group
        summ = {h: orc.groups[layer][h // g].summary[h] for h in range(wl.n_q_heads)}
        prob = O.route_layer(to64(q), to64(p), np.full(wl.n_q_heads, 2.0), summ, seg, wl.gamma,
                             wl.n_kv_heads).prob
        tau = torch.tensor([float(np.quantile(prob[h], 0.75)) for h in range(wl.n_q_heads)],
                           dtype=torch.float32).cuda()
        rb = S.RouteBuffers.allocate(cache, with_prob=True)
        o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
        ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
        S.sekv_route_attn(cache, layer, q, p, tau, rb, o, ws)
        torch.cuda.synchronize()
        route = O.route_layer(to64(q), to64(p), to64(tau), summ, seg, wl.gamma, wl.n_kv_heads)
        n_tie = compare_route(rb, route, to64(tau), wl)
        ref = O.decode_layer(to64(q), route_from_gpu(rb, route.prob, wl.n_kv_heads),
                             orc.groups[layer], seg, n_kv_heads=wl.n_kv_heads)
        err = max(attn_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads))
        log(f"[append] layer {layer}: spans {build.n_compressed} -> {seg.n_compressed}, dense "
            f"{build.dense_pos.size} -> {seg.dense_pos.size}, open run {seg.open_len}, zoomed "
            f"pairs {int(route.mask.sum())}, ties {n_tie}, attention err {err:.2e}")
        assert err <= (1e-5 if wl.kv_dtype == "f32" else 2e-3)


def test_append_full_rank_all_zoomed_is_dense(S):
    wl = workload(n_layers=1)
    log("[append] full rank, every span zoomed after appends")
    inp = Inputs(wl, 32)
    full = torch.full_like(inp.ranks, 128)
    cache = build_and_append(S, wl, inp, capacity=400, max_rank=128, ranks=full,
                             steps=(7, 1, 1, 91, 300))
    q = inp.query(0)[0].contiguous()
    rb = S.RouteBuffers.allocate(cache)
    o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(cache, 0, q, inp.p[0].contiguous(),
                      torch.full((wl.n_q_heads,), -1.0, device="cuda"), rb, o, ws)
    torch.cuda.synchronize()
    assert int(rb.mask.sum()) == wl.n_q_heads * cache.info.n_compressed
    G = wl.group
    kt = torch.from_numpy(np.repeat(to64(inp.k[0]), G, axis=0))
    vt = torch.from_numpy(np.repeat(to64(inp.v[0]), G, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(to64(q))[:, None, :], kt, vt)[:, 0, :].numpy()
    err = max(attn_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads))
    log(f"[append] dense check over {N1} tokens: spans {cache.info.n_compressed} err={err:.2e}")
    assert err <= 2e-3


def test_append_errors_change_nothing(S):
    wl = workload(n_layers=1, n_tokens=N0 + 40)
    inp = Inputs(wl, 33)
    cfg = make_cfg(S, wl)
    plain = S.sekv_build_spans(cfg, inp.s[:N0].contiguous(), inp.k[:, :, :N0].contiguous(),
                               inp.v[:, :, :N0].contiguous(), inp.w, inp.ranks[:, :, :N0].contiguous())
    one = lambda t, n: (inp.s[t:t + n].contiguous(), inp.k[:, :, t:t + n].contiguous(),  # noqa
                        inp.v[:, :, t:t + n].contiguous(), inp.w)
    with pytest.raises(S.SekvError, match="append_capacity"):
        S.sekv_append_tokens(plain, *one(N0, 1))
    cfg.append_capacity = 16
    cache = S.sekv_build_spans(cfg, inp.s[:N0].contiguous(), inp.k[:, :, :N0].contiguous(),
                               inp.v[:, :, :N0].contiguous(), inp.w, inp.ranks[:, :, :N0].contiguous())
    S.sekv_append_tokens(cache, *one(N0, 10))
    before = cache.spans()
    with pytest.raises(S.SekvError, match="capacity"):
        S.sekv_append_tokens(cache, *one(N0 + 10, 7))
    bad = one(N0 + 10, 2)
    s_bad = bad[0].clone()
    s_bad[1] = float("nan")
    with pytest.raises(S.SekvError, match="finite"):
        S.sekv_append_tokens(cache, s_bad, *bad[1:])
    after = cache.spans()
    assert cache.info.n_appended == 10 and cache.info.n_tokens == N0 + 10
    for key in before:
        assert torch.equal(before[key], after[key]), key
    S.sekv_append_tokens(cache, *one(N0 + 10, 6))
    assert cache.info.n_appended == 16


def test_appended_caches_in_batched_and_noalloc_calls(S):
    """Caches grown by different appends keep working through the batched
    call (bit-identical to the single calls) and the allocation-free call
    (bit-identical to the workspace call)."""
    wl = workload(n_layers=1)
    log("[append] batched and allocation-free calls after appends")
    caches, inps = [], []
    for seed, steps in ((41, (1,) * 20 + (250, 130)), (42, (120, 3, 47, 230)), (43, (400,))):
        inp = Inputs(wl, seed)
        caches.append(build_and_append(S, wl, inp, capacity=512, steps=steps))
        inps.append(inp)
    p = inps[0].p[0].contiguous()
    tau = torch.full((wl.n_q_heads,), 0.7, device="cuda")
    qs = [inp.query(3)[0].contiguous() for inp in inps]
    single = []
    for c, q in zip(caches, qs):
        rb = S.RouteBuffers.allocate(c)
        o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
        ws = torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda")
        S.sekv_route_attn(c, 0, q, p, tau, rb, o, ws)
        single.append((rb, o))
    rbs = [S.RouteBuffers.allocate(c) for c in caches]
    outs = [torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda") for _ in caches]
    wss = [torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda") for c in caches]
    S.sekv_route_attn_batch(caches, 0, qs, p, tau, rbs, outs, wss)
    torch.cuda.synchronize()
    for (rb, o), rbb, ob in zip(single, rbs, outs):
        assert torch.equal(rb.mask, rbb.mask) and torch.equal(o, ob)
    for c, q, (rb, o) in zip(caches, qs, single):
        rbn = S.RouteBuffers.allocate(c)
        on = torch.zeros_like(o)
        S.sekv_route_attn_noalloc(c, 0, q, p, tau, rbn, on)
        torch.cuda.synchronize()
        assert torch.equal(rb.mask, rbn.mask) and torch.equal(o, on)
    log(f"[append] spans after appends: {[c.info.n_compressed for c in caches]}")
