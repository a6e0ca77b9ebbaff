"""Parity of the matched-budget cap (SeKV paper Sec. 3.3, zoom-in decoding)
through the C ABI: sekv_cap_budget (per KV head) and sekv_cap_budget_layer
(one budget and one order for the whole layer) against the oracle's
cap_budget on the same gate values and masks, bit-exact (masks, per-head
lists, unions), and the attention over the capped route against the oracle's
mixed attention."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import Inputs, OracleSide, attn_err, log, make_cfg, rel_err, to64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def clone_route(S, rb):
    return S.RouteBuffers(mask=rb.mask.clone(), list=rb.list.clone(), count=rb.count.clone(),
                          union_list=rb.union_list.clone(), union_count=rb.union_count.clone(),
                          prob=rb.prob.clone())


def gpu_route_as_oracle(rb, sc: int, hq: int, hkv: int) -> O.LayerRoute:
    """The GPU's uncapped route in the oracle's form (its own gate values)."""
    prob = rb.prob.cpu().numpy()[:, :sc].astype(np.float64)
    mask = rb.mask.cpu().numpy().astype(bool)[:, :sc]
    g = hq // hkv
    return O.LayerRoute(prob=prob, mask=mask, lists=[O.compact(mask[h]) for h in range(hq)],
                        unions=[O.union_lists(list(mask[k * g:(k + 1) * g])) for k in range(hkv)])


def assert_route_equals(rb, ref: O.LayerRoute, hq: int, hkv: int):
    sc = ref.mask.shape[1]
    assert np.array_equal(rb.mask.cpu().numpy().astype(bool)[:, :sc], ref.mask)
    cnt, lst = rb.count.cpu().numpy(), rb.list.cpu().numpy()
    for h in range(hq):
        assert lst[h, :cnt[h]].tolist() == ref.lists[h].tolist(), f"head {h}"
    uc, ul = rb.union_count.cpu().numpy(), rb.union_list.cpu().numpy()
    for g in range(hkv):
        assert ul[g, :uc[g]].tolist() == ref.unions[g].tolist(), f"group {g}"


@pytest.mark.parametrize("name,kw,zoom", [
    ("llama3_8b_128k", dict(n_layers=1, n_tokens=20000), 0.3),
    ("qwen25_14b_128k_b4", dict(n_layers=1, n_tokens=9000, batch=1), 0.5),
    ("llama3_8b_128k", dict(n_layers=1, n_tokens=5000, n_q_heads=24, n_kv_heads=8), 0.2),
])
def test_layer_budget_cap_matches_oracle(S, name, kw, zoom):
    """One budget for the layer: the kept (KV head, span) pairs are the longest
    prefix of one order over every KV head's candidates (key descending, ties
    to the lower KV head, then the lower span id)."""
    wl = synth.workload(name, **kw)
    hq, hkv = wl.n_q_heads, wl.n_kv_heads
    log(f"[budget] layer scope {name} {kw} zoom={zoom}")
    inp = Inputs(wl, 10)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    sc = cache.info.n_compressed
    q = inp.query(0)[0].contiguous()
    p = inp.p[0].contiguous()
    # uneven zoom across KV heads: head 0 of every other KV head zooms 3x the share
    prob = orc.route(0, to64(q), to64(p), np.full(hq, 2.0), wl.gamma).prob
    g = wl.group
    share = [min(0.9, zoom * (3.0 if (h // g) % 2 == 0 and h % g == 0 else 1.0)) for h in range(hq)]
    tau = torch.tensor([float(np.quantile(prob[h], 1.0 - share[h])) for h in range(hq)],
                       dtype=torch.float32).cuda()
    base = S.RouteBuffers.allocate(cache, with_prob=True)
    S.sekv_route(cache, 0, q, p, tau, base)
    torch.cuda.synchronize()
    uncapped = gpu_route_as_oracle(base, sc, hq, hkv)
    n = orc.seg.span_len[orc.seg.cspan].astype(np.int64)
    total = sum(int(n[u].sum()) for u in uncapped.unions)
    assert total > 0
    budgets = sorted({0, 1, total // 5, total // 2, total - 1, total, 10 ** 12})
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    for budget in budgets:
        rb = clone_route(S, base)
        S.sekv_cap_budget(cache, rb, budget, scope="layer")
        o = torch.zeros(hq, wl.head_dim, device="cuda")
        S.sekv_decode_attn(cache, 0, q, rb, o, ws)
        torch.cuda.synchronize()
        ref = O.cap_budget(uncapped, orc.seg, hkv, budget, scope="layer")
        assert_route_equals(rb, ref, hq, hkv)
        assert torch.equal(rb.prob, base.prob)
        kept = [int(n[u].sum()) for u in ref.unions]
        assert sum(kept) <= budget
        out = orc.decode(0, to64(q), ref)
        worst = max(attn_err(to64(o)[h], out[h]) for h in range(hq))
        log(f"[budget] layer budget={budget} kept tokens per group {kept} (total {total}) "
            f"zoomed pairs {int(ref.mask.sum())} err={worst:.2e}")
        assert worst <= TOL[wl.kv_dtype]
        if budget >= total:
            assert torch.equal(rb.mask, base.mask) and torch.equal(rb.count, base.count)
        if budget == 0:
            assert int(rb.count.sum()) == 0 and int(rb.union_count.sum()) == 0


@pytest.mark.parametrize("hq,hkv", [(64, 64), (256, 128)])
def test_layer_budget_cap_many_kv_heads(S, hq, hkv):
    """The layer scope with 64 and 128 KV heads, whose decisions are spread
    over 4 and 2 workgroups per KV head (8 up to 32 KV heads), each taking a
    share of its KV head's candidates: masks, per-head lists and unions
    against the oracle's cap on the GPU's own route, at budgets across the
    range (the attention over capped routes is checked above)."""
    wl = synth.workload("tiny", n_q_heads=hq, n_kv_heads=hkv, n_tokens=2048)
    log(f"[budget] layer scope, {hq}/{hkv} heads")
    inp = Inputs(wl, 14)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank, with_factors=False)
    sc = cache.info.n_compressed
    assert sc > 0
    q = inp.query(0)[0].contiguous()
    p = inp.p[0].contiguous()
    prob = orc.route(0, to64(q), to64(p), np.full(hq, 2.0), wl.gamma).prob
    g = wl.group
    # uneven zoom: every third KV head's heads zoom 40% of the spans, the rest 10%
    share = [0.4 if (h // g) % 3 == 0 else 0.1 for h in range(hq)]
    tau = torch.tensor([float(np.quantile(prob[h], 1.0 - share[h])) for h in range(hq)],
                       dtype=torch.float32).cuda()
    base = S.RouteBuffers.allocate(cache, with_prob=True)
    S.sekv_route(cache, 0, q, p, tau, base)
    torch.cuda.synchronize()
    uncapped = gpu_route_as_oracle(base, sc, hq, hkv)
    n = orc.seg.span_len[orc.seg.cspan].astype(np.int64)
    total = sum(int(n[u].sum()) for u in uncapped.unions)
    assert total > 0
    for budget in sorted({0, total // 7, total // 3, total - 1, total}):
        rb = clone_route(S, base)
        S.sekv_cap_budget(cache, rb, budget, scope="layer")
        torch.cuda.synchronize()
        ref = O.cap_budget(uncapped, orc.seg, hkv, budget, scope="layer")
        assert_route_equals(rb, ref, hq, hkv)
        kept = sum(int(n[u].sum()) for u in ref.unions)
        assert kept <= budget
        log(f"[budget] {hkv} KV heads, layer budget={budget}: kept {kept} of {total} tokens, "
            f"zoomed pairs {int(ref.mask.sum())}")


@pytest.mark.parametrize("name,kw,zoom", [
    ("tiny", dict(), None),
    ("llama3_8b_128k", dict(n_layers=1, n_tokens=20000), 0.3),
    ("qwen25_14b_128k_b4", dict(n_layers=1, n_tokens=9000, batch=1), 0.5),
])
def test_budget_cap_matches_oracle(S, name, kw, zoom):
    wl = synth.workload(name, **kw)
    hq, hkv = wl.n_q_heads, wl.n_kv_heads
    log(f"[budget] {name} {kw} zoom={zoom}")
    inp = Inputs(wl, 9)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    sc = cache.info.n_compressed
    q = inp.query(0)[0].contiguous()
    p = inp.p[0].contiguous()
    if zoom is None:
        tau = synth.tau_uniform(wl, 9, device="cuda")[0].contiguous()
    else:
        prob = orc.route(0, to64(q), to64(p), np.full(hq, 2.0), wl.gamma).prob
        tau = torch.tensor([float(np.quantile(prob[h], 1.0 - zoom)) for h in range(hq)],
                           dtype=torch.float32).cuda()
    base = S.RouteBuffers.allocate(cache, with_prob=True)
    S.sekv_route(cache, 0, q, p, tau, base)
    torch.cuda.synchronize()
    uncapped = gpu_route_as_oracle(base, sc, hq, hkv)
    n = orc.seg.span_len[orc.seg.cspan].astype(np.int64)
    totals = [int(n[u].sum()) for u in uncapped.unions]
    assert max(totals) > 0
    budgets = sorted({0, 1, int(np.median(totals)) // 3, int(np.median(totals)) // 2,
                      max(totals) - 1, max(totals), 10 ** 12})
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    for budget in budgets:
        rb = clone_route(S, base)
        S.sekv_cap_budget(cache, rb, budget)
        o = torch.zeros(hq, wl.head_dim, device="cuda")
        S.sekv_decode_attn(cache, 0, q, rb, o, ws)
        torch.cuda.synchronize()
        ref = O.cap_budget(uncapped, orc.seg, hkv, budget)
        assert_route_equals(rb, ref, hq, hkv)
        assert torch.equal(rb.prob, base.prob)
        kept = [int(n[u].sum()) for u in ref.unions]
        assert all(k <= budget for k in kept)
        out = orc.decode(0, to64(q), ref)
        worst = max(attn_err(to64(o)[h], out[h]) for h in range(hq))
        if hkv == 1:   # one KV head: the layer scope is the per-KV-head cap
            rl = clone_route(S, base)
            S.sekv_cap_budget(cache, rl, budget, scope="layer")
            torch.cuda.synchronize()
            assert torch.equal(rl.mask, rb.mask) and torch.equal(rl.union_count, rb.union_count)
        log(f"[budget] budget={budget} kept tokens per group {kept} (of {totals}) "
            f"zoomed pairs {int(ref.mask.sum())} err={worst:.2e}")
        assert worst <= TOL[wl.kv_dtype]
        if budget >= max(totals):
            for a, b in ((rb.mask, base.mask), (rb.count, base.count),
                         (rb.union_count, base.union_count)):
                assert torch.equal(a, b)
        if budget == 0:
            assert int(rb.count.sum()) == 0 and int(rb.union_count.sum()) == 0


def test_budget_cap_after_single_launch_and_repeat(S):
    """The route written by the single-launch call caps the same way as the
    two-call route; capping twice with the same budget changes nothing more;
    reruns are bit-identical."""
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=12000)
    log("[budget] single-launch route, idempotence, repeat")
    inp = Inputs(wl, 2)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    q, p = inp.query(3)[0].contiguous(), inp.p[0].contiguous()
    tau = torch.full((wl.n_q_heads,), 0.55, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    a = S.RouteBuffers.allocate(cache, with_prob=True)
    b = S.RouteBuffers.allocate(cache, with_prob=True)
    o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
    S.sekv_route(cache, 0, q, p, tau, a)
    S.sekv_route_attn(cache, 0, q, p, tau, b, o, ws)
    torch.cuda.synchronize()
    assert int(a.union_count.sum()) > 0
    budget = 500
    outs = []
    for rb in (a, b):
        S.sekv_cap_budget(cache, rb, budget)
        once = clone_route(S, rb)
        S.sekv_cap_budget(cache, rb, budget)
        torch.cuda.synchronize()
        for x, y in ((rb.mask, once.mask), (rb.count, once.count),
                     (rb.union_count, once.union_count), (rb.union_list, once.union_list)):
            assert torch.equal(x, y)
        oo = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
        S.sekv_decode_attn(cache, 0, q, rb, oo, ws)
        torch.cuda.synchronize()
        outs.append(oo)
    assert torch.equal(a.mask, b.mask) and torch.equal(a.union_count, b.union_count)
    assert torch.equal(outs[0], outs[1])


def test_budget_cap_rejects_bad_arguments(S):
    wl = synth.workload("tiny")
    inp = Inputs(wl, 1)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    rb = S.RouteBuffers.allocate(cache, with_prob=False)
    with pytest.raises(ValueError, match="gate values"):
        S.sekv_cap_budget(cache, rb, 10)
    rb = S.RouteBuffers.allocate(cache, with_prob=True)
    with pytest.raises(S.SekvError, match="budget_tokens"):
        S.sekv_cap_budget(cache, rb, -1)
    st = S.RouteBuffers.allocate(cache, with_prob=False).struct()
    import ctypes
    assert S.lib().sekv_cap_budget(cache.handle, ctypes.byref(st), 5, None) == S.SEKV_ERR_INVALID
    assert b"prob" in S.lib().sekv_last_error()


def test_budget_cap_large_union(S):
    """A union of thousands of spans (short spans, every span zoomed), so the
    cap runs its multi-tile comparison and multi-block compaction, per KV head
    and for the layer: masks, lists and unions bit-exact against the oracle's
    cap on the GPU's gates."""
    wl = synth.workload("tiny", n_tokens=40000, min_span_len=1)
    hq, hkv = wl.n_q_heads, wl.n_kv_heads
    inp = Inputs(wl, 4)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    seg = O.segment(to64(inp.s), wl.window, wl.alpha, wl.min_span_len)
    sc = cache.info.n_compressed
    assert sc == seg.n_compressed and sc > 4096
    q = inp.query(0)[0].contiguous()
    # every span zoomed by head 0, the others above their median gate
    base = S.RouteBuffers.allocate(cache, with_prob=True)
    S.sekv_route(cache, 0, q, inp.p[0].contiguous(), torch.full((hq,), 2.0, device="cuda"), base)
    torch.cuda.synchronize()
    med = base.prob[:, :sc].median(dim=1).values.float()
    tau = torch.where(torch.arange(hq, device="cuda") == 0, torch.full_like(med, -1.0), med)
    S.sekv_route(cache, 0, q, inp.p[0].contiguous(), tau.contiguous(), base)
    torch.cuda.synchronize()
    uncapped = gpu_route_as_oracle(base, sc, hq, hkv)
    assert uncapped.unions[0].size == sc
    n = seg.span_len[seg.cspan].astype(np.int64)
    total = int(n.sum())
    log(f"[budget] large union: {sc} spans, {total} tokens")
    for budget in (total // 5, total // 2, total - 1):
        rb = clone_route(S, base)
        S.sekv_cap_budget(cache, rb, budget)
        torch.cuda.synchronize()
        ref = O.cap_budget(uncapped, seg, hkv, budget)
        assert_route_equals(rb, ref, hq, hkv)
        # the layer scope over more candidates than one LDS tile holds
        rl = clone_route(S, base)
        S.sekv_cap_budget(cache, rl, budget, scope="layer")
        torch.cuda.synchronize()
        assert_route_equals(rl, O.cap_budget(uncapped, seg, hkv, budget, scope="layer"), hq, hkv)
        log(f"[budget] budget={budget}: kept {ref.unions[0].size} of {sc} spans")
