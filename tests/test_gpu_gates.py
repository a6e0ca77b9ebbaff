"""Soft-gated reconstruction (Eq. 8) through the C ABI: sekv_apply_gates
repacks the factor pool with each matrix's kept components and gate-scaled
singular values, keys gated by their own gates and values by theirs (the SeKV
page, Sec. 3.2: the value matrix has gates and factors of its own).  Against
the oracle's gate_group on the same gates: key and value ranks exact, factors
by reconstruction and singular values, attention over the gated cache within
the attention tolerance (with the GPU's zoom mask, so every head is
compared); all-one gates change nothing bit for bit, and value-only gates
leave the key factors bit-identical."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import (Inputs, OracleSide, attn_err, compare_group, log, make_cfg,
                          route_from_gpu, to64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def layer_out(S, cache, q, p, tau, with_prob=False):
    rb = S.RouteBuffers.allocate(cache, with_prob=with_prob)
    o = torch.zeros(cache.cfg.n_q_heads, cache.cfg.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(cache, 0, q.contiguous(), p.contiguous(), tau.contiguous(), rb, o, ws)
    torch.cuda.synchronize()
    return rb, o


@pytest.mark.parametrize("name,kw,eps", [("tiny", dict(), 0.3),
                                         ("llama3_8b_128k", dict(n_layers=1, n_tokens=9000), 0.5),
                                         ("llama3_8b_128k", dict(n_layers=1, n_tokens=5000,
                                                                 n_q_heads=24, n_kv_heads=4), 0.4)])
def test_gates_match_oracle(S, name, kw, eps):
    wl = synth.workload(name, **kw)
    log(f"[gates] {name} {kw} eps={eps}")
    inp = Inputs(wl, 7)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    sc = cache.info.n_compressed
    before = cache.info.factor_bytes
    kg = synth.span_gates(wl, 7, sc, "k", device="cuda")
    vg = synth.span_gates(wl, 7, sc, "v", device="cuda")
    S.sekv_apply_gates(cache, kg, vg, eps)
    kh_, vh_ = kg.cpu().double().numpy(), vg.cpu().double().numpy()
    n_diff = 0
    worst_rec = 0.0
    for kh in range(wl.n_kv_heads):
        gg = O.gate_group(orc.groups[0][kh], kh_[0, kh], vh_[0, kh], eps)
        orc.groups[0][kh] = gg
        n_diff += int((gg.rank != gg.vrank).sum())
        # ranks exact for keys and values, factors by reconstruction (1e-4)
        # and singular values (1e-5) on sampled spans of each matrix
        _, rec = compare_group(cache, orc, 0, kh, n_factor_checks=40)
        worst_rec = max(worst_rec, rec)
    assert n_diff > 0, "the gates should leave some spans with different key and value ranks"
    assert cache.info.factor_bytes < before
    # attention over the gated cache, about a third of the spans zoomed
    q = inp.query(0)[0]
    p = inp.p[0]
    prob = orc.route(0, to64(q), to64(p), np.full(wl.n_q_heads, 2.0), wl.gamma).prob
    tau = torch.tensor([float(np.quantile(prob[h], 0.67)) for h in range(wl.n_q_heads)],
                       dtype=torch.float32).cuda()
    rb, o = layer_out(S, cache, q, p, tau)
    route = orc.route(0, to64(q), to64(p), to64(tau), wl.gamma)
    ref = orc.decode(0, to64(q), route_from_gpu(rb, route.prob, wl.n_kv_heads))
    worst = max(attn_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads))
    log(f"[gates] factor bytes {before} -> {cache.info.factor_bytes}, spans with rK != rV "
        f"{n_diff}, rec err {worst_rec:.1e}, zoomed pairs {int(route.mask.sum())}, "
        f"attention err {worst:.2e}")
    assert worst <= TOL[wl.kv_dtype]


def test_value_gates_leave_keys_and_unit_gates_change_nothing(S):
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=9000)
    inp = Inputs(wl, 8)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    q, p = inp.query(0)[0], inp.p[0]
    tau = torch.full((wl.n_q_heads,), 0.55, device="cuda")
    _, o0 = layer_out(S, cache, q, p, tau)
    before = cache.info.factor_bytes
    sc = cache.info.n_compressed
    ones = torch.ones(1, wl.n_kv_heads, sc, wl.max_rank, device="cuda")
    S.sekv_apply_gates(cache, ones, ones, 0.5)
    _, o1 = layer_out(S, cache, q, p, tau)
    assert cache.info.factor_bytes == before
    assert torch.equal(o0, o1)
    # value gates only: every key factor stays bit for bit, value ranks drop
    spans = [0, sc // 3, sc - 1]
    kfac = {j: cache.factors(0, 1, j, 0, int(cache.group_data(0, 1)[3][j]),
                             int(cache.spans()["span_len"][cache.spans()["cspan"][j]]))
            for j in spans}
    vg = synth.span_gates(wl, 8, sc, "v", device="cuda")
    S.sekv_apply_gates(cache, ones, vg, 0.5)
    rk, rv = cache.group_data(0, 1)[3:5]
    assert int((rv < rk).sum()) > 0 and torch.all(rv <= rk)
    for j in spans:
        u, sg, vt = cache.factors(0, 1, j, 0, int(rk[j]), kfac[j][0].shape[0])
        assert torch.equal(u, kfac[j][0]) and torch.equal(sg, kfac[j][1])
        assert torch.equal(vt, kfac[j][2])
    bad = ones.clone()
    bad[0, 0, 0, 0] = 1.5
    with pytest.raises(S.SekvError, match="value gate.*outside"):
        S.sekv_apply_gates(cache, ones, bad, 0.5)
    with pytest.raises(S.SekvError, match="key gate.*outside"):
        S.sekv_apply_gates(cache, bad, ones, 0.5)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    with pytest.raises(S.SekvError, match="host memory"):
        S.sekv_apply_gates(host, ones, ones, 0.5)
