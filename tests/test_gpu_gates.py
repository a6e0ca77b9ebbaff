"""Soft-gated reconstruction (Eq. 8) through the C ABI: sekv_apply_gates
repacks the factor pool with the kept components and gate-scaled singular
values.  Against the oracle's gate_factors on the same gates: ranks exact,
factors by reconstruction and singular values, attention over the gated cache
within the attention tolerance; all-one gates change nothing bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import Inputs, OracleSide, log, make_cfg, rel_err, to64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def layer_out(S, cache, q, p, tau):
    rb = S.RouteBuffers.allocate(cache)
    o = torch.zeros(cache.cfg.n_q_heads, cache.cfg.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(cache, 0, q.contiguous(), p.contiguous(), tau.contiguous(), rb, o, ws)
    torch.cuda.synchronize()
    return rb, o


@pytest.mark.parametrize("name,kw,eps", [("tiny", dict(), 0.3),
                                         ("llama3_8b_128k", dict(n_layers=1, n_tokens=9000), 0.5)])
def test_gates_match_oracle(S, name, kw, eps):
    wl = synth.workload(name, **kw)
    log(f"[gates] {name} {kw} eps={eps}")
    inp = Inputs(wl, 7)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0], wl.max_rank)
    sc = cache.info.n_compressed
    before = cache.info.factor_bytes
    gates = synth.span_gates(wl, 7, sc, device="cuda")
    S.sekv_apply_gates(cache, gates, eps)
    gh = gates.cpu().double().numpy()
    worst_rec = 0.0
    for kh in range(wl.n_kv_heads):
        gg = O.gate_group(orc.groups[0][kh], gh[0, kh], eps)
        orc.groups[0][kh] = gg
        rk = cache.group_data(0, kh)[3].numpy()
        assert rk.tolist() == gg.rank.tolist()
        idx = np.unique(np.linspace(0, sc - 1, min(sc, 40)).astype(int))
        for i in idx:
            n = int(orc.seg.span_len[orc.seg.cspan[i]])
            r = int(gg.rank[i])
            for kv, fac in ((0, gg.kfac[i]), (1, gg.vfac[i])):
                u, sg, vt = cache.factors(0, kh, int(i), kv, r, n)
                rec = (u.double() * sg.double()) @ vt.double()
                ref = fac.reconstruct()
                worst_rec = max(worst_rec, float(np.linalg.norm(rec.numpy() - ref) /
                                                 max(np.linalg.norm(ref), 1e-300)))
                big = np.abs(fac.sigma) > 1e-6 * np.max(np.abs(fac.sigma))
                assert np.allclose(sg.double().numpy()[big], fac.sigma[big], rtol=1e-5, atol=0)
    assert worst_rec <= 1e-4, worst_rec
    assert cache.info.factor_bytes < before
    # attention over the gated cache, about a third of the spans zoomed
    q = inp.query(0)[0]
    p = inp.p[0]
    prob = orc.route(0, to64(q), to64(p), np.full(wl.n_q_heads, 2.0), wl.gamma).prob
    tau = torch.tensor([float(np.quantile(prob[h], 0.67)) for h in range(wl.n_q_heads)],
                       dtype=torch.float32).cuda()
    rb, o = layer_out(S, cache, q, p, tau)
    route = orc.route(0, to64(q), to64(p), to64(tau), wl.gamma)
    tie = np.abs(route.prob - to64(tau)[:, None]) < 1e-5
    ref = orc.decode(0, to64(q), route)
    worst = max(rel_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads) if not tie[h].any())
    log(f"[gates] factor bytes {before} -> {cache.info.factor_bytes}, rec err {worst_rec:.1e}, "
        f"zoomed pairs {int(route.mask.sum())}, attention err {worst:.2e}")
    assert worst <= TOL[wl.kv_dtype]


def test_unit_gates_change_nothing_and_host_tier_is_rejected(S):
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=9000)
    inp = Inputs(wl, 8)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    q, p = inp.query(0)[0], inp.p[0]
    tau = torch.full((wl.n_q_heads,), 0.55, device="cuda")
    _, o0 = layer_out(S, cache, q, p, tau)
    before = cache.info.factor_bytes
    ones = torch.ones(1, wl.n_kv_heads, cache.info.n_compressed, wl.max_rank, device="cuda")
    S.sekv_apply_gates(cache, ones, 0.5)
    _, o1 = layer_out(S, cache, q, p, tau)
    assert cache.info.factor_bytes == before
    assert torch.equal(o0, o1)
    bad = ones.clone()
    bad[0, 0, 0, 0] = 1.5
    with pytest.raises(S.SekvError, match="outside"):
        S.sekv_apply_gates(cache, bad, 0.5)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    with pytest.raises(S.SekvError, match="host memory"):
        S.sekv_apply_gates(host, ones, 0.5)
