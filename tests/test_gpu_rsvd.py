"""Randomized truncated SVD build (svd_mode = SEKV_SVD_RANDOMIZED) through the
C ABI, held to the build acceptance bounds against the oracle's exact SVD on
the same stored inputs: singular values within 1e-5 relative, the
reconstruction error within (1 + 1e-4) of the Eckart-Young optimum plus
1e-6 of the span's energy, reconstructions within 1e-4 of the oracle's; and
attention over the randomized cache within the attention tolerance."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.parity import (Inputs, OracleSide, attn_err, log, make_cfg, rel_err, route_from_gpu,
                          to64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def rsvd_cfg(S, wl):
    c = make_cfg(S, wl)
    c.svd_mode = S.SEKV_SVD_RANDOMIZED
    return c


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_128k", dict(n_layers=2, n_tokens=16384 + 77)),
    ("llama32_3b_32k", dict(n_layers=1, n_tokens=8192 + 5)),
    ("llama3_8b_128k", dict(n_layers=1, n_tokens=16384 + 77, kv_dtype="f32")),
])
def test_randomized_svd_bounds_and_attention(S, name, kw):
    wl = synth.workload(name, **kw)
    seed = synth.default_seed(wl)
    log(f"[rsvd] {name} {kw}")
    inp = Inputs(wl, seed)
    cache = S.sekv_build_spans(rsvd_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    exact = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    layers = list(range(wl.n_layers))
    orc = OracleSide(inp, layers, wl.max_rank)
    seg = orc.seg
    n_all = seg.span_len[seg.cspan]
    cand = np.flatnonzero((n_all > 40) & (n_all <= 640))
    assert cand.size > 0
    # an even sample, plus every span of the 256- and 640-row launches
    idx = np.union1d(cand[np.unique(np.linspace(0, cand.size - 1, min(cand.size, 48)).astype(int))],
                     np.flatnonzero((n_all > 128) & (n_all <= 640)))
    log(f"[rsvd] spans checked: {idx.size}, longest {int(n_all[idx].max())} tokens")
    worst = {"sigma": 0.0, "excess": 0.0, "rec": 0.0}
    for layer in layers:
        for kh in range(wl.n_kv_heads):
            gc = orc.groups[layer][kh]
            for i in idx:
                n = int(n_all[i])
                r = int(gc.rank[i])
                b = int(seg.span_start[seg.cspan[i]])
                for kv, fac in ((0, gc.kfac[i]), (1, gc.vfac[i])):
                    x = to64((inp.k if kv == 0 else inp.v)[layer, kh, b:b + n])
                    u, sg, vt = cache.factors(layer, kh, int(i), kv, r, n)
                    rec = ((u.double() * sg.double()) @ vt.double()).numpy()
                    big = fac.sigma > 1e-6 * fac.sigma[0]
                    es = np.max(np.abs(sg.double().numpy()[big] - fac.sigma[big]) / fac.sigma[big])
                    err2 = float(np.linalg.norm(x - rec) ** 2)
                    bound = (1 + 1e-4) * fac.tail2 + 1e-6 * float(np.linalg.norm(x) ** 2)
                    ref = fac.reconstruct()
                    er = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
                    worst["sigma"] = max(worst["sigma"], float(es))
                    worst["excess"] = max(worst["excess"], (err2 - fac.tail2) /
                                          float(np.linalg.norm(x) ** 2))
                    worst["rec"] = max(worst["rec"], er)
                    assert es <= 1e-5, (layer, kh, i, kv, es)
                    assert err2 <= bound, (layer, kh, i, kv, err2, bound)
                    assert er <= 1e-4, (layer, kh, i, kv, er)
    log(f"[rsvd] {idx.size} spans x {len(layers) * wl.n_kv_heads} groups: worst sigma rel "
        f"{worst['sigma']:.1e}, excess error / |K|^2 {worst['excess']:.1e}, "
        f"reconstruction rel {worst['rec']:.1e}")
    # attention over the randomized cache, against the oracle and the exact cache
    tau = torch.full((wl.n_q_heads,), 0.55, device="cuda")
    for layer in layers:
        q = inp.query(0)[layer].contiguous()
        p = inp.p[layer].contiguous()
        outs, rbs = [], []
        for c in (cache, exact):
            rb = S.RouteBuffers.allocate(c)
            o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
            ws = torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda")
            S.sekv_route_attn(c, layer, q, p, tau, rb, o, ws)
            torch.cuda.synchronize()
            outs.append(to64(o))
            rbs.append(rb)
        route = orc.route(layer, to64(q), to64(p), to64(tau), wl.gamma)
        ref = orc.decode(layer, to64(q), route_from_gpu(rbs[0], route.prob, wl.n_kv_heads))
        err = max(attn_err(outs[0][h], ref[h]) for h in range(wl.n_q_heads))
        diff = max(rel_err(outs[0][h], outs[1][h]) for h in range(wl.n_q_heads))
        log(f"[rsvd] layer {layer}: zoomed pairs {int(route.mask.sum())}, attention err {err:.2e}, "
            f"vs exact-SVD cache {diff:.1e}")
        assert err <= 2e-3
        assert diff <= 1e-4


def test_randomized_mode_rejects_high_rank(S):
    wl = synth.workload("tiny")
    inp = Inputs(wl, 1)
    c = rsvd_cfg(S, wl)
    c.max_rank = 64
    with pytest.raises(S.SekvError, match="max_rank"):
        S.sekv_build_spans(c, inp.s, inp.k, inp.v, inp.w, inp.ranks)
