"""The HBM residency cache of host-tier factors (sekv_set_residency) through
the C ABI: routes and outputs against the CPU oracle (outputs over the GPU's
zoom mask, cache hits and misses alike), bit-identical to the host tier
without the cache (a block is the same bytes wherever it is read from) and
equal to the device tier up to the float32 merge order; a span zoomed again in
a later call of the same layer is read from the cache; set conflicts, tiny
capacities and blocks larger than a slot fall back to staging and stay
correct."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.parity import (Inputs, OracleSide, attn_err, compare_route, log, make_cfg,
                          route_from_gpu, to64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


@pytest.fixture(scope="module")
def setup(S):
    wl = synth.workload("llama3_8b_128k", n_layers=2, n_tokens=9000)
    inp = Inputs(wl, 4)
    dev = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    host = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    res = S.sekv_build_spans(make_cfg(S, wl, tier="host"), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    orc = OracleSide(inp, [0, 1], wl.max_rank)
    return wl, inp, dev, host, res, orc


def attend(S, cache, layer, q, p, tau, side):
    rb = S.RouteBuffers.allocate(cache)
    o = torch.zeros(cache.cfg.n_q_heads, cache.cfg.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(cache, layer, q.contiguous(), p.contiguous(), tau, rb, o, ws,
                      fetch_stream=side)
    torch.cuda.synchronize()
    return rb, o


def union_bytes(cache, rb, layer):
    sp = cache.spans()
    clen = sp["span_len"][sp["cspan"].long()].numpy().astype(np.int64)
    tot, n = 0, 0
    for g in range(cache.cfg.n_kv_heads):
        gd = cache.group_data(layer, g)
        rk, rv = gd[3].numpy().astype(np.int64), gd[4].numpy().astype(np.int64)
        ids = rb.union_list[g, :int(rb.union_count[g])].cpu().numpy()
        tot += int((4 * (rk[ids] + rv[ids]) * (clen[ids] + 128 + 1)).sum())
        n += ids.size
    return n, tot


def test_residency_rejects_device_tier_and_bad_sizes(S, setup):
    _, _, dev, _, res, _ = setup
    with pytest.raises(S.SekvError, match="host-tier"):
        dev.set_residency(1 << 20)
    with pytest.raises(S.SekvError, match="below one slot"):
        res.set_residency(1000, 64 * 1024)
    with pytest.raises(S.SekvError, match="residency sets"):
        res.set_residency((1 << 31) * 256, 256)   # 2^31 sets of 256 bytes, before any allocation
    with pytest.raises(S.SekvError, match="not enabled"):
        res.residency_stats()


@pytest.mark.parametrize("capacity,slot", [(256 << 20, 64 << 10), (4 * (64 << 10), 64 << 10),
                                           (64 << 20, 4 << 10)])
def test_residency_outputs_and_hits(S, setup, capacity, slot):
    wl, inp, dev, host, res, orc = setup
    log(f"[residency] capacity={capacity} slot={slot}")
    res.set_residency(capacity, slot)
    side = torch.cuda.Stream()
    tau = torch.full((wl.n_q_heads,), 0.7, device="cuda")
    calls = [(0, 1), (1, 1), (0, 1), (1, 2), (0, 1)]   # (layer, query step); repeats hit
    seen = {}
    for layer, step in calls:
        q = inp.query(step)[layer]
        p = inp.p[layer]
        rbh, oh = attend(S, host, layer, q, p, tau, side)
        rbr, orr = attend(S, res, layer, q, p, tau, side)
        rbd, od = attend(S, dev, layer, q, p, tau, side)
        st = res.residency_stats(reset=True)
        n, nbytes = union_bytes(res, rbr, layer)
        assert torch.equal(rbr.mask, rbh.mask) and torch.equal(rbr.union_count, rbh.union_count)
        assert torch.equal(orr, oh), "residency changed the output"
        err = float((orr - od).abs().max() / od.abs().max())
        assert err <= 1e-6
        # against the oracle: the route outside the tie band, every head's
        # output over the GPU's mask
        route = orc.route(layer, to64(q), to64(p), to64(tau), wl.gamma)
        compare_route(rbr, route, to64(tau), wl)
        ref = orc.decode(layer, to64(q), route_from_gpu(rbr, route.prob, wl.n_kv_heads))
        err_o = max(attn_err(to64(orr)[h], ref[h]) for h in range(wl.n_q_heads))
        assert err_o <= 2e-3, err_o
        assert st["hit_blocks"] + st["fetched_blocks"] == n
        assert st["hit_bytes"] + st["fetched_bytes"] == nbytes
        key = (layer, step)
        if slot < 8 * 1024:
            assert st["hit_blocks"] == 0        # no block fits a 4 KB slot
        elif key in seen and capacity >= (256 << 20):
            # the same union again, nothing else evicted it in between beyond
            # set conflicts: most blocks are hits
            assert st["hit_blocks"] >= 0.5 * n, st
        if key not in seen and capacity >= (256 << 20) and (layer, step) == (0, 1):
            assert st["hit_blocks"] == 0
        seen[key] = st
        log(f"[residency] layer={layer} step={step} union={n} hits={st['hit_blocks']} "
            f"fetched={st['fetched_blocks']} fetched MB={st['fetched_bytes'] / 1e6:.2f} "
            f"err vs oracle={err_o:.1e} rel diff vs device={err:.1e}")
    res.set_residency(0, 0)
    with pytest.raises(S.SekvError, match="not enabled"):
        res.residency_stats()
    rbr, orr = attend(S, res, 0, inp.query(1)[0], inp.p[0], tau, side)
    rbh, oh = attend(S, host, 0, inp.query(1)[0], inp.p[0], tau, side)
    assert torch.equal(orr, oh)
