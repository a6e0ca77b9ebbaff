"""The allocation-free route + attention (sekv_route_attn_noalloc) through the
C ABI: on two calls in a row, the second on a smaller cache (so the shared
scratch holds the first call's larger contents), its routes and outputs equal
sekv_route_attn's with a caller workspace bit for bit (the same kernels write
and merge the same partial slots); a host-tier cache too; a cache whose
partial states exceed the scratch is rejected before anything runs."""
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.parity import Inputs, log, make_cfg

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


def both_calls(S, cache, inp, layer, tau, side=None):
    q = inp.query(3)[layer].contiguous()
    p = inp.p[layer].contiguous()
    rb_w = S.RouteBuffers.allocate(cache, with_prob=True)
    o_w = torch.zeros(cache.cfg.n_q_heads, cache.cfg.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn(cache, layer, q, p, tau, rb_w, o_w, ws, fetch_stream=side)
    rb_n = S.RouteBuffers.allocate(cache, with_prob=True)
    o_n = torch.full_like(o_w, float("nan"))
    S.sekv_route_attn_noalloc(cache, layer, q, p, tau, rb_n, o_n, fetch_stream=side)
    torch.cuda.synchronize()
    return rb_w, o_w, rb_n, o_n


def same_route(a, b):
    assert torch.equal(a.mask, b.mask) and torch.equal(a.prob, b.prob)
    assert torch.equal(a.count, b.count) and torch.equal(a.union_count, b.union_count)
    for h in range(a.count.numel()):
        assert torch.equal(a.list[h, :int(a.count[h])], b.list[h, :int(b.count[h])])
    for g in range(a.union_count.numel()):
        n = int(a.union_count[g])
        assert torch.equal(a.union_list[g, :n], b.union_list[g, :n])


def test_noalloc_equals_workspace_call_larger_then_smaller(S):
    tau = None
    for n_tokens, tier in ((24000, "device"), (3000, "device"), (9000, "host")):
        wl = synth.workload("llama3_8b_128k", n_layers=2, n_tokens=n_tokens)
        log(f"[noalloc] {tier} tier, {n_tokens} tokens")
        inp = Inputs(wl, 13)
        cache = S.sekv_build_spans(make_cfg(S, wl, tier=tier), inp.s, inp.k, inp.v, inp.w,
                                   inp.ranks)
        assert cache.workspace_bytes() <= S.SEKV_NOALLOC_SCRATCH_BYTES
        tau = torch.full((wl.n_q_heads,), 0.6, device="cuda")
        side = torch.cuda.Stream() if tier == "host" else None
        for layer in range(wl.n_layers):
            rb_w, o_w, rb_n, o_n = both_calls(S, cache, inp, layer, tau, side)
            assert int(rb_w.union_count.sum()) > 0
            same_route(rb_w, rb_n)
            assert torch.equal(o_w, o_n), "allocation-free output differs"
            log(f"[noalloc] layer {layer}: workspace {cache.workspace_bytes()} B, zoomed pairs "
                f"{int(rb_n.mask.sum())}, outputs bit-identical")


def test_noalloc_rejects_caches_beyond_its_scratch(S):
    # 8 query heads per KV head and ~4500 compressed spans: the partial states
    # need more than the scratch holds
    wl = synth.workload("llama3_8b_128k", n_layers=1, n_tokens=400000, n_q_heads=64,
                        n_kv_heads=8)
    log("[noalloc] oversized cache")
    inp = Inputs(wl, 14)
    cache = S.sekv_build_spans(make_cfg(S, wl), inp.s, inp.k, inp.v, inp.w, inp.ranks)
    assert cache.workspace_bytes() > S.SEKV_NOALLOC_SCRATCH_BYTES
    rb = S.RouteBuffers.allocate(cache)
    o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
    tau = torch.full((wl.n_q_heads,), 0.6, device="cuda")
    with pytest.raises(S.SekvError, match="scratch"):
        S.sekv_route_attn_noalloc(cache, 0, inp.query(0)[0].contiguous(), inp.p[0].contiguous(),
                                  tau, rb, o)
