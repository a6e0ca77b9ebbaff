"""The batch-4 Qwen2.5-14B workload (40 query / 8 KV heads, G = 5) at a
context of 32768 tokens per sequence, through the batched call the bench
times: for sampled (sequence, layer, KV head) groups the oracle rebuilds the
group from the same inputs and checks its stored representation, the zoom
masks and lists of its query heads (outside the tie band) and every head's
output (over the GPU's mask); and the sweep's 100% point at full rank, which
is dense attention over all 32768 tokens (torch SDPA on the CPU, float64)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.conftest import gpu_available
from tests.parity import Inputs, attn_err, compare_group, compare_spans, log, make_cfg, to64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BF16 = 2e-3
CTX = 32768


@pytest.fixture(scope="module")
def S():
    import compressed_kv_attention_sekv_amd as S
    S.lib()
    return S


@pytest.fixture(scope="module")
def batch4(S):
    base = synth.workload("qwen25_14b_128k_b4", n_layers=2, n_tokens=CTX)
    seed = synth.default_seed(base)
    log(f"[batch4] building 4 sequences of {CTX} tokens")
    inps, caches = [], []
    for i in range(4):
        inp = Inputs(base, seed, seq=i)
        inps.append(inp)
        caches.append(S.sekv_build_spans(make_cfg(S, base), inp.s, inp.k, inp.v, inp.w,
                                         inp.ranks))
    return base, inps, caches


def gpu_tau(S, cache, layer, q, p, share):
    """Per-head thresholds at the (1 - share) quantile of the library's own gate
    values for this query (thresholds are inputs of the step)."""
    rb = S.RouteBuffers.allocate(cache, with_prob=True)
    S.sekv_route(cache, layer, q.contiguous(), p.contiguous(),
                 torch.full((cache.cfg.n_q_heads,), 2.0, device="cuda"), rb)
    torch.cuda.synchronize()
    return torch.quantile(rb.prob.float(), 1.0 - share, dim=1).float().contiguous()


@pytest.mark.parametrize("layer", [0, 1])
def test_batch4_32k_sampled_groups(S, batch4, layer):
    base, inps, caches = batch4
    Hq, d, G = base.n_q_heads, base.head_dim, base.group
    p = inps[0].p[layer].contiguous()   # one model layer's projections, shared
    qs = [inp.query(20 + layer)[layer].contiguous() for inp in inps]
    tau = gpu_tau(S, caches[0], layer, qs[0], p, 0.10)   # ~10% of spans per head
    rbs = [S.RouteBuffers.allocate(c, with_prob=True) for c in caches]
    outs = [torch.zeros(Hq, d, device="cuda") for _ in caches]
    wss = [torch.empty(c.workspace_bytes(), dtype=torch.uint8, device="cuda") for c in caches]
    S.sekv_route_attn_batch(caches, layer, qs, p, tau, rbs, outs, wss)
    torch.cuda.synchronize()
    for i, kv_head in ((0, 1), (1, 6), (2, 3), (3, 7)):
        inp, cache, rb = inps[i], caches[i], rbs[i]
        s64 = to64(inp.s)
        seg = O.segment(s64, base.window, base.alpha, base.min_span_len)
        w = to64(inp.w[layer])
        heads = list(range(kv_head * G, kv_head * G + G))
        gc = O.build_group(seg, s64, to64(inp.k[layer, kv_head]), to64(inp.v[layer, kv_head]),
                           {h: w[h] for h in heads}, inp.ranks[layer, kv_head].cpu().numpy(),
                           base.kv_dtype, base.max_rank)

        class One:
            pass
        orc = One()
        orc.wl, orc.seg, orc.groups = base, seg, {layer: {kv_head: gc}}
        compare_spans(cache, orc)
        nmis, rec = compare_group(cache, orc, layer, kv_head, n_factor_checks=8)
        qn, tn, pr = to64(qs[i]), to64(tau), to64(p)
        h0, h1 = heads[0], heads[-1] + 1
        route = O.route_layer(qn[h0:h1], pr[h0:h1], tn[h0:h1],
                              {k: gc.summary[h] for k, h in enumerate(heads)}, seg, base.gamma, 1)
        mask = rb.mask.cpu().numpy().astype(bool)[h0:h1, :seg.n_compressed]
        tie = np.abs(route.prob - tn[h0:h1, None]) < 1e-5
        assert np.array_equal(mask[~tie], route.mask[~tie])
        assert np.max(np.abs(rb.prob.cpu().numpy()[h0:h1, :seg.n_compressed] - route.prob)) <= 1e-12
        if not tie.any():
            cnt, lst = rb.count.cpu().numpy(), rb.list.cpu().numpy()
            for k, h in enumerate(heads):
                assert lst[h, :cnt[h]].tolist() == route.lists[k].tolist()
            uc, ul = rb.union_count.cpu().numpy(), rb.union_list.cpu().numpy()
            assert ul[kv_head, :uc[kv_head]].tolist() == route.unions[0].tolist()
        og = to64(outs[i])
        err = max(attn_err(og[h], O.mixed_attention(qn[h], gc, seg, mask[k]))
                  for k, h in enumerate(heads))
        log(f"[batch4] seq={i} layer={layer} kv_head={kv_head}: spans={seg.n_compressed} "
            f"zoom={mask.mean():.3f} union={int(rb.union_count[kv_head])} ties={int(tie.sum())} "
            f"storage mismatches={nmis} rec={rec:.1e} attention err={err:.2e}")
        assert err <= TOL_BF16


def test_batch4_32k_full_rank_all_zoomed_is_dense(S):
    """The sweep's 100% point at full rank: every span zoomed with every
    component kept gives textbook attention over all 32768 tokens."""
    wl = synth.workload("qwen25_14b_128k_b4", n_layers=1, n_tokens=CTX, batch=1)
    log("[batch4] full rank, every span zoomed, 32768 tokens")
    inp = Inputs(wl, 9)
    cache = S.sekv_build_spans(make_cfg(S, wl, max_rank=128), inp.s, inp.k, inp.v, inp.w,
                               torch.full_like(inp.ranks, 128))
    q = inp.query(0)[0].contiguous()
    rb = S.RouteBuffers.allocate(cache)
    o = torch.zeros(wl.n_q_heads, wl.head_dim, device="cuda")
    ws = torch.empty(cache.workspace_bytes(), dtype=torch.uint8, device="cuda")
    S.sekv_route_attn_batch([cache], 0, [q], inp.p[0].contiguous(),
                            torch.full((wl.n_q_heads,), -1.0, device="cuda"), [rb], [o], [ws])
    torch.cuda.synchronize()
    assert int(rb.mask.sum()) == wl.n_q_heads * cache.info.n_compressed
    k, v = to64(inp.k[0]), to64(inp.v[0])
    G = wl.group
    kt = torch.from_numpy(np.repeat(k, G, axis=0))
    vt = torch.from_numpy(np.repeat(v, G, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(to64(q))[:, None, :], kt, vt)[:, 0, :].numpy()
    err = max(attn_err(to64(o)[h], ref[h]) for h in range(wl.n_q_heads))
    log(f"[batch4] dense check: spans={cache.info.n_compressed} err={err:.2e}")
    assert err <= TOL_BF16
