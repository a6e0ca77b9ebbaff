"""Shared helpers of the parity tests: draw one workload's inputs on the
device, run the HIP library through its C ABI, run the CPU oracle on the same
inputs (copied to the host), and compare stage by stage."""
from __future__ import annotations

import math
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle as O
import synth

TIE_BAND = 1e-5  # |p - tau| below this: the zoom decision is not compared


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


class Inputs:
    """Seeded inputs of one workload, on the device."""

    def __init__(self, wl: synth.Workload, seed: int, device="cuda", seq: int = 0,
                 surprisal: Optional[torch.Tensor] = None):
        self.wl, self.seed = wl, seed
        if surprisal is None:
            self.s, self.spike = synth.surprisal(wl, seed, seq=seq, device=device)
        else:
            self.s = surprisal.to(device=device, dtype=torch.float32).contiguous()
            self.spike = torch.zeros(wl.n_tokens, dtype=torch.bool, device=device)
        self.k, self.v, self.ranks = synth.kv_cache(wl, seed, self.spike, seq=seq, device=device)
        self.w, self.p = synth.route_weights(wl, seed, device=device)

    def query(self, step: int) -> torch.Tensor:
        return synth.queries(self.wl, self.seed, step, device=self.s.device)


def make_cfg(S, wl: synth.Workload, max_rank=None, tier="device", gamma=None):
    return S.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, head_dim=wl.head_dim,
                         route_dim=wl.route_dim, window=wl.window,
                         max_rank=wl.max_rank if max_rank is None else max_rank,
                         min_span_len=wl.min_span_len, alpha=wl.alpha,
                         gamma=wl.gamma if gamma is None else gamma, kv_dtype=wl.kv_dtype,
                         factor_tier=tier)


class OracleSide:
    """The oracle's cache for a chosen set of layers (all KV heads)."""

    def __init__(self, inp: Inputs, layers: Sequence[int], rank_cap: int, with_factors=True):
        wl = inp.wl
        self.wl = wl
        s = to64(inp.s)
        self.seg = O.segment(s, wl.window, wl.alpha, wl.min_span_len)
        self.groups: Dict[int, Dict[int, O.GroupCache]] = {}
        g = wl.group
        for layer in layers:
            w = to64(inp.w[layer])
            self.groups[layer] = {}
            for kh in range(wl.n_kv_heads):
                k = to64(inp.k[layer, kh])
                v = to64(inp.v[layer, kh])
                rk = inp.ranks[layer, kh].cpu().numpy()
                heads = {h: w[h] for h in range(kh * g, kh * g + g)}
                self.groups[layer][kh] = O.build_group(self.seg, s, k, v, heads, rk, wl.kv_dtype,
                                                       rank_cap, with_factors=with_factors)

    def summaries(self, layer: int) -> Dict[int, np.ndarray]:
        g = self.wl.group
        return {h: self.groups[layer][h // g].summary[h] for h in range(self.wl.n_q_heads)}

    def route(self, layer: int, q: np.ndarray, p: np.ndarray, tau: np.ndarray, gamma: float):
        return O.route_layer(q, p, tau, self.summaries(layer), self.seg, gamma, self.wl.n_kv_heads)

    def decode(self, layer: int, q: np.ndarray, route: O.LayerRoute, heads=None):
        return O.decode_layer(q, route, self.groups[layer], self.seg, heads=heads,
                              n_kv_heads=self.wl.n_kv_heads)


def calibrate_tau(orc: OracleSide, inp: Inputs, layers, targets: torch.Tensor, gamma: float,
                  n_queries: int = 16) -> torch.Tensor:
    """Per-(layer, head) thresholds: the (1 - f) quantile of the oracle's gate
    values over calibration queries (targets f [L][Hq])."""
    wl = inp.wl
    cq = synth.calibration_queries(wl, inp.seed, n_queries, device=inp.s.device)
    tau = torch.full((wl.n_layers, wl.n_q_heads), 1.0, dtype=torch.float32)
    for layer in layers:
        pr = to64(inp.p[layer])
        probs = [orc.route(layer, to64(cq[i, layer]), pr, np.full(wl.n_q_heads, 2.0), gamma).prob
                 for i in range(n_queries)]
        allp = np.concatenate(probs, axis=1)
        for h in range(wl.n_q_heads):
            f = float(targets[layer, h])
            tau[layer, h] = float(np.quantile(allp[h], 1.0 - f)) if f > 0 else 1.0
    return tau


def rel_err(a: np.ndarray, b: np.ndarray) -> float:
    """Norm-wise relative error max|a - b| / max|b|."""
    den = float(np.max(np.abs(b)))
    return float(np.max(np.abs(a - b))) / (den if den > 0 else 1.0)


ELEM_FLOOR = 0.1


def elem_err(a: np.ndarray, b: np.ndarray, floor: float = ELEM_FLOOR) -> float:
    """Element-wise relative error max_i |a_i - b_i| / max(|b_i|, floor max|b|):
    each output element against its own magnitude, with an absolute floor of
    10% of the head's largest element where the reference is near zero."""
    b = np.asarray(b, dtype=np.float64)
    den = np.maximum(np.abs(b), floor * float(np.max(np.abs(b))))
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - b) / den))


def attn_err(a: np.ndarray, b: np.ndarray) -> float:
    """The larger of the norm-wise and the floored element-wise error."""
    return max(rel_err(a, b), elem_err(a, b))


def route_from_gpu(rb, prob: np.ndarray, n_kv_heads: int) -> O.LayerRoute:
    """An oracle route carrying the GPU's zoom mask (lists and unions formed by
    the oracle's own compaction), so attention parity covers every head: a
    decision inside the tie band is taken as the GPU took it."""
    hq, sc = prob.shape
    mask = rb.mask.cpu().numpy().astype(bool)[:, :sc]
    g = hq // n_kv_heads
    return O.LayerRoute(prob=prob, mask=mask, lists=[O.compact(mask[h]) for h in range(hq)],
                        unions=[O.union_lists(list(mask[k * g:(k + 1) * g]))
                                for k in range(n_kv_heads)])


def compare_spans(cache, orc: OracleSide):
    sp = cache.spans()
    seg = orc.seg
    thr = seg.threshold
    s = seg  # noqa
    assert cache.info.mu == seg.mu or abs(cache.info.mu - seg.mu) <= 1e-13 * max(1, abs(seg.mu))
    assert abs(cache.info.sigma - seg.sigma) <= 1e-12 * max(1, seg.sigma)
    assert sp["anchors"].numpy().tolist() == seg.anchors.tolist()
    assert sp["span_start"].numpy().tolist() == seg.span_start.tolist()
    assert sp["span_len"].numpy().tolist() == seg.span_len.tolist()
    assert sp["kind"].numpy().astype(int).tolist() == seg.kind.tolist()
    assert sp["cspan"].numpy().tolist() == seg.cspan.tolist()
    assert sp["dense_pos"].numpy().tolist() == seg.dense_pos.tolist()
    return thr


def storage_mismatch(gpu: np.ndarray, ref: np.ndarray, kv_dtype: str) -> int:
    """Count entries that differ; every difference must be one storage ulp
    (a float64 rounding-order tie at the storage rounding point)."""
    diff = gpu != ref
    n = int(diff.sum())
    if n:
        ulp = np.abs(ref[diff]) * (2.0 ** -7 if kv_dtype == "bf16" else 2.0 ** -23)
        assert np.all(np.abs(gpu[diff] - ref[diff]) <= ulp * 1.01), "difference above one ulp"
    return n


def compare_group(cache, orc: OracleSide, layer: int, kv_head: int, n_factor_checks: int = 24):
    wl = orc.wl
    kb, vb, sm, rk, rv = cache.group_data(layer, kv_head)
    gc = orc.groups[layer][kv_head]
    assert rk.numpy().tolist() == gc.rank.tolist()
    assert rv.numpy().tolist() == gc.vrank.tolist()
    nmis = storage_mismatch(to64(kb), gc.kbar, wl.kv_dtype)
    nmis += storage_mismatch(to64(vb), gc.vbar, wl.kv_dtype)
    g = wl.group
    for hl in range(g):
        nmis += storage_mismatch(to64(sm[hl]), gc.summary[kv_head * g + hl], wl.kv_dtype)
    total = kb.numel() * 2 + sm.numel()
    assert nmis <= max(2, total * 1e-6), f"{nmis} storage mismatches of {total}"
    # factors: compare reconstructions and singular values, never raw vectors
    sc = len(gc.rank)
    worst = 0.0
    if gc.kfac:
        idx = np.unique(np.linspace(0, sc - 1, min(sc, n_factor_checks)).astype(int)) if sc else []
        for i in idx:
            n = int(orc.seg.span_len[orc.seg.cspan[i]])
            for kv, fac in ((0, gc.kfac[i]), (1, gc.vfac[i])):
                r = int(gc.rank[i] if kv == 0 else gc.vrank[i])
                u, sg, vt = cache.factors(layer, kv_head, int(i), kv, r, n)
                rec = (u.double() * sg.double()) @ vt.double()
                ref = fac.reconstruct()
                e = np.linalg.norm(rec.numpy() - ref) / max(np.linalg.norm(ref), 1e-300)
                worst = max(worst, e)
                big = np.abs(fac.sigma) > 1e-6 * np.max(np.abs(fac.sigma))
                assert np.allclose(sg.double().numpy()[big], fac.sigma[big], rtol=1e-5, atol=0)
    assert worst <= 1e-4, f"factor reconstruction differs by {worst}"
    return nmis, worst


def compare_route(rb, route: O.LayerRoute, tau: np.ndarray, wl) -> int:
    """Masks bit-exact outside the tie band; lists and unions exact when the
    band is empty.  Returns the number of (head, span) pairs in the band."""
    mask = rb.mask.cpu().numpy().astype(bool)
    sc = route.mask.shape[1]
    mask = mask[:, :sc]
    tie = np.abs(route.prob - tau[:, None].astype(np.float64)) < TIE_BAND
    assert np.array_equal(mask[~tie], route.mask[~tie])
    if rb.prob is not None and sc:
        gp = rb.prob.cpu().numpy()[:, :sc]
        assert np.max(np.abs(gp - route.prob)) <= 1e-12
    n_tie = int(tie.sum())
    if n_tie == 0:
        cnt = rb.count.cpu().numpy()
        lst = rb.list.cpu().numpy()
        for h in range(wl.n_q_heads):
            assert lst[h, :cnt[h]].tolist() == route.lists[h].tolist()
        uc = rb.union_count.cpu().numpy()
        ul = rb.union_list.cpu().numpy()
        for g in range(wl.n_kv_heads):
            assert ul[g, :uc[g]].tolist() == route.unions[g].tolist()
    return n_tie


def tied_heads(route: O.LayerRoute, tau: np.ndarray) -> List[int]:
    tie = np.abs(route.prob - tau[:, None].astype(np.float64)) < TIE_BAND
    return [h for h in range(tie.shape[0]) if tie[h].any()]
