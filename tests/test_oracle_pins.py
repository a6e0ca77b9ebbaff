"""Pins of the CPU oracle against what the SeKV pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
derived by hand from the definitions (tests/golden), closed forms, invariants,
special cases that reduce to a textbook routine (torch's scaled-dot-product
attention, numpy's std, LAPACK eigenvalues), or brute force on tiny inputs.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# segmentation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("segmentation_tiny.json")["cases"], ids=lambda c: c["name"])
def test_segmentation_golden(case):
    seg = O.segment(np.array(case["surprisal"], float), case["window"], case["alpha"],
                    case["min_span_len"])
    assert seg.mu == pytest.approx(case["mu"], abs=1e-15)
    assert seg.sigma == pytest.approx(case["sigma"], rel=1e-14)
    assert seg.anchors.tolist() == case["anchors"]
    assert seg.span_start.tolist() == case["span_start"]
    assert seg.span_len.tolist() == case["span_len"]
    assert seg.kind.tolist() == case["kind"]
    assert seg.dense_pos.tolist() == case["dense_pos"]


def _numpy_segmentation(s, window, alpha, min_len):
    """Brute force through different routines: numpy's std, flatnonzero and
    diff of a padded indicator."""
    s = np.asarray(s, float)
    thr = np.mean(s) + alpha * np.std(s)
    limit = max(s.size - window, 0)
    anch = np.flatnonzero(s[:limit] > thr)
    inside = np.ones(limit + 2, dtype=np.int8)
    inside[1:limit + 1] = (s[:limit] > thr).astype(np.int8)  # 1 = anchor / outside
    edges = np.diff(inside)
    starts = np.flatnonzero(edges == -1)
    ends = np.flatnonzero(edges == 1)
    lens = ends - starts
    return anch, starts, lens, (lens < min_len).astype(int)


@pytest.mark.parametrize("seed", range(12))
def test_segmentation_brute_force_random(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 40))
    s = r.gamma(2.0, 1.5, n).astype(np.float32).astype(float)
    s[r.random(n) < 0.1] += 6
    window = int(r.integers(0, 6))
    min_len = int(r.integers(1, 5))
    seg = O.segment(s, window, 1.0, min_len)
    anch, starts, lens, kind = _numpy_segmentation(s, window, 1.0, min_len)
    # the two thresholds differ only by summation order; skip razor-thin ties
    if np.any(np.abs(s - seg.threshold) < 1e-12 * max(1.0, abs(seg.threshold))):
        pytest.skip("tie at the threshold")
    assert seg.anchors.tolist() == anch.tolist()
    assert seg.span_start.tolist() == starts.tolist()
    assert seg.span_len.tolist() == lens.tolist()
    assert seg.kind.tolist() == kind.tolist()


def test_segmentation_closed_forms():
    # constant sequence: std 0, nothing exceeds the mean
    seg = O.segment(np.full(1000, 0.1, dtype=np.float32), 100, 1.0, 8)
    assert seg.sigma == 0.0 and seg.anchors.size == 0
    assert seg.span_start.tolist() == [0] and seg.span_len.tolist() == [900]
    # a single spike in a constant sequence is the single anchor
    s = np.full(300, 2.0)
    s[77] = 9.0
    seg = O.segment(s, 50, 1.0, 8)
    assert seg.anchors.tolist() == [77]
    assert seg.span_start.tolist() == [0, 78] and seg.span_len.tolist() == [77, 172]
    # fewer tokens than the window: no spans, everything dense
    seg = O.segment(np.arange(10.0), 512, 1.0, 8)
    assert seg.span_start.size == 0 and seg.dense_pos.tolist() == list(range(10))


def test_segmentation_partition():
    r = np.random.default_rng(5)
    s = r.gamma(2.0, 1.5, 5000)
    s[r.random(5000) < 0.02] += 6
    seg = O.segment(s, 512, 1.0, 8)
    covered = np.zeros(5000, int)
    covered[seg.anchors] += 1
    for b, n in zip(seg.span_start, seg.span_len):
        covered[b:b + n] += 1
    covered[5000 - 512:] += 1
    assert np.all(covered == 1)
    assert seg.anchors.size + seg.span_len.sum() + 512 == 5000
    # anchor share close to P(s > T) of the sample itself
    assert seg.anchors.size == int(np.sum(s[:-512] > seg.threshold))


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_values():
    r = np.random.default_rng(0)
    x = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    mine = O.round_bf16(x.astype(float))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_round_bf16_single_rounding_from_float64():
    # halfway cases go to even; a float64 value just above a halfway point must
    # round up, which rounding through float32 first would get wrong
    assert O.round_bf16(1 + 2.0 ** -8) == 1.0
    assert O.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert O.round_bf16(1 + 2.0 ** -8 + 2.0 ** -40) == 1 + 2.0 ** -7
    assert O.round_bf16(-(1 + 2.0 ** -8 + 2.0 ** -40)) == -(1 + 2.0 ** -7)
    assert O.round_bf16(255.5) == 256.0
    assert O.round_store(1 + 2.0 ** -30, "f32") == 1.0


# ---------------------------------------------------------------------------
# weights, means, summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("span_summary_tiny.json")["cases"], ids=lambda c: c["name"])
def test_summary_golden(case):
    w = O.span_weights(case["surprisal"])
    assert np.allclose(w, case["weights"], atol=1e-15)
    km = O.weighted_mean(w, case["keys"])
    vm = O.weighted_mean(w, case["values"])
    assert np.allclose(km, case["kbar"], atol=1e-14)
    assert np.allclose(vm, case["vbar"], atol=1e-14)
    assert np.allclose(np.array(case["w_route"], float) @ km, case["summary"], atol=1e-14)


def test_build_group_means_and_summaries_follow_span_table():
    # a hand-built sequence: anchor at 2, spans [0,2) and [3,7), window 1
    s = np.array([1.0, 3.0, 50.0, 2.0, 2.0, 4.0, 0.0, 1.0])
    seg = O.segment(s, 1, 1.0, 2)
    assert seg.anchors.tolist() == [2]
    assert seg.span_start.tolist() == [0, 3] and seg.span_len.tolist() == [2, 4]
    k = np.arange(16, dtype=float).reshape(8, 2)
    v = -k
    wh = {0: np.array([[1.0, 0.0]]), 1: np.array([[0.0, 2.0]])}
    gc = O.build_group(seg, s, k, v, wh, np.full(8, 32), "f32", 32)
    # span 0: weights [.25, .75] over rows [0,1],[2,3] -> [1.5, 2.5]
    assert np.allclose(gc.kbar[0], [1.5, 2.5])
    # span 1: weights [.25,.25,.5,0] over rows 3..6 -> [8.5, 9.5]
    assert np.allclose(gc.kbar[1], [8.5, 9.5])
    assert np.allclose(gc.vbar, -gc.kbar)
    assert np.allclose(gc.summary[0][:, 0], gc.kbar[:, 0])
    assert np.allclose(gc.summary[1][:, 0], 2 * gc.kbar[:, 1])
    assert gc.dense_k.tolist() == k[[2, 7]].tolist()


def test_summary_linearity_and_constant_span():
    r = np.random.default_rng(3)
    n, d, dr = 37, 128, 32
    x = r.standard_normal((n, d))
    sp = r.gamma(2, 1.0, n)
    w = O.span_weights(sp)
    wh = r.standard_normal((dr, d))
    # W applied to the weighted mean == weighted mean of the projected keys
    per_token = np.array([wh @ x[t] for t in range(n)])
    assert np.allclose(wh @ O.weighted_mean(w, x), (w[:, None] * per_token).sum(0), atol=1e-12)
    assert abs(w.sum() - 1) < 1e-15
    # identical tokens: the mean is the token, whatever the weights
    row = O.round_bf16(r.standard_normal(d))
    assert np.array_equal(O.round_bf16(O.weighted_mean(w, np.tile(row, (n, 1)))), row)
    assert O.span_weights([7.0]).tolist() == [1.0]


# ---------------------------------------------------------------------------
# truncated SVD
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,r", [(5, 3), (40, 8), (128, 32), (300, 17), (9, 9)])
def test_svd_identities(n, r):
    rng = np.random.default_rng(n * 7 + r)
    d = 128
    x = rng.standard_normal((n, 6)) @ rng.standard_normal((6, d)) + 0.05 * rng.standard_normal((n, d))
    full = O.truncated_svd(x, min(n, d))
    assert np.linalg.norm(x - full.reconstruct()) <= 1e-12 * np.linalg.norm(x)
    f = O.truncated_svd(x, r)
    err2 = np.linalg.norm(x - f.reconstruct()) ** 2
    # Eckart-Young: the error of the rank-r truncation is the discarded energy
    assert err2 == pytest.approx(f.tail2, rel=1e-10, abs=1e-20)
    assert np.allclose(f.u.T @ f.u, np.eye(r), atol=1e-12)
    assert np.allclose(f.vt @ f.vt.T, np.eye(r), atol=1e-12)
    # singular values against a different LAPACK routine (symmetric eigensolver)
    ev = np.sort(np.linalg.eigvalsh(x @ x.T if n <= d else x.T @ x))[::-1]
    assert np.allclose(f.sigma ** 2, ev[:r], rtol=1e-9, atol=1e-9)
    assert np.all(np.diff(f.sigma) <= 0)


def test_svd_planted_rank():
    rng = np.random.default_rng(11)
    n, d, k = 90, 128, 5
    x = rng.standard_normal((n, k)) @ rng.standard_normal((k, d)) + 1e-3 * rng.standard_normal((n, d))
    f = O.truncated_svd(x, 32)
    assert f.sigma[k - 1] > 1.0 and f.sigma[k] < 0.03
    assert O.span_rank(40, 6, 128, 32) == 6 and O.span_rank(0, 50, 128, 32) == 1
    assert O.span_rank(20, 50, 128, 32) == 20 and O.span_rank(99, 500, 128, 32) == 32


# ---------------------------------------------------------------------------
# soft gates (Eq. 8)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,r", [(40, 8), (128, 32), (300, 17)])
def test_gate_factors_closed_forms(n, r):
    rng = np.random.default_rng(n + 3 * r)
    d = 128
    x = rng.standard_normal((n, 6)) @ rng.standard_normal((6, d)) + 0.05 * rng.standard_normal((n, d))
    f = O.truncated_svd(x, r)
    full = O.truncated_svd(x, min(n, d))
    # gates of one change nothing
    g1 = O.gate_factors(f, np.ones(r), 0.5)
    assert np.array_equal(g1.u, f.u) and np.array_equal(g1.sigma, f.sigma)
    assert np.array_equal(g1.vt, f.vt)
    # 0/1 gates on a prefix are the truncation to that prefix (Eckart-Young pins it)
    k = max(1, r // 2)
    gp = O.gate_factors(f, np.r_[np.ones(k), np.zeros(r - k)], 0.5)
    assert gp.sigma.size == k
    assert np.linalg.norm(gp.reconstruct() - O.truncated_svd(x, k).reconstruct()) <= \
        1e-12 * np.linalg.norm(x)
    # soft gates: with orthonormal factors the error splits component by
    # component, (1 - g_i)^2 sigma_i^2 for a kept one and sigma_i^2 for every
    # dropped or never-retained one (the full spectrum from LAPACK)
    g = rng.uniform(0.0, 1.0, r)
    eps = 0.3
    gf = O.gate_factors(f, g, eps)
    kept = g >= eps
    assert gf.sigma.size == int(kept.sum())
    s_all = full.sigma
    want = float(np.sum(((1.0 - g[kept]) * s_all[:r][kept]) ** 2) +
                 np.sum(s_all[:r][~kept] ** 2) + np.sum(s_all[r:] ** 2))
    got = float(np.linalg.norm(x - gf.reconstruct()) ** 2)
    assert got == pytest.approx(want, rel=1e-9)


def test_gate_factors_keeps_one_component():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((20, 128))
    f = O.truncated_svd(x, 6)
    g = np.array([0.01, 0.05, 0.02, 0.05, 0.0, 0.03])
    gf = O.gate_factors(f, g, 0.5)
    assert gf.sigma.size == 1
    assert gf.sigma[0] == pytest.approx(0.05 * f.sigma[1])   # largest gate, lowest index
    assert np.array_equal(gf.vt[0], f.vt[1])


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def test_route_golden():
    c = _golden("route_attention_tiny.json")["route"]
    for tau, want in c["zoom_at_tau"].items():
        p, z = O.route_head(c["q"], c["p_proj"], c["summary"], c["log_len"], c["gamma"], float(tau))
        assert np.allclose(p, c["p"], rtol=0, atol=1e-16)
        assert z.tolist() == want


def test_route_special_cases():
    r = np.random.default_rng(2)
    sc, dr, d = 50, 32, 128
    summ = O.round_bf16(r.standard_normal((sc, dr)) * 0.3)
    ll = np.log(r.integers(8, 600, sc).astype(float))
    q = r.standard_normal(d)
    pp = r.standard_normal((dr, d)) / math.sqrt(d)
    # strict threshold: p <= 1 never exceeds 1; p > 0 always exceeds -1
    assert not O.route_head(q, pp, summ, ll, 0.1, 1.0)[1].any()
    assert O.route_head(q, pp, summ, ll, 0.1, -1.0)[1].all()
    # sets grow as the threshold falls
    prev = np.zeros(sc, bool)
    for tau in np.linspace(0.99, 0.01, 30):
        z = O.route_head(q, pp, summ, ll, 0.1, tau)[1]
        assert np.all(z >= prev)
        prev = z
    # zero summaries: the gate is the size prior alone (scipy's expit)
    from scipy.special import expit
    p, _ = O.route_head(q, pp, np.zeros((sc, dr)), ll, 0.37, 0.5)
    assert np.allclose(p, expit(0.37 * ll), rtol=1e-15, atol=0)
    # zero size prior and a one-hot projection: x is one summary coordinate times q_0
    e0 = np.zeros((dr, d))
    e0[3, 0] = 1.0
    p, _ = O.route_head(np.eye(d)[0] * 2.0, e0, summ, ll, 0.0, 0.5)
    assert np.allclose(p, expit(2.0 * summ[:, 3]), rtol=1e-15, atol=0)


def test_compaction_and_union():
    r = np.random.default_rng(9)
    m = r.random((4, 200)) < 0.1
    for h in range(4):
        assert O.compact(m[h]).tolist() == np.flatnonzero(m[h]).tolist()
    assert O.union_lists(list(m)).tolist() == np.flatnonzero(m.any(0)).tolist()
    assert O.union_lists([]).size == 0


# ---------------------------------------------------------------------------
# mixed-resolution attention
# ---------------------------------------------------------------------------

def test_attention_golden():
    c = _golden("route_attention_tiny.json")["attention"]
    seg = O.Segmentation(n_tokens=3, window=1, mu=0, sigma=0, threshold=0,
                         anchors=np.zeros(0, np.int64), span_start=np.array([0]),
                         span_len=np.array(c["span_len"]), kind=np.array([0]),
                         cspan=np.array([0]), dense_pos=np.array([2]))
    gc = O.GroupCache(dense_k=np.array(c["dense_k"], float), dense_v=np.array(c["dense_v"], float),
                      kbar=np.array(c["kbar"], float), vbar=np.array(c["vbar"], float),
                      summary={}, kfac=[None], vfac=[None], rank=np.array([1]), vrank=np.array([1]))
    o = O.mixed_attention(c["q"], gc, seg, [False])
    assert np.allclose(o, c["o"], atol=1e-15)


def _problem(seed, n=1500, hq=4, hkv=2, window=128, min_len=8, constant_spans=False,
             kv_dtype="f32", rank_cap=32):
    r = np.random.default_rng(seed)
    d, dr = 128, 32
    s = r.gamma(2.0, 0.05, n)
    s[r.random(n) < 1 / 40] += 6.0
    seg = O.segment(s, window, 1.0, min_len)
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    if constant_spans:
        for b, ln in zip(seg.span_start, seg.span_len):
            k[:, b:b + ln] = k[:, b:b + 1]
            v[:, b:b + ln] = v[:, b:b + 1]
    k = O.round_store(k, kv_dtype)
    v = O.round_store(v, kv_dtype)
    w = r.standard_normal((hq, dr, d)) / math.sqrt(d)
    p = r.standard_normal((hq, dr, d)) / math.sqrt(d)
    q = r.standard_normal((hq, d))
    g = hq // hkv
    groups = {kh: O.build_group(seg, s, k[kh], v[kh], {h: w[h] for h in range(kh * g, kh * g + g)},
                                np.full(n, 999), kv_dtype, rank_cap) for kh in range(hkv)}
    summ = {h: groups[h // g].summary[h] for h in range(hq)}
    return seg, k, v, q, p, summ, groups, s


def _sdpa(q, k, v, bias=None):
    """Textbook attention through torch (CPU, float64); grouped-query layout
    by repeating each KV head over its query heads."""
    hq, hkv = q.shape[0], k.shape[0]
    kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=0))
    vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=0))
    qt = torch.from_numpy(q)[:, None, :]
    mask = None if bias is None else torch.from_numpy(bias)[:, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[:, 0, :].numpy()


def test_all_zoomed_at_full_rank_is_dense_attention():
    seg, k, v, q, p, summ, groups, _ = _problem(21, rank_cap=128)
    route = O.route_layer(q, p, np.full(4, -1.0), summ, seg, 0.1, 2)
    assert route.mask.all()
    out = O.decode_layer(q, route, groups, seg, n_kv_heads=2)
    ref = _sdpa(q, k, v)
    for h in range(4):
        assert np.allclose(out[h], ref[h], rtol=1e-10, atol=1e-12)


def test_none_zoomed_with_constant_spans_is_dense_attention():
    # a span of identical tokens weighs n e^{q.k/sqrt d}: the coarse entry with
    # + ln n carries exactly that mass
    seg, k, v, q, p, summ, groups, _ = _problem(22, constant_spans=True)
    route = O.route_layer(q, p, np.full(4, 1.0), summ, seg, 0.1, 2)
    assert not route.mask.any()
    out = O.decode_layer(q, route, groups, seg, n_kv_heads=2)
    ref = _sdpa(q, k, v)
    for h in range(4):
        assert np.allclose(out[h], ref[h], rtol=1e-10, atol=1e-12)


def test_mixed_zoom_matches_explicit_entry_list():
    """Some spans zoomed at full rank, the rest coarse: the same as textbook
    attention over an explicit entry list built from the raw rows (dense rows,
    zoomed spans' exact rows, one mean row per other span with an additive
    ln n bias)."""
    seg, k, v, q, p, summ, groups, s = _problem(23, kv_dtype="bf16", rank_cap=128)
    tau = np.array([0.45, 0.55, 0.5, 0.6])
    route = O.route_layer(q, p, tau, summ, seg, 0.1, 2)
    assert 0 < route.mask.sum() < route.mask.size
    out = O.decode_layer(q, route, groups, seg, n_kv_heads=2)
    for h in range(4):
        kh = h // 2
        rows_k, rows_v, bias = [k[kh, seg.dense_pos]], [v[kh, seg.dense_pos]], [np.zeros(seg.dense_pos.size)]
        for i, j in enumerate(seg.cspan):
            b, n = seg.span_start[j], seg.span_len[j]
            if route.mask[h, i]:
                rows_k.append(k[kh, b:b + n])
                rows_v.append(v[kh, b:b + n])
                bias.append(np.zeros(n))
            else:
                rows_k.append(groups[kh].kbar[i:i + 1])
                rows_v.append(groups[kh].vbar[i:i + 1])
                bias.append(np.array([math.log(n)]))
        ref = _sdpa(q[h:h + 1], np.concatenate(rows_k)[None], np.concatenate(rows_v)[None],
                    np.concatenate(bias)[None])
        assert np.allclose(out[h], ref[0], rtol=1e-9, atol=1e-11)
    # the union of a group is the OR of its heads' masks
    for g in range(2):
        assert route.unions[g].tolist() == np.flatnonzero(route.mask[2 * g:2 * g + 2].any(0)).tolist()


def test_short_context_is_dense_attention_over_window():
    seg, k, v, q, p, summ, groups, _ = _problem(24, n=300, window=512)
    assert seg.span_start.size == 0
    route = O.route_layer(q, p, np.full(4, 0.5), summ, seg, 0.1, 2)
    out = O.decode_layer(q, route, groups, seg, n_kv_heads=2)
    ref = _sdpa(q, k, v)
    for h in range(4):
        assert np.allclose(out[h], ref[h], rtol=1e-10, atol=1e-12)


def test_truncation_moves_output_by_bounded_amount():
    """Rank-r zoom vs full-rank zoom: the output changes, and by less as r grows."""
    errs = []
    for cap in (4, 16, 64, 128):
        seg, k, v, q, p, summ, groups, _ = _problem(25, n=800, rank_cap=cap)
        route = O.route_layer(q, p, np.full(4, -1.0), summ, seg, 0.1, 2)
        out = O.decode_layer(q, route, groups, seg, n_kv_heads=2)
        ref = _sdpa(q, k, v)
        errs.append(max(np.abs(out[h] - ref[h]).max() for h in range(4)))
    assert errs[-1] < 1e-10
    assert errs[0] > errs[1] > errs[2] > errs[3]


# ---------------------------------------------------------------------------
# budget cap (Sec. 3.3, matched-budget paragraph)
# ---------------------------------------------------------------------------

def _route_of(prob, tau):
    prob = np.asarray(prob, dtype=np.float64)
    mask = prob > tau
    return O.LayerRoute(prob=prob, mask=mask, lists=[O.compact(z) for z in mask], unions=[])


def _seg_of(span_len):
    n = np.asarray(span_len, dtype=np.int64)
    return types.SimpleNamespace(span_len=n, cspan=np.arange(n.size), n_compressed=n.size)


@pytest.mark.parametrize("case", _golden("budget_cap_tiny.json")["cases"], ids=lambda c: str(c["budget"]))
def test_budget_cap_golden(case):
    gold = _golden("budget_cap_tiny.json")
    route = _route_of(gold["prob"], gold["tau"])
    capped = O.cap_budget(route, _seg_of(gold["span_len"]), gold["n_kv_heads"], case["budget"])
    assert capped.mask.astype(int).tolist() == case["mask"]
    assert [u.tolist() for u in capped.unions] == case["unions"]
    assert [l.tolist() for l in capped.lists] == [list(np.flatnonzero(m)) for m in case["mask"]]


@pytest.mark.parametrize("case", _golden("budget_cap_tiny.json")["layer_scope"]["cases"],
                         ids=lambda c: f"layer-{c['budget']}")
def test_budget_cap_layer_scope_golden(case):
    gold = _golden("budget_cap_tiny.json")
    route = _route_of(gold["prob"], gold["tau"])
    capped = O.cap_budget(route, _seg_of(gold["span_len"]), gold["n_kv_heads"], case["budget"],
                          scope="layer")
    assert capped.mask.astype(int).tolist() == case["mask"]
    assert [u.tolist() for u in capped.unions] == case["unions"]
    assert [l.tolist() for l in capped.lists] == [list(np.flatnonzero(m)) for m in case["mask"]]


def test_budget_cap_layer_scope_properties():
    """Layer scope: one KV head reduces to the per-KV-head cap; the kept total
    never exceeds the budget and is a prefix (adding the next candidate in
    key order would exceed it); larger budgets keep supersets."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        hkv, g, sc = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(5, 40))
        prob = rng.uniform(0, 1, (hkv * g, sc))
        lens = rng.integers(1, 50, sc)
        route = _route_of(prob.tolist(), 0.5)
        seg = _seg_of(lens.tolist())
        prev = None
        for budget in sorted(rng.integers(0, int(lens.sum()) * hkv + 1, 6).tolist()):
            capped = O.cap_budget(route, seg, hkv, budget, scope="layer")
            if hkv == 1:
                same = O.cap_budget(route, seg, hkv, budget)
                assert np.array_equal(capped.mask, same.mask)
            total = sum(int(lens[j]) for u in capped.unions for j in u)
            assert total <= budget
            assert np.all(capped.mask <= route.mask)
            if prev is not None:
                assert np.all(prev <= capped.mask)
            prev = capped.mask


def test_budget_cap_properties():
    """On random routes: the kept spans of each group are a prefix of the
    order (key descending, id ascending) whose total fits and whose next span
    would not; the cap only removes zooms; it is monotone in the budget and
    leaves a route unchanged once the budget covers the whole union."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        hkv, grp, sc = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 40))
        hq = hkv * grp
        prob = rng.random((hq, sc))
        if trial % 3 == 0:
            prob = np.round(prob, 1)   # many ties
        n = rng.integers(1, 60, sc)
        route = _route_of(prob, rng.random())
        seg = _seg_of(n)
        full = [int(n[O.union_lists(list(route.mask[g * grp:(g + 1) * grp]))].sum()) for g in range(hkv)]
        prev = None
        for budget in sorted(int(b) for b in rng.integers(0, max(full) + 2, 5)):
            capped = O.cap_budget(route, seg, hkv, budget)
            assert not (capped.mask & ~route.mask).any()
            for g in range(hkv):
                hs = slice(g * grp, (g + 1) * grp)
                cand = O.union_lists(list(route.mask[hs]))
                kept = set(O.union_lists(list(capped.mask[hs])).tolist())
                assert sum(n[j] for j in kept) <= budget
                if not cand.size:
                    continue
                key = {j: prob[hs][route.mask[hs][:, j], j].max() for j in cand}
                order = sorted(cand, key=lambda j: (-key[j], j))
                k = len(kept)
                assert set(order[:k]) == kept
                if k < len(order):
                    assert sum(n[j] for j in order[:k + 1]) > budget
                # a kept span stays zoomed for exactly the heads that chose it
                for j in kept:
                    assert (capped.mask[hs][:, j] == route.mask[hs][:, j]).all()
            if prev is not None:
                assert not (prev & ~capped.mask).any()
            prev = capped.mask
        big = O.cap_budget(route, seg, hkv, max(full))
        assert (big.mask == route.mask).all()


def _two_spans(seed, n=60):
    """A span's key and value matrices with different planted spectra."""
    rng = np.random.default_rng(seed)
    d = 128
    k = rng.standard_normal((n, 7)) @ rng.standard_normal((7, d)) + 0.05 * rng.standard_normal((n, d))
    v = 3.0 * rng.standard_normal((n, 4)) @ rng.standard_normal((4, d)) + \
        0.2 * rng.standard_normal((n, d))
    return k, v


def _energy(x):
    """Squared singular values of x, descending, from LAPACK's symmetric
    eigensolver (a routine other than the oracle's SVD)."""
    return np.sort(np.clip(np.linalg.eigvalsh(x.T @ x), 0.0, None))[::-1]


def test_gate_group_keys_and_values_have_their_own_gates():
    """Sec. 3.2 low-rank paragraph: the value matrix gets the gated
    decomposition with gates and factors of its own.  Value-only gates leave
    the keys bit-identical; distinct key and value gates give distinct ranks;
    and each matrix's error is its own closed form sum_kept (1 - g)^2 s^2 +
    sum_dropped s^2 + sum_beyond_r s^2 (orthonormal factors), so gates applied
    to the wrong matrix, or one vector for both, fail."""
    n, r, eps = 60, 12, 0.3
    k, v = _two_spans(3, n)
    seg = types.SimpleNamespace()
    kf, vf = O.truncated_svd(k, r), O.truncated_svd(v, r)
    gc = O.GroupCache(dense_k=np.zeros((0, 128)), dense_v=np.zeros((0, 128)),
                      kbar=np.zeros((1, 128)), vbar=np.zeros((1, 128)), summary={},
                      kfac=[kf], vfac=[vf], rank=np.array([r]), vrank=np.array([r]))
    ones = np.ones((1, 32))
    rng = np.random.default_rng(9)
    gv = np.r_[rng.uniform(0.35, 1.0, 4), rng.uniform(0.0, 0.25, r - 4), np.zeros(32 - r)][None, :]
    gk = np.r_[rng.uniform(0.35, 1.0, 9), rng.uniform(0.0, 0.25, r - 9), np.zeros(32 - r)][None, :]
    # value gates only: keys untouched, bit for bit
    g1 = O.gate_group(gc, ones, gv, eps)
    assert np.array_equal(g1.kfac[0].u, kf.u) and np.array_equal(g1.kfac[0].sigma, kf.sigma)
    assert np.array_equal(g1.kfac[0].vt, kf.vt)
    assert g1.rank.tolist() == [r] and g1.vrank.tolist() == [4]
    # distinct gates: distinct ranks, each matrix's error its own closed form
    g2 = O.gate_group(gc, gk, gv, eps)
    assert g2.rank.tolist() == [9] and g2.vrank.tolist() == [4]
    for x, fac, g in ((k, g2.kfac[0], gk[0]), (v, g2.vfac[0], gv[0])):
        s2 = _energy(x)
        kept = g[:r] >= eps
        want = float(np.sum((1.0 - g[:r][kept]) ** 2 * s2[:r][kept]) + np.sum(s2[:r][~kept]) +
                     np.sum(s2[r:]))
        got = float(np.linalg.norm(x - fac.reconstruct()) ** 2)
        assert got == pytest.approx(want, rel=1e-8)
    # the closed forms tell the two matrices apart: the key error under the
    # value gates is not the key error under the key gates
    swapped = O.gate_group(gc, gv, gk, eps)
    ek = float(np.linalg.norm(k - swapped.kfac[0].reconstruct()) ** 2)
    s2 = _energy(k)
    kept = gk[0, :r] >= eps
    want_k = float(np.sum((1.0 - gk[0, :r][kept]) ** 2 * s2[:r][kept]) + np.sum(s2[:r][~kept]) +
                   np.sum(s2[r:]))
    assert abs(ek - want_k) > 1e-3 * want_k
    del seg


def test_gated_attention_uses_each_matrix_reconstruction():
    """A zoomed span with value gates of zero everywhere but one component
    attends to values rebuilt from that component alone, while its scores
    still use the ungated keys: checked against torch's SDPA over the rows the
    two reconstructions give."""
    n, r = 40, 10
    k, v = _two_spans(4, n)
    seg = O.Segmentation(n_tokens=n, window=0, mu=0.0, sigma=0.0, threshold=0.0,
                         anchors=np.zeros(0, np.int64), span_start=np.array([0]),
                         span_len=np.array([n]), kind=np.array([0]), cspan=np.array([0]),
                         dense_pos=np.zeros(0, np.int64))
    kf, vf = O.truncated_svd(k, r), O.truncated_svd(v, r)
    gc = O.GroupCache(dense_k=np.zeros((0, 128)), dense_v=np.zeros((0, 128)),
                      kbar=np.zeros((1, 128)), vbar=np.zeros((1, 128)), summary={},
                      kfac=[kf], vfac=[vf], rank=np.array([r]), vrank=np.array([r]))
    gv = np.zeros((1, 32))
    gv[0, 2] = 0.7
    gg = O.gate_group(gc, np.ones((1, 32)), gv, 0.5)
    assert gg.rank.tolist() == [r] and gg.vrank.tolist() == [1]
    q = np.random.default_rng(5).standard_normal(128)
    o = O.mixed_attention(q, gg, seg, np.array([True]))
    kr = (kf.u * kf.sigma) @ kf.vt
    vr = 0.7 * vf.sigma[2] * np.outer(vf.u[:, 2], vf.vt[2])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, :], torch.from_numpy(kr)[None], torch.from_numpy(vr)[None])
    assert np.allclose(o, ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# window append and retire
# ---------------------------------------------------------------------------

def _append_case(seed, n_build=300, n_total=420, window=40, min_len=4):
    rng = np.random.default_rng(seed)
    s = rng.gamma(2.0, 0.3, n_total)
    s[rng.choice(n_total, n_total // 12, replace=False)] += 3.0
    build = O.segment(s[:n_build], window, 1.0, min_len)
    return s, build


@pytest.mark.parametrize("seed", range(6))
def test_append_partition_and_brute_force(seed):
    """After appends, anchors, every span, the open run and the window
    partition [0, N); the spans and anchors the appends add equal an
    independent formulation: in the retired positions, the anchors are those
    above the build's threshold and the new spans are the maximal runs of
    other positions that an anchor follows (found with numpy run boundaries)."""
    n_build, window, min_len = 300, 40, 4
    s, build = _append_case(seed, n_build=n_build, window=window, min_len=min_len)
    for n in (n_build, n_build + 1, n_build + 17, s.size):
        seg = O.segment_appended(s[:n], n_build, build, min_len)
        covered = np.zeros(n, dtype=int)
        covered[seg.anchors] += 1
        for b, ln in zip(seg.span_start, seg.span_len):
            covered[b:b + ln] += 1
        covered[seg.open_start:seg.open_start + seg.open_len] += 1
        covered[max(n - window, 0):] += 1
        assert np.all(covered == 1)
        assert seg.anchors.size + int(seg.span_len.sum()) + seg.open_len + min(window, n) == n
        # brute force over the retired positions
        r0, r1 = n_build - window, n - window
        above = s[r0:r1] > build.threshold
        assert seg.anchors[build.anchors.size:].tolist() == (r0 + np.flatnonzero(above)).tolist()
        low = np.r_[False, ~above, False].astype(int)
        edges = np.diff(low)
        starts, ends = np.flatnonzero(edges == 1), np.flatnonzero(edges == -1)
        closed = [(r0 + a, b - a) for a, b in zip(starts, ends) if b < r1 - r0]
        new = list(zip(seg.span_start[build.span_start.size:].tolist(),
                       seg.span_len[build.span_len.size:].tolist()))
        assert new == closed
        tail = [(r0 + a, b - a) for a, b in zip(starts, ends) if b == r1 - r0]
        assert (seg.open_start, seg.open_len) == (tail[0] if tail else (0, 0))
        # short new spans stay at full resolution
        assert set(seg.dense_pos.tolist()) == set(range(n)) - {
            t for i in seg.cspan for t in range(seg.span_start[i], seg.span_start[i] + seg.span_len[i])}


def test_append_closed_forms():
    """No appended token above the threshold: the spans stay, every retired
    token sits in the open run; every retired token above it: each becomes an
    anchor, no span is added; appending nothing returns the build."""
    n_build, window = 200, 30
    s, build = _append_case(1, n_build=n_build, n_total=260, window=window)
    same = O.segment_appended(s[:n_build], n_build, build, 4)
    for f in ("anchors", "span_start", "span_len", "kind", "cspan", "dense_pos"):
        assert np.array_equal(getattr(same, f), getattr(build, f))
    low = s.copy()
    low[n_build:] = build.threshold - 1.0
    low[n_build - window:n_build] = np.minimum(low[n_build - window:n_build], build.threshold)
    seg = O.segment_appended(low, n_build, build, 4)
    assert np.array_equal(seg.span_start, build.span_start)
    assert seg.open_len == 60 and seg.open_start == n_build - window
    high = s.copy()
    high[n_build - window:] = build.threshold + 1.0
    seg = O.segment_appended(high, n_build, build, 4)
    assert seg.anchors.size == build.anchors.size + 60 and seg.open_len == 0
    assert np.array_equal(seg.span_len, build.span_len)


def test_append_full_rank_all_zoomed_is_dense_attention():
    """Every span of the appended cache zoomed at full rank: textbook attention
    over all N tokens (torch SDPA), whatever was retired."""
    n_build, window, min_len = 300, 40, 4
    s, build = _append_case(3, n_build=n_build, window=window, min_len=min_len)
    seg = O.segment_appended(s, n_build, build, min_len)
    assert seg.n_compressed > build.n_compressed
    rng = np.random.default_rng(8)
    k = rng.standard_normal((s.size, 128))
    v = rng.standard_normal((s.size, 128))
    gc = O.build_group(seg, s, k, v, {}, np.full(s.size, 128), "f32", 128)
    q = rng.standard_normal(128)
    o = O.mixed_attention(q, gc, seg, np.ones(seg.n_compressed, dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, :], torch.from_numpy(k)[None], torch.from_numpy(v)[None])
    assert np.allclose(o, ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)
