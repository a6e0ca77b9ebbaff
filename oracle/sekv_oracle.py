"""Plain, slow CPU oracle of SeKV's build step and decode-time attention.

TEST INFRASTRUCTURE.  Only the test suite, the graft entry's smoke check and the
bench's CPU-baseline leg may import or call this module.  The HIP library never
does, and this module imports nothing from it: the two share no code.

Everything is computed in float64 with numpy, in the order the method states
its steps, one span and one head at a time.  Stored quantities the method keeps
in a narrower type (means and summaries in the key/value storage type) are
rounded once, to nearest even, exactly where the method stores them; every
later step reads the rounded value widened back to float64.

Sources (SeKV: Resolution-Adaptive KV Cache with Hierarchical Semantic Memory
for Long-Context LLM Inference, arXiv 2606.31145, and its Chinese-language
summary page).  Most inline symbols are lost in the extracted text; each
function names the passage it follows and the reading taken where the text is
silent.  The readings are:

  * statistics: population mean and std of the surprisal over the whole
    sequence, in float64, two passes; threshold mean + alpha * std (Sec. 3.1;
    summary page sec. 2 gives alpha = 1.0);
  * boundary: strictly greater than the threshold (summary sec. 2 says the
    surprisal must exceed it);
  * the last ``window`` positions are the local window (summary sec. 2: the
    most recent 512 tokens stay at full resolution) and are never anchors or
    span members;
  * spans are the maximal runs of non-anchor positions before the window,
    including a leading and a trailing run (Sec. 3.3: no span is dropped);
  * spans shorter than ``min_span_len`` stay at full resolution (Sec. 3.2 low-
    rank paragraph; the length symbol is lost, 8 is taken);
  * span-local weights w_t = s_t / sum of s over the span, 1/n if that sum is
    zero (Sec. 3.2 summary paragraph: normalized, surprisal-weighted);
  * summary s_{h,j} = W_h kbar_j, which equals the weighted average of the
    projected keys by linearity (Sec. 3.2);
  * gate p = sigmoid(q~ . s + gamma ln n), q~ = P q, no 1/sqrt(d_r) scale,
    natural log; zoom iff p > tau strictly (Sec. 3.2, Sec. 3.3 Eq. 9);
  * factors: exact SVD, hard gates (keep the top r_j components,
    r_j = min(requested rank, n_j, d, R), at least 1); the build takes one
    requested rank per span for its keys and its values alike (Sec. 3.2
    low-rank paragraph, Eq. 8 with 0/1 gates), and soft gates may then leave
    the two with different ranks;
  * attention: one softmax over dense tokens (window, anchors, short-span
    tokens), one coarse entry per non-zoomed span with + ln n_j added to its
    scaled score, and the rank-r reconstruction of every zoomed span's tokens;
    score scale 1/sqrt(d) (Sec. 3.3; summary sec. 3);
  * soft gates (optional, Eq. 8): each retained component i is scaled by its
    gate g_i, components with g_i below a threshold are dropped, at least one
    (the largest gate) is kept; the key matrix and the value matrix of a span
    carry their own gate vectors (Sec. 3.2 low-rank paragraph: the value
    matrix gets the same gated decomposition with its own gates and factors),
    so each keeps its own rank;
  * window append and retire (optional): appended tokens enter the window;
    a token leaving it is an anchor if its surprisal exceeds the build's
    threshold, else it joins the open run, which stays at full resolution
    until the next retired anchor closes it into a span;
  * budget cap (optional): the reconstructed spans' total length is capped,
    per KV head or over the whole layer (one order across its KV heads, the
    step-peak reading of the budget); spans are kept by decreasing gate value
    (the largest over the group's heads that selected them), ties by lower KV
    head then lower id, as long as the total fits (Sec. 3.3, the
    matched-budget paragraph).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round float64 values once, to nearest even, onto the bfloat16 grid
    (8 significant bits), returned as float64.  Valid for zero and for
    magnitudes in the bfloat16 normal range, which is all this method stores."""
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)                 # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)             # numpy rint rounds half to even
    out = np.ldexp(r, e - 8)
    nz = x != 0
    if np.any(nz):
        ax = np.abs(x[nz])
        if ax.min() < 2.0 ** -126 or ax.max() >= 2.0 ** 128:
            raise ValueError("value outside the bfloat16 normal range")
    return out


def round_store(x, dtype: str) -> np.ndarray:
    """Round to the storage type ("bf16" or "f32") and widen back to float64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# segmentation (Sec. 3.1; summary page sec. 2)
# ---------------------------------------------------------------------------

def surprisal_threshold(s, alpha: float) -> Tuple[float, float, float]:
    """Mean, population std and boundary threshold mean + alpha * std of the
    surprisal over the whole sequence, all in float64 (two passes)."""
    s = np.asarray(s, dtype=F64)
    n = s.size
    if n == 0:
        raise ValueError("empty sequence")
    total = 0.0
    for v in s:
        total += float(v)
    mu = total / n
    ss = 0.0
    for v in s:
        ss += (float(v) - mu) ** 2
    sigma = math.sqrt(ss / n)
    return mu, sigma, mu + float(alpha) * sigma


@dataclasses.dataclass
class Segmentation:
    n_tokens: int
    window: int
    mu: float
    sigma: float
    threshold: float
    anchors: np.ndarray        # ascending anchor positions, int64
    span_start: np.ndarray     # every span, ascending, int64
    span_len: np.ndarray
    kind: np.ndarray           # 0 = compressed (summary + factors), 1 = short (full resolution)
    cspan: np.ndarray          # indices (into span_*) of the compressed spans, ascending
    dense_pos: np.ndarray      # ascending positions kept at full resolution
    open_start: int = 0        # after appends: the open run of retired tokens (not yet a span)
    open_len: int = 0

    @property
    def n_compressed(self) -> int:
        return int(self.cspan.size)


def segment(s, window: int, alpha: float, min_span_len: int) -> Segmentation:
    """Anchors are positions before the window whose surprisal exceeds the
    threshold; spans are the maximal runs of other positions before the window;
    spans of at least ``min_span_len`` tokens are compressed, shorter ones join
    the full-resolution set together with the anchors and the window."""
    s = np.asarray(s, dtype=F64)
    n = s.size
    mu, sigma, thr = surprisal_threshold(s, alpha)
    limit = max(n - int(window), 0)
    is_anchor = [float(s[t]) > thr for t in range(limit)]
    anchors = [t for t in range(limit) if is_anchor[t]]
    starts: List[int] = []
    lens: List[int] = []
    t = 0
    while t < limit:
        if is_anchor[t]:
            t += 1
            continue
        begin = t
        while t < limit and not is_anchor[t]:
            t += 1
        starts.append(begin)
        lens.append(t - begin)
    kind = [0 if ln >= min_span_len else 1 for ln in lens]
    dense = set(anchors)
    for b, ln, k in zip(starts, lens, kind):
        if k == 1:
            dense.update(range(b, b + ln))
    dense.update(range(limit, n))
    return Segmentation(
        n_tokens=n, window=int(window), mu=mu, sigma=sigma, threshold=thr,
        anchors=np.array(anchors, dtype=np.int64),
        span_start=np.array(starts, dtype=np.int64),
        span_len=np.array(lens, dtype=np.int64),
        kind=np.array(kind, dtype=np.int64),
        cspan=np.array([i for i, k in enumerate(kind) if k == 0], dtype=np.int64),
        dense_pos=np.array(sorted(dense), dtype=np.int64),
    )


def segment_appended(s, n_build: int, build: Segmentation, min_span_len: int) -> Segmentation:
    """The segmentation of a cache built over the first ``n_build`` tokens of
    ``s`` after the remaining tokens were appended one decode step at a time.

    Reading taken (the pages say every decode step attends over the
    mixed-resolution memory and the most recent ``window`` tokens stay at full
    resolution, and are silent on how tokens leave the window): an appended
    token enters the window at full resolution; a token that leaves the window
    is compared with the build's threshold (the prompt's statistics, which the
    method computes once): above it, it becomes an anchor; otherwise it joins
    the open run, the retired non-anchor tokens since the last retired anchor,
    which stay at full resolution until the next retired anchor closes the run
    into a span (compressed if at least ``min_span_len`` tokens long, else kept
    at full resolution like any short span).  What the build made stays as it
    is."""
    s = np.asarray(s, dtype=F64)
    n = s.size
    w = build.window
    thr = build.threshold
    r0, r1 = max(n_build - w, 0), max(n - w, 0)   # positions retired by the appends
    anchors = list(build.anchors)
    starts, lens = list(build.span_start), list(build.span_len)
    run_start, run_len = r0, 0
    for t in range(r0, r1):
        if float(s[t]) > thr:
            if run_len:
                starts.append(run_start)
                lens.append(run_len)
            anchors.append(t)
            run_start, run_len = t + 1, 0
        else:
            if run_len == 0:
                run_start = t
            run_len += 1
    kind = [0 if ln >= min_span_len else 1 for ln in lens]
    dense = set(anchors)
    for b, ln, k in zip(starts, lens, kind):
        if k == 1:
            dense.update(range(b, b + ln))
    dense.update(range(run_start, run_start + run_len))
    dense.update(range(r1, n))
    return Segmentation(
        n_tokens=n, window=w, mu=build.mu, sigma=build.sigma, threshold=thr,
        anchors=np.array(anchors, dtype=np.int64),
        span_start=np.array(starts, dtype=np.int64), span_len=np.array(lens, dtype=np.int64),
        kind=np.array(kind, dtype=np.int64),
        cspan=np.array([i for i, k in enumerate(kind) if k == 0], dtype=np.int64),
        dense_pos=np.array(sorted(dense), dtype=np.int64),
        open_start=run_start if run_len else 0, open_len=run_len)


# ---------------------------------------------------------------------------
# span representations (Sec. 3.2)
# ---------------------------------------------------------------------------

def span_weights(s_span) -> np.ndarray:
    """Normalized span-local surprisal weights: w_t = s_t / sum_span s."""
    s_span = np.asarray(s_span, dtype=F64)
    total = float(np.sum(s_span))
    if total == 0.0:
        return np.full(s_span.size, 1.0 / s_span.size)
    return s_span / total


def weighted_mean(w, x) -> np.ndarray:
    """sum_t w_t x_t over the span's token rows (float64)."""
    return np.asarray(w, dtype=F64) @ np.asarray(x, dtype=F64)


def span_rank(requested: int, n: int, d: int, rank_cap: int) -> int:
    """Retained rank: the request capped by span length, head dim and the rank
    cap R, and at least one component."""
    return int(max(1, min(int(requested), n, d, rank_cap)))


@dataclasses.dataclass
class Factors:
    u: np.ndarray      # [n][r] left singular vectors
    sigma: np.ndarray  # [r]    singular values, descending
    vt: np.ndarray     # [r][d] right singular vectors (rows)
    tail2: float       # sum of the discarded sigma^2

    def reconstruct(self) -> np.ndarray:
        return (self.u * self.sigma) @ self.vt


def truncated_svd(x, r: int) -> Factors:
    """Exact SVD of the span's [n][d] token matrix, keeping the top r
    components (hard gates in the gated reconstruction, Eq. 8)."""
    x = np.asarray(x, dtype=F64)
    u, sig, vt = np.linalg.svd(x, full_matrices=False)
    return Factors(u=u[:, :r].copy(), sigma=sig[:r].copy(), vt=vt[:r].copy(),
                   tail2=float(np.sum(sig[r:] ** 2)))


def gate_factors(f: Factors, gates, eps: float) -> Factors:
    """Gated reconstruction (Eq. 8): component i of the retained factors is
    scaled by its gate g_i in [0, 1], K^ = U diag(g * sigma) V^T, and
    components whose gate is negligible (g_i < eps) are dropped from storage.

    Reading taken: gate i belongs to the i-th largest singular value; the kept
    components keep their order; a span keeps at least one component (as the
    hard-gate rank is at least one), the one with the largest gate (lowest
    index on ties), when every gate is negligible.  ``tail2`` of the result is
    not set (nan): the reconstruction error of soft gates is no longer the
    discarded energy alone."""
    r = f.sigma.size
    g = np.asarray(gates, dtype=F64)[:r]
    kept = [i for i in range(r) if g[i] >= eps]
    if not kept:
        kept = [int(np.argmax(g))]
    kept = np.array(kept, dtype=np.int64)
    return Factors(u=f.u[:, kept].copy(), sigma=f.sigma[kept] * g[kept], vt=f.vt[kept].copy(),
                   tail2=float("nan"))


def gate_group(gc: "GroupCache", key_gates, value_gates, eps: float) -> "GroupCache":
    """The group with every span's key factors gated by its key gates and its
    value factors by its value gates (Eq. 8 applied to each matrix, Sec. 3.2:
    the value matrix has gates and factors of its own).  ``key_gates`` and
    ``value_gates`` are [S_c][R]; gate i of a span belongs to the i-th largest
    singular value of that matrix.  Keys and values then keep their own ranks
    (``rank`` and ``vrank``)."""
    kf = [gate_factors(f, key_gates[i], eps) for i, f in enumerate(gc.kfac)]
    vf = [gate_factors(f, value_gates[i], eps) for i, f in enumerate(gc.vfac)]
    return dataclasses.replace(gc, kfac=kf, vfac=vf,
                               rank=np.array([f.sigma.size for f in kf], dtype=np.int64),
                               vrank=np.array([f.sigma.size for f in vf], dtype=np.int64))


@dataclasses.dataclass
class GroupCache:
    """What one (layer, KV head) keeps: the full-resolution rows, each
    compressed span's coarse mean key/value (rounded to storage), the routing
    summaries of every query head in the group (rounded to storage), and the
    span factors of keys and values."""
    dense_k: np.ndarray              # [D][d]
    dense_v: np.ndarray
    kbar: np.ndarray                 # [S_c][d], rounded to storage
    vbar: np.ndarray
    summary: Dict[int, np.ndarray]   # query head -> [S_c][d_r], rounded to storage
    kfac: List[Factors]
    vfac: List[Factors]
    rank: np.ndarray                 # [S_c] retained rank of the key factors
    vrank: np.ndarray                # [S_c] retained rank of the value factors


def build_group(seg: Segmentation, s, k, v, w_route: Dict[int, np.ndarray], ranks_by_pos,
                kv_dtype: str, rank_cap: int, with_factors: bool = True) -> GroupCache:
    """Build the cache of one (layer, KV head) from its keys and values
    ``k``, ``v`` [N][d] (stored values widened to float64), the surprisal ``s``,
    each of its query heads' summary projection W_h [d_r][d], and the
    requested rank of the span that starts at each position."""
    s = np.asarray(s, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    d = k.shape[1]
    kbar, vbar, ranks, kfac, vfac = [], [], [], [], []
    summ = {h: [] for h in w_route}
    for j in seg.cspan:
        b, n = int(seg.span_start[j]), int(seg.span_len[j])
        w = span_weights(s[b:b + n])
        km = weighted_mean(w, k[b:b + n])
        vm = weighted_mean(w, v[b:b + n])
        kbar.append(round_store(km, kv_dtype))
        vbar.append(round_store(vm, kv_dtype))
        for h, wh in w_route.items():
            summ[h].append(round_store(np.asarray(wh, dtype=F64) @ km, kv_dtype))
        r = span_rank(int(ranks_by_pos[b]), n, d, rank_cap)
        ranks.append(r)
        if with_factors:
            kfac.append(truncated_svd(k[b:b + n], r))
            vfac.append(truncated_svd(v[b:b + n], r))
    sc = len(kbar)
    dr = next(iter(w_route.values())).shape[0] if w_route else 0
    return GroupCache(
        dense_k=k[seg.dense_pos], dense_v=v[seg.dense_pos],
        kbar=np.array(kbar).reshape(sc, d), vbar=np.array(vbar).reshape(sc, d),
        summary={h: np.array(x).reshape(sc, dr) for h, x in summ.items()},
        kfac=kfac, vfac=vfac, rank=np.array(ranks, dtype=np.int64),
        vrank=np.array(ranks, dtype=np.int64))


# ---------------------------------------------------------------------------
# decode: routing (Sec. 3.2 gate, Sec. 3.3 Eq. 9)
# ---------------------------------------------------------------------------

def span_log_len(seg: Segmentation) -> np.ndarray:
    """ln n_j of every compressed span, float64."""
    return np.log(seg.span_len[seg.cspan].astype(F64))


def route_head(q, p_proj, summary, log_len, gamma: float, tau: float):
    """Gate and zoom decision of every compressed span for one query head.

    q~ = P q; x_j = q~ . s_j + gamma ln n_j; p_j = 1 / (1 + e^-x_j);
    zoom iff p_j > tau.  Returns (p [S_c] float64, zoom [S_c] bool)."""
    qt = np.asarray(p_proj, dtype=F64) @ np.asarray(q, dtype=F64)
    x = np.asarray(summary, dtype=F64) @ qt + float(gamma) * np.asarray(log_len, dtype=F64)
    p = 1.0 / (1.0 + np.exp(-x))
    return p, p > float(tau)


def compact(mask) -> np.ndarray:
    """Ascending ids of the set entries."""
    return np.array([j for j, z in enumerate(mask) if z], dtype=np.int64)


def union_lists(masks: Sequence[np.ndarray]) -> np.ndarray:
    """Ascending ids zoomed by at least one head of a group."""
    if not masks:
        return np.zeros(0, dtype=np.int64)
    return compact(np.logical_or.reduce([np.asarray(m, dtype=bool) for m in masks]))


# ---------------------------------------------------------------------------
# decode: mixed-resolution attention (Sec. 3.3; summary sec. 3)
# ---------------------------------------------------------------------------

def mixed_attention(q, gc: GroupCache, seg: Segmentation, zoom) -> np.ndarray:
    """One softmax over every entry the head sees: full-resolution rows; one
    coarse entry (kbar_j, vbar_j) with + ln n_j for each non-zoomed span; the
    rank-r_j reconstructed rows of each zoomed span.  Returns o [d] float64."""
    q = np.asarray(q, dtype=F64)
    d = q.size
    scale = 1.0 / math.sqrt(d)
    log_len = span_log_len(seg)
    keys = [gc.dense_k]
    vals = [gc.dense_v]
    bias = [np.zeros(gc.dense_k.shape[0])]
    for i in range(seg.n_compressed):
        if zoom[i]:
            kr = gc.kfac[i].reconstruct()
            keys.append(kr)
            vals.append(gc.vfac[i].reconstruct())
            bias.append(np.zeros(kr.shape[0]))
        else:
            keys.append(gc.kbar[i:i + 1])
            vals.append(gc.vbar[i:i + 1])
            bias.append(np.array([log_len[i]]))
    kk = np.concatenate(keys, axis=0)
    vv = np.concatenate(vals, axis=0)
    e = scale * (kk @ q) + np.concatenate(bias)
    m = np.max(e)
    a = np.exp(e - m)
    return (a @ vv) / np.sum(a)


# ---------------------------------------------------------------------------
# one decode step of one layer
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LayerRoute:
    prob: np.ndarray      # [Hq][S_c] float64
    mask: np.ndarray      # [Hq][S_c] bool
    lists: List[np.ndarray]
    unions: List[np.ndarray]


def route_layer(q, p_proj, tau, summaries: Dict[int, np.ndarray], seg: Segmentation,
                gamma: float, n_kv_heads: int) -> LayerRoute:
    """Route every query head of a layer and form the per-group unions.
    ``summaries`` maps each query head to its [S_c][d_r] summaries."""
    hq = len(q)
    group = hq // n_kv_heads
    ll = span_log_len(seg)
    probs, masks = [], []
    for h in range(hq):
        p, z = route_head(q[h], p_proj[h], summaries[h], ll, gamma, float(tau[h]))
        probs.append(p)
        masks.append(z)
    lists = [compact(z) for z in masks]
    unions = [union_lists(masks[g * group:(g + 1) * group]) for g in range(n_kv_heads)]
    sc = seg.n_compressed
    return LayerRoute(prob=np.array(probs).reshape(hq, sc), mask=np.array(masks).reshape(hq, sc),
                      lists=lists, unions=unions)


def cap_budget(route: LayerRoute, seg: Segmentation, n_kv_heads: int, budget: int,
               scope: str = "kv_head") -> LayerRoute:
    """The matched-budget cap of the zoom decisions (Sec. 3.3, zoom-in decoding:
    when the selected spans exceed the budget, spans are kept in decreasing
    order of their gate value until the budget is filled).

    Reading taken: a candidate is a span in a KV head's union; its order key is
    the largest gate value among the group's heads that selected it; its cost is
    its length n_j (the tokens that KV head reconstructs).  With scope
    "kv_head" each KV head is capped on its own, ties going to the lower span
    id.  With scope "layer" one order runs over the candidates of every KV head
    of the layer (ties to the lower KV head, then the lower span id) and the
    budget bounds their total: Sec. 3.3 defines the budget as the peak
    GPU-resident KV of a decoding step including the spans reconstructed at
    that step, and a step reaches its peak inside one layer, whose
    reconstructed spans are needed only while it attends.  The kept
    candidates are the longest prefix of the order whose total length is at
    most ``budget``; a kept span stays zoomed for the heads that selected it,
    a dropped one reverts to its coarse entry for all of them."""
    if scope not in ("kv_head", "layer"):
        raise ValueError(scope)
    hq = route.mask.shape[0]
    group = hq // n_kv_heads
    n = seg.span_len[seg.cspan].astype(np.int64)
    mask = route.mask.copy()
    cands = []   # (key, g, j)
    for g in range(n_kv_heads):
        heads = range(g * group, (g + 1) * group)
        for j in union_lists([route.mask[h] for h in heads]):
            key = max(route.prob[h, j] for h in heads if route.mask[h, j])
            cands.append((float(key), g, int(j)))
    kept = set()
    groups = [list(range(n_kv_heads))] if scope == "layer" else [[g] for g in range(n_kv_heads)]
    for gs in groups:
        order = sorted((c for c in cands if c[1] in gs), key=lambda c: (-c[0], c[1], c[2]))
        total = 0
        for key, g, j in order:
            if total + n[j] > budget:
                break
            total += n[j]
            kept.add((g, j))
    for h in range(hq):
        g = h // group
        for j in np.flatnonzero(mask[h]):
            if (g, int(j)) not in kept:
                mask[h, j] = False
    lists = [compact(z) for z in mask]
    unions = [union_lists(list(mask[g * group:(g + 1) * group])) for g in range(n_kv_heads)]
    return LayerRoute(prob=route.prob, mask=mask, lists=lists, unions=unions)


def decode_layer(q, route: LayerRoute, groups: Dict[int, GroupCache], seg: Segmentation,
                 heads: Optional[Sequence[int]] = None, n_kv_heads: int = 1) -> Dict[int, np.ndarray]:
    """Attention output of the given query heads of one layer (all by default);
    ``groups`` maps KV head -> GroupCache."""
    hq = len(q)
    group = hq // n_kv_heads
    heads = range(hq) if heads is None else heads
    return {h: mixed_attention(q[h], groups[h // group], seg, route.mask[h]) for h in heads}
