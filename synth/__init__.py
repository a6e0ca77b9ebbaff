"""Seeded synthetic inputs for the SeKV decode path and its build step.

This module draws random numbers and nothing else.  It holds no step of the
method: no surprisal statistics, no boundary thresholding, no weighting, no
SVD, no routing and no attention.  Both the CPU oracle (through the tests) and
the HIP library (through the bench and the tests) take their inputs from here,
so the two sides always see the same tensors.

Every tensor is a pure function of (workload, seed, stream name, indices): each
stream gets its own ``torch.Generator`` seeded from a BLAKE2b hash of those
keys, so any (layer, KV head) slice can be regenerated alone, on the CPU or on
a device.  Values drawn on a device differ from those drawn on the CPU; a
parity run draws once, on the device, and copies what the oracle needs.

Workload shapes follow the configurations SeKV is evaluated at (Llama-3.2-3B,
Llama-3-8B and Qwen2.5-14B grouped-query shapes, head dim 128, routing dim 32,
rank cap 32, window 512; SeKV paper, Sec. 3 and the Chinese summary page,
sections 2 and 8).  The surprisal law is the one the workloads name:
Gamma(k=2, theta) plus +6 spikes.  Span keys and values are planted low-rank
blocks plus Gaussian noise, so a truncated SVD has structure to find.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "rng", "surprisal", "planted_segments",
    "span_kv", "kv_cache", "rank_by_pos", "route_weights", "tau_uniform",
    "zoom_targets", "queries", "correlated_queries", "span_gates", "calibration_queries",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    n_tokens: int
    kv_dtype: str                 # "f32" or "bf16": keys, values, means, summaries
    gamma_theta: float            # base surprisal ~ Gamma(k=2, theta)
    spike_frac: float             # fraction of positions that carry a spike
    planted_rank: Tuple[int, int]  # span K/V planted rank, inclusive range
    rank_mode: str                # "uniform": ranks ~ U[4,32] per span start; "planted"
    tau_mode: str                 # "uniform", "calibrated", "skewed", "sweep"
    steps: int
    batch: int = 1
    head_dim: int = 128
    route_dim: int = 32
    window: int = 512
    max_rank: int = 32
    min_span_len: int = 8
    alpha: float = 1.0
    gamma: float = 0.1
    spike_height: float = 6.0
    noise_std: float = 0.05
    zoom_frac: float = 0.05       # calibrated mode: per-head zoom target
    heavy_frac: float = 0.10      # skewed mode: share of (layer, head) pairs that zoom a lot
    heavy_zoom: float = 0.20
    light_zoom: float = 0.01

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Mean span length L gives a spike rate of 1/(L+1): with the small-theta base
# law, spikes are the only positions above mean + 1.0 * std, so the boundaries
# fall on them and spans average L tokens.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        name="tiny", n_layers=1, n_q_heads=4, n_kv_heads=1, n_tokens=4096,
        kv_dtype="f32", gamma_theta=1.5, spike_frac=0.02, planted_rank=(8, 8),
        rank_mode="uniform", tau_mode="uniform", steps=1),
    "llama32_3b_32k": Workload(
        name="llama32_3b_32k", n_layers=28, n_q_heads=24, n_kv_heads=8,
        n_tokens=32768, kv_dtype="bf16", gamma_theta=0.05, spike_frac=1.0 / 61,
        planted_rank=(4, 24), rank_mode="planted", tau_mode="calibrated",
        zoom_frac=0.05, steps=256),
    "llama3_8b_128k": Workload(
        name="llama3_8b_128k", n_layers=32, n_q_heads=32, n_kv_heads=8,
        n_tokens=131072, kv_dtype="bf16", gamma_theta=0.05, spike_frac=1.0 / 81,
        planted_rank=(4, 32), rank_mode="planted", tau_mode="skewed", steps=512),
    "qwen25_14b_128k_b4": Workload(
        name="qwen25_14b_128k_b4", n_layers=48, n_q_heads=40, n_kv_heads=8,
        n_tokens=131072, kv_dtype="bf16", gamma_theta=0.05, spike_frac=1.0 / 81,
        planted_rank=(4, 32), rank_mode="planted", tau_mode="sweep",
        zoom_frac=0.10, batch=4, steps=1024),
    "build_8b_128k": Workload(
        name="build_8b_128k", n_layers=32, n_q_heads=32, n_kv_heads=8,
        n_tokens=131072, kv_dtype="bf16", gamma_theta=0.05, spike_frac=1.0 / 81,
        planted_rank=(4, 32), rank_mode="planted", tau_mode="skewed", steps=1),
}

_SEEDS = {name: i + 1 for i, name in enumerate(WORKLOADS)}


def workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.with_(**overrides) if overrides else wl


def default_seed(wl: Workload) -> int:
    return _SEEDS.get(wl.name, 97)


def rng(seed: int, *keys, device="cpu") -> torch.Generator:
    """A generator private to one stream: BLAKE2b(seed, keys) -> 63-bit seed."""
    h = hashlib.blake2b(repr((int(seed),) + tuple(keys)).encode(), digest_size=8)
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h.digest(), "little") & ((1 << 63) - 1))
    return g


def _uniform_open0(n, g, device):
    # (0, 1]: 1 - U[0, 1) never reaches 0, so its log is finite
    return 1.0 - torch.rand(n, generator=g, device=device, dtype=torch.float64)


def surprisal(wl: Workload, seed: int, seq: int = 0, device="cpu"):
    """Per-token surprisal [N] float32 and the planted spike mask [N] bool.

    Base values are Gamma(k=2, theta), drawn as theta times the sum of two
    unit exponentials; an exact count round(spike_frac * N) of distinct
    positions gets +spike_height on top.
    """
    n = wl.n_tokens
    g = rng(seed, "surprisal", seq, device=device)
    e = -torch.log(_uniform_open0(n, g, device)) - torch.log(_uniform_open0(n, g, device))
    base = wl.gamma_theta * e
    n_spikes = int(round(wl.spike_frac * n))
    pos = torch.randperm(n, generator=g, device=device)[:n_spikes]
    spike = torch.zeros(n, dtype=torch.bool, device=device)
    spike[pos] = True
    s = base + wl.spike_height * spike.to(torch.float64)
    return s.to(torch.float32), spike


def planted_segments(wl: Workload, spike: torch.Tensor):
    """Generator-side block structure: runs of non-spike positions, also cut at
    the start of the last ``window`` positions.  Returns (seg_id [N] int64 with
    -1 on spikes, number of segments).  This is how the K/V blocks are planted,
    not how the method segments (that thresholds surprisal statistics)."""
    n = spike.numel()
    dev = spike.device
    t = torch.arange(n, device=dev)
    prev_spike = torch.ones(n, dtype=torch.bool, device=dev)
    prev_spike[1:] = spike[:-1]
    start = (~spike) & (prev_spike | (t == max(n - wl.window, 0)))
    seg = torch.cumsum(start.to(torch.int64), 0) - 1
    seg = torch.where(spike, torch.full_like(seg, -1), seg)
    return seg, int(start.sum().item())


def span_kv(wl: Workload, seed: int, layer: int, kvh: int, spike: torch.Tensor,
            seg: torch.Tensor, n_seg: int, seq: int = 0, device="cpu", chunk: int = 8192):
    """Keys and values [N][d] float32 for one (layer, KV head), plus the planted
    rank per segment [n_seg] int64.

    Inside each planted segment, X = A B^T + E with A ~ N(0,1) [n x r*],
    B ~ N(0, 1/r*) [d x r*], E ~ N(0, noise_std^2); spike tokens are N(0, 1).
    K and V share r* but draw their own A, B, E.
    """
    n, d = wl.n_tokens, wl.head_dim
    lo, hi = wl.planted_rank
    g = rng(seed, "rank", seq, layer, kvh, device=device)
    r_star = torch.randint(lo, hi + 1, (max(n_seg, 1),), generator=g, device=device)
    seg_c = seg.clamp(min=0)
    cols = torch.arange(hi, device=device)
    out = []
    for which in ("k", "v"):
        g = rng(seed, "kv", which, seq, layer, kvh, device=device)
        a = torch.randn(n, hi, generator=g, device=device)
        a = a * (cols.unsqueeze(0) < r_star[seg_c].unsqueeze(1))
        b = torch.randn(max(n_seg, 1), d, hi, generator=g, device=device)
        b = b * (cols.view(1, 1, -1) < r_star.view(-1, 1, 1))
        b = b / torch.sqrt(r_star.to(torch.float32)).view(-1, 1, 1)
        noise = torch.randn(n, d, generator=g, device=device) * wl.noise_std
        lone = torch.randn(n, d, generator=g, device=device)
        x = torch.empty(n, d, device=device)
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            bg = b[seg_c[c0:c1]].contiguous()
            x[c0:c1] = torch.bmm(bg, a[c0:c1].unsqueeze(-1).contiguous()).squeeze(-1)
        x = x + noise
        x = torch.where(spike.unsqueeze(1), lone, x)
        out.append(x)
    return out[0], out[1], r_star


def _store(x: torch.Tensor, wl: Workload) -> torch.Tensor:
    return x.to(torch.bfloat16) if wl.kv_dtype == "bf16" else x.to(torch.float32)


def kv_cache(wl: Workload, seed: int, spike: torch.Tensor, seq: int = 0, device="cpu",
             layers=None):
    """Full keys and values [L][Hkv][N][d] in the workload's storage dtype
    (bf16 draws are rounded to nearest even from float32 by torch), and the
    per-position rank table [L][Hkv][N] int32.  ``layers`` restricts the draw
    to a subset of layers (the result then has len(layers) layers)."""
    layers = list(range(wl.n_layers)) if layers is None else list(layers)
    seg, n_seg = planted_segments(wl, spike)
    dt = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    L, H, n, d = len(layers), wl.n_kv_heads, wl.n_tokens, wl.head_dim
    k = torch.empty(L, H, n, d, dtype=dt, device=device)
    v = torch.empty(L, H, n, d, dtype=dt, device=device)
    ranks = torch.empty(L, H, n, dtype=torch.int32, device=device)
    for li, layer in enumerate(layers):
        for h in range(H):
            kk, vv, r_star = span_kv(wl, seed, layer, h, spike, seg, n_seg, seq, device)
            k[li, h] = _store(kk, wl)
            v[li, h] = _store(vv, wl)
            ranks[li, h] = rank_by_pos(wl, seed, layer, h, seg, r_star, seq, device)
            del kk, vv
    return k, v, ranks


def rank_by_pos(wl: Workload, seed: int, layer: int, kvh: int, seg: torch.Tensor,
                r_star: torch.Tensor, seq: int = 0, device="cpu") -> torch.Tensor:
    """Requested SVD rank for a span that starts at each position [N] int32.

    "uniform": an independent U[4, 32] draw per position (the tiny workload).
    "planted": the planted rank of the position's segment, so truncation keeps
    the signal and drops only noise.  Capping by the span length and by the
    rank cap is the method's job, not the generator's.
    """
    if wl.rank_mode == "uniform":
        g = rng(seed, "svd_rank", seq, layer, kvh, device=device)
        return torch.randint(4, wl.max_rank + 1, (wl.n_tokens,), generator=g,
                             device=device).to(torch.int32)
    r = r_star[seg.clamp(min=0)]
    r = torch.where(seg < 0, torch.full_like(r, wl.max_rank), r)
    return r.to(torch.int32)


def route_weights(wl: Workload, seed: int, device="cpu"):
    """Summary projection W and query projection P, each [L][Hq][dr][d]
    float32 ~ N(0, std^2) with std = 1/sqrt(d)."""
    shape = (wl.n_layers, wl.n_q_heads, wl.route_dim, wl.head_dim)
    std = 1.0 / math.sqrt(wl.head_dim)
    w = torch.randn(shape, generator=rng(seed, "w_route", device=device), device=device) * std
    p = torch.randn(shape, generator=rng(seed, "p_query", device=device), device=device) * std
    return w, p


def tau_uniform(wl: Workload, seed: int, device="cpu") -> torch.Tensor:
    """Per-(layer, query head) thresholds ~ U(0.4, 0.6), float32 [L][Hq]."""
    g = rng(seed, "tau", device=device)
    u = torch.rand(wl.n_layers, wl.n_q_heads, generator=g, device=device)
    return (0.4 + 0.2 * u).to(torch.float32)


def zoom_targets(wl: Workload, seed: int, frac: Optional[float] = None) -> torch.Tensor:
    """Target share of spans each (layer, query head) should zoom, [L][Hq]
    float64 on the CPU.

    "calibrated"/"sweep": the same share for every head.  "skewed": a random
    heavy_frac of the (layer, head) pairs, taken from layers >= L/3 (zoom-heavy
    heads sit in middle and deep layers), zoom heavy_zoom; the rest light_zoom.
    """
    L, H = wl.n_layers, wl.n_q_heads
    if wl.tau_mode != "skewed":
        f = wl.zoom_frac if frac is None else frac
        return torch.full((L, H), float(f), dtype=torch.float64)
    t = torch.full((L, H), wl.light_zoom, dtype=torch.float64)
    first = L // 3
    pool = (L - first) * H
    n_heavy = int(round(wl.heavy_frac * L * H))
    g = rng(seed, "heavy_heads")
    pick = torch.randperm(pool, generator=g)[:min(n_heavy, pool)]
    t.view(-1)[first * H + pick] = wl.heavy_zoom
    return t


def queries(wl: Workload, seed: int, step: int, seq: int = 0, device="cpu") -> torch.Tensor:
    """Decode query for one step, [L][Hq][d] float32 ~ N(0, 1)."""
    g = rng(seed, "query", seq, step, device=device)
    return torch.randn(wl.n_layers, wl.n_q_heads, wl.head_dim, generator=g, device=device)


def correlated_queries(wl: Workload, seed: int, n: int, rho: float, seq: int = 0,
                       device="cpu") -> torch.Tensor:
    """n consecutive decode queries [n][L][Hq][d] from a stationary AR(1)
    process, q_0 = e_0 and q_t = rho q_{t-1} + sqrt(1 - rho^2) e_t with the
    e_t those of ``queries``: each q_t ~ N(0, 1), neighbouring steps
    correlated by rho (real decoding keeps zooming into many of the same
    spans; independent queries do not).  rho = 0 gives ``queries``."""
    out = torch.empty(n, wl.n_layers, wl.n_q_heads, wl.head_dim, device=device)
    c = math.sqrt(max(0.0, 1.0 - rho * rho))
    for t in range(n):
        e = queries(wl, seed, t, seq=seq, device=device)
        out[t] = e if t == 0 else rho * out[t - 1] + c * e
    return out


def span_gates(wl: Workload, seed: int, n_compressed: int, which: str = "k",
               device="cpu") -> torch.Tensor:
    """Per-component gates of the key (``which`` "k") or value ("v") factors of
    every (layer, KV head, compressed span), [L][Hkv][S_c][max_rank] float32
    in (0, 1): g_i = sigmoid(z_i) with z_i ~ N(3 - 6 i / (R - 1), 1), so
    leading components mostly stay open and trailing ones mostly close (a
    stand-in for a trained gate predictor).  Keys and values draw from streams
    of their own."""
    if which not in ("k", "v"):
        raise ValueError(which)
    R = wl.max_rank
    g = rng(seed, "span_gates", which, device=device)
    mu = 3.0 - 6.0 * torch.arange(R, device=device, dtype=torch.float32) / max(R - 1, 1)
    z = torch.randn(wl.n_layers, wl.n_kv_heads, n_compressed, R, generator=g, device=device)
    return torch.sigmoid(z + mu)


def calibration_queries(wl: Workload, seed: int, n: int = 16, seq: int = 0, device="cpu"):
    """Queries for threshold calibration, [n][L][Hq][d], from a stream of their
    own so measured steps never reuse them."""
    g = rng(seed, "calib", seq, device=device)
    return torch.randn(n, wl.n_layers, wl.n_q_heads, wl.head_dim, generator=g, device=device)
