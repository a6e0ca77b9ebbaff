"""SeKV decode-time attention on AMD Instinct MI355X: Python binding.

A thin ctypes layer over ``libsekv.so`` (the C ABI of include/sekv.h).  The
functions here marshal torch tensors into device pointers and streams and call
the library; every step of the build and of the decode step runs in the HIP
kernels behind that ABI.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "SekvError", "SekvConfig", "SekvCacheInfo", "SekvRouteOut", "lib", "library_path",
    "make_config", "Cache", "RouteBuffers", "sekv_segment", "sekv_build_spans", "sekv_route",
    "sekv_decode_attn", "sekv_route_attn", "sekv_decode_attn_batch", "sekv_route_attn_batch",
    "sekv_cap_budget", "sekv_cap_budget_layer", "sekv_decode_workspace_bytes",
    "sekv_append_tokens", "sekv_test_fail_fetch",
    "EXPORTED_SYMBOLS",
    "sekv_set_residency", "sekv_residency_stats", "sekv_apply_gates", "SEKV_MAX_BATCH",
    "SEKV_F32", "SEKV_BF16", "SEKV_TIER_DEVICE", "SEKV_TIER_HOST_PINNED",
    "SEKV_SVD_EXACT", "SEKV_SVD_RANDOMIZED", "sekv_route_attn_noalloc",
    "SEKV_NOALLOC_SCRATCH_BYTES", "SEKV_FETCH_GATHER", "SEKV_FETCH_MEMCPY",
]

SEKV_OK, SEKV_ERR_INVALID, SEKV_ERR_NOMEM, SEKV_ERR_HIP, SEKV_ERR_UNSUPPORTED = range(5)
SEKV_F32, SEKV_BF16 = 0, 1
SEKV_TIER_DEVICE, SEKV_TIER_HOST_PINNED = 0, 1
SEKV_FETCH_GATHER, SEKV_FETCH_MEMCPY = 0, 1
SEKV_SVD_EXACT, SEKV_SVD_RANDOMIZED = 0, 1
SEKV_MAX_BATCH = 8
SEKV_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024

EXPORTED_SYMBOLS = (
    "sekv_segment", "sekv_build_spans", "sekv_cache_info_get", "sekv_cache_copy_spans",
    "sekv_cache_copy_group", "sekv_cache_copy_factors", "sekv_route",
    "sekv_decode_workspace_bytes", "sekv_decode_attn", "sekv_route_attn",
    "sekv_decode_attn_batch", "sekv_route_attn_batch", "sekv_cap_budget", "sekv_set_residency",
    "sekv_residency_stats", "sekv_apply_gates", "sekv_cache_destroy", "sekv_last_error",
    "sekv_route_attn_noalloc", "sekv_cap_budget_layer", "sekv_append_tokens",
    "sekv_test_fail_fetch", "sekv_set_fetch_mode",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("SEKV_LIBRARY", os.path.join(_HERE, "libsekv.so"))


class SekvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sekv status {status}: {msg}")
        self.status = status


class SekvConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("route_dim", ctypes.c_int32), ("window", ctypes.c_int32),
        ("max_rank", ctypes.c_int32), ("min_span_len", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("gamma", ctypes.c_double),
        ("kv_dtype", ctypes.c_int32), ("factor_tier", ctypes.c_int32),
        ("host_pool_cap_bytes", ctypes.c_uint64),
        ("svd_mode", ctypes.c_int32), ("append_capacity", ctypes.c_int32),
    ]


class SekvCacheInfo(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int32), ("n_anchors", ctypes.c_int32),
        ("n_spans", ctypes.c_int32), ("n_compressed", ctypes.c_int32),
        ("n_dense", ctypes.c_int32), ("factor_tier", ctypes.c_int32),
        ("mu", ctypes.c_double), ("sigma", ctypes.c_double), ("threshold", ctypes.c_double),
        ("resident_bytes", ctypes.c_uint64), ("factor_bytes", ctypes.c_uint64),
        ("factor_pool_bytes", ctypes.c_uint64),
        ("open_start", ctypes.c_int32), ("open_len", ctypes.c_int32),
        ("n_appended", ctypes.c_int32), ("append_capacity", ctypes.c_int32),
    ]


class SekvRouteOut(ctypes.Structure):
    _fields_ = [
        ("mask", ctypes.c_void_p), ("list", ctypes.c_void_p), ("count", ctypes.c_void_p),
        ("union_list", ctypes.c_void_p), ("union_count", ctypes.c_void_p),
        ("prob", ctypes.c_void_p),
    ]


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libsekv.so (once) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"SeKV HIP library not found at {path}; build it with "
                          "`python -m compressed_kv_attention_sekv_amd.build`")
    L = ctypes.CDLL(path)
    P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    I32P = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "sekv_segment": (I32, [ctypes.POINTER(SekvConfig), I32, P, I32P, I32P, I32P, P]),
        "sekv_build_spans": (I32, [ctypes.POINTER(SekvConfig), I32, P, P, P, P, P, P,
                                   ctypes.POINTER(P)]),
        "sekv_cache_info_get": (I32, [P, ctypes.POINTER(SekvCacheInfo)]),
        "sekv_cache_copy_spans": (I32, [P, P, P, P, P, P, P]),
        "sekv_cache_copy_group": (I32, [P, I32, I32, P, P, P, P, P]),
        "sekv_cache_copy_factors": (I32, [P, I32, I32, I32, I32, P, P, P]),
        "sekv_route": (I32, [P, I32, P, P, P, ctypes.POINTER(SekvRouteOut), P]),
        "sekv_decode_workspace_bytes": (SZ, [P]),
        "sekv_decode_attn": (I32, [P, I32, P, ctypes.POINTER(SekvRouteOut), P, P, SZ, P, P]),
        "sekv_route_attn": (I32, [P, I32, P, P, P, ctypes.POINTER(SekvRouteOut), P, P, SZ, P,
                                  P]),
        "sekv_route_attn_noalloc": (I32, [P, I32, P, P, P, ctypes.POINTER(SekvRouteOut), P,
                                          P, P]),
        "sekv_route_attn_batch": (I32, [ctypes.POINTER(P), I32, I32, ctypes.POINTER(P), P, P,
                                        ctypes.POINTER(SekvRouteOut), ctypes.POINTER(P),
                                        ctypes.POINTER(P), ctypes.POINTER(SZ), P]),
        "sekv_decode_attn_batch": (I32, [ctypes.POINTER(P), I32, I32, ctypes.POINTER(P),
                                         ctypes.POINTER(SekvRouteOut), ctypes.POINTER(P),
                                         ctypes.POINTER(P), ctypes.POINTER(SZ), P]),
        "sekv_cap_budget": (I32, [P, ctypes.POINTER(SekvRouteOut), ctypes.c_int64, P]),
        "sekv_cap_budget_layer": (I32, [P, ctypes.POINTER(SekvRouteOut), ctypes.c_int64, P]),
        "sekv_append_tokens": (I32, [P, I32, P, P, P, P, P, P]),
        "sekv_set_residency": (I32, [P, U64, U64]),
        "sekv_apply_gates": (I32, [P, P, P, ctypes.c_float, P]),
        "sekv_residency_stats": (I32, [P, ctypes.POINTER(U64), I32]),
        "sekv_test_fail_fetch": (I32, [I32]),
        "sekv_set_fetch_mode": (I32, [P, I32]),
        "sekv_cache_destroy": (None, [P]),
        "sekv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    del U64
    _LIB = L
    return L


def _check(status: int) -> None:
    if status != SEKV_OK:
        raise SekvError(status, lib().sekv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_config(n_layers: int, n_q_heads: int, n_kv_heads: int, *, head_dim: int = 128,
                route_dim: int = 32, window: int = 512, max_rank: int = 32,
                min_span_len: int = 8, alpha: float = 1.0, gamma: float = 0.1,
                kv_dtype: str = "bf16", factor_tier: str = "device",
                host_pool_cap_bytes: int = 0, svd: str = "exact",
                append_capacity: int = 0) -> SekvConfig:
    return SekvConfig(n_layers, n_q_heads, n_kv_heads, head_dim, route_dim, window, max_rank,
                      min_span_len, float(alpha), float(gamma),
                      SEKV_BF16 if kv_dtype == "bf16" else SEKV_F32,
                      SEKV_TIER_HOST_PINNED if factor_tier == "host" else SEKV_TIER_DEVICE,
                      int(host_pool_cap_bytes),
                      SEKV_SVD_RANDOMIZED if svd == "randomized" else SEKV_SVD_EXACT,
                      int(append_capacity))


def sekv_segment(cfg: SekvConfig, surprisal: torch.Tensor, stream=None):
    """(n_anchors, n_spans, n_compressed) of a surprisal sequence."""
    _need(surprisal, "surprisal", torch.float32)
    a, s, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().sekv_segment(ctypes.byref(cfg), surprisal.numel(), _ptr(surprisal),
                              ctypes.byref(a), ctypes.byref(s), ctypes.byref(c), _stream(stream)))
    return a.value, s.value, c.value


@dataclasses.dataclass
class RouteBuffers:
    """Device buffers of one layer's route output, allocated with torch."""
    mask: torch.Tensor
    list: torch.Tensor
    count: torch.Tensor
    union_list: torch.Tensor
    union_count: torch.Tensor
    prob: Optional[torch.Tensor]

    @classmethod
    def allocate(cls, cache: "Cache", with_prob: bool = False, device="cuda"):
        hq, hkv, sc = cache.cfg.n_q_heads, cache.cfg.n_kv_heads, max(cache.info.n_compressed, 1)
        return cls(
            mask=torch.zeros(hq, sc, dtype=torch.uint8, device=device),
            list=torch.zeros(hq, sc, dtype=torch.int32, device=device),
            count=torch.zeros(hq, dtype=torch.int32, device=device),
            union_list=torch.zeros(hkv, sc, dtype=torch.int32, device=device),
            union_count=torch.zeros(hkv, dtype=torch.int32, device=device),
            prob=torch.zeros(hq, sc, dtype=torch.float64, device=device) if with_prob else None)

    def struct(self) -> SekvRouteOut:
        return SekvRouteOut(self.mask.data_ptr(), self.list.data_ptr(), self.count.data_ptr(),
                            self.union_list.data_ptr(), self.union_count.data_ptr(),
                            self.prob.data_ptr() if self.prob is not None else None)


class Cache:
    """Owns an sekv_cache handle; destroyed with the object."""

    def __init__(self, handle: ctypes.c_void_p, cfg: SekvConfig):
        self.handle = handle
        self.cfg = cfg
        info = SekvCacheInfo()
        _check(lib().sekv_cache_info_get(handle, ctypes.byref(info)))
        self.info = info

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _LIB is not None:
            _LIB.sekv_cache_destroy(h)
            self.handle = None

    @property
    def group(self) -> int:
        return self.cfg.n_q_heads // self.cfg.n_kv_heads

    def spans(self):
        """Span table as CPU int tensors."""
        i = self.info
        t = {k: torch.zeros(max(n, 1), dtype=torch.int32) for k, n in (
            ("anchors", i.n_anchors), ("span_start", i.n_spans), ("span_len", i.n_spans),
            ("cspan", i.n_compressed), ("dense_pos", i.n_dense))}
        kind = torch.zeros(max(i.n_spans, 1), dtype=torch.uint8)
        _check(lib().sekv_cache_copy_spans(self.handle, _ptr(t["anchors"]), _ptr(t["span_start"]),
                                           _ptr(t["span_len"]), _ptr(kind), _ptr(t["cspan"]),
                                           _ptr(t["dense_pos"])))
        out = {"anchors": t["anchors"][:i.n_anchors], "span_start": t["span_start"][:i.n_spans],
               "span_len": t["span_len"][:i.n_spans], "kind": kind[:i.n_spans],
               "cspan": t["cspan"][:i.n_compressed], "dense_pos": t["dense_pos"][:i.n_dense]}
        return out

    def group_data(self, layer: int, kv_head: int):
        """(kbar, vbar, summaries [G][S_c][dr], key ranks, value ranks) of one
        (layer, KV head), CPU tensors."""
        sc, d, dr, g = self.info.n_compressed, self.cfg.head_dim, self.cfg.route_dim, self.group
        dt = torch.bfloat16 if self.cfg.kv_dtype == SEKV_BF16 else torch.float32
        kb = torch.zeros(max(sc, 1), d, dtype=dt)
        vb = torch.zeros(max(sc, 1), d, dtype=dt)
        sm = torch.zeros(g, max(sc, 1), dr, dtype=dt)
        rk = torch.zeros(max(sc, 1), dtype=torch.int32)
        rv = torch.zeros(max(sc, 1), dtype=torch.int32)
        _check(lib().sekv_cache_copy_group(self.handle, layer, kv_head, _ptr(kb), _ptr(vb),
                                           _ptr(sm), _ptr(rk), _ptr(rv)))
        return kb[:sc], vb[:sc], sm[:, :sc].contiguous() if sc else sm[:, :0], rk[:sc], rv[:sc]

    def factors(self, layer: int, kv_head: int, span: int, kv: int, rank: int, n: int):
        u = torch.zeros(n, rank, dtype=torch.float32)
        s = torch.zeros(rank, dtype=torch.float32)
        vt = torch.zeros(rank, self.cfg.head_dim, dtype=torch.float32)
        _check(lib().sekv_cache_copy_factors(self.handle, layer, kv_head, span, kv, _ptr(u),
                                             _ptr(s), _ptr(vt)))
        return u, s, vt

    def workspace_bytes(self) -> int:
        return int(lib().sekv_decode_workspace_bytes(self.handle))

    def set_residency(self, capacity_bytes: int, slot_bytes: int = 64 * 1024) -> None:
        """Enable (capacity > 0) or disable the HBM residency cache of a
        host-tier cache's factor blocks."""
        _check(lib().sekv_set_residency(self.handle, int(capacity_bytes), int(slot_bytes)))

    def set_fetch_mode(self, mode: str) -> None:
        """Host tier: "gather" (one kernel, default) or "memcpy" (hipMemcpyAsync
        per run of union spans) for the factor fetch."""
        modes = {"gather": SEKV_FETCH_GATHER, "memcpy": SEKV_FETCH_MEMCPY}
        if mode not in modes:
            raise ValueError(f"fetch mode must be one of {sorted(modes)}")
        _check(lib().sekv_set_fetch_mode(self.handle, modes[mode]))

    def residency_stats(self, reset: bool = False) -> dict:
        out = (ctypes.c_uint64 * 6)()
        _check(lib().sekv_residency_stats(self.handle, out, 1 if reset else 0))
        return {"hit_blocks": out[0], "fetched_blocks": out[1], "hit_bytes": out[2],
                "fetched_bytes": out[3], "sets": out[4], "slot_bytes": out[5]}


def sekv_build_spans(cfg: SekvConfig, surprisal: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     w_route: torch.Tensor, rank_by_pos: Optional[torch.Tensor] = None,
                     stream=None) -> Cache:
    """Build the cache; shapes as in include/sekv.h."""
    _need(surprisal, "surprisal", torch.float32)
    kv_dt = torch.bfloat16 if cfg.kv_dtype == SEKV_BF16 else torch.float32
    _need(k, "k", kv_dt)
    _need(v, "v", kv_dt)
    _need(w_route, "w_route", torch.float32)
    n = surprisal.numel()
    shape = (cfg.n_layers, cfg.n_kv_heads, n, cfg.head_dim)
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError(f"k and v must be {shape}")
    if tuple(w_route.shape) != (cfg.n_layers, cfg.n_q_heads, cfg.route_dim, cfg.head_dim):
        raise ValueError("w_route must be [L][Hq][dr][d]")
    if rank_by_pos is not None:
        _need(rank_by_pos, "rank_by_pos", torch.int32)
        if tuple(rank_by_pos.shape) != (cfg.n_layers, cfg.n_kv_heads, n):
            raise ValueError("rank_by_pos must be [L][Hkv][N]")
    h = ctypes.c_void_p()
    _check(lib().sekv_build_spans(ctypes.byref(cfg), n, _ptr(surprisal), _ptr(k), _ptr(v),
                                  _ptr(w_route), _ptr(rank_by_pos), _stream(stream),
                                  ctypes.byref(h)))
    return Cache(h, cfg)


def sekv_test_fail_fetch(n: int) -> None:
    """Test hook: the next ``n`` host-tier factor fetches fail (SekvError)."""
    _check(lib().sekv_test_fail_fetch(int(n)))


def sekv_append_tokens(cache: Cache, surprisal: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       w_route: torch.Tensor, rank: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """Append decode tokens to the window and retire those that leave it
    (shapes as in include/sekv.h); refreshes ``cache.info``."""
    c = cache.cfg
    _need(surprisal, "surprisal", torch.float32)
    kv_dt = torch.bfloat16 if c.kv_dtype == SEKV_BF16 else torch.float32
    _need(k, "k", kv_dt)
    _need(v, "v", kv_dt)
    _need(w_route, "w_route", torch.float32)
    n = surprisal.numel()
    shape = (c.n_layers, c.n_kv_heads, n, c.head_dim)
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError(f"k and v must be {shape}")
    if tuple(w_route.shape) != (c.n_layers, c.n_q_heads, c.route_dim, c.head_dim):
        raise ValueError("w_route must be [L][Hq][dr][d]")
    if rank is not None:
        _need(rank, "rank", torch.int32)
        if tuple(rank.shape) != (c.n_layers, c.n_kv_heads, n):
            raise ValueError("rank must be [L][Hkv][n_new]")
    _check(lib().sekv_append_tokens(cache.handle, n, _ptr(surprisal), _ptr(k), _ptr(v),
                                    _ptr(w_route), _ptr(rank), _stream(stream)))
    info = SekvCacheInfo()
    _check(lib().sekv_cache_info_get(cache.handle, ctypes.byref(info)))
    cache.info = info


def sekv_route(cache: Cache, layer: int, q: torch.Tensor, proj: torch.Tensor, tau: torch.Tensor,
               out: RouteBuffers, stream=None) -> None:
    _need(q, "q", torch.float32)
    _need(proj, "proj", torch.float32)
    _need(tau, "tau", torch.float32)
    c = cache.cfg
    if tuple(q.shape) != (c.n_q_heads, c.head_dim) or tuple(tau.shape) != (c.n_q_heads,) or \
            tuple(proj.shape) != (c.n_q_heads, c.route_dim, c.head_dim):
        raise ValueError("q [Hq][d], proj [Hq][dr][d], tau [Hq] expected")
    st = out.struct()
    _check(lib().sekv_route(cache.handle, layer, _ptr(q), _ptr(proj), _ptr(tau),
                            ctypes.byref(st), _stream(stream)))


def sekv_decode_workspace_bytes(cache: Cache) -> int:
    return cache.workspace_bytes()


def sekv_decode_attn(cache: Cache, layer: int, q: torch.Tensor, route: RouteBuffers,
                     o: torch.Tensor, workspace: torch.Tensor, stream=None,
                     fetch_stream=None) -> None:
    _need(q, "q", torch.float32)
    _need(o, "o", torch.float32)
    _need(workspace, "workspace")
    c = cache.cfg
    if tuple(q.shape) != (c.n_q_heads, c.head_dim) or tuple(o.shape) != (c.n_q_heads, c.head_dim):
        raise ValueError("q and o must be [Hq][d]")
    st = route.struct()
    fst = None if fetch_stream is None else _stream(fetch_stream)
    _check(lib().sekv_decode_attn(cache.handle, layer, _ptr(q), ctypes.byref(st), _ptr(o),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream), fst))


def sekv_route_attn(cache: Cache, layer: int, q: torch.Tensor, proj: torch.Tensor,
                    tau: torch.Tensor, route: RouteBuffers, o: torch.Tensor,
                    workspace: torch.Tensor, stream=None, fetch_stream=None) -> None:
    """Route and attend one layer in one call (three launches with device-tier factors)."""
    _need(q, "q", torch.float32)
    _need(proj, "proj", torch.float32)
    _need(tau, "tau", torch.float32)
    _need(o, "o", torch.float32)
    _need(workspace, "workspace")
    c = cache.cfg
    if tuple(q.shape) != (c.n_q_heads, c.head_dim) or tuple(o.shape) != (c.n_q_heads, c.head_dim):
        raise ValueError("q and o must be [Hq][d]")
    if tuple(tau.shape) != (c.n_q_heads,) or \
            tuple(proj.shape) != (c.n_q_heads, c.route_dim, c.head_dim):
        raise ValueError("proj [Hq][dr][d] and tau [Hq] expected")
    st = route.struct()
    fst = None if fetch_stream is None else _stream(fetch_stream)
    _check(lib().sekv_route_attn(cache.handle, layer, _ptr(q), _ptr(proj), _ptr(tau),
                                 ctypes.byref(st), _ptr(o), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream),
                                 fst))


def sekv_route_attn_noalloc(cache: Cache, layer: int, q: torch.Tensor, proj: torch.Tensor,
                            tau: torch.Tensor, route: RouteBuffers, o: torch.Tensor, stream=None,
                            fetch_stream=None) -> None:
    """sekv_route_attn without a workspace: the partial states go to the
    library's per-device scratch (no allocation; calls on one device must not
    overlap)."""
    _need(q, "q", torch.float32)
    _need(proj, "proj", torch.float32)
    _need(tau, "tau", torch.float32)
    _need(o, "o", torch.float32)
    c = cache.cfg
    if tuple(q.shape) != (c.n_q_heads, c.head_dim) or tuple(o.shape) != (c.n_q_heads, c.head_dim):
        raise ValueError("q and o must be [Hq][d]")
    if tuple(tau.shape) != (c.n_q_heads,) or \
            tuple(proj.shape) != (c.n_q_heads, c.route_dim, c.head_dim):
        raise ValueError("proj [Hq][dr][d] and tau [Hq] expected")
    st = route.struct()
    fst = None if fetch_stream is None else _stream(fetch_stream)
    _check(lib().sekv_route_attn_noalloc(cache.handle, layer, _ptr(q), _ptr(proj), _ptr(tau),
                                         ctypes.byref(st), _ptr(o), _stream(stream), fst))


def sekv_cap_budget(cache: Cache, route: RouteBuffers, budget_tokens: int, stream=None,
                    scope: str = "kv_head") -> None:
    """Cap one layer's zoom decisions to ``budget_tokens`` reconstructed tokens
    per KV head (scope "kv_head") or for the whole layer (scope "layer"), in
    place (``route`` must carry gate values)."""
    if route.prob is None:
        raise ValueError("the budget cap needs the route's gate values: allocate with_prob=True")
    if scope not in ("kv_head", "layer"):
        raise ValueError(f"scope must be 'kv_head' or 'layer', got {scope!r}")
    st = route.struct()
    fn = lib().sekv_cap_budget_layer if scope == "layer" else lib().sekv_cap_budget
    _check(fn(cache.handle, ctypes.byref(st), int(budget_tokens), _stream(stream)))


def sekv_apply_gates(cache: Cache, key_gates: torch.Tensor, value_gates: torch.Tensor,
                     eps: float, stream=None) -> None:
    """Soft-gate the cache's key factors with ``key_gates`` and its value
    factors with ``value_gates`` (Eq. 8), each [L][Hkv][S_c][max_rank] float32
    on the device.  Refreshes ``cache.info``."""
    c = cache.cfg
    shape = (c.n_layers, c.n_kv_heads, cache.info.n_compressed, c.max_rank)
    for name, g in (("key_gates", key_gates), ("value_gates", value_gates)):
        _need(g, name, torch.float32)
        if tuple(g.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    _check(lib().sekv_apply_gates(cache.handle, _ptr(key_gates), _ptr(value_gates), float(eps),
                                  _stream(stream)))
    info = SekvCacheInfo()
    _check(lib().sekv_cache_info_get(cache.handle, ctypes.byref(info)))
    cache.info = info


def _batch_arrays(caches, qs, routes, os_, workspaces):
    n = len(caches)
    if not (len(qs) == len(routes) == len(os_) == len(workspaces) == n):
        raise ValueError("caches, q, routes, o and workspaces must have one entry per sequence")
    for c, q, o, w in zip(caches, qs, os_, workspaces):
        _need(q, "q", torch.float32)
        _need(o, "o", torch.float32)
        _need(w, "workspace")
        shape = (c.cfg.n_q_heads, c.cfg.head_dim)
        if tuple(q.shape) != shape or tuple(o.shape) != shape:
            raise ValueError("q and o must be [Hq][d]")
    P = ctypes.c_void_p
    return ((P * n)(*[c.handle for c in caches]), (P * n)(*[_ptr(q) for q in qs]),
            (SekvRouteOut * n)(*[r.struct() for r in routes]), (P * n)(*[_ptr(o) for o in os_]),
            (P * n)(*[_ptr(w) for w in workspaces]),
            (ctypes.c_size_t * n)(*[w.numel() * w.element_size() for w in workspaces]))


def sekv_route_attn_batch(caches: Sequence[Cache], layer: int, qs: Sequence[torch.Tensor],
                          proj: torch.Tensor, tau: torch.Tensor, routes: Sequence[RouteBuffers],
                          os_: Sequence[torch.Tensor], workspaces: Sequence[torch.Tensor],
                          stream=None) -> None:
    """Route and attend one layer of several sequences (one cache each): one route launch,
    one attend launch and one tail launch for all of them."""
    _need(proj, "proj", torch.float32)
    _need(tau, "tau", torch.float32)
    cs, qp, rs, op, wp, wb = _batch_arrays(caches, qs, routes, os_, workspaces)
    _check(lib().sekv_route_attn_batch(cs, len(caches), layer, qp, _ptr(proj), _ptr(tau), rs, op,
                                       wp, wb, _stream(stream)))


def sekv_decode_attn_batch(caches: Sequence[Cache], layer: int, qs: Sequence[torch.Tensor],
                           routes: Sequence[RouteBuffers], os_: Sequence[torch.Tensor],
                           workspaces: Sequence[torch.Tensor], stream=None) -> None:
    """Attend one layer of several sequences (routes given): one chunk-mask launch, one
    attend launch and one tail launch."""
    cs, qp, rs, op, wp, wb = _batch_arrays(caches, qs, routes, os_, workspaces)
    _check(lib().sekv_decode_attn_batch(cs, len(caches), layer, qp, rs, op, wp, wb,
                                        _stream(stream)))
