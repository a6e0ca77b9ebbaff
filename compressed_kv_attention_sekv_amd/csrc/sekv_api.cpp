// Host runtime and C ABI of the SeKV library: argument validation, the cache
// handle (device tables, full-resolution rows, means, summaries, factor pool
// in HBM or pinned host memory), and the launch sequence of the build and of
// each decode step.  See include/sekv.h for the contract of every call.
#include "sekv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "sekv_internal.h"

using namespace sekv;

namespace {

thread_local std::string g_err;

// SEKV_LOG=1 in the environment: one line per build, append, error and
// configuration change on stderr (read once, at the first message)
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("SEKV_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void slog(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[640];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[sekv] %s\n", buf);
}

sekv_status fail(sekv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  slog("error %d: %s", (int)st, buf);
  return st;
}

// sekv_test_fail_fetch: host-tier factor fetches still to fail on purpose
std::atomic<int> g_fail_fetch{0};

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

#define SEKV_HIP(expr)                                                                        \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return fail(SEKV_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),        \
                  __FILE__, __LINE__);                                                        \
  } while (0)

sekv_status check_config(const sekv_config* c) {
  if (!c) return fail(SEKV_ERR_INVALID, "config is NULL");
  if (c->n_layers < 1) return fail(SEKV_ERR_INVALID, "n_layers must be >= 1");
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return fail(SEKV_ERR_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->n_kv_heads > kMaxKvHeads)
    return fail(SEKV_ERR_INVALID, "at most %d KV heads", kMaxKvHeads);
  if (c->n_q_heads / c->n_kv_heads > kMaxGroup)
    return fail(SEKV_ERR_INVALID, "at most %d query heads per KV head", kMaxGroup);
  if (c->head_dim != kHeadDim) return fail(SEKV_ERR_INVALID, "head_dim must be %d", kHeadDim);
  if (c->route_dim < 1 || c->route_dim > kMaxRouteDim)
    return fail(SEKV_ERR_INVALID, "route_dim must be in [1, %d]", kMaxRouteDim);
  if (c->window < 0) return fail(SEKV_ERR_INVALID, "window must be >= 0");
  if (c->max_rank < 1 || c->max_rank > kHeadDim)
    return fail(SEKV_ERR_INVALID, "max_rank must be in [1, %d]", kHeadDim);
  if (c->min_span_len < 1) return fail(SEKV_ERR_INVALID, "min_span_len must be >= 1");
  if (!std::isfinite(c->alpha) || !std::isfinite(c->gamma))
    return fail(SEKV_ERR_INVALID, "alpha and gamma must be finite");
  if (c->kv_dtype != SEKV_F32 && c->kv_dtype != SEKV_BF16)
    return fail(SEKV_ERR_INVALID, "kv_dtype must be SEKV_F32 or SEKV_BF16");
  if (c->factor_tier != SEKV_TIER_DEVICE && c->factor_tier != SEKV_TIER_HOST_PINNED)
    return fail(SEKV_ERR_INVALID, "factor_tier must be SEKV_TIER_DEVICE or SEKV_TIER_HOST_PINNED");
  if (c->svd_mode != SEKV_SVD_EXACT && c->svd_mode != SEKV_SVD_RANDOMIZED)
    return fail(SEKV_ERR_INVALID, "svd_mode must be SEKV_SVD_EXACT or SEKV_SVD_RANDOMIZED");
  if (c->svd_mode == SEKV_SVD_RANDOMIZED && c->max_rank > kRsvdMaxRank)
    return fail(SEKV_ERR_INVALID, "the randomized SVD supports max_rank <= %d", kRsvdMaxRank);
  if (c->append_capacity < 0) return fail(SEKV_ERR_INVALID, "append_capacity must be >= 0");
  if (c->append_capacity > 0 && c->factor_tier != SEKV_TIER_DEVICE)
    return fail(SEKV_ERR_UNSUPPORTED, "append_capacity needs device-tier factors");
  return SEKV_OK;
}

// device buffers owned by a scope; freed on every exit path
struct Scratch {
  std::vector<void*> ptrs;
  ~Scratch() {
    for (void* p : ptrs) (void)hipFree(p);
  }
  template <typename T>
  sekv_status alloc(T** out, size_t bytes, const char* what) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes ? bytes : 256);
    if (e != hipSuccess)
      return fail(SEKV_ERR_NOMEM, "hipMalloc(%zu) for %s failed: %s", bytes, what,
                  hipGetErrorString(e));
    ptrs.push_back(p);
    *out = (T*)p;
    return SEKV_OK;
  }
  void release(void* p) {
    ptrs.erase(std::remove(ptrs.begin(), ptrs.end(), p), ptrs.end());
  }
};

size_t elem_bytes(int dtype) { return dtype == SEKV_BF16 ? 2 : 4; }

sekv_status run_segment(const sekv_config* cfg, int n, const float* s, Scratch& sc, SegOut& o,
                        int32_t counts[4], double stats[3], hipStream_t st, int extra = 0) {
  sekv_status r;
  const int n_tab = n;   // the segmentation kernel's own length
  n = n + extra;         // table capacity: room for appended tokens
  if ((r = sc.alloc(&o.stats, 3 * sizeof(double), "stats"))) return r;
  if ((r = sc.alloc(&o.counts, 4 * sizeof(int32_t), "counts"))) return r;
  if ((r = sc.alloc(&o.anchors, (size_t)n * 4, "anchors"))) return r;
  if ((r = sc.alloc(&o.span_start, (size_t)n * 4, "span_start"))) return r;
  if ((r = sc.alloc(&o.span_len, (size_t)n * 4, "span_len"))) return r;
  if ((r = sc.alloc(&o.kind, (size_t)n, "kind"))) return r;
  if ((r = sc.alloc(&o.cspan, (size_t)n * 4, "cspan"))) return r;
  if ((r = sc.alloc(&o.cstart, (size_t)n * 4, "cstart"))) return r;
  if ((r = sc.alloc(&o.clen, (size_t)n * 4, "clen"))) return r;
  if ((r = sc.alloc(&o.dense_pos, (size_t)n * 4, "dense_pos"))) return r;
  if ((r = sc.alloc(&o.flag, (size_t)n, "flag"))) return r;
  SEKV_HIP(launch_segment(s, n_tab, cfg->window, cfg->alpha, cfg->min_span_len, o, st));
  SEKV_HIP(hipMemcpyAsync(counts, o.counts, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, st));
  SEKV_HIP(hipMemcpyAsync(stats, o.stats, 3 * sizeof(double), hipMemcpyDeviceToHost, st));
  SEKV_HIP(hipStreamSynchronize(st));
  return SEKV_OK;
}

}  // namespace

struct sekv_cache {
  sekv_config cfg{};
  int device = 0;                  // the device the cache was built on
  int n_tokens = 0, n_anchors = 0, n_spans = 0, sc = 0, n_dense = 0;
  // strides of the span arrays ([..][scs]) and of the full-resolution rows
  // ([..][ds][d]): the counts plus room for appended tokens (window append)
  int scs = 0, ds = 0;
  // window append (append_capacity > 0): host copies of what the appends
  // read and extend, and the device buffers they add
  int n_appended = 0, open_start = 0, open_len = 0;
  uint64_t pool_cap_floats = 0;       // pool allocation, in floats (>= pool_floats)
  std::vector<int32_t> h_dense_pos;   // ascending positions of the full-resolution rows
  std::vector<float> h_tail_s;        // surprisal of positions tail_base .. n_tokens - 1
  int tail_base = 0;
  float* dense_s = nullptr;           // [ds] surprisal of each full-resolution row
  int32_t* rank_by_dense = nullptr;   // [L][Hkv][ds] rank requested at each row
  int32_t* app_start = nullptr;       // [scs] first full-resolution row of appended spans
  int32_t* app_ranges = nullptr;      // [2 capacity] row ranges removed by one append
  int group = 1;
  double stats[3] = {0, 0, 0};
  std::vector<void*> dev;  // every device allocation, freed on destroy
  // span tables (device)
  int32_t *anchors = nullptr, *span_start = nullptr, *span_len = nullptr, *cspan = nullptr;
  int32_t *cstart = nullptr, *clen = nullptr, *dense_pos = nullptr;
  uint8_t* kind = nullptr;
  double* lnn64 = nullptr;
  float* lnn32 = nullptr;
  // representations (device)
  void *dense_k = nullptr, *dense_v = nullptr, *kbar = nullptr, *vbar = nullptr, *summ = nullptr;
  int32_t* rank = nullptr;        // [L][Hkv][Sc]
  uint64_t* fac_off = nullptr;    // [L][Hkv][Sc] float offset of each block
  std::vector<int32_t> h_rank;
  std::vector<int32_t> h_clen;
  std::vector<uint64_t> h_fac_off;
  std::vector<uint64_t> layer_base;  // [L + 1] first float of each layer's blocks
  uint64_t factor_bytes = 0, pool_floats = 0;
  float* pool_dev = nullptr;      // device tier
  float* pool_host = nullptr;     // host tier (pinned, mapped)
  int fetch_mode = SEKV_FETCH_GATHER;  // host tier: how the union blocks reach staging
  std::vector<int32_t> h_ulist;   // memcpy fetch: the route's union lists, on the host
  std::vector<int32_t> h_ucount;
  float* pool_host_dev = nullptr; // device view of pool_host
  float* stage = nullptr;         // host tier: device staging for one layer
  uint64_t stage_floats = 0;
  uint32_t* chunk_bits = nullptr;  // [Hkv][n_work][kListWords] zoom bit masks of each chunk
  int32_t* zcount = nullptr;       // [Hkv] zoom workgroups per KV head of the last zoom launch
  uint8_t* cap_drop = nullptr;     // [Hkv][S_c] decisions of the layer-wide budget cap
  float* zero_block = nullptr;     // kZeroBlockFloats zeros: a valid source for idle prefetches
  LayerGeom geom{};
  hipEvent_t ev_route = nullptr, ev_fetch = nullptr;
  // host tier: HBM residency cache of factor blocks (sekv_set_residency)
  std::vector<void*> res_dev;
  ResidencyView res{};
  bool res_on = false;
  uint64_t res_epoch = 0;

  void residency_free() {
    for (void* p : res_dev) (void)hipFree(p);
    res_dev.clear();
    res = ResidencyView{};
    res_on = false;
    res_epoch = 0;
  }
  ~sekv_cache() {
    residency_free();
    for (void* p : dev) (void)hipFree(p);
    if (pool_host) (void)hipHostFree(pool_host);
    if (ev_route) (void)hipEventDestroy(ev_route);
    if (ev_fetch) (void)hipEventDestroy(ev_fetch);
  }
  template <typename T>
  sekv_status alloc(T** out, size_t bytes, const char* what) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes ? bytes : 256);
    if (e != hipSuccess)
      return fail(SEKV_ERR_NOMEM, "hipMalloc(%zu) for %s failed: %s", bytes, what,
                  hipGetErrorString(e));
    dev.push_back(p);
    *out = (T*)p;
    return SEKV_OK;
  }
  size_t kv_elem() const { return elem_bytes(cfg.kv_dtype); }
  int bf16() const { return cfg.kv_dtype == SEKV_BF16; }
};

extern "C" {

const char* sekv_last_error(void) { return g_err.c_str(); }

sekv_status sekv_segment(const sekv_config* cfg, int32_t n_tokens, const float* surprisal_dev,
                         int32_t* n_anchors, int32_t* n_spans, int32_t* n_compressed,
                         hipStream_t stream) {
  sekv_status r = check_config(cfg);
  if (r) return r;
  if (n_tokens < 1) return fail(SEKV_ERR_INVALID, "n_tokens must be >= 1");
  if (!surprisal_dev) return fail(SEKV_ERR_INVALID, "surprisal_dev is NULL");
  Scratch scr;
  SegOut o{};
  int32_t counts[4];
  double stats[3];
  if ((r = run_segment(cfg, n_tokens, surprisal_dev, scr, o, counts, stats, stream))) return r;
  if (n_anchors) *n_anchors = counts[0];
  if (n_spans) *n_spans = counts[1];
  if (n_compressed) *n_compressed = counts[2];
  return SEKV_OK;
}

static sekv_status build_impl(const sekv_config* cfg, int32_t n_tokens, const float* s,
                              const void* k_dev, const void* v_dev, const float* w_route,
                              const int32_t* rank_by_pos, hipStream_t st,
                              std::unique_ptr<sekv_cache>& out) {
  auto c = std::make_unique<sekv_cache>();
  c->cfg = *cfg;
  SEKV_HIP(hipGetDevice(&c->device));
  c->n_tokens = n_tokens;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  const int L = cfg->n_layers, Hkv = cfg->n_kv_heads, Hq = cfg->n_q_heads, dr = cfg->route_dim;
  const int n_lg = L * Hkv;
  sekv_status r;

  // ---- segmentation: tables stay in the cache (capacity n_tokens) ---------
  Scratch scr;
  SegOut o{};
  int32_t counts[4];
  const int cap = cfg->append_capacity;
  if ((r = run_segment(cfg, n_tokens, s, scr, o, counts, c->stats, st, cap))) return r;
  for (void* p : {(void*)o.anchors, (void*)o.span_start, (void*)o.span_len, (void*)o.kind,
                  (void*)o.cspan, (void*)o.cstart, (void*)o.clen, (void*)o.dense_pos}) {
    scr.release(p);
    c->dev.push_back(p);
  }
  c->anchors = o.anchors;
  c->span_start = o.span_start;
  c->span_len = o.span_len;
  c->kind = o.kind;
  c->cspan = o.cspan;
  c->cstart = o.cstart;
  c->clen = o.clen;
  c->dense_pos = o.dense_pos;
  c->n_anchors = counts[0];
  c->n_spans = counts[1];
  c->sc = counts[2];
  c->n_dense = counts[3];
  const int sc = c->sc, D = c->n_dense;
  const size_t eb = c->kv_elem();
  c->scs = sc + (cap > 0 ? cap / cfg->min_span_len + 1 : 0);
  c->ds = D + cap;
  const int scs = c->scs, ds = c->ds;

  if ((r = c->alloc(&c->lnn64, (size_t)scs * 8, "lnn64"))) return r;
  if ((r = c->alloc(&c->lnn32, (size_t)scs * 4, "lnn32"))) return r;
  SEKV_HIP(launch_log_len(c->clen, sc, c->lnn64, c->lnn32, st));
  if ((r = c->alloc(&c->rank, (size_t)n_lg * scs * 4, "rank"))) return r;
  SEKV_HIP(launch_span_rank(rank_by_pos, c->cstart, c->clen, n_tokens, 0, sc, scs, n_lg,
                            cfg->max_rank, c->rank, st));

  // ---- full-resolution rows ------------------------------------------------
  if ((r = c->alloc(&c->dense_k, (size_t)n_lg * ds * kHeadDim * eb, "dense_k"))) return r;
  if ((r = c->alloc(&c->dense_v, (size_t)n_lg * ds * kHeadDim * eb, "dense_v"))) return r;
  SEKV_HIP(launch_gather_dense(c->bf16(), k_dev, n_tokens, c->dense_pos, D, ds, n_lg, c->dense_k,
                               st));
  SEKV_HIP(launch_gather_dense(c->bf16(), v_dev, n_tokens, c->dense_pos, D, ds, n_lg, c->dense_v,
                               st));

  // ---- means and summaries -------------------------------------------------
  if ((r = c->alloc(&c->kbar, (size_t)n_lg * scs * kHeadDim * eb, "kbar"))) return r;
  if ((r = c->alloc(&c->vbar, (size_t)n_lg * scs * kHeadDim * eb, "vbar"))) return r;
  if ((r = c->alloc(&c->summ, (size_t)L * Hq * scs * dr * eb, "summaries"))) return r;
  SEKV_HIP(launch_span_summarize(c->bf16(), s, k_dev, v_dev, w_route, n_tokens, c->cstart,
                                 c->clen, 0, sc, scs, L, Hkv, c->group, dr, c->kbar, c->vbar,
                                 c->summ, st));

  // ---- factor pool layout (host) ---------------------------------------------
  c->h_rank.assign((size_t)n_lg * scs, 0);
  c->h_clen.resize(sc);
  if (sc) {
    SEKV_HIP(hipMemcpyAsync(c->h_rank.data(), c->rank, c->h_rank.size() * 4,
                            hipMemcpyDeviceToHost, st));
    SEKV_HIP(hipMemcpyAsync(c->h_clen.data(), c->clen, (size_t)sc * 4, hipMemcpyDeviceToHost, st));
  }
  SEKV_HIP(hipStreamSynchronize(st));
  c->h_fac_off.assign((size_t)n_lg * scs, 0);
  c->layer_base.assign(L + 1, 0);
  uint64_t off = 0, fbytes = 0, stage_max = 0;
  for (int l = 0; l < L; ++l) {
    c->layer_base[l] = off;
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < sc; ++j) {
        const size_t idx = ((size_t)l * Hkv + g) * scs + j;
        const FactorView fv = FactorView::packed(c->h_rank[idx], c->h_clen[j]);
        c->h_fac_off[idx] = off;
        off += fv.block_floats();
        fbytes += fv.alg_bytes();
      }
    stage_max = std::max(stage_max, off - c->layer_base[l]);
  }
  c->layer_base[L] = off;
  c->pool_floats = off;
  c->factor_bytes = fbytes;
  if ((r = c->alloc(&c->fac_off, c->h_fac_off.size() * 8, "fac_off"))) return r;
  if (!c->h_fac_off.empty())
    SEKV_HIP(hipMemcpyAsync(c->fac_off, c->h_fac_off.data(), c->h_fac_off.size() * 8,
                            hipMemcpyHostToDevice, st));

  // ---- per-span SVD, spans bucketed by Gram size m = min(n, d) --------------
  float* pool_build = nullptr;
  const size_t pool_bytes = (size_t)c->pool_floats * 4;
  if (cfg->factor_tier == SEKV_TIER_HOST_PINNED && cfg->host_pool_cap_bytes &&
      pool_bytes > cfg->host_pool_cap_bytes)
    return fail(SEKV_ERR_NOMEM, "factor pool needs %zu bytes, host pool cap is %llu", pool_bytes,
                (unsigned long long)cfg->host_pool_cap_bytes);
  if (cfg->factor_tier == SEKV_TIER_DEVICE) {
    // with append capacity, room for the blocks of every span the appends
    // can close: at most cap / min_span_len + 1 spans per (layer, KV head),
    // of at most cap tokens together, each at most at the rank cap
    c->pool_cap_floats = c->pool_floats;
    if (cap > 0) {
      const uint64_t R = (uint64_t)std::min(cfg->max_rank, kHeadDim), R4 = (R + 3) & ~3ull;
      const uint64_t spans = (uint64_t)cap / cfg->min_span_len + 1;
      c->pool_cap_floats += (uint64_t)n_lg * (spans * (2 * R * kHeadDim + 2 * R4 + 63) +
                                              2 * R4 * (uint64_t)cap);
    }
    if ((r = c->alloc(&c->pool_dev, (size_t)c->pool_cap_floats * 4, "factor pool"))) return r;
    pool_build = c->pool_dev;
  } else {
    if ((r = scr.alloc(&pool_build, pool_bytes, "factor build buffer"))) return r;
  }
  {
    std::vector<int32_t> ids[3], rs_ids[3];
    const int rs_rows[3] = {128, 256, kRsvdMaxRows};
    const bool rsvd = cfg->svd_mode == SEKV_SVD_RANDOMIZED;
    for (int j = 0; j < sc; ++j) {
      const int n = c->h_clen[j];
      if (rsvd && n > kRsvdMinRows && n <= kRsvdMaxRows) {
        rs_ids[n <= 128 ? 0 : (n <= 256 ? 1 : 2)].push_back(j);
        continue;
      }
      const int m = std::min(n, kHeadDim);
      ids[m <= 32 ? 0 : (m <= 64 ? 1 : 2)].push_back(j);
    }
    for (int b = 0; b < 3; ++b) {
      if (rs_ids[b].empty()) continue;
      int32_t* d_ids = nullptr;
      if ((r = scr.alloc(&d_ids, rs_ids[b].size() * 4, "randomized svd span ids"))) return r;
      SEKV_HIP(hipMemcpyAsync(d_ids, rs_ids[b].data(), rs_ids[b].size() * 4,
                              hipMemcpyHostToDevice, st));
      for (int which = 0; which < 2; ++which)
        SEKV_HIP(launch_span_rsvd(c->bf16(), which ? v_dev : k_dev, n_tokens, c->cstart, c->clen,
                                  d_ids, (int)rs_ids[b].size(), scs, n_lg, c->rank, c->fac_off,
                                  pool_build, which, rs_rows[b], st));
    }
    const int max_m[3] = {32, 64, 128};
    for (int b = 0; b < 3; ++b) {
      if (ids[b].empty()) continue;
      int32_t* d_ids = nullptr;
      if ((r = scr.alloc(&d_ids, ids[b].size() * 4, "svd span ids"))) return r;
      SEKV_HIP(hipMemcpyAsync(d_ids, ids[b].data(), ids[b].size() * 4, hipMemcpyHostToDevice, st));
      for (int which = 0; which < 2; ++which)
        SEKV_HIP(launch_span_svd(c->bf16(), which ? v_dev : k_dev, n_tokens, c->cstart, c->clen,
                                 d_ids, (int)ids[b].size(), scs, n_lg, c->rank, c->fac_off,
                                 pool_build, which, max_m[b], st));
    }
  }
  if (cfg->factor_tier == SEKV_TIER_HOST_PINNED) {
    hipError_t e = hipHostMalloc((void**)&c->pool_host, pool_bytes ? pool_bytes : 256,
                                 hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) {
      c->pool_host = nullptr;
      return fail(SEKV_ERR_NOMEM, "hipHostMalloc(%zu) for the factor pool failed: %s",
                  pool_bytes, hipGetErrorString(e));
    }
    SEKV_HIP(hipHostGetDevicePointer((void**)&c->pool_host_dev, c->pool_host, 0));
    if (pool_bytes)
      SEKV_HIP(hipMemcpyAsync(c->pool_host, pool_build, pool_bytes, hipMemcpyDeviceToHost, st));
    c->stage_floats = stage_max;
    if ((r = c->alloc(&c->stage, (size_t)stage_max * 4, "fetch staging"))) return r;
  }

  // ---- decode geometry and chunk bit masks --------------------------------------
  c->geom = make_layer_geom(Hq, Hkv, dr, D, sc, ds, scs);
  // chunk masks for the geometry at full append capacity (the most workgroups)
  const int nw_max = make_layer_geom(Hq, Hkv, dr, ds, scs, ds, scs).n_work;
  if ((r = c->alloc(&c->chunk_bits, (size_t)Hkv * nw_max * kListWords * 4, "chunk bits")))
    return r;
  if (cap > 0) {
    // what the appends read: each full-resolution row's surprisal and
    // requested rank, and on the host the row positions and the surprisal
    // from the window on
    if ((r = c->alloc(&c->dense_s, (size_t)ds * 4, "row surprisal"))) return r;
    if ((r = c->alloc(&c->rank_by_dense, (size_t)n_lg * ds * 4, "row ranks"))) return r;
    if ((r = c->alloc(&c->app_start, (size_t)scs * 4, "appended span rows"))) return r;
    if ((r = c->alloc(&c->app_ranges, (size_t)2 * (cap / cfg->min_span_len + 2) * 4,
                      "removed row ranges")))
      return r;
    SEKV_HIP(launch_gather_words((const uint32_t*)s, 0, c->dense_pos, D, ds, 1,
                                 (uint32_t*)c->dense_s, st));
    if (rank_by_pos)
      SEKV_HIP(launch_gather_words((const uint32_t*)rank_by_pos, n_tokens, c->dense_pos, D, ds,
                                   n_lg, (uint32_t*)c->rank_by_dense, st));
    else
      SEKV_HIP(launch_fill_i32(c->rank_by_dense, n_lg * ds, cfg->max_rank, st));
    c->h_dense_pos.resize(D);
    if (D)
      SEKV_HIP(hipMemcpyAsync(c->h_dense_pos.data(), c->dense_pos, (size_t)D * 4,
                              hipMemcpyDeviceToHost, st));
    c->tail_base = std::max(n_tokens - cfg->window, 0);
    c->h_tail_s.resize(n_tokens - c->tail_base);
    if (!c->h_tail_s.empty())
      SEKV_HIP(hipMemcpyAsync(c->h_tail_s.data(), s + c->tail_base, c->h_tail_s.size() * 4,
                              hipMemcpyDeviceToHost, st));
  }
  if ((r = c->alloc(&c->zero_block, (size_t)kZeroBlockFloats * 4, "zero block"))) return r;
  if ((r = c->alloc(&c->zcount, (size_t)Hkv * 4, "zoom counts"))) return r;
  if ((r = c->alloc(&c->cap_drop, (size_t)Hkv * std::max(scs, 1), "budget decisions"))) return r;
  SEKV_HIP(hipMemsetAsync(c->zcount, 0, (size_t)Hkv * 4, st));
  SEKV_HIP(hipMemsetAsync(c->zero_block, 0, (size_t)kZeroBlockFloats * 4, st));
  SEKV_HIP(hipEventCreateWithFlags(&c->ev_route, hipEventDisableTiming));
  SEKV_HIP(hipEventCreateWithFlags(&c->ev_fetch, hipEventDisableTiming));
  SEKV_HIP(hipStreamSynchronize(st));
  out = std::move(c);
  return SEKV_OK;
}

sekv_status sekv_build_spans(const sekv_config* cfg, int32_t n_tokens, const float* surprisal_dev,
                             const void* k_dev, const void* v_dev, const float* w_route_dev,
                             const int32_t* rank_by_pos_dev, hipStream_t stream,
                             sekv_cache** out) {
  if (!out) return fail(SEKV_ERR_INVALID, "out is NULL");
  *out = nullptr;
  sekv_status r = check_config(cfg);
  if (r) return r;
  if (n_tokens < 1) return fail(SEKV_ERR_INVALID, "n_tokens must be >= 1");
  if (!surprisal_dev || !k_dev || !v_dev || !w_route_dev)
    return fail(SEKV_ERR_INVALID, "surprisal, keys, values and w_route must be non-NULL");
  std::unique_ptr<sekv_cache> c;
  const auto t0 = std::chrono::steady_clock::now();
  r = build_impl(cfg, n_tokens, surprisal_dev, k_dev, v_dev, w_route_dev, rank_by_pos_dev, stream,
                 c);
  if (r) {
    (void)hipStreamSynchronize(stream);  // nothing queued may outlive the freed buffers
    return r;
  }
  slog("build: %d tokens, %d layers x %d KV heads: %d anchors, %d spans (%d compressed), %d "
       "full-resolution rows; factor pool %.3f GB (%s tier, %s SVD), %.1f ms",
       n_tokens, cfg->n_layers, cfg->n_kv_heads, c->n_anchors, c->n_spans, c->sc, c->n_dense,
       (double)c->pool_floats * 4e-9, cfg->factor_tier == SEKV_TIER_DEVICE ? "device" : "host",
       cfg->svd_mode == SEKV_SVD_EXACT ? "exact" : "randomized", ms_since(t0));
  *out = c.release();
  return SEKV_OK;
}

// ---- window append ----------------------------------------------------------------
static sekv_status append_impl(sekv_cache* c, int n_new, const float* s_new, const void* k_new,
                               const void* v_new, const float* w_route, const int32_t* rank_new,
                               hipStream_t st) {
  const sekv_config& cfg = c->cfg;
  const int L = cfg.n_layers, Hkv = cfg.n_kv_heads, Hq = cfg.n_q_heads, dr = cfg.route_dim;
  const int n_lg = L * Hkv, W = cfg.window;
  const size_t eb = c->kv_elem();
  const int ds = c->ds, scs = c->scs;
  sekv_status r;
  // the new tokens' surprisal decides the retirements on the host
  std::vector<float> sn(n_new);
  SEKV_HIP(hipMemcpyAsync(sn.data(), s_new, (size_t)n_new * 4, hipMemcpyDeviceToHost, st));
  SEKV_HIP(hipStreamSynchronize(st));
  for (int t = 0; t < n_new; ++t)
    if (!std::isfinite(sn[t]))
      return fail(SEKV_ERR_INVALID, "surprisal of new token %d is not finite", t);

  // ---- 1. the new tokens join the full-resolution rows (the window) ---------
  const int D0 = c->n_dense, N0 = c->n_tokens;
  SEKV_HIP(hipMemcpy2DAsync((char*)c->dense_k + (size_t)D0 * kHeadDim * eb,
                            (size_t)ds * kHeadDim * eb, k_new, (size_t)n_new * kHeadDim * eb,
                            (size_t)n_new * kHeadDim * eb, n_lg, hipMemcpyDeviceToDevice, st));
  SEKV_HIP(hipMemcpy2DAsync((char*)c->dense_v + (size_t)D0 * kHeadDim * eb,
                            (size_t)ds * kHeadDim * eb, v_new, (size_t)n_new * kHeadDim * eb,
                            (size_t)n_new * kHeadDim * eb, n_lg, hipMemcpyDeviceToDevice, st));
  SEKV_HIP(hipMemcpyAsync(c->dense_s + D0, s_new, (size_t)n_new * 4, hipMemcpyDeviceToDevice, st));
  if (rank_new)
    SEKV_HIP(hipMemcpy2DAsync(c->rank_by_dense + D0, (size_t)ds * 4, rank_new, (size_t)n_new * 4,
                              (size_t)n_new * 4, n_lg, hipMemcpyDeviceToDevice, st));

  Scratch scr_rank;
  if (!rank_new) {   // max_rank for every new token: one fill, then a strided copy
    int32_t* tmp = nullptr;
    if ((r = scr_rank.alloc(&tmp, (size_t)n_lg * n_new * 4, "requested ranks"))) return r;
    SEKV_HIP(launch_fill_i32(tmp, n_lg * n_new, cfg.max_rank, st));
    SEKV_HIP(hipMemcpy2DAsync(c->rank_by_dense + D0, (size_t)ds * 4, tmp, (size_t)n_new * 4,
                              (size_t)n_new * 4, n_lg, hipMemcpyDeviceToDevice, st));
  }
  // host state changes below are undone if the append fails before the device
  // copies of the span table change (only the pool room and scratch can fail)
  const size_t hp0 = c->h_dense_pos.size(), ht0 = c->h_tail_s.size();
  auto undo = [&](sekv_status e) {
    c->h_dense_pos.resize(hp0);
    c->h_tail_s.resize(ht0);
    return e;
  };
  for (int t = 0; t < n_new; ++t) {
    c->h_dense_pos.push_back(N0 + t);
    c->h_tail_s.push_back(sn[t]);
  }
  int D = D0 + n_new;
  const int N = N0 + n_new;

  // ---- 2. retire the tokens that leave the window ----------------------------
  struct NewSpan { int start, len, row; bool compressed; };
  std::vector<NewSpan> closed;
  std::vector<int32_t> new_anchors;
  const double thr = c->stats[2];
  const int r_old = std::max(N0 - W, 0), r_new = std::max(N - W, 0);
  // the row of position p among the full-resolution rows (ascending)
  auto row_of = [&](int p) {
    return (int)(std::lower_bound(c->h_dense_pos.begin(), c->h_dense_pos.end(), p) -
                 c->h_dense_pos.begin());
  };
  int open_start = c->open_start, open_len = c->open_len;
  for (int t = r_old; t < r_new; ++t) {
    const double sv = (double)c->h_tail_s[t - c->tail_base];
    if (sv > thr) {
      if (open_len > 0) {
        closed.push_back(NewSpan{open_start, open_len, row_of(open_start),
                                 open_len >= cfg.min_span_len});
        open_len = 0;
      }
      new_anchors.push_back(t);
    } else {
      if (open_len == 0) open_start = t;
      ++open_len;
    }
  }
  // spans now stored compressed: ids sc0 .. sc0 + nc - 1, in order
  const int sc0 = c->sc;
  std::vector<NewSpan> comp;
  for (const NewSpan& sp : closed)
    if (sp.compressed) comp.push_back(sp);
  const int nc = (int)comp.size();
  if (nc > 0) {
    std::vector<int32_t> hstart(nc), hlen(nc);
    for (int i = 0; i < nc; ++i) {
      hstart[i] = comp[i].row;
      hlen[i] = comp[i].len;
    }
    SEKV_HIP(hipMemcpyAsync(c->app_start + sc0, hstart.data(), (size_t)nc * 4,
                            hipMemcpyHostToDevice, st));
    SEKV_HIP(hipMemcpyAsync(c->clen + sc0, hlen.data(), (size_t)nc * 4, hipMemcpyHostToDevice, st));
    SEKV_HIP(launch_log_len(c->clen + sc0, nc, c->lnn64 + sc0, c->lnn32 + sc0, st));
    // retained ranks, then the blocks' place in the pool
    SEKV_HIP(launch_span_rank(c->rank_by_dense, c->app_start, c->clen, ds, sc0, nc, scs, n_lg,
                              cfg.max_rank, c->rank, st));
    std::vector<int32_t> hr((size_t)n_lg * nc);
    SEKV_HIP(hipMemcpy2DAsync(hr.data(), (size_t)nc * 4, c->rank + sc0, (size_t)scs * 4,
                              (size_t)nc * 4, n_lg, hipMemcpyDeviceToHost, st));
    SEKV_HIP(hipStreamSynchronize(st));
    uint64_t off = c->pool_floats, fbytes = 0;
    std::vector<uint64_t> hoff((size_t)n_lg * nc);
    for (int lg = 0; lg < n_lg; ++lg)
      for (int i = 0; i < nc; ++i) {
        const FactorView fv = FactorView::packed(hr[(size_t)lg * nc + i], hlen[i]);
        hoff[(size_t)lg * nc + i] = off;
        off += fv.block_floats();
        fbytes += fv.alg_bytes();
      }
    if (off > c->pool_cap_floats)
      return undo(fail(SEKV_ERR_NOMEM, "the factor pool's append room is exhausted"));
    int32_t* d_ids = nullptr;
    Scratch scr;
    if ((r = scr.alloc(&d_ids, (size_t)nc * 4, "appended span ids"))) return undo(r);
    SEKV_HIP(hipMemcpy2DAsync(c->fac_off + sc0, (size_t)scs * 8, hoff.data(), (size_t)nc * 8,
                              (size_t)nc * 8, n_lg, hipMemcpyHostToDevice, st));
    for (int lg = 0; lg < n_lg; ++lg)
      for (int i = 0; i < nc; ++i) {
        c->h_rank[(size_t)lg * scs + sc0 + i] = hr[(size_t)lg * nc + i];
        c->h_fac_off[(size_t)lg * scs + sc0 + i] = hoff[(size_t)lg * nc + i];
      }
    for (int i = 0; i < nc; ++i) c->h_clen.push_back(hlen[i]);
    c->pool_floats = off;
    c->factor_bytes += fbytes;
    // means, summaries and factors from the spans' full-resolution rows
    SEKV_HIP(launch_span_summarize(c->bf16(), c->dense_s, c->dense_k, c->dense_v, w_route, ds,
                                   c->app_start, c->clen, sc0, nc, scs, L, Hkv, c->group, dr,
                                   c->kbar, c->vbar, c->summ, st));
    std::vector<int32_t> ids[3];
    for (int i = 0; i < nc; ++i) {
      const int m = std::min(hlen[i], kHeadDim);
      ids[m <= 32 ? 0 : (m <= 64 ? 1 : 2)].push_back(sc0 + i);
    }
    const int max_m[3] = {32, 64, 128};
    std::vector<int32_t> all_ids;
    for (int b = 0; b < 3; ++b) all_ids.insert(all_ids.end(), ids[b].begin(), ids[b].end());
    SEKV_HIP(hipMemcpyAsync(d_ids, all_ids.data(), (size_t)nc * 4, hipMemcpyHostToDevice, st));
    for (int b = 0, at = 0; b < 3; at += (int)ids[b].size(), ++b) {
      if (ids[b].empty()) continue;
      for (int which = 0; which < 2; ++which)
        SEKV_HIP(launch_span_svd(c->bf16(), which ? c->dense_v : c->dense_k, ds, c->app_start,
                                 c->clen, d_ids + at, (int)ids[b].size(), scs, n_lg, c->rank,
                                 c->fac_off, c->pool_dev, which, max_m[b], st));
    }
    // the compressed spans' rows leave the full-resolution set
    std::vector<int32_t> ranges;
    for (const NewSpan& sp : comp) {
      ranges.push_back(sp.row);
      ranges.push_back(sp.len);
    }
    SEKV_HIP(hipMemcpyAsync(c->app_ranges, ranges.data(), ranges.size() * 4,
                            hipMemcpyHostToDevice, st));
    const int vec = (int)(kHeadDim * eb / 16);
    SEKV_HIP(launch_compact_rows(c->dense_k, 16, ds, vec, D, n_lg, c->app_ranges, nc, st));
    SEKV_HIP(launch_compact_rows(c->dense_v, 16, ds, vec, D, n_lg, c->app_ranges, nc, st));
    SEKV_HIP(launch_compact_rows(c->dense_s, 4, ds, 1, D, 1, c->app_ranges, nc, st));
    SEKV_HIP(launch_compact_rows(c->rank_by_dense, 4, ds, 1, D, n_lg, c->app_ranges, nc, st));
    for (int i = nc - 1; i >= 0; --i)
      c->h_dense_pos.erase(c->h_dense_pos.begin() + comp[i].row,
                           c->h_dense_pos.begin() + comp[i].row + comp[i].len);
    for (const NewSpan& sp : comp) D -= sp.len;
    SEKV_HIP(hipStreamSynchronize(st));  // the host staging vectors of this block end here
  }

  // ---- 3. the span table, anchors and row positions on the device -----------
  std::vector<int32_t> hs, hl, hcs;
  std::vector<uint8_t> hk;
  for (const NewSpan& sp : closed) {
    hs.push_back(sp.start);
    hl.push_back(sp.len);
    hk.push_back(sp.compressed ? 0 : 1);
  }
  for (size_t i = 0; i < closed.size(); ++i)
    if (closed[i].compressed) hcs.push_back(c->n_spans + (int)i);
  if (!closed.empty()) {
    const size_t k = closed.size();
    SEKV_HIP(hipMemcpyAsync(c->span_start + c->n_spans, hs.data(), k * 4, hipMemcpyHostToDevice, st));
    SEKV_HIP(hipMemcpyAsync(c->span_len + c->n_spans, hl.data(), k * 4, hipMemcpyHostToDevice, st));
    SEKV_HIP(hipMemcpyAsync(c->kind + c->n_spans, hk.data(), k, hipMemcpyHostToDevice, st));
  }
  if (!hcs.empty()) {
    SEKV_HIP(hipMemcpyAsync(c->cspan + sc0, hcs.data(), hcs.size() * 4, hipMemcpyHostToDevice, st));
    std::vector<int32_t> cst(nc);
    for (int i = 0; i < nc; ++i) cst[i] = comp[i].start;
    SEKV_HIP(hipMemcpyAsync(c->cstart + sc0, cst.data(), (size_t)nc * 4, hipMemcpyHostToDevice, st));
  }
  if (!new_anchors.empty())
    SEKV_HIP(hipMemcpyAsync(c->anchors + c->n_anchors, new_anchors.data(), new_anchors.size() * 4,
                            hipMemcpyHostToDevice, st));
  // the row positions changed from the first removed row (or the new rows) on
  const int first = nc > 0 ? comp[0].row : D0;
  if (D > first)
    SEKV_HIP(hipMemcpyAsync(c->dense_pos + first, c->h_dense_pos.data() + first,
                            (size_t)(D - first) * 4, hipMemcpyHostToDevice, st));
  SEKV_HIP(hipStreamSynchronize(st));
  c->open_start = open_start;
  c->open_len = open_len;
  c->n_spans += (int)closed.size();
  c->n_anchors += (int)new_anchors.size();
  c->sc += nc;
  c->n_dense = D;
  c->n_tokens = N;
  c->n_appended += n_new;
  c->geom = make_layer_geom(Hq, Hkv, dr, D, c->sc, ds, scs);
  slog("append: %d tokens (%d of %d appended), %d retired: %d anchors and %d spans (%d "
       "compressed) closed, open run %d; %d full-resolution rows", n_new, c->n_appended,
       cfg.append_capacity, r_new - r_old, (int)new_anchors.size(), (int)closed.size(), nc,
       c->open_len, D);
  return SEKV_OK;
}

sekv_status sekv_set_fetch_mode(sekv_cache* c, int32_t mode) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (mode != SEKV_FETCH_GATHER && mode != SEKV_FETCH_MEMCPY)
    return fail(SEKV_ERR_INVALID, "fetch mode must be SEKV_FETCH_GATHER or SEKV_FETCH_MEMCPY");
  if (c->cfg.factor_tier != SEKV_TIER_HOST_PINNED)
    return fail(SEKV_ERR_INVALID, "the fetch mode is a host-tier setting; this cache keeps its "
                "factors in HBM");
  c->fetch_mode = mode;
  slog("fetch mode: %s", mode == SEKV_FETCH_GATHER ? "gather kernel" : "hipMemcpyAsync per run");
  return SEKV_OK;
}

sekv_status sekv_test_fail_fetch(int32_t n) {
  if (n < 0) return fail(SEKV_ERR_INVALID, "n must be >= 0 (got %d)", n);
  g_fail_fetch.store(n);
  slog("test hook: the next %d host-tier factor fetches fail", n);
  return SEKV_OK;
}

sekv_status sekv_append_tokens(sekv_cache* c, int32_t n_new, const float* surprisal_dev,
                               const void* k_dev, const void* v_dev, const float* w_route_dev,
                               const int32_t* rank_dev, hipStream_t stream) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (!surprisal_dev || !k_dev || !v_dev || !w_route_dev)
    return fail(SEKV_ERR_INVALID, "surprisal, keys, values and w_route must be non-NULL");
  if (n_new < 1) return fail(SEKV_ERR_INVALID, "n_new must be >= 1 (got %d)", n_new);
  if (c->cfg.append_capacity <= 0)
    return fail(SEKV_ERR_UNSUPPORTED, "the cache was built without append_capacity");
  if ((long long)c->n_appended + n_new > c->cfg.append_capacity)
    return fail(SEKV_ERR_NOMEM, "appending %d tokens exceeds the append capacity (%d of %d used)",
                n_new, c->n_appended, c->cfg.append_capacity);
  return append_impl(c, n_new, surprisal_dev, k_dev, v_dev, w_route_dev, rank_dev, stream);
}

sekv_status sekv_cache_info_get(const sekv_cache* c, sekv_cache_info* out) {
  if (!c || !out) return fail(SEKV_ERR_INVALID, "cache and out must be non-NULL");
  const int L = c->cfg.n_layers, Hkv = c->cfg.n_kv_heads, Hq = c->cfg.n_q_heads;
  const size_t eb = c->kv_elem();
  out->n_tokens = c->n_tokens;
  out->n_anchors = c->n_anchors;
  out->n_spans = c->n_spans;
  out->n_compressed = c->sc;
  out->n_dense = c->n_dense;
  out->factor_tier = c->cfg.factor_tier;
  out->mu = c->stats[0];
  out->sigma = c->stats[1];
  out->threshold = c->stats[2];
  out->resident_bytes = (uint64_t)L * Hkv * ((uint64_t)c->n_dense * 2 + (uint64_t)c->sc * 2) *
                            kHeadDim * eb +
                        (uint64_t)L * Hq * c->sc * c->cfg.route_dim * eb;
  out->factor_bytes = c->factor_bytes;
  out->factor_pool_bytes = (uint64_t)c->pool_floats * 4;
  out->open_start = c->open_start;
  out->open_len = c->open_len;
  out->n_appended = c->n_appended;
  out->append_capacity = c->cfg.append_capacity;
  return SEKV_OK;
}

sekv_status sekv_cache_copy_spans(const sekv_cache* c, int32_t* anchors, int32_t* span_start,
                                  int32_t* span_len, uint8_t* kind, int32_t* cspan,
                                  int32_t* dense_pos) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (anchors && c->n_anchors)
    SEKV_HIP(hipMemcpy(anchors, c->anchors, (size_t)c->n_anchors * 4, hipMemcpyDeviceToHost));
  if (span_start && c->n_spans)
    SEKV_HIP(hipMemcpy(span_start, c->span_start, (size_t)c->n_spans * 4, hipMemcpyDeviceToHost));
  if (span_len && c->n_spans)
    SEKV_HIP(hipMemcpy(span_len, c->span_len, (size_t)c->n_spans * 4, hipMemcpyDeviceToHost));
  if (kind && c->n_spans)
    SEKV_HIP(hipMemcpy(kind, c->kind, (size_t)c->n_spans, hipMemcpyDeviceToHost));
  if (cspan && c->sc)
    SEKV_HIP(hipMemcpy(cspan, c->cspan, (size_t)c->sc * 4, hipMemcpyDeviceToHost));
  if (dense_pos && c->n_dense)
    SEKV_HIP(hipMemcpy(dense_pos, c->dense_pos, (size_t)c->n_dense * 4, hipMemcpyDeviceToHost));
  return SEKV_OK;
}

sekv_status sekv_cache_copy_group(const sekv_cache* c, int32_t layer, int32_t kv_head, void* kbar,
                                  void* vbar, void* summary, int32_t* rank_k, int32_t* rank_v) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers || kv_head < 0 || kv_head >= c->cfg.n_kv_heads)
    return fail(SEKV_ERR_INVALID, "layer %d / kv_head %d out of range", layer, kv_head);
  const size_t eb = c->kv_elem();
  const int sc = c->sc, G = c->group, dr = c->cfg.route_dim;
  const size_t lg = (size_t)layer * c->cfg.n_kv_heads + kv_head;
  const size_t scs = c->scs;
  if (!sc) return SEKV_OK;
  if (kbar)
    SEKV_HIP(hipMemcpy(kbar, (const char*)c->kbar + lg * scs * kHeadDim * eb,
                       (size_t)sc * kHeadDim * eb, hipMemcpyDeviceToHost));
  if (vbar)
    SEKV_HIP(hipMemcpy(vbar, (const char*)c->vbar + lg * scs * kHeadDim * eb,
                       (size_t)sc * kHeadDim * eb, hipMemcpyDeviceToHost));
  if (summary) {
    const size_t h0 = (size_t)layer * c->cfg.n_q_heads + (size_t)kv_head * G;
    for (int hl = 0; hl < G; ++hl)
      SEKV_HIP(hipMemcpy((char*)summary + (size_t)hl * sc * dr * eb,
                         (const char*)c->summ + (h0 + hl) * scs * dr * eb, (size_t)sc * dr * eb,
                         hipMemcpyDeviceToHost));
  }
  for (int j = 0; j < sc; ++j) {
    if (rank_k) rank_k[j] = rank_of(c->h_rank[lg * scs + j], 0);
    if (rank_v) rank_v[j] = rank_of(c->h_rank[lg * scs + j], 1);
  }
  return SEKV_OK;
}

sekv_status sekv_cache_copy_factors(const sekv_cache* c, int32_t layer, int32_t kv_head,
                                    int32_t span, int32_t kv, float* u, float* sigma, float* vt) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers || kv_head < 0 || kv_head >= c->cfg.n_kv_heads ||
      span < 0 || span >= c->sc || (kv != 0 && kv != 1))
    return fail(SEKV_ERR_INVALID, "layer/kv_head/span/kv out of range");
  const size_t idx = ((size_t)layer * c->cfg.n_kv_heads + kv_head) * c->scs + span;
  const int n = c->h_clen[span];
  const FactorView fv = FactorView::packed(c->h_rank[idx], n);
  const int r = fv.r(kv), r4 = fv.r4(kv);
  std::vector<float> blk(fv.block_floats());
  const float* src = (c->cfg.factor_tier == SEKV_TIER_DEVICE ? c->pool_dev : c->pool_host) +
                     c->h_fac_off[idx];
  if (c->cfg.factor_tier == SEKV_TIER_DEVICE)
    SEKV_HIP(hipMemcpy(blk.data(), src, blk.size() * 4, hipMemcpyDeviceToHost));
  else
    std::memcpy(blk.data(), src, blk.size() * 4);
  if (u)
    for (int t = 0; t < n; ++t)
      for (int i = 0; i < r; ++i) u[(size_t)t * r + i] = blk[fv.u(kv) + (size_t)t * r4 + i];
  if (sigma)
    for (int i = 0; i < r; ++i) sigma[i] = blk[fv.sigma(kv) + i];
  if (vt) std::memcpy(vt, blk.data() + fv.vt(kv), (size_t)r * kHeadDim * 4);
  return SEKV_OK;
}

namespace {

sekv_status check_layer_call(const sekv_cache* c, int32_t layer) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers)
    return fail(SEKV_ERR_INVALID, "layer %d out of range [0, %d)", layer, c->cfg.n_layers);
  return SEKV_OK;
}

sekv_status check_route_out(const sekv_route_out* out) {
  if (!out) return fail(SEKV_ERR_INVALID, "route output is NULL");
  if (!out->mask || !out->list || !out->count || !out->union_list || !out->union_count)
    return fail(SEKV_ERR_INVALID, "route output buffers must be non-NULL (prob may be NULL)");
  return SEKV_OK;
}

// layer slices of the cache, in the layout the layer kernel reads
LayerArgs layer_args(const sekv_cache* c, int32_t layer, const float* q, const float* proj,
                     const float* tau, const sekv_route_out* ro, float* o, void* ws) {
  const int Hq = c->cfg.n_q_heads, Hkv = c->cfg.n_kv_heads;
  const size_t eb = c->kv_elem();
  const size_t lg0 = (size_t)layer * Hkv;
  const bool host_tier = c->cfg.factor_tier == SEKV_TIER_HOST_PINNED;
  LayerArgs a{};
  a.q = q;
  a.proj = proj;
  a.tau = tau;
  a.summ = (const char*)c->summ + (size_t)layer * Hq * c->scs * c->cfg.route_dim * eb;
  a.lnn64 = c->lnn64;
  a.lnn32 = c->lnn32;
  a.gamma = c->cfg.gamma;
  a.dense_k = (const char*)c->dense_k + lg0 * c->ds * kHeadDim * eb;
  a.dense_v = (const char*)c->dense_v + lg0 * c->ds * kHeadDim * eb;
  a.kbar = (const char*)c->kbar + lg0 * c->scs * kHeadDim * eb;
  a.vbar = (const char*)c->vbar + lg0 * c->scs * kHeadDim * eb;
  a.clen = c->clen;
  a.rank = c->rank + lg0 * c->scs;
  a.fac_off = c->fac_off + lg0 * c->scs;
  a.pool = host_tier ? c->stage : c->pool_dev;
  a.off_base = host_tier ? c->layer_base[layer] : 0;
  if (ro) {
    a.mask = ro->mask;
    a.prob = ro->prob;
    a.list = ro->list;
    a.count = ro->count;
    a.ulist = ro->union_list;
    a.ucount = ro->union_count;
  }
  a.o = o;
  a.part = (float*)ws;
  a.chunk_bits = c->chunk_bits;
  a.zcount = c->zcount;
  a.zero_block = c->zero_block;
  return a;
}

}  // namespace

sekv_status sekv_route(const sekv_cache* c, int32_t layer, const float* q_dev,
                       const float* proj_dev, const float* tau_dev, const sekv_route_out* out,
                       hipStream_t stream) {
  sekv_status r;
  if ((r = check_layer_call(c, layer))) return r;
  if (!q_dev || !proj_dev || !tau_dev)
    return fail(SEKV_ERR_INVALID, "q, proj and tau must be non-NULL");
  if ((r = check_route_out(out))) return r;
  if (c->sc == 0) {
    SEKV_HIP(launch_fill_i32(out->count, c->cfg.n_q_heads, 0, stream));
    SEKV_HIP(launch_fill_i32(out->union_count, c->cfg.n_kv_heads, 0, stream));
    return SEKV_OK;
  }
  const LayerArgs a = layer_args(c, layer, q_dev, proj_dev, tau_dev, out, nullptr, nullptr);
  SEKV_HIP(launch_route(c->bf16(), c->geom, a, stream));
  SEKV_HIP(launch_layer_tail(kLists, c->geom, a, stream));
  return SEKV_OK;
}

size_t sekv_decode_workspace_bytes(const sekv_cache* c) {
  if (!c) return 0;
  const size_t b =
      (size_t)c->cfg.n_kv_heads * c->geom.n_slots() * c->group * kPartStride * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

static sekv_status attn_impl(const sekv_cache* c, int32_t layer, const float* q_dev,
                             const sekv_route_out* route, float* o_dev, void* ws_dev,
                             hipStream_t stream, hipStream_t fetch_stream) {
  const LayerArgs a = layer_args(c, layer, q_dev, nullptr, nullptr, route, o_dev, ws_dev);
  const int sc = c->sc;
  if (sc == 0) {
    SEKV_HIP(launch_layer(c->bf16(), kDense, c->geom, a, stream));
    SEKV_HIP(launch_layer_tail(kMerge, c->geom, a, stream));
    return SEKV_OK;
  }
  if (c->cfg.factor_tier == SEKV_TIER_DEVICE) {
    // the chunk masks from the given mask, then as sekv_route_attn after its route
    SEKV_HIP(launch_layer(c->bf16(), kMaskBits, c->geom, a, stream));
    SEKV_HIP(launch_attend(c->bf16(), kDense, c->geom, a, stream));
    SEKV_HIP(launch_layer_tail(kMerge | kZoomSplit, c->geom, a, stream));
    return SEKV_OK;
  }
  // host tier: the zoomed spans' factors are gathered into device staging on
  // the fetch stream while full-resolution rows and coarse entries are
  // attended on `stream`; the zoomed spans and the merge follow the fetch
  for (int n = g_fail_fetch.load(); n > 0;)
    if (g_fail_fetch.compare_exchange_weak(n, n - 1))
      return fail(SEKV_ERR_HIP, "factor fetch of layer %d failed (injected by sekv_test_fail_fetch)",
                  layer);
  const size_t lg0 = (size_t)layer * c->cfg.n_kv_heads;
  hipStream_t fst = fetch_stream ? fetch_stream : stream;
  if (fst != stream) {
    SEKV_HIP(hipEventRecord(c->ev_route, stream));
    SEKV_HIP(hipStreamWaitEvent(fst, c->ev_route, 0));
  }
  // with the residency cache the zoomed spans read their blocks through the
  // offset table the fetch writes (cache slots or the arena's staging)
  LayerArgs az = a;
  if (c->res_on) {
    sekv_cache* cm = const_cast<sekv_cache*>(c);   // per-cache call counter
    if (++cm->res_epoch > kResMaxEpoch) {
      // a fill kernel, not a memset, so that a captured step replays it correctly
      SEKV_HIP(launch_fill_i32((int32_t*)c->res.claim, (int)(c->res.n_sets * 2), 0, fst));
      cm->res_epoch = 1;
    }
    SEKV_HIP(launch_resident_fetch(c->geom, layer, route->union_list, route->union_count,
                                   c->clen, c->rank + lg0 * c->scs, c->fac_off + lg0 * c->scs,
                                   c->layer_base[layer], c->pool_host_dev, c->res, c->res_epoch,
                                   fst));
    az.pool = c->res.arena;
    az.fac_off = c->res.off;
    az.off_base = 0;
  } else if (c->fetch_mode == SEKV_FETCH_MEMCPY) {
    // one hipMemcpyAsync per run of consecutive union spans (their blocks
    // are adjacent in the pool); the union lists must reach the host first,
    // so the host waits for the route
    sekv_cache* cm = const_cast<sekv_cache*>(c);
    const int Hkv = c->cfg.n_kv_heads, sc = c->sc;
    cm->h_ucount.resize(Hkv);
    cm->h_ulist.resize((size_t)Hkv * sc);
    SEKV_HIP(hipMemcpyAsync(cm->h_ucount.data(), route->union_count, (size_t)Hkv * 4,
                            hipMemcpyDeviceToHost, fst));
    SEKV_HIP(hipMemcpyAsync(cm->h_ulist.data(), route->union_list, (size_t)Hkv * sc * 4,
                            hipMemcpyDeviceToHost, fst));
    SEKV_HIP(hipStreamSynchronize(fst));
    const uint64_t base = c->layer_base[layer];
    for (int g = 0; g < Hkv; ++g) {
      const int n = std::min(std::max(cm->h_ucount[g], 0), sc);
      const size_t row = (lg0 + g) * (size_t)c->scs;
      for (int k = 0; k < n;) {
        const int j0 = cm->h_ulist[(size_t)g * sc + k];
        if (j0 < 0 || j0 >= sc) return fail(SEKV_ERR_INVALID, "union list entry %d out of range", j0);
        int j1 = j0 + 1;   // the run j0 .. j1 - 1
        while (k + (j1 - j0) < n && cm->h_ulist[(size_t)g * sc + k + (j1 - j0)] == j1 && j1 < sc)
          ++j1;
        const uint64_t o0 = c->h_fac_off[row + j0];
        const uint64_t o1 = o0 + (uint64_t)FactorView::packed(c->h_rank[row + j1 - 1],
                                                               c->h_clen[j1 - 1]).block_floats() +
                            (c->h_fac_off[row + j1 - 1] - o0);
        SEKV_HIP(hipMemcpyAsync(c->stage + (o0 - base), c->pool_host + o0, (size_t)(o1 - o0) * 4,
                                hipMemcpyHostToDevice, fst));
        k += j1 - j0;
      }
    }
  } else {
    SEKV_HIP(launch_fetch_gather(c->geom, route->union_list, route->union_count, c->clen,
                                 c->rank + lg0 * c->scs, c->fac_off + lg0 * c->scs,
                                 c->layer_base[layer],
                                 c->pool_host_dev, c->stage, fst));
  }
  if (fst != stream) SEKV_HIP(hipEventRecord(c->ev_fetch, fst));
  SEKV_HIP(launch_layer(c->bf16(), kDense, c->geom, a, stream));
  if (fst != stream) SEKV_HIP(hipStreamWaitEvent(stream, c->ev_fetch, 0));
  SEKV_HIP(launch_zoom(c->geom, az, stream));
  SEKV_HIP(launch_layer_tail(kZoomSplit | kMerge, c->geom, az, stream));
  return SEKV_OK;
}

static sekv_status check_workspace(const sekv_cache* c, const void* ws_dev, size_t ws_bytes) {
  if (!ws_dev) return fail(SEKV_ERR_INVALID, "workspace is NULL");
  if (ws_bytes < sekv_decode_workspace_bytes(c))
    return fail(SEKV_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                sekv_decode_workspace_bytes(c));
  return SEKV_OK;
}

sekv_status sekv_decode_attn(const sekv_cache* c, int32_t layer, const float* q_dev,
                             const sekv_route_out* route, float* o_dev, void* ws_dev,
                             size_t ws_bytes, hipStream_t stream, hipStream_t fetch_stream) {
  sekv_status r;
  if ((r = check_layer_call(c, layer))) return r;
  if (!q_dev || !route || !o_dev)
    return fail(SEKV_ERR_INVALID, "q, route and o must be non-NULL");
  if (!route->mask || !route->union_list || !route->union_count)
    return fail(SEKV_ERR_INVALID, "route mask and union lists must be non-NULL");
  if ((r = check_workspace(c, ws_dev, ws_bytes))) return r;
  return attn_impl(c, layer, q_dev, route, o_dev, ws_dev, stream, fetch_stream);
}

sekv_status sekv_route_attn(const sekv_cache* c, int32_t layer, const float* q_dev,
                            const float* proj_dev, const float* tau_dev,
                            const sekv_route_out* route, float* o_dev, void* ws_dev,
                            size_t ws_bytes, hipStream_t stream, hipStream_t fetch_stream) {
  sekv_status r;
  if ((r = check_layer_call(c, layer))) return r;
  if (!q_dev || !proj_dev || !tau_dev || !o_dev)
    return fail(SEKV_ERR_INVALID, "q, proj, tau and o must be non-NULL");
  if ((r = check_route_out(route))) return r;
  if ((r = check_workspace(c, ws_dev, ws_bytes))) return r;
  if (c->cfg.factor_tier == SEKV_TIER_HOST_PINNED || c->sc == 0) {
    if ((r = sekv_route(c, layer, q_dev, proj_dev, tau_dev, route, stream))) return r;
    return attn_impl(c, layer, q_dev, route, o_dev, ws_dev, stream, fetch_stream);
  }
  // route; then rows, coarse entries and zoomed spans side by side; then the
  // merge and lists
  const LayerArgs a = layer_args(c, layer, q_dev, proj_dev, tau_dev, route, o_dev, ws_dev);
  SEKV_HIP(launch_route(c->bf16(), c->geom, a, stream));
  SEKV_HIP(launch_attend(c->bf16(), kDense | kLists, c->geom, a, stream));
  SEKV_HIP(launch_layer_tail(kMerge | kZoomSplit, c->geom, a, stream));
  return SEKV_OK;
}

// ---- the allocation-free route + attention --------------------------------------
// The partial softmax states of sekv_route_attn_noalloc live in this file-scope
// device array instead of a caller workspace.  Each device holds its own copy
// until the process ends.  Host code never uses the array's name as an address:
// its device address is looked up once per device (with that device current)
// and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SEKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sekv_status scratch_for_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SEKV_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    SEKV_HIP(hipGetDevice(&cur));
    if (cur != dev) SEKV_HIP(hipSetDevice(dev));
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) SEKV_HIP(hipSetDevice(cur));
    if (e != hipSuccess)
      return fail(SEKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SEKV_OK;
}
}  // namespace

sekv_status sekv_route_attn_noalloc(const sekv_cache* c, int32_t layer, const float* q_dev,
                                    const float* proj_dev, const float* tau_dev,
                                    const sekv_route_out* route, float* o_dev, hipStream_t stream,
                                    hipStream_t fetch_stream) {
  sekv_status r;
  if ((r = check_layer_call(c, layer))) return r;
  const size_t need = sekv_decode_workspace_bytes(c);
  if (need > (size_t)SEKV_NOALLOC_SCRATCH_BYTES)
    return fail(SEKV_ERR_UNSUPPORTED, "this cache needs %zu bytes of partial states, more than the "
                "%d-byte scratch of the allocation-free call; use sekv_route_attn with a workspace",
                need, (int)SEKV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((r = scratch_for_device(c->device, &ws))) return r;
  return sekv_route_attn(c, layer, q_dev, proj_dev, tau_dev, route, o_dev, ws,
                         (size_t)SEKV_NOALLOC_SCRATCH_BYTES, stream, fetch_stream);
}

static sekv_status cap_impl(const sekv_cache* c, const sekv_route_out* route,
                            int64_t budget_tokens, hipStream_t stream, bool layer_scope) {
  sekv_status r;
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if ((r = check_route_out(route))) return r;
  if (!route->prob)
    return fail(SEKV_ERR_INVALID, "the budget cap orders spans by gate value: route prob is NULL");
  if (budget_tokens < 0)
    return fail(SEKV_ERR_INVALID, "budget_tokens must be >= 0 (got %lld)",
                (long long)budget_tokens);
  if (c->sc > kCapMaxSpans)
    return fail(SEKV_ERR_UNSUPPORTED, "the budget cap handles at most %d compressed spans (cache "
                "has %d)", kCapMaxSpans, c->sc);
  if (c->sc == 0) return SEKV_OK;
  SEKV_HIP(launch_cap_budget(c->sc, c->cfg.n_kv_heads, c->group, (long long)budget_tokens,
                             c->clen, route->prob, route->mask, route->list, route->count,
                             route->union_list, route->union_count,
                             layer_scope ? c->cap_drop : nullptr, stream));
  return SEKV_OK;
}

sekv_status sekv_cap_budget(const sekv_cache* c, const sekv_route_out* route,
                            int64_t budget_tokens, hipStream_t stream) {
  return cap_impl(c, route, budget_tokens, stream, false);
}

sekv_status sekv_cap_budget_layer(const sekv_cache* c, const sekv_route_out* route,
                                  int64_t budget_tokens, hipStream_t stream) {
  return cap_impl(c, route, budget_tokens, stream, true);
}

sekv_status sekv_apply_gates(sekv_cache* c, const float* key_gates_dev,
                             const float* value_gates_dev, float eps, hipStream_t st) {
  if (!c || !key_gates_dev || !value_gates_dev)
    return fail(SEKV_ERR_INVALID, "cache, key gates and value gates must be non-NULL");
  if (!std::isfinite(eps)) return fail(SEKV_ERR_INVALID, "eps must be finite");
  if (c->cfg.factor_tier != SEKV_TIER_DEVICE)
    return fail(SEKV_ERR_UNSUPPORTED, "soft gates repack the device factor pool; this cache keeps "
                "its factors in host memory");
  const int L = c->cfg.n_layers, Hkv = c->cfg.n_kv_heads, sc = c->sc, R = c->cfg.max_rank;
  if (sc == 0) return SEKV_OK;
  const size_t nb = (size_t)L * Hkv * sc;      // gate rows [L][Hkv][S_c]
  const size_t nbs = (size_t)L * Hkv * c->scs;  // table entries [L][Hkv][scs]
  std::vector<float> hg[2];
  for (int kv = 0; kv < 2; ++kv) {
    hg[kv].resize(nb * R);
    SEKV_HIP(hipMemcpyAsync(hg[kv].data(), kv ? value_gates_dev : key_gates_dev,
                            hg[kv].size() * 4, hipMemcpyDeviceToHost, st));
  }
  SEKV_HIP(hipStreamSynchronize(st));
  // which components stay, per matrix: gate >= eps, at least one (the largest
  // gate, the lowest index on ties); the new pool keeps the layout of the old one
  std::vector<uint8_t> kept(nbs * 2 * R, 0);
  std::vector<int32_t> nr(nbs, 0);
  std::vector<uint64_t> noff(nbs, 0), nbase(L + 1, 0);
  uint64_t off = 0, fbytes = 0;
  for (int l = 0; l < L; ++l) {
    nbase[l] = off;
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < sc; ++j) {
        const size_t idx = ((size_t)l * Hkv + g) * c->scs + j;
        const size_t gi = ((size_t)l * Hkv + g) * sc + j;
        const int n = c->h_clen[j];
        int nk[2];
        for (int kv = 0; kv < 2; ++kv) {
          const int r = rank_of(c->h_rank[idx], kv);
          const float* gg = &hg[kv][gi * R];
          uint8_t* kp = &kept[(idx * 2 + kv) * R];
          int k = 0, best = 0;
          for (int i = 0; i < r; ++i) {
            if (!(gg[i] >= 0.f && gg[i] <= 1.f))
              return fail(SEKV_ERR_INVALID, "%s gate %d of (layer %d, KV head %d, span %d) is %g, "
                          "outside [0, 1]", kv ? "value" : "key", i, l, g, j, (double)gg[i]);
            if (gg[i] >= eps) kp[k++] = (uint8_t)i;
            if (gg[i] > gg[best]) best = i;
          }
          if (k == 0) {
            kp[0] = (uint8_t)best;
            k = 1;
          }
          nk[kv] = k;
        }
        const FactorView fv(nk[0], nk[1], n);
        nr[idx] = pack_ranks(nk[0], nk[1]);
        noff[idx] = off;
        off += fv.block_floats();
        fbytes += fv.alg_bytes();
      }
  }
  nbase[L] = off;
  Scratch scr;
  sekv_status r;
  uint8_t* d_kept = nullptr;
  int32_t* d_rank = nullptr;
  uint64_t* d_off = nullptr;
  float* npool = nullptr;
  if ((r = scr.alloc(&d_kept, kept.size(), "gate kept components"))) return r;
  if ((r = scr.alloc(&d_rank, nbs * 4, "gated ranks"))) return r;
  if ((r = scr.alloc(&d_off, nbs * 8, "gated offsets"))) return r;
  // the repacked pool keeps the room an append capacity reserved
  const uint64_t room = c->pool_cap_floats - c->pool_floats;
  if ((r = scr.alloc(&npool, (size_t)(off + room) * 4, "gated factor pool"))) return r;
  SEKV_HIP(hipMemcpyAsync(d_kept, kept.data(), kept.size(), hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemcpyAsync(d_rank, nr.data(), nbs * 4, hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemcpyAsync(d_off, noff.data(), nbs * 8, hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemsetAsync(npool, 0, (size_t)(off + room) * 4, st));
  SEKV_HIP(launch_gate_repack(c->pool_dev, c->fac_off, c->rank, npool, d_off, d_rank, d_kept,
                              key_gates_dev, value_gates_dev, c->clen, sc, c->scs, R, nbs, st));
  SEKV_HIP(hipMemcpyAsync(c->rank, d_rank, nbs * 4, hipMemcpyDeviceToDevice, st));
  SEKV_HIP(hipMemcpyAsync(c->fac_off, d_off, nbs * 8, hipMemcpyDeviceToDevice, st));
  SEKV_HIP(hipStreamSynchronize(st));
  // the new pool replaces the old one
  scr.release(npool);
  c->dev.erase(std::remove(c->dev.begin(), c->dev.end(), (void*)c->pool_dev), c->dev.end());
  (void)hipFree(c->pool_dev);
  c->pool_dev = npool;
  c->dev.push_back(npool);
  c->h_rank = std::move(nr);
  c->h_fac_off = std::move(noff);
  c->layer_base = std::move(nbase);
  c->pool_floats = off;
  c->pool_cap_floats = off + room;
  c->factor_bytes = fbytes;
  return SEKV_OK;
}

// sets of one residency cache, at most (the claims are cleared as 32-bit words)
constexpr uint64_t kResMaxSets = 1ull << 30;

sekv_status sekv_set_residency(sekv_cache* c, uint64_t capacity_bytes, uint64_t slot_bytes) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (c->cfg.factor_tier != SEKV_TIER_HOST_PINNED)
    return fail(SEKV_ERR_INVALID, "the residency cache holds host-tier factors; this cache keeps "
                "its factors in HBM");
  const uint64_t keys = (uint64_t)c->cfg.n_layers * c->cfg.n_kv_heads * (uint64_t)c->sc;
  if (keys > kResKeyMask)
    return fail(SEKV_ERR_UNSUPPORTED, "too many (layer, KV head, span) blocks for the cache keys");
  uint64_t slot_floats = 0, n_sets = 0;
  if (capacity_bytes) {
    if (slot_bytes == 0) return fail(SEKV_ERR_INVALID, "slot_bytes must be > 0");
    slot_floats = ((slot_bytes + 255) / 256) * 64;
    n_sets = capacity_bytes / (slot_floats * 4);
    if (n_sets == 0)
      return fail(SEKV_ERR_INVALID, "capacity of %llu bytes is below one slot of %llu bytes",
                  (unsigned long long)capacity_bytes, (unsigned long long)(slot_floats * 4));
    if (n_sets > kResMaxSets)
      return fail(SEKV_ERR_UNSUPPORTED, "%llu residency sets; at most %llu are supported",
                  (unsigned long long)n_sets, (unsigned long long)kResMaxSets);
  }
  // nothing queued may still use the old tables
  SEKV_HIP(hipDeviceSynchronize());
  c->residency_free();
  if (!capacity_bytes) return SEKV_OK;
  const uint64_t slots_off = (c->stage_floats + 63) / 64 * 64;
  const size_t n_off = std::max<size_t>((size_t)c->cfg.n_kv_heads * c->scs, 1);
  struct Buf { void** p; size_t bytes; const char* what; } bufs[] = {
      {(void**)&c->res.arena, (size_t)(slots_off + n_sets * slot_floats) * 4, "residency arena"},
      {(void**)&c->res.claim, (size_t)n_sets * 8, "residency claims"},
      {(void**)&c->res.tag, (size_t)n_sets * 8, "residency tags"},
      {(void**)&c->res.off, n_off * 8, "residency offsets"},
      {(void**)&c->res.stats, 4 * 8, "residency counters"}};
  for (const Buf& b : bufs) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, b.bytes);
    if (e != hipSuccess) {
      c->residency_free();
      return fail(SEKV_ERR_NOMEM, "hipMalloc(%zu) for %s failed: %s", b.bytes, b.what,
                  hipGetErrorString(e));
    }
    c->res_dev.push_back(p);
    *b.p = p;
  }
  c->res.slots_off = slots_off;
  c->res.slot_floats = slot_floats;
  c->res.n_sets = n_sets;
  hipError_t e = hipMemset(c->res.claim, 0, n_sets * 8);
  if (e == hipSuccess) e = hipMemset(c->res.tag, 0xff, n_sets * 8);
  if (e == hipSuccess) e = hipMemset(c->res.stats, 0, 4 * 8);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    c->residency_free();
    return fail(SEKV_ERR_HIP, "clearing the residency tables failed: %s", hipGetErrorString(e));
  }
  c->res_on = true;
  return SEKV_OK;
}

sekv_status sekv_residency_stats(const sekv_cache* c, uint64_t* out, int32_t reset) {
  if (!c || !out) return fail(SEKV_ERR_INVALID, "cache and out must be non-NULL");
  if (!c->res_on) return fail(SEKV_ERR_INVALID, "the residency cache is not enabled");
  SEKV_HIP(hipDeviceSynchronize());
  SEKV_HIP(hipMemcpy(out, c->res.stats, 4 * 8, hipMemcpyDeviceToHost));
  out[4] = c->res.n_sets;
  out[5] = c->res.slot_floats * 4;
  if (reset) {
    SEKV_HIP(hipMemset(c->res.stats, 0, 4 * 8));
    SEKV_HIP(hipDeviceSynchronize());
  }
  return SEKV_OK;
}

// ---- batches of sequences -------------------------------------------------------
static_assert(kMaxBatch == SEKV_MAX_BATCH, "one batch limit");

static sekv_status batch_impl(const sekv_cache* const* caches, int32_t batch, int32_t layer,
                              const float* const* q_devs, const float* proj_dev,
                              const float* tau_dev, const sekv_route_out* routes,
                              float* const* o_devs, void* const* ws_devs, const size_t* ws_bytes,
                              hipStream_t stream, bool with_route) {
  if (!caches || !q_devs || !routes || !o_devs || !ws_devs || !ws_bytes)
    return fail(SEKV_ERR_INVALID, "caches, q, routes, o, workspace arrays must be non-NULL");
  if (batch < 1 || batch > SEKV_MAX_BATCH)
    return fail(SEKV_ERR_INVALID, "batch %d outside [1, %d]", batch, SEKV_MAX_BATCH);
  if (with_route && (!proj_dev || !tau_dev))
    return fail(SEKV_ERR_INVALID, "proj and tau must be non-NULL");
  sekv_status r;
  for (int i = 0; i < batch; ++i) {
    const sekv_cache* c = caches[i];
    if ((r = check_layer_call(c, layer))) return r;
    const sekv_config& a = c->cfg;
    const sekv_config& b = caches[0]->cfg;
    if (a.n_layers != b.n_layers || a.n_q_heads != b.n_q_heads || a.n_kv_heads != b.n_kv_heads ||
        a.head_dim != b.head_dim || a.route_dim != b.route_dim || a.kv_dtype != b.kv_dtype)
      return fail(SEKV_ERR_INVALID, "cache %d has another model shape than cache 0", i);
    for (int k = 0; k < i; ++k)
      if (caches[k] == c)
        return fail(SEKV_ERR_INVALID, "cache %d appears twice in the batch (slots %d and %d)", i,
                    k, i);
    if (!q_devs[i] || !o_devs[i])
      return fail(SEKV_ERR_INVALID, "q and o of sequence %d must be non-NULL", i);
    if (with_route) {
      if ((r = check_route_out(&routes[i]))) return r;
    } else if (!routes[i].mask || !routes[i].union_list || !routes[i].union_count) {
      return fail(SEKV_ERR_INVALID, "route mask and union lists of sequence %d must be non-NULL",
                  i);
    }
    if ((r = check_workspace(c, ws_devs[i], ws_bytes[i]))) return r;
  }
  // every device-tier sequence with compressed spans goes into the one launch;
  // the others take the single-sequence path (also on `stream`)
  BatchLayerArgs b{};
  int nb = 0;
  for (int i = 0; i < batch; ++i) {
    const sekv_cache* c = caches[i];
    if (c->cfg.factor_tier == SEKV_TIER_HOST_PINNED || c->sc == 0) {
      r = with_route ? sekv_route_attn(c, layer, q_devs[i], proj_dev, tau_dev, &routes[i],
                                       o_devs[i], ws_devs[i], ws_bytes[i], stream, stream)
                     : sekv_decode_attn(c, layer, q_devs[i], &routes[i], o_devs[i], ws_devs[i],
                                        ws_bytes[i], stream, stream);
      if (r) return r;
      continue;
    }
    b.geo[nb] = c->geom;
    b.arg[nb] = layer_args(c, layer, q_devs[i], with_route ? proj_dev : nullptr,
                           with_route ? tau_dev : nullptr, &routes[i], o_devs[i], ws_devs[i]);
    ++nb;
  }
  if (nb > 0) {
    // as the single calls: route (or the chunk masks of the given routes), then
    // zoomed spans beside rows and coarse entries, then merge (and lists)
    const int grp = caches[0]->geom.group;
    if (with_route)
      SEKV_HIP(launch_route_batch(caches[0]->bf16(), grp, b, nb, stream));
    else
      SEKV_HIP(launch_layer_batch(caches[0]->bf16(), kMaskBits, grp, b, nb, stream));
    SEKV_HIP(launch_attend_batch(caches[0]->bf16(), kDense | (with_route ? kLists : 0), grp, b,
                                 nb, stream));
    SEKV_HIP(launch_layer_tail_batch(kMerge | kZoomSplit, grp, b, nb, stream));
  }
  return SEKV_OK;
}

sekv_status sekv_route_attn_batch(const sekv_cache* const* caches, int32_t batch, int32_t layer,
                                  const float* const* q_devs, const float* proj_dev,
                                  const float* tau_dev, const sekv_route_out* routes,
                                  float* const* o_devs, void* const* ws_devs,
                                  const size_t* ws_bytes, hipStream_t stream) {
  return batch_impl(caches, batch, layer, q_devs, proj_dev, tau_dev, routes, o_devs, ws_devs,
                    ws_bytes, stream, true);
}

sekv_status sekv_decode_attn_batch(const sekv_cache* const* caches, int32_t batch, int32_t layer,
                                   const float* const* q_devs, const sekv_route_out* routes,
                                   float* const* o_devs, void* const* ws_devs,
                                   const size_t* ws_bytes, hipStream_t stream) {
  return batch_impl(caches, batch, layer, q_devs, nullptr, nullptr, routes, o_devs, ws_devs,
                    ws_bytes, stream, false);
}

void sekv_cache_destroy(sekv_cache* c) { delete c; }

}  // extern "C"
