// Host runtime and C ABI of the SeKV library: argument validation, the cache
// handle (device tables, full-resolution rows, means, summaries, factor pool
// in HBM or pinned host memory), and the launch sequence of the build and of
// each decode step.  See include/sekv.h for the contract of every call.
#include "sekv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "sekv_internal.h"

using namespace sekv;

namespace {

thread_local std::string g_err;

sekv_status fail(sekv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
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
  if (c->reserved != 0) return fail(SEKV_ERR_INVALID, "reserved must be 0");
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
                        int32_t counts[4], double stats[3], hipStream_t st) {
  sekv_status r;
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
  SEKV_HIP(launch_segment(s, n, cfg->window, cfg->alpha, cfg->min_span_len, o, st));
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
  float* pool_host_dev = nullptr; // device view of pool_host
  float* stage = nullptr;         // host tier: device staging for one layer
  uint64_t stage_floats = 0;
  uint32_t* chunk_bits = nullptr;  // [Hkv][n_work][kListWords] zoom bit masks of each chunk
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
  if ((r = run_segment(cfg, n_tokens, s, scr, o, counts, c->stats, st))) return r;
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

  if ((r = c->alloc(&c->lnn64, (size_t)sc * 8, "lnn64"))) return r;
  if ((r = c->alloc(&c->lnn32, (size_t)sc * 4, "lnn32"))) return r;
  SEKV_HIP(launch_log_len(c->clen, sc, c->lnn64, c->lnn32, st));
  if ((r = c->alloc(&c->rank, (size_t)n_lg * sc * 4, "rank"))) return r;
  SEKV_HIP(launch_span_rank(rank_by_pos, c->cstart, c->clen, n_tokens, sc, n_lg, cfg->max_rank,
                            c->rank, st));

  // ---- full-resolution rows ------------------------------------------------
  if ((r = c->alloc(&c->dense_k, (size_t)n_lg * D * kHeadDim * eb, "dense_k"))) return r;
  if ((r = c->alloc(&c->dense_v, (size_t)n_lg * D * kHeadDim * eb, "dense_v"))) return r;
  SEKV_HIP(launch_gather_dense(c->bf16(), k_dev, n_tokens, c->dense_pos, D, n_lg, c->dense_k, st));
  SEKV_HIP(launch_gather_dense(c->bf16(), v_dev, n_tokens, c->dense_pos, D, n_lg, c->dense_v, st));

  // ---- means and summaries -------------------------------------------------
  if ((r = c->alloc(&c->kbar, (size_t)n_lg * sc * kHeadDim * eb, "kbar"))) return r;
  if ((r = c->alloc(&c->vbar, (size_t)n_lg * sc * kHeadDim * eb, "vbar"))) return r;
  if ((r = c->alloc(&c->summ, (size_t)L * Hq * sc * dr * eb, "summaries"))) return r;
  SEKV_HIP(launch_span_summarize(c->bf16(), s, k_dev, v_dev, w_route, n_tokens, c->cstart,
                                 c->clen, sc, L, Hkv, c->group, dr, c->kbar, c->vbar, c->summ, st));

  // ---- factor pool layout (host) ---------------------------------------------
  c->h_rank.resize((size_t)n_lg * sc);
  c->h_clen.resize(sc);
  if (sc) {
    SEKV_HIP(hipMemcpyAsync(c->h_rank.data(), c->rank, c->h_rank.size() * 4,
                            hipMemcpyDeviceToHost, st));
    SEKV_HIP(hipMemcpyAsync(c->h_clen.data(), c->clen, (size_t)sc * 4, hipMemcpyDeviceToHost, st));
  }
  SEKV_HIP(hipStreamSynchronize(st));
  c->h_fac_off.resize((size_t)n_lg * sc);
  c->layer_base.assign(L + 1, 0);
  uint64_t off = 0, fbytes = 0, stage_max = 0;
  for (int l = 0; l < L; ++l) {
    c->layer_base[l] = off;
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < sc; ++j) {
        const size_t idx = ((size_t)l * Hkv + g) * sc + j;
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
    if ((r = c->alloc(&c->pool_dev, pool_bytes, "factor pool"))) return r;
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
                                  d_ids, (int)rs_ids[b].size(), sc, n_lg, c->rank, c->fac_off,
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
                                 d_ids, (int)ids[b].size(), sc, n_lg, c->rank, c->fac_off,
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
  c->geom = make_layer_geom(Hq, Hkv, dr, D, sc);
  if ((r = c->alloc(&c->chunk_bits, (size_t)Hkv * c->geom.n_work * kListWords * 4, "chunk bits")))
    return r;
  if ((r = c->alloc(&c->zero_block, (size_t)kZeroBlockFloats * 4, "zero block"))) return r;
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
  r = build_impl(cfg, n_tokens, surprisal_dev, k_dev, v_dev, w_route_dev, rank_by_pos_dev, stream,
                 c);
  if (r) {
    (void)hipStreamSynchronize(stream);  // nothing queued may outlive the freed buffers
    return r;
  }
  *out = c.release();
  return SEKV_OK;
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
  if (!sc) return SEKV_OK;
  if (kbar)
    SEKV_HIP(hipMemcpy(kbar, (const char*)c->kbar + lg * sc * kHeadDim * eb, (size_t)sc * kHeadDim * eb,
                       hipMemcpyDeviceToHost));
  if (vbar)
    SEKV_HIP(hipMemcpy(vbar, (const char*)c->vbar + lg * sc * kHeadDim * eb, (size_t)sc * kHeadDim * eb,
                       hipMemcpyDeviceToHost));
  if (summary) {
    const size_t h0 = (size_t)layer * c->cfg.n_q_heads + (size_t)kv_head * G;
    SEKV_HIP(hipMemcpy(summary, (const char*)c->summ + h0 * sc * dr * eb, (size_t)G * sc * dr * eb,
                       hipMemcpyDeviceToHost));
  }
  for (int j = 0; j < sc; ++j) {
    if (rank_k) rank_k[j] = rank_of(c->h_rank[lg * sc + j], 0);
    if (rank_v) rank_v[j] = rank_of(c->h_rank[lg * sc + j], 1);
  }
  return SEKV_OK;
}

sekv_status sekv_cache_copy_factors(const sekv_cache* c, int32_t layer, int32_t kv_head,
                                    int32_t span, int32_t kv, float* u, float* sigma, float* vt) {
  if (!c) return fail(SEKV_ERR_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers || kv_head < 0 || kv_head >= c->cfg.n_kv_heads ||
      span < 0 || span >= c->sc || (kv != 0 && kv != 1))
    return fail(SEKV_ERR_INVALID, "layer/kv_head/span/kv out of range");
  const size_t idx = ((size_t)layer * c->cfg.n_kv_heads + kv_head) * c->sc + span;
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
  const int Hq = c->cfg.n_q_heads, Hkv = c->cfg.n_kv_heads, sc = c->sc, D = c->n_dense;
  const size_t eb = c->kv_elem();
  const size_t lg0 = (size_t)layer * Hkv;
  const bool host_tier = c->cfg.factor_tier == SEKV_TIER_HOST_PINNED;
  LayerArgs a{};
  a.q = q;
  a.proj = proj;
  a.tau = tau;
  a.summ = (const char*)c->summ + (size_t)layer * Hq * sc * c->cfg.route_dim * eb;
  a.lnn64 = c->lnn64;
  a.lnn32 = c->lnn32;
  a.gamma = c->cfg.gamma;
  a.dense_k = (const char*)c->dense_k + lg0 * D * kHeadDim * eb;
  a.dense_v = (const char*)c->dense_v + lg0 * D * kHeadDim * eb;
  a.kbar = (const char*)c->kbar + lg0 * sc * kHeadDim * eb;
  a.vbar = (const char*)c->vbar + lg0 * sc * kHeadDim * eb;
  a.clen = c->clen;
  a.rank = c->rank + lg0 * sc;
  a.fac_off = c->fac_off + lg0 * sc;
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
  SEKV_HIP(launch_layer(c->bf16(), kRoute, c->geom, a, stream));
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
  if (c->cfg.factor_tier == SEKV_TIER_DEVICE || sc == 0) {
    SEKV_HIP(launch_layer(c->bf16(), kDense | kZoom, c->geom, a, stream));
    SEKV_HIP(launch_layer_tail(kMerge, c->geom, a, stream));
    return SEKV_OK;
  }
  // host tier: the zoomed spans' factors are gathered into device staging on
  // the fetch stream while full-resolution rows and coarse entries are
  // attended on `stream`; the zoomed spans and the merge follow the fetch
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
                                   c->clen, c->rank + lg0 * sc, c->fac_off + lg0 * sc,
                                   c->layer_base[layer], c->pool_host_dev, c->res, c->res_epoch,
                                   fst));
    az.pool = c->res.arena;
    az.fac_off = c->res.off;
    az.off_base = 0;
  } else {
    SEKV_HIP(launch_fetch_gather(c->geom, route->union_list, route->union_count, c->clen,
                                 c->rank + lg0 * sc, c->fac_off + lg0 * sc, c->layer_base[layer],
                                 c->pool_host_dev, c->stage, fst));
  }
  if (fst != stream) SEKV_HIP(hipEventRecord(c->ev_fetch, fst));
  SEKV_HIP(launch_layer(c->bf16(), kDense, c->geom, a, stream));
  if (fst != stream) SEKV_HIP(hipStreamWaitEvent(stream, c->ev_fetch, 0));
  SEKV_HIP(launch_layer(c->bf16(), kZoom | kZoomSplit, c->geom, az, stream));
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
  const LayerArgs a = layer_args(c, layer, q_dev, proj_dev, tau_dev, route, o_dev, ws_dev);
  SEKV_HIP(launch_layer(c->bf16(), kRoute | kDense | kZoom, c->geom, a, stream));
  SEKV_HIP(launch_layer_tail(kMerge | kLists, c->geom, a, stream));
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

sekv_status sekv_cap_budget(const sekv_cache* c, const sekv_route_out* route,
                            int64_t budget_tokens, hipStream_t stream) {
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
                             route->union_list, route->union_count, stream));
  return SEKV_OK;
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
  const size_t nb = (size_t)L * Hkv * sc;
  std::vector<float> hg[2];
  for (int kv = 0; kv < 2; ++kv) {
    hg[kv].resize(nb * R);
    SEKV_HIP(hipMemcpyAsync(hg[kv].data(), kv ? value_gates_dev : key_gates_dev,
                            hg[kv].size() * 4, hipMemcpyDeviceToHost, st));
  }
  SEKV_HIP(hipStreamSynchronize(st));
  // which components stay, per matrix: gate >= eps, at least one (the largest
  // gate, the lowest index on ties); the new pool keeps the layout of the old one
  std::vector<uint8_t> kept(nb * 2 * R, 0);
  std::vector<int32_t> nr(nb);
  std::vector<uint64_t> noff(nb), nbase(L + 1, 0);
  uint64_t off = 0, fbytes = 0;
  for (int l = 0; l < L; ++l) {
    nbase[l] = off;
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < sc; ++j) {
        const size_t idx = ((size_t)l * Hkv + g) * sc + j;
        const int n = c->h_clen[j];
        int nk[2];
        for (int kv = 0; kv < 2; ++kv) {
          const int r = rank_of(c->h_rank[idx], kv);
          const float* gg = &hg[kv][idx * R];
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
  if ((r = scr.alloc(&d_rank, nb * 4, "gated ranks"))) return r;
  if ((r = scr.alloc(&d_off, nb * 8, "gated offsets"))) return r;
  if ((r = scr.alloc(&npool, (size_t)off * 4, "gated factor pool"))) return r;
  SEKV_HIP(hipMemcpyAsync(d_kept, kept.data(), kept.size(), hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemcpyAsync(d_rank, nr.data(), nb * 4, hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemcpyAsync(d_off, noff.data(), nb * 8, hipMemcpyHostToDevice, st));
  SEKV_HIP(hipMemsetAsync(npool, 0, (size_t)off * 4, st));
  SEKV_HIP(launch_gate_repack(c->pool_dev, c->fac_off, c->rank, npool, d_off, d_rank, d_kept,
                              key_gates_dev, value_gates_dev, c->clen, sc, R, nb, st));
  SEKV_HIP(hipMemcpyAsync(c->rank, d_rank, nb * 4, hipMemcpyDeviceToDevice, st));
  SEKV_HIP(hipMemcpyAsync(c->fac_off, d_off, nb * 8, hipMemcpyDeviceToDevice, st));
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
  const size_t n_off = std::max<size_t>((size_t)c->cfg.n_kv_heads * c->sc, 1);
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
    const int mode = with_route ? (kRoute | kDense | kZoom) : (kDense | kZoom);
    const int tail = with_route ? (kMerge | kLists) : kMerge;
    SEKV_HIP(launch_layer_batch(caches[0]->bf16(), mode, caches[0]->geom.group, b, nb, stream));
    SEKV_HIP(launch_layer_tail_batch(tail, caches[0]->geom.group, b, nb, stream));
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
