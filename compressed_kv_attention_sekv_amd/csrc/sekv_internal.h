// Internal declarations shared by the host runtime and the HIP kernels of the
// SeKV library (gfx950).  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sekv {

constexpr int kHeadDim = 128;     // d: the kernels are written for 128-wide heads
constexpr int kMaxGroup = 8;      // query heads per KV head
constexpr int kMaxRouteDim = 64;  // dr

// ---------------------------------------------------------------------------
// Factor block of one (layer, KV head, compressed span), float32, in the pool:
//   [ VKt r x d | UK r x n4 | sK r4 | VVt r x d | UV r x n4 | sV r4 ]
// VKt/VVt hold the right singular vectors as rows, UK/UV the left singular
// vectors component-major (entry [i][t] is token t of component i, so a wave
// reading one component over consecutive tokens is coalesced), sK/sV the
// singular values.  n4 = n rounded up to 4, r4 = r rounded up to 4, so every
// sub-array starts on a 16-byte boundary; padding entries are zero.  Blocks
// start on 256-byte boundaries.  Algorithmic size: 8 r (n + d + 1) bytes.
// ---------------------------------------------------------------------------
__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }

struct FactorView {
  int r, n, n4, r4;
  __host__ __device__ FactorView(int r_, int n_) : r(r_), n(n_), n4(round4(n_)), r4(round4(r_)) {}
  __host__ __device__ int half() const { return r * kHeadDim + r * n4 + r4; }
  __host__ __device__ int vt(int kv) const { return kv * half(); }
  __host__ __device__ int u(int kv) const { return kv * half() + r * kHeadDim; }
  __host__ __device__ int sigma(int kv) const { return kv * half() + r * kHeadDim + r * n4; }
  __host__ __device__ uint64_t block_floats() const {
    return (uint64_t)((2 * half() + 63) & ~63);
  }
};

// ---------------------------------------------------------------------------
// bfloat16 helpers (storage as uint16_t bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round a double once, to nearest even, to bfloat16.  Inputs are finite; the
// method stores values far inside the bf16 normal range, and values below it
// are flushed to signed zero.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t sign = u >> 63;
  int64_t e = (int64_t)((u >> 52) & 0x7ff);
  if (e == 0) return (uint16_t)(sign << 15);
  int64_t eb = e - 1023 + 127;  // bf16 biased exponent
  if (eb <= 0) return (uint16_t)(sign << 15);
  // 52 mantissa bits -> keep 7: round on the 45 dropped bits, ties to even
  uint64_t mant = u & ((1ull << 52) - 1);
  uint64_t keep = mant >> 45;
  uint64_t rest = mant & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rest > half || (rest == half && (keep & 1))) {
    keep += 1;
    if (keep == 128) { keep = 0; eb += 1; }
  }
  if (eb >= 255) return (uint16_t)((sign << 15) | 0x7f80);
  return (uint16_t)((sign << 15) | ((uint64_t)eb << 7) | keep);
}

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static float from_f64(double x) { return (float)x; }  // IEEE RNE
};
template <> struct Store<uint16_t> {
  __device__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static uint16_t from_f64(double x) { return f64_to_bf16_rne(x); }
};

// ---------------------------------------------------------------------------
// Device views handed to the launchers
// ---------------------------------------------------------------------------
struct SegOut {          // all device, capacity N unless noted
  double* stats;         // [3] mu, sigma, threshold
  int32_t* counts;       // [4] anchors, spans, compressed, dense
  int32_t* anchors;
  int32_t* span_start;
  int32_t* span_len;
  uint8_t* kind;
  int32_t* cspan;        // compressed -> span index
  int32_t* cstart;
  int32_t* clen;
  int32_t* dense_pos;
  uint8_t* flag;         // scratch [N]
};

struct DecodeGeom {
  int n_q_heads, n_kv_heads, group, route_dim;
  int n_dense, n_compressed;
  int dense_tiles, coarse_tiles, zoom_slots, n_slots;
};

// launchers (return hipError_t of the launch)
hipError_t launch_segment(const float* s, int n, int window, double alpha, int min_len,
                          const SegOut& o, hipStream_t st);
hipError_t launch_log_len(const int32_t* clen, int sc, double* lnn64, float* lnn32,
                          hipStream_t st);
hipError_t launch_span_rank(const int32_t* rank_by_pos, const int32_t* cstart,
                            const int32_t* clen, int n_tokens, int sc, int n_lg, int max_rank,
                            int32_t* rank, hipStream_t st);
hipError_t launch_gather_dense(int bf16, const void* src, int n_tokens, const int32_t* pos,
                               int n_dense, int n_lg, void* dst, hipStream_t st);
hipError_t launch_span_summarize(int bf16, const float* s, const void* k, const void* v,
                                 const float* w_route, int n_tokens, const int32_t* cstart,
                                 const int32_t* clen, int sc, int n_layers, int hkv, int group,
                                 int dr, void* kbar, void* vbar, void* summ, hipStream_t st);
hipError_t launch_span_svd(int bf16, const void* x, int n_tokens, const int32_t* cstart,
                           const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                           int n_lg, const int32_t* rank, const uint64_t* fac_off, float* pool,
                           int which, int max_m, hipStream_t st);

hipError_t launch_route(int bf16, const DecodeGeom& g, const float* q, const float* proj,
                        const float* tau, const void* summ, const double* lnn64, double gamma,
                        uint8_t* mask, double* prob, int32_t* list, int32_t* count,
                        int32_t* ulist, int32_t* ucount, int32_t* scratch, uint32_t* tickets,
                        hipStream_t st);
hipError_t launch_attn_tiles(int bf16, const DecodeGeom& g, const float* q, const void* dense_k,
                             const void* dense_v, const void* kbar, const void* vbar,
                             const float* lnn32, const uint8_t* mask, float* part,
                             hipStream_t st);
hipError_t launch_attn_zoom(const DecodeGeom& g, const float* q, const uint8_t* mask,
                            const int32_t* ulist, const int32_t* ucount, const int32_t* clen,
                            const int32_t* rank, const uint64_t* fac_off, const float* pool,
                            uint64_t off_base, float* part, hipStream_t st);
hipError_t launch_attn_merge(const DecodeGeom& g, const float* part, float* o, hipStream_t st);
hipError_t launch_fetch_gather(const DecodeGeom& g, const int32_t* ulist, const int32_t* ucount,
                               const int32_t* clen, const int32_t* rank,
                               const uint64_t* fac_off, uint64_t layer_base,
                               const float* host_pool_mapped, float* stage, hipStream_t st);

}  // namespace sekv
