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
//   [ VKt rK x d | UK n x rK4 | sK rK4 | VVt rV x d | UV n x rV4 | sV rV4 ]
// The key and value matrices of a span are factored separately and keep their
// own ranks rK and rV (equal after the build; soft gates may make them
// differ).  VKt/VVt hold the right singular vectors as rows; UK/UV hold the
// left singular vectors token-major (row t is token t's coefficients, padded
// to r4 = r rounded up to 4), so one lane reads a token's whole row with
// 16-byte loads and the rows of consecutive tokens are contiguous; sK/sV hold
// the singular values.  Every sub-array starts on a 16-byte boundary and
// padding entries are zero.  Blocks start on 256-byte boundaries.
// Algorithmic size: 4 (rK + rV) (n + d + 1) bytes.
//
// The rank table holds one int32 per block: rK in the low 16 bits, rV in the
// high 16 bits.
// ---------------------------------------------------------------------------
__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }
__host__ __device__ inline int32_t pack_ranks(int rk, int rv) {
  return (int32_t)((uint32_t)rk | ((uint32_t)rv << 16));
}
// rank of the key (kv = 0) or value (kv = 1) factors of a packed entry
__host__ __device__ inline int rank_of(int32_t packed, int kv) {
  return kv ? (int)((uint32_t)packed >> 16) : (int)((uint32_t)packed & 0xffffu);
}
__host__ __device__ inline int rank_max(int32_t packed) {
  const int a = rank_of(packed, 0), b = rank_of(packed, 1);
  return a > b ? a : b;
}

struct FactorView {
  int rk, rv, n;
  __host__ __device__ FactorView(int rk_, int rv_, int n_) : rk(rk_), rv(rv_), n(n_) {}
  __host__ __device__ static FactorView packed(int32_t ranks, int n_) {
    return FactorView(rank_of(ranks, 0), rank_of(ranks, 1), n_);
  }
  __host__ __device__ int r(int kv) const { return kv ? rv : rk; }
  __host__ __device__ int r4(int kv) const { return round4(r(kv)); }
  __host__ __device__ int half(int kv) const { return r(kv) * kHeadDim + n * r4(kv) + r4(kv); }
  __host__ __device__ int vt(int kv) const { return kv ? half(0) : 0; }
  __host__ __device__ int u(int kv) const { return vt(kv) + r(kv) * kHeadDim; }
  __host__ __device__ int sigma(int kv) const { return u(kv) + n * r4(kv); }
  __host__ __device__ uint64_t block_floats() const {
    return (uint64_t)((half(0) + half(1) + 63) & ~63);
  }
  // algorithmic bytes of the block: 4 (rK + rV) (n + d + 1)
  __host__ __device__ uint64_t alg_bytes() const {
    return 4ull * (uint64_t)(rk + rv) * (uint64_t)(n + kHeadDim + 1);
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

// ---------------------------------------------------------------------------
// Decode geometry of a cache.  Per KV head the layer kernel runs n_work
// workgroups; workgroup w owns
//   compressed spans [kChunk w, kChunk (w + 1)) (routing, coarse entries and
//   the zoomed spans among them), and
//   full-resolution rows [dense_rows w, dense_rows (w + 1)).
// The zoomed spans of a layer run in a launch of their own, z_total
// workgroups dealt to the KV heads in proportion to their union sizes.
// Partial softmax states live in the workspace as
//   part[Hkv][n_work + z_total][G][kPartStride] floats: m, l, -, -, acc[d]
// slot w < n_work holds layer workgroup w's rows and coarse entries, slot
// n_work + i the spans of the KV head's i-th zoom workgroup; zcount[g] (per
// cache) records how many zoom workgroups KV head g got in the last launch.
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;                 // waves per workgroup of the layer kernel
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 32;                // compressed spans per workgroup
constexpr int kRowBlock = 16;             // full-resolution rows per wave per pass
constexpr int kMaxDenseRows = 256;        // full-resolution rows per workgroup, at most
constexpr int kPartStride = kHeadDim + 4;
constexpr int kMaxRank = kHeadDim;
constexpr int kListWords = kMaxGroup + 1; // zoom bit masks per chunk: heads, then union
// A block of zeros each cache owns: the source of the layer kernel's prefetches
// when a wave has nothing to prefetch, so that every wave issues the same
// loads and the compiler counts outstanding loads exactly.  It holds a factor
// block of one token at rank 1 and a full V_K stage (32 rows of d floats).
constexpr int kZeroBlockFloats = 32 * kHeadDim;
constexpr int kMaxKvHeads = 256;          // KV heads of a layer, at most
constexpr int kZoomWgMax = 512;           // zoom workgroups filling the GPU (two per CU)
constexpr int kAttendZoomWgs = 256;       // zoom workgroups beside the rows: one per CU of
                                          // MI355X (two ~80 KB workgroups fit a CU)
constexpr int kZoomBatchMax = 64;         // zoomed spans of one zoom workgroup, at most
constexpr int kRouteChunks = 4;           // chunks per route workgroup for the largest grids

struct LayerGeom {
  int n_q_heads, n_kv_heads, group, route_dim;
  int n_dense, n_compressed;
  int dense_stride;  // rows between the full-resolution sets of two KV heads (>= n_dense)
  int sc_stride;     // entries between two (layer, head) rows of the span arrays (>= S_c)
  int n_chunks;      // ceil(S_c / kChunk)
  int n_work;        // workgroups per KV head: max(1, n_chunks, ceil(D / kMaxDenseRows))
  int dense_rows;    // full-resolution rows per workgroup, a multiple of kWaves * kRowBlock
  int z_total;       // zoom workgroups (see make_layer_geom)
  int z_attend;      // zoom workgroups of launch_attend (<= z_total)
  int z_slots;       // zoom partial slots per KV head: z_total as built (launch_attend
                     // deals the spans to fewer workgroups, into the same slots)
  __host__ __device__ int n_slots() const { return n_work + z_slots; }
};

__host__ inline LayerGeom make_layer_geom(int hq, int hkv, int dr, int n_dense, int sc,
                                          int dense_stride, int sc_stride) {
  LayerGeom g{};
  g.dense_stride = dense_stride;
  g.sc_stride = sc_stride;
  g.n_q_heads = hq;
  g.n_kv_heads = hkv;
  g.group = hq / hkv;
  g.route_dim = dr;
  g.n_dense = n_dense;
  g.n_compressed = sc;
  g.n_chunks = (sc + kChunk - 1) / kChunk;
  int w = (n_dense + kMaxDenseRows - 1) / kMaxDenseRows;
  if (w < g.n_chunks) w = g.n_chunks;
  if (w < 1) w = 1;
  g.n_work = w;
  const int unit = kWaves * kRowBlock;
  const int rows = (n_dense + w - 1) / w;
  g.dense_rows = (rows + unit - 1) / unit * unit;
  // zoom workgroups: enough to fill the GPU (at most kZoomWgMax unless more
  // are needed), and never fewer than Hkv S_c / kZoomBatchMax + Hkv, so that
  // no workgroup's share of a layer's zoomed spans exceeds kZoomBatchMax
  int z = hkv * g.n_chunks;
  if (z > kZoomWgMax) z = kZoomWgMax;
  const long long need = ((long long)hkv * sc + kZoomBatchMax - 1) / kZoomBatchMax + hkv;
  if (z < need) z = (int)need;
  g.z_total = z;
  g.z_slots = z;
  // beside the rows in one launch (launch_attend): one zoom workgroup per CU,
  // the other slot of each CU taking row workgroups (measured at 128K: 188,
  // 256, 320 and 512 zoom workgroups gave 37.1, 35.7, 36.4 and 37.0 us per
  // layer), within the same bounds
  long long za = kAttendZoomWgs;
  if (za < need) za = need;
  if (za > z) za = z;
  g.z_attend = (int)za;
  return g;
}

// What one launch of the layer kernel does (bit set).
enum LayerMode : int {
  kDense = 2,      // layer launch: attend the workgroup's full-resolution rows and coarse
                   // entries (and write the chunk's zoom masks from the mask)
  kZoomSplit = 8,  // tail launch: merge the zoom workgroups' slots too
  kMerge = 16,     // tail launch: merge each query head's partials into o
  kLists = 32,     // tail or attend launch: write the ascending zoom lists and union
  kKeepBits = 64,  // with kDense: leave the chunk masks the route launch wrote
  kMaskBits = 128, // layer launch, alone: write the chunk masks from a given route's mask
};

struct LayerArgs {
  const float* q;          // [Hq][d]
  const float* proj;       // [Hq][dr][d]
  const float* tau;        // [Hq]
  const void* summ;        // [Hq][S_c][dr] storage type
  const double* lnn64;     // [S_c]
  const float* lnn32;      // [S_c]
  double gamma;
  const void* dense_k;     // [Hkv][D][d]
  const void* dense_v;
  const void* kbar;        // [Hkv][S_c][d]
  const void* vbar;
  const int32_t* clen;     // [S_c]
  const int32_t* rank;     // [Hkv][sc_stride] packed key and value ranks
  const uint64_t* fac_off; // [Hkv][sc_stride] float offsets
  const float* pool;       // factor blocks, addressed as pool + (fac_off - off_base)
  uint64_t off_base;
  uint8_t* mask;           // [Hq][S_c] (written by the route launch, read otherwise)
  double* prob;            // [Hq][S_c] or NULL
  int32_t* list;           // [Hq][S_c]
  int32_t* count;          // [Hq]
  int32_t* ulist;          // [Hkv][S_c]
  int32_t* ucount;         // [Hkv]
  float* o;                // [Hq][d]
  float* part;             // workspace
  uint32_t* chunk_bits;    // [Hkv][n_work][kListWords] zoom bit masks of each chunk
  int32_t* zcount;         // [Hkv] zoom workgroups of each KV head (written by the zoom kernel)
  const float* zero_block; // kZeroBlockFloats zeros
};

// A batch of independent sequences (one cache each, same model shape) through
// one launch per layer: every sequence's geometry and pointers travel in the
// kernel arguments.
constexpr int kMaxBatch = 8;
struct BatchLayerArgs {
  LayerGeom geo[kMaxBatch];
  LayerArgs arg[kMaxBatch];
};
static_assert(sizeof(BatchLayerArgs) + 16 <= 4096, "kernel arguments fit 4 KB");

// launchers (return hipError_t of the launch)
hipError_t launch_segment(const float* s, int n, int window, double alpha, int min_len,
                          const SegOut& o, hipStream_t st);
hipError_t launch_log_len(const int32_t* clen, int sc, double* lnn64, float* lnn32,
                          hipStream_t st);
// spans j0 .. j0 + n - 1; `stride` separates the (layer, head) rows of the
// span arrays, n_tokens the rows of the K/V (or dense) source
hipError_t launch_span_rank(const int32_t* rank_by_pos, const int32_t* cstart,
                            const int32_t* clen, int n_tokens, int j0, int n, int stride,
                            int n_lg, int max_rank, int32_t* rank, hipStream_t st);
hipError_t launch_gather_dense(int bf16, const void* src, int n_tokens, const int32_t* pos,
                               int n_dense, int dst_stride, int n_lg, void* dst, hipStream_t st);
// window append: per-row 32-bit gather, and removal of sorted row ranges
// ([a, len] pairs, device int32) from [0, n_rows) of each of n_lg blocks of
// stride rows (rows of elems_per_row elements of elem_bytes 4 or 16)
hipError_t launch_gather_words(const uint32_t* src, int src_stride, const int32_t* pos, int n,
                               int dst_stride, int n_lg, uint32_t* dst, hipStream_t st);
hipError_t launch_compact_rows(void* base, int elem_bytes, int stride, int elems_per_row,
                               int n_rows, int n_lg, const int32_t* ranges, int n_ranges,
                               hipStream_t st);
hipError_t launch_span_summarize(int bf16, const float* s, const void* k, const void* v,
                                 const float* w_route, int n_tokens, const int32_t* cstart,
                                 const int32_t* clen, int j0, int n, int sc, int n_layers,
                                 int hkv, int group, int dr, void* kbar, void* vbar, void* summ,
                                 hipStream_t st);
hipError_t launch_span_svd(int bf16, const void* x, int n_tokens, const int32_t* cstart,
                           const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                           int n_lg, const int32_t* rank, const uint64_t* fac_off, float* pool,
                           int which, int max_m, hipStream_t st);

// randomized truncated SVD (build option): spans of kRsvdMinRows < n <=
// kRsvdMaxRows tokens, ranks up to kRsvdMaxRank; other spans take the exact path
// (launches sized for 128, 256 and kRsvdMaxRows rows)
constexpr int kRsvdMaxRank = 32;
constexpr int kRsvdMinRows = 40;
constexpr int kRsvdMaxRows = 640;
hipError_t launch_span_rsvd(int bf16, const void* x, int n_tokens, const int32_t* cstart,
                            const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                            int n_lg, const int32_t* rank, const uint64_t* fac_off, float* pool,
                            int which, int max_rows, hipStream_t st);

hipError_t launch_layer(int bf16, int mode, const LayerGeom& g, const LayerArgs& a,
                        hipStream_t st);
// the route of a layer alone (mask, gate values, chunk masks): 1, 2 or
// kRouteChunks chunks per workgroup as the grid grows
hipError_t launch_route(int bf16, const LayerGeom& g, const LayerArgs& a, hipStream_t st);
hipError_t launch_route_batch(int bf16, int group, const BatchLayerArgs& b, int batch,
                              hipStream_t st);
hipError_t launch_layer_batch(int bf16, int mode, int group, const BatchLayerArgs& b, int batch,
                              hipStream_t st);
// the merge and lists of a layer (kMerge, kLists, kZoomSplit bits of mode) in a
// launch of their own, after a layer launch without those bits
hipError_t launch_layer_tail(int mode, const LayerGeom& g, const LayerArgs& a, hipStream_t st);
hipError_t launch_layer_tail_batch(int mode, int group, const BatchLayerArgs& b, int batch,
                                   hipStream_t st);
// the zoomed spans of a layer, after a layer launch that wrote its chunk masks
hipError_t launch_zoom(const LayerGeom& g, const LayerArgs& a, hipStream_t st);
// rows, coarse entries (mode kDense) and the zoomed spans of a layer in one
// launch, after a route-only layer launch (which wrote mask and chunk masks)
hipError_t launch_attend(int bf16, int mode, const LayerGeom& g, const LayerArgs& a,
                         hipStream_t st);
hipError_t launch_attend_batch(int bf16, int mode, int group, const BatchLayerArgs& b, int batch,
                               hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);
// matched-budget cap of one layer's route output (in place); the kernel keeps
// one bit per union entry in LDS, so S_c is limited to kCapMaxSpans
constexpr int kCapMaxSpans = 1 << 19;
size_t cap_budget_lds_bytes(int sc);
// drop == NULL caps each KV head on its own; else drop [Hkv][S_c] bytes of
// scratch and one budget for the whole layer
hipError_t launch_cap_budget(int sc, int hkv, int group, long long budget, const int32_t* clen,
                             const double* prob, uint8_t* mask, int32_t* list, int32_t* count,
                             int32_t* ulist, int32_t* ucount, uint8_t* drop, hipStream_t st);
// HBM residency cache of host-tier factor blocks (two-choice: a block may sit
// in either of two hashed sets, one slot per set).  A block's key is
// (layer * Hkv + g) * S_c + j, below 2^kResKeyBits; a set's claim is
// (epoch << (kResKeyBits + 1)) | (holds << kResKeyBits) | (kResKeyMask - key)
// of its winner, holds = 1 if the set already holds that block.
constexpr int kResKeyBits = 39;
constexpr uint64_t kResKeyMask = (1ull << kResKeyBits) - 1;
constexpr uint64_t kResMaxEpoch = (1ull << (64 - kResKeyBits - 1)) - 1;
struct ResidencyView {
  float* arena;                // [staging of one layer | n_sets slots]
  uint64_t slots_off;          // first float of slot 0
  uint64_t slot_floats;        // multiple of 64
  uint64_t n_sets;
  unsigned long long* claim;   // [n_sets]
  long long* tag;              // [n_sets], -1 = empty
  uint64_t* off;               // [Hkv][S_c] arena offset of each union block, this call
  unsigned long long* stats;   // hit blocks, fetched blocks, hit bytes, fetched bytes
};
hipError_t launch_resident_fetch(const LayerGeom& g, int layer, const int32_t* ulist,
                                 const int32_t* ucount, const int32_t* clen, const int32_t* rank,
                                 const uint64_t* fac_off, uint64_t layer_base,
                                 const float* host_pool_mapped, const ResidencyView& rv,
                                 uint64_t epoch, hipStream_t st);
// soft gates: repack every (layer, KV head, span) block of the device pool
// into a new pool with the kept components (gate-scaled sigma); kept is
// [blocks][2][max_rank] (keys, then values), the gates [blocks][max_rank] each
hipError_t launch_gate_repack(const float* old_pool, const uint64_t* old_off,
                              const int32_t* old_rank, float* new_pool, const uint64_t* new_off,
                              const int32_t* new_rank, const uint8_t* kept, const float* key_gates,
                              const float* value_gates, const int32_t* clen, int sc, int scs,
                              int max_rank, uint64_t n_blocks, hipStream_t st);
hipError_t launch_fetch_gather(const LayerGeom& g, const int32_t* ulist, const int32_t* ucount,
                               const int32_t* clen, const int32_t* rank,
                               const uint64_t* fac_off, uint64_t layer_base,
                               const float* host_pool_mapped, float* stage, hipStream_t st);

}  // namespace sekv
