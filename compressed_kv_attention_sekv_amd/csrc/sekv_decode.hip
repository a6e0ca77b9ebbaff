// Decode-step kernels of the SeKV cache (gfx950).  A layer is three launches:
// the route gates every compressed span; the attend launch attends the zoomed
// spans beside the full-resolution rows and coarse entries; a small tail
// merges the partial softmax states.
//
// SeKV paper Sec. 3.2 (query projected into the routing space; independent
// sigmoid gate with a gamma ln n size prior) and Sec. 3.3 (Eq. 9 zoom decision
// per head; one softmax over anchors, window, tokens of zoomed spans rebuilt
// from their low-rank factors (Eq. 8 with hard gates), and one coarse entry per
// other span whose scaled score gets + ln n_j).
//
// Per KV head g:
//   - route: each workgroup projects the group's queries into routing space
//     (float64), gates chunks of 32 compressed spans and writes their zoom mask
//     and one bit mask per list (per head, and their union) for each chunk;
//   - attend: zoom workgroups share out the union's spans and attend each one
//     straight from its factors, one wave per span:
//       b_h = sigma_K * (V_K^T q_h) / sqrt(d);  e_{h,t} = U_K[t] . b_h;
//       c_h = U_V^T p_h;  acc_h += V_V^T (sigma_V * c_h)
//     so the factors are read once for all heads and no token row is formed;
//     row workgroups stream a slice of the full-resolution rows (window,
//     anchors, short-span tokens) with 16-byte loads shared by the G query
//     heads, and the coarse entries of a chunk that a head did not zoom;
//     list workgroups write the ascending zoom lists from the bit masks;
//   - tail: one workgroup per query head merges the partial (m, l, acc) of
//     every attend workgroup of its KV head into o.
// The kernel boundaries make every workgroup's stores visible to the next
// launch, so no workgroup waits on another and no agent-scope fence (an L2
// write-back or invalidation, which stalls the workgroups still streaming
// factors through that L2) sits inside a launch.
#include <hip/hip_runtime.h>
#include <math.h>

#include "sekv_internal.h"

namespace sekv {

// ---------------------------------------------------------------------------
// Time stamps of a diagnostic build (compiled with SEKV_TIMELINE, into its own
// library): workgroups of the route, attend and tail launches record
// s_memrealtime (a 100 MHz clock) at fixed points of their work into device
// tables that sekv_timeline_read copies out; one table row per workgroup.
// The product build compiles every stamp away.
//   route:  0 start, 1 end, 2 projections done, 3 first chunk gated, 4 query in LDS
//   attend: 0 start, 1 kind (0 zoom, 1 rows, 2 lists), 2 end;
//           zoom: 3 allocated, 4 spans found, 5 metadata, 6..9 each wave's
//           pipeline done, 10 KV head + 1 (0: no share), 11 spans in the share;
//           rows: 3 prologue done, 4 rows and coarse entries done
//   tail:   0 start, 1 end
// ---------------------------------------------------------------------------
#ifdef SEKV_TIMELINE
constexpr int kTlWgs = 4096, kTlSlots = 16;
__device__ unsigned long long g_tl_route[kTlWgs * kTlSlots];
__device__ unsigned long long g_tl_attend[kTlWgs * kTlSlots];
__device__ unsigned long long g_tl_tail[kTlWgs * kTlSlots];
#define SEKV_NOW() __builtin_amdgcn_s_memrealtime()
#define SEKV_TL(table, slot, value)                                               \
  do {                                                                            \
    if (threadIdx.x == 0 && blockIdx.x < kTlWgs && blockIdx.y == 0)               \
      table[blockIdx.x * kTlSlots + (slot)] = (unsigned long long)(value);         \
  } while (0)
#define SEKV_TL_WAVE(table, slot, value)                                          \
  do {                                                                            \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < kTlWgs && blockIdx.y == 0)        \
      table[blockIdx.x * kTlSlots + (slot) + (threadIdx.x >> 6)] =                \
          (unsigned long long)(value);                                            \
  } while (0)
#else
#define SEKV_TL(table, slot, value) ((void)0)
#define SEKV_TL_WAVE(table, slot, value) ((void)0)
#endif

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// Cross-lane moves inside a row of 16 lanes go through DPP (an ALU operand
// modifier), moves between rows through the gfx950 permlane swaps; neither
// touches the LDS permute unit.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)__double2loint(x), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)__double2hiint(x), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within 16
constexpr int kDppRor8 = 0x128;       // lane i <- (i + 8) mod 16 (= i xor 8)

// The values of a lane and of its partner 16 (or 32) lanes away, in a fixed
// order: lo from the lower row (half), hi from the upper one, the same on
// both lanes.  v_permlane16_swap exchanges the odd rows of one operand with
// the even rows of the other; applied to one value twice it yields rows
// (x0, x0, x2, x2) and (x1, x1, x3, x3).  v_permlane32_swap does the same
// with the two halves of the wave.  No LDS access is involved.
struct Pair { float lo, hi; };
template <int OFF>
__device__ __forceinline__ Pair pair_xor(float x) {
  static_assert(OFF == 16 || OFF == 32, "row or half exchange");
  const uint32_t u = __float_as_uint(x);
  const auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float xor16_sum(float x) { const Pair p = pair_xor<16>(x); return p.lo + p.hi; }
__device__ __forceinline__ float xor32_sum(float x) { const Pair p = pair_xor<32>(x); return p.lo + p.hi; }
__device__ __forceinline__ double xor16_sum(double x) { return x + __shfl_xor(x, 16, 64); }
__device__ __forceinline__ double xor32_sum(double x) { return x + __shfl_xor(x, 32, 64); }

// sum over aligned groups of N lanes (N = 4, 8, 16, 32, 64); every lane of a
// group receives the group's total
template <int N, typename F>
__device__ __forceinline__ F group_sum(F x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if (N >= 8) x += dpp<kDppHalfMirror>(x);
  if (N >= 16) x += dpp<kDppMirror>(x);
  if (N >= 32) x = xor16_sum(x);
  if (N >= 64) x = xor32_sum(x);
  return x;
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float readlane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// A float as an int of the same order (for every value but NaN): the sign
// bit stays, the other bits of a negative value are flipped.  A max taken on
// these keys is the float max, with neither operand canonicalised, and the
// DPP move folds into the integer max.  The map is its own inverse.
__device__ __forceinline__ int fkey(float x) {
  const int i = __float_as_int(x);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float funkey(int k) { return __int_as_float(fkey(__int_as_float(k))); }
template <int CTRL>
__device__ __forceinline__ int kmax_dpp(int k) {
  // the patterns used stay inside a row, so no lane reads out of bounds
  return max(k, __builtin_amdgcn_mov_dpp(k, CTRL, 0xF, 0xF, true));
}
// wave-wide max / sum, the total on every lane
__device__ __forceinline__ float wave_max(float x) {
  int k = fkey(x);
  k = kmax_dpp<kDppXor1>(k);
  k = kmax_dpp<kDppXor2>(k);
  k = kmax_dpp<kDppHalfMirror>(k);
  k = kmax_dpp<kDppMirror>(k);
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
  k = max((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
  return funkey(max((int)r[0], (int)r[1]));
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
// weights of two online-softmax states under their common max; -inf = empty
__device__ __forceinline__ float merge_w(float m1, float m2, float& w1, float& w2) {
  const float M = fmaxf(m1, m2);
  w1 = (m1 == -INFINITY) ? 0.f : __expf(m1 - M);
  w2 = (m2 == -INFINITY) ? 0.f : __expf(m2 - M);
  return M;
}

template <typename T> struct Lanes {
  static constexpr int EPL = 16 / sizeof(T);        // elements per 16-byte lane load
  static constexpr int LPR = kHeadDim / EPL;        // lanes per row
  static constexpr int RPW = 64 / LPR;              // rows per wave load
};

__device__ __forceinline__ void unpack16(const uint4& raw, float* out, uint16_t) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& raw, float* out, float) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

// ---------------------------------------------------------------------------
// shared memory of the layer kernel
// ---------------------------------------------------------------------------
// scratch of one zoomed span of any rank
template <int G> struct ZoomScratchAny {
  float bsh[G][kMaxRank];
  float csh[G][kMaxRank];
  float psh[64][G];
};
// an online softmax state of G heads: (m, l, acc[d]) per head
template <int G> struct WaveState {
  float acc[G][kHeadDim];
  float m[G];
  float l[G];
};
template <int G>
struct alignas(16) WaveScratch {
  WaveState<G> st;                 // the wave's state before and after its spans
};

// Rows of V_K a wave can stage in LDS for its next zoomed span: all 32 while
// two workgroups still fit in a CU's 160 KB, fewer for large groups.
template <int G> constexpr int stage_rows() { return G <= 5 ? 32 : 24; }
// a stage: SR rows of V_K, then 64 floats of sigma_K and 64 of sigma_V
template <int SR> constexpr int stage_floats() { return SR * kHeadDim + 128; }

// The tail's merge, one workgroup per query head: thread = (4 dims, stripe of
// slots); the stripes are combined through LDS.
constexpr int kMergeQuads = kHeadDim / 4;
constexpr int kMergeStripes = kThreads / kMergeQuads;
struct MergeScratch {
  float4 red[kMergeStripes * kMergeQuads];   // each stripe's acc
  float m[kMergeStripes], l[kMergeStripes];
};

template <int G>
struct alignas(16) Smem {
  float qs[G][kHeadDim];           // query * 1/sqrt(d)
  int bits[kChunk];                // heads of the group that zoom span j0 + i
  union {
    struct {                       // routing (dead once the gates are taken)
      float qu[G][kHeadDim];       // query as given
      double qt[G][kMaxRouteDim + 1];  // P_h q_h (rows padded: the gates of G heads read
                                       // G rows at once, on different LDS banks)
    } rt;
    WaveScratch<G> w[kWaves];      // written from the rows phase on
  };
};

// Shared memory of the zoom kernel: the query, a batch of the workgroup's
// zoomed spans (factor block, length, packed ranks, heads that zoom it), each
// KV head's union size, and each wave's state / span scratch.
constexpr int kZoomBatch = kZoomBatchMax;
template <int G>
struct alignas(16) ZSmem {
  float qs[G][kHeadDim];
  uint64_t m_off[kZoomBatch];
  int m_n[kZoomBatch], m_r[kZoomBatch], bits[kZoomBatch];
  int g, i, zg, lo, hi;            // this workgroup's KV head, index among its
                                   // zoom workgroups, their count, span range
  union {
    int cnt[kMaxKvHeads];          // union size of each KV head (dead once shared out)
    WaveScratch<G> w[kWaves];      // the waves' states and span scratch
  };
};
// Per wave: V_K of its next zoomed span, written by LDS DMA while the current
// span is processed, or the scratch of a span of rank > 32.  An array of its
// own, so the compiler can tell the DMA's LDS writes from every other LDS
// access and waits for them only where the stage is read.
template <int G> struct alignas(16) Stage {
  float v[kWaves][stage_floats<stage_rows<G>()>()];
};

// ---------------------------------------------------------------------------
// Rows of K/V (full-resolution rows, or a chunk's coarse entries), one wave:
// LOADS wave-wide 16-byte loads of K and of V, RPW rows each.  Each row slot
// (LPR lanes) keeps its own online state across calls; rows_finish combines
// the slots, after which every lane holds the wave's state for its EPL dims.
// ---------------------------------------------------------------------------
template <typename T, int G>
struct RowState {
  float m[G], l[G], acc[G][Lanes<T>::EPL];
  __device__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < Lanes<T>::EPL; ++e) acc[h][e] = 0.f;
    }
  }
};

template <typename T, int LOADS>
__device__ __forceinline__ void rows_load(const T* __restrict__ K, const T* __restrict__ V, int r0,
                                          int r1, uint4 (&kr)[LOADS], uint4 (&vr)[LOADS]) {
  using Ln = Lanes<T>;
  const int lane = threadIdx.x & 63, sub = lane / Ln::LPR, sl = lane % Ln::LPR;
  if (r1 > r0) {
    // rows past the range load row r1 - 1 (always valid) and are masked later
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int row = min(r0 + u * Ln::RPW + sub, r1 - 1);
      kr[u] = *(const uint4*)(K + (size_t)row * kHeadDim + sl * Ln::EPL);
      vr[u] = *(const uint4*)(V + (size_t)row * kHeadDim + sl * Ln::EPL);
    }
  } else {   // nothing for this wave (uniform)
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Coarse entries add lnn[row - bias0] to their scaled score and are skipped by
// the heads whose bit is set in skip[row - bias0]; full-resolution rows pass
// lnn = NULL.
// this lane's EPL query dims of every head of the group, in registers
template <typename T, int G>
struct QSlice {
  float v[G][Lanes<T>::EPL];
  __device__ void load(const float (*qs)[kHeadDim]) {
    using Ln = Lanes<T>;
    const int sl = (threadIdx.x & 63) % Ln::LPR;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < Ln::EPL; e += 4) {
        const float4 x = *(const float4*)&qs[h][sl * Ln::EPL + e];
        v[h][e] = x.x;
        v[h][e + 1] = x.y;
        v[h][e + 2] = x.z;
        v[h][e + 3] = x.w;
      }
  }
};

template <typename T, int G, int LOADS>
__device__ __forceinline__ void rows_accumulate(const uint4 (&kr)[LOADS], const uint4 (&vr)[LOADS],
                                                int r0, int r1, const QSlice<T, G>& q,
                                                const float (&bias)[LOADS], const int* skip,
                                                int skip0, RowState<T, G>& s) {
  using Ln = Lanes<T>;
  constexpr int EPL = Ln::EPL;
  const int lane = threadIdx.x & 63, sub = lane / Ln::LPR;
  float sc[LOADS][G];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    float kf[EPL];
    unpack16(kr[u], kf, T());
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d += q.v[h][e] * kf[e];
      sc[u][h] = group_sum<Ln::LPR>(d);
    }
    const int row = r0 + u * Ln::RPW + sub;
    const bool valid = row < r1;
    const int sk = (skip != nullptr && valid) ? skip[row - skip0] : 0;
#pragma unroll
    for (int h = 0; h < G; ++h)
      sc[u][h] = (valid && !((sk >> h) & 1)) ? sc[u][h] + bias[u] : -INFINITY;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sc[0][h];
#pragma unroll
    for (int u = 1; u < LOADS; ++u) mx = fmaxf(mx, sc[u][h]);
    if (mx == -INFINITY) continue;
    const float M = fmaxf(s.m[h], mx);
    const float wo = (s.m[h] == -INFINITY) ? 0.f : __expf(s.m[h] - M);
    s.l[h] *= wo;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s.acc[h][e] *= wo;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const float p = (sc[u][h] == -INFINITY) ? 0.f : __expf(sc[u][h] - M);
      float vf[EPL];
      unpack16(vr[u], vf, T());
      s.l[h] += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s.acc[h][e] += p * vf[e];
    }
    s.m[h] = M;
  }
}

// merge the states of lanes OFF apart (both lanes end with the same state)
template <int OFF, typename T, int G>
__device__ __forceinline__ void rows_merge_xor(RowState<T, G>& s) {
  using Ln = Lanes<T>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const Pair m = pair_xor<OFF>(s.m[h]);
    const Pair l = pair_xor<OFF>(s.l[h]);
    float w1, w2;
    const float M = merge_w(m.lo, m.hi, w1, w2);
    s.l[h] = l.lo * w1 + l.hi * w2;
#pragma unroll
    for (int e = 0; e < Ln::EPL; ++e) {
      const Pair x = pair_xor<OFF>(s.acc[h][e]);
      s.acc[h][e] = x.lo * w1 + x.hi * w2;
    }
    s.m[h] = M;
  }
}

template <typename T, int G>
__device__ __forceinline__ void rows_finish(RowState<T, G>& s) {
  static_assert(Lanes<T>::LPR == 16 || Lanes<T>::LPR == 32, "row slots are 16 or 32 lanes apart");
  if (Lanes<T>::LPR == 16) rows_merge_xor<16>(s);
  rows_merge_xor<32>(s);
}

template <typename T, int G>
__device__ __forceinline__ void rows_store(const RowState<T, G>& s, float (*acc)[kHeadDim],
                                           float* m, float* l) {
  using Ln = Lanes<T>;
  const int lane = threadIdx.x & 63, sub = lane / Ln::LPR, sl = lane % Ln::LPR;
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < Ln::EPL; ++e) acc[h][sl * Ln::EPL + e] = s.acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = s.m[h];
      l[h] = s.l[h];
    }
  }
}

// ---------------------------------------------------------------------------
// One zoomed span, one wave: factored attention of the heads in `hm`, merged
// into the wave's running state (zm, zl, za: lane holds dims 2 lane, 2 lane+1).
// ---------------------------------------------------------------------------
template <int G>
__device__ __attribute__((always_inline)) void zoom_span(const float* __restrict__ blk, int n, int rk, int rv, unsigned hm,
                          const float (*qs)[kHeadDim], ZoomScratchAny<G>& zs, float* zm, float* zl,
                          float (*za)[2]) {
  const int lane = threadIdx.x & 63;
  const FactorView fv(rk, rv, n);
  const int rk4 = fv.r4(0), rv4 = fv.r4(1);
  const float* vk = blk + fv.vt(0);
  const float* uk = blk + fv.u(0);
  const float* sk = blk + fv.sigma(0);
  const float* vv = blk + fv.vt(1);
  const float* uv = blk + fv.u(1);
  const float* sv = blk + fv.sigma(1);

  // (A) b_h[i] = sigma_K[i] * (V_K^T q_h)[i]: 8 lanes per component, 16 dims per lane
  {
    const int part = lane & 7, ci = lane >> 3;
    for (int i0 = 0; i0 < rk; i0 += 8) {
      const int i = i0 + ci;
      float pa[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pa[h] = 0.f;
      if (i < rk) {
        const float* row = vk + (size_t)i * kHeadDim + part * 4;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const float4 x = *(const float4*)(row + 32 * c4);
          const int d0 = part * 4 + c4 * 32;
#pragma unroll
          for (int h = 0; h < G; ++h)
            pa[h] += x.x * qs[h][d0] + x.y * qs[h][d0 + 1] + x.z * qs[h][d0 + 2] +
                     x.w * qs[h][d0 + 3];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pa[h] = group_sum<8>(pa[h]);
      }
      if (part == 0 && i < rk) {
        const float sg = sk[i];
#pragma unroll
        for (int h = 0; h < G; ++h) zs.bsh[h][i] = pa[h] * sg;
      }
    }
    // padding components and the value-side coefficients start at zero
    for (int idx = lane; idx < G * rk4; idx += 64) {
      const int h = idx / rk4, i = idx % rk4;
      if (i >= rk) zs.bsh[h][i] = 0.f;
    }
    for (int idx = lane; idx < G * rv4; idx += 64) zs.csh[idx / rv4][idx % rv4] = 0.f;
  }
  __builtin_amdgcn_wave_barrier();

  // (B, C) 64 tokens at a time: scores, online softmax, c_h += U_V^T p_h
  float ms[G], ls[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ms[h] = -INFINITY;
    ls[h] = 0.f;
  }
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    float e[G];
#pragma unroll
    for (int h = 0; h < G; ++h) e[h] = 0.f;
    if (t < n) {
      const float4* ur = (const float4*)(uk + (size_t)t * rk4);
      for (int i4 = 0; i4 < rk4 / 4; ++i4) {
        const float4 u = ur[i4];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float4 b = *(const float4*)&zs.bsh[h][4 * i4];
          e[h] += u.x * b.x + u.y * b.y + u.z * b.z + u.w * b.w;
        }
      }
    }
    float corr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (t >= n || !((hm >> h) & 1u)) e[h] = -INFINITY;
      const float mx = wave_max(e[h]);
      const float mn = fmaxf(ms[h], mx);
      corr[h] = (ms[h] == -INFINITY) ? 0.f : __expf(ms[h] - mn);
      const float p = (e[h] == -INFINITY) ? 0.f : __expf(e[h] - mn);
      ls[h] = ls[h] * corr[h] + wave_sum(p);
      ms[h] = mn;
      zs.psh[lane][h] = p;
    }
    __builtin_amdgcn_wave_barrier();
    const int tn = min(64, n - t0);
    const int i4 = lane & 7, ts = lane >> 3;
    for (int cb = 0; cb < rv4; cb += 32) {
      const int i = cb + 4 * i4;
      float c4[G][4];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) c4[h][q] = 0.f;
      if (i < rv4) {
        for (int k = ts; k < tn; k += 8) {
          const float4 u = *(const float4*)(uv + (size_t)(t0 + k) * rv4 + i);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = zs.psh[k][h];
            c4[h][0] += p * u.x;
            c4[h][1] += p * u.y;
            c4[h][2] += p * u.z;
            c4[h][3] += p * u.w;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c4[h][q] += dpp<kDppRor8>(c4[h][q]);
          c4[h][q] = xor32_sum(xor16_sum(c4[h][q]));
        }
      if (ts == 0 && i < rv4) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int q = 0; q < 4; ++q) zs.csh[h][i + q] = zs.csh[h][i + q] * corr[h] + c4[h][q];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // (D) a_h[dim] = sum_i V_V[i][dim] sigma_V[i] c_h[i]; merge into the running state
  float a[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) a[h][0] = a[h][1] = 0.f;
  for (int i = 0; i < rv; ++i) {
    const float2 x = *(const float2*)(vv + (size_t)i * kHeadDim + 2 * lane);
    const float sg = sv[i];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = sg * zs.csh[h][i];
      a[h][0] += w * x.x;
      a[h][1] += w * x.y;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hm >> h) & 1u)) continue;
    float w1, w2;
    const float M = merge_w(zm[h], ms[h], w1, w2);
    za[h][0] = za[h][0] * w1 + a[h][0] * w2;
    za[h][1] = za[h][1] * w1 + a[h][1] * w2;
    zl[h] = zl[h] * w1 + ls[h] * w2;
    zm[h] = M;
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Zoomed spans of rank <= 32, processed by one wave as a pipeline over its
// list of spans.  While span i is processed, the loads of span i + 1 are in
// flight: its V_K by LDS DMA into the wave's stage (issued once phase (A) of
// span i has read the stage), its first 64 rows of U_K into the registers ub
// (issued once span i's last rows there are consumed).  Span i's own U_V and
// V_V, needed last, are loaded at its start, ahead of all of these.
//
// Loads complete in issue order and the wait for one load is a count of the
// loads issued after it, so every wave issues the same loads whatever it has
// to prefetch: a wave with no next span prefetches its current one again, or
// the cache's zero block.  The compiler then counts exactly, and no wait for
// a span's own data also waits for the next span's.  Every load reads a
// clamped, valid address; values past a span's rank or length are left in
// place and excluded where they are used (an overwrite would wait for the load).
// ---------------------------------------------------------------------------
struct SpanRef {        // a zoomed span, the same on every lane of the wave
  const float* blk;     // its factor block
  int n, rk, rv;        // length, ranks of its key and value factors
  unsigned hm;          // heads of the group that zoom it
};

template <int G>
__device__ __forceinline__ SpanRef span_ref(const ZSmem<G>& s, const float* pool, int jl) {
  SpanRef sp;
  jl = uniform(jl);
  sp.blk = pool + uniform64(s.m_off[jl]);
  sp.n = uniform(s.m_n[jl]);
  const int32_t rr = uniform(s.m_r[jl]);
  sp.rk = rank_of(rr, 0);
  sp.rv = rank_of(rr, 1);
  sp.hm = (unsigned)uniform(s.bits[jl]);
  return sp;
}

// A span's V_K (rK rows of d floats at the start of its block) and its
// sigma_K and sigma_V into a stage: SR rows, then 64 floats of sigma_K and 64
// of sigma_V (entry i holds sigma[min(i, r4 - 1)] with r4 of that matrix;
// entries r .. r4 - 1 are the block's zero padding).  Each row instruction
// moves 1 KB (two rows) straight from memory to LDS, lane l writing bytes
// [16 l, 16 l + 16) of it; always SR / 2 of them, those past the span's rows
// copying its last two rows again (an odd rK also moves the 512 bytes after
// V_K, still inside the block: the value half that follows holds at least
// one row of d floats).
//
// The DMA instructions are written as inline assembly.  The compiler then
// does not count them among the wave's outstanding loads: its own waits for
// registers loaded before a DMA stay exact (with the DMA counted, every such
// wait becomes a wait for all loads, the DMA of the next span included), and
// a DMA it does not see only makes those waits stricter, never too weak.  The
// waits for the DMA itself are explicit: wait_lds() before a stage is
// overwritten, wait_vm<48>() before it is read.  M0 holds the LDS address of
// each instruction and is restored after it.
// the LDS address of p, in a scalar register (p is the same on every lane)
__device__ __forceinline__ uint32_t lds_addr(const float* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)p);
}
__device__ __forceinline__ void dma_x4(const float* g, const float* lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(lds)), "v"(g)
      : "memory");
}
__device__ __forceinline__ void dma_x1(const float* g, const float* lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(lds)), "v"(g)
      : "memory");
}
template <int SR>
__device__ __forceinline__ void stage_vk(const SpanRef& sp, float* stage) {
  const int lane = threadIdx.x & 63;
  const int nk = (sp.rk + 1) >> 1;
  const FactorView fv(sp.rk, sp.rv, sp.n);
#pragma unroll
  for (int k = 0; k < SR / 2; ++k) dma_x4(sp.blk + min(k, nk - 1) * 256 + lane * 4, stage + k * 256);
  dma_x1(sp.blk + fv.sigma(0) + min(lane, fv.r4(0) - 1), stage + SR * kHeadDim);
  dma_x1(sp.blk + fv.sigma(1) + min(lane, fv.r4(1) - 1), stage + SR * kHeadDim + 64);
}

// LDS reads of this wave complete before the stage is overwritten by DMA
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// token rows t0 .. t0 + 63 of U (n rows of r4 floats), lane = token: 8
// 16-byte loads of components 4 q .. 4 q + 3 (clamped to valid rows and
// components)
template <int NQ, int M>
__device__ __forceinline__ void load_u_tile(const float* u, int n, int r4, int t0, float4 (&x)[M]) {
  static_assert(NQ <= M, "tile registers");
  const int lane = threadIdx.x & 63;
  const int nq = r4 / 4, tl = min(t0 + lane, n - 1);
#pragma unroll
  for (int q = 0; q < NQ; ++q) x[q] = *(const float4*)(u + (size_t)tl * r4 + 4 * min(q, nq - 1));
}
// what a wave prefetches of its next span into registers: the first rows of
// U_K (always 8 loads, so the waits that count them stay exact)
__device__ __forceinline__ void prefetch_span(const SpanRef& sp, float4 (&ub)[8]) {
  const FactorView fv(sp.rk, sp.rv, sp.n);
  load_u_tile<8>(sp.blk + fv.u(0), sp.n, fv.r4(0), 0, ub);
}

// Keep the loads issued so far ahead of everything after (the waits below
// count loads in issue order).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most N of this wave's vector memory operations (loads, and
// LDS DMA) are outstanding.  Operations complete in issue order, so this
// waits for everything issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Rows t0 .. t0 + 63 of U_V (n rows of r4 floats) in the layout of (C):
// lane = (component group cg, token group tg), lane = cg TG + tg with TG =
// 64 / (RC / 4); x[k] holds components 4 cg .. 4 cg + 3 of token
// t0 + k TG + tg, k < RC / 4 (rows clamped to the span, component groups to
// r4).  For each k the wave reads TG consecutive rows whole: one contiguous
// piece of memory.
template <int RC>
__device__ __forceinline__ void load_uv_tile(const float* u, int n, int r4, int t0,
                                             float4 (&x)[RC / 4]) {
  constexpr int CG = RC / 4, TG = 64 / CG;
  const int lane = threadIdx.x & 63;
  const int cg = min(lane / TG, r4 / 4 - 1), tg = lane % TG;
#pragma unroll
  for (int k = 0; k < CG; ++k)
    x[k] = *(const float4*)(u + (size_t)min(t0 + k * TG + tg, n - 1) * r4 + 4 * cg);
}

// One span of the pipeline, for key and value ranks up to RC (16 or 32):
// loads are sized to RC (U rows of RC / 4 16-byte pieces, V_V in RC / 2
// 16-byte loads of two rows each), whatever the two ranks below it.  On entry
// ub holds the span's first rows of U_K and, if rK <= SR, the stage holds (or
// is receiving) its V_K; on return ub holds the
// first rows of U_K of `nxp` (8 loads, whatever its rank) and the stage
// receives the V_K of `nxs` (the next span, or a stand-in when it has none of
// the kind).
//
//  (A) b_h[i] = sigma_K[i] (V_K q_h)[i]: lane (part, ci) sums dims 4 part + 32 c
//      .. + 3, c < 4, of rows ci + 8 p (eight lanes read 128 contiguous bytes,
//      free of LDS bank conflicts); b goes to the wave's scratch scr[h][0..32),
//      which (B) reads broadcast.
//  (B) e[t] = U_K[t] . b_h with lane = token t, then the online softmax.
//  (C) c_h[i] = sum_t p_h[t] U_V[t][i]: p goes through the wave's scratch
//      to lane (cg, tg), which keeps components 4 cg .. 4 cg + 3 of the sum
//      over its RC / 4 tokens of each block (rescaled with the softmax);
//      once per span the GL token groups are added, which leaves components
//      4 g .. 4 g + 3 in lanes GL g .. GL g + GL - 1.  The softmax sum l
//      likewise stays a per-lane partial until then.
//  (D) a_h = V_V^T (sigma_V c_h) with sigma_V c_h read out as scalars; lane
//      (half, dq) sums rows 2 k + half of dims 4 dq .. 4 dq + 3, the two
//      halves of the wave are added, and scr[h] turns the result into the
//      state's layout (dims 2 lane, 2 lane + 1).
template <int G, int SR, int RC>
__device__ __attribute__((always_inline)) void zoom_span32(const SpanRef& cu, const SpanRef& nxp, const SpanRef& nxs,
                            float4 (&ub)[8], float* stage, float (*scr)[kHeadDim],
                            const float (*qs)[kHeadDim], float* zm, float* zl, float (*za)[2]) {
  static_assert(RC == 16 || RC == 32, "rank class");
  constexpr int UQ = RC / 4;          // 16-byte pieces of a U row
  constexpr int VK = RC / 2;          // 16-byte loads of V_V
  constexpr int GL = 64 / (RC / 4);   // lanes holding each 4 components of c
  const int lane = threadIdx.x & 63;
  const int n = cu.n, rk = cu.rk, rv = cu.rv;
  const unsigned hm = cu.hm;
  const FactorView fv(rk, rv, n);
  const int rk4 = fv.r4(0), rv4 = fv.r4(1);
  const float* vk = cu.blk + fv.vt(0);
  const float* vv = cu.blk + fv.vt(1);
  const int part = lane & 7, ci = lane >> 3;   // (A): component ci + 8 p, dims 4 part + 32 c
  const int half = lane >> 5, dq = lane & 31;  // (D): rows 2 k + half, dims 4 dq ..
  const int cg = lane / GL;                    // (C): components 4 cg .. 4 cg + 3
  const int tg = lane % GL;                    // (C): tokens tg, tg + GL, ... of a block
  const bool staged = SR >= 32 || rk <= SR;    // always, when the stage holds 32 rows

  // this span's own loads, needed last: the first rows of U_V, all of V_V
  float4 uc[UQ];
  load_uv_tile<RC>(cu.blk + fv.u(1), n, rv4, 0, uc);
  float4 vd[VK];
#pragma unroll
  for (int k = 0; k < VK; ++k)
    vd[k] = *(const float4*)(vv + (size_t)min(2 * k + half, rv - 1) * kHeadDim + 4 * dq);
  float4 va[4][4];   // V_K from memory, only when it is not staged
  float sgm[4];      // and then sigma_K and sigma_V too (the stage holds another span's)
  float4 svm = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!staged) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = min(ci + 8 * p, rk - 1);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        va[p][c4] = *(const float4*)(vk + (size_t)i * kHeadDim + part * 4 + c4 * 32);
    }
    // entries clamped to each matrix's r4 (as the stage copy is)
    const float* sk = cu.blk + fv.sigma(0);
    const float* sv = cu.blk + fv.sigma(1);
#pragma unroll
    for (int p = 0; p < 4; ++p) sgm[p] = sk[min(ci + 8 * p, rk4 - 1)];
    svm = make_float4(sv[min(4 * cg, rv4 - 1)], sv[min(4 * cg + 1, rv4 - 1)],
                      sv[min(4 * cg + 2, rv4 - 1)], sv[min(4 * cg + 3, rv4 - 1)]);
  }

  // sigma_K of the lane's components in (A) (ci + 8 p) and sigma_V of its
  // components after (C) (4 cg ..), from the stage (for a span too large for
  // the stage, from its block, loaded above).  The stage's DMA was followed by
  // the 8 loads of U_K rows prefetched for this span and the UQ + VK above,
  // so once at most that many are outstanding the DMA has landed.
  issue_fence();
  wait_vm<8 + UQ + VK>();
  float sg[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) sg[p] = staged ? stage[SR * kHeadDim + ci + 8 * p] : sgm[p];
  const float4 svg = staged ? *(const float4*)(stage + SR * kHeadDim + 64 + 4 * cg) : svm;

  // (A) components at or past rK get exactly 0 (a stage row past rK may hold
  // anything)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hm >> h) & 1u)) continue;
#pragma unroll
    for (int p = 0; p < RC / 8; ++p) {
      const int i = ci + 8 * p;
      float acc = 0.f;
      if (8 * p < rk) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const float4 x =
              staged ? *(const float4*)(stage + i * kHeadDim + part * 4 + c4 * 32) : va[p][c4];
          const float4 qv = *(const float4*)&qs[h][part * 4 + c4 * 32];
          acc += x.x * qv.x + x.y * qv.y + x.z * qv.z + x.w * qv.w;
        }
        acc = group_sum<8>(acc);
      }
      if (part == 0) scr[h][i] = i < rk ? acc * sg[p] : 0.f;
    }
  }
  // the stage is free: the next span's V_K goes in while this one proceeds
  wait_lds();
  issue_fence();
  stage_vk<SR>(nxs, stage);
  issue_fence();
  __builtin_amdgcn_wave_barrier();

  float ms[G], ls[G], cacc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ms[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) cacc[h][k] = 0.f;
  }
  // (B) scores of tokens t0 + lane from the rows in ub
  auto scores = [&](int t0, float (&e)[G]) {
    const int tn = min(64, n - t0);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      e[h] = -INFINITY;
      if (!((hm >> h) & 1u)) continue;
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const float4 b = *(const float4*)&scr[h][4 * q];   // the same address on every lane
        if (q < rk4 / 4) acc += ub[q].x * b.x + ub[q].y * b.y + ub[q].z * b.z + ub[q].w * b.w;
      }
      if (lane < tn) e[h] = acc;
    }
  };
  // online softmax and (C) from the rows in uc
  auto accumulate = [&](const float (&e)[G]) {
    float corr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      corr[h] = 1.f;
      if (!((hm >> h) & 1u)) continue;
      // every block has a token, so mx and mn are finite, and the empty
      // state (ms = -inf) and the lanes past the span (e = -inf) get exp(-inf) = 0
      const float mx = wave_max(e[h]);
      const float mn = fmaxf(ms[h], mx);
      corr[h] = __expf(ms[h] - mn);
      const float p = __expf(e[h] - mn);
      ls[h] = ls[h] * corr[h] + p;   // the lane's part of l
      ms[h] = mn;
      // token `lane` to lane (tg, k) = (lane mod GL, lane / GL), k-th of its tokens
      scr[h][64 + (lane % GL) * (RC / 4) + lane / GL] = p;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((hm >> h) & 1u)) continue;
      float pk[RC / 4];
#pragma unroll
      for (int q = 0; q < RC / 16; ++q) {
        const float4 v = *(const float4*)&scr[h][64 + tg * (RC / 4) + 4 * q];
        pk[4 * q] = v.x;
        pk[4 * q + 1] = v.y;
        pk[4 * q + 2] = v.z;
        pk[4 * q + 3] = v.w;
      }
      float c0 = cacc[h][0] * corr[h], c1 = cacc[h][1] * corr[h];
      float c2 = cacc[h][2] * corr[h], c3 = cacc[h][3] * corr[h];
#pragma unroll
      for (int k = 0; k < RC / 4; ++k) {
        c0 += pk[k] * uc[k].x;
        c1 += pk[k] * uc[k].y;
        c2 += pk[k] * uc[k].z;
        c3 += pk[k] * uc[k].w;
      }
      cacc[h][0] = c0;
      cacc[h][1] = c1;
      cacc[h][2] = c2;
      cacc[h][3] = c3;
    }
    __builtin_amdgcn_wave_barrier();
  };
  // every 64 tokens but the last: the next 64 rows of U_K and U_V follow
  // (the same loads on every pass, so the compiler's waits stay exact)
  int t0 = 0;
  for (; t0 + 64 < n; t0 += 64) {
    float e[G];
    scores(t0, e);
    issue_fence();
    load_u_tile<UQ>(cu.blk + fv.u(0), n, rk4, t0 + 64, ub);
    issue_fence();
    accumulate(e);
    issue_fence();
    load_uv_tile<RC>(cu.blk + fv.u(1), n, rv4, t0 + 64, uc);
    issue_fence();
  }
  // the last 64: then what the next span needs first
  {
    float e[G];
    scores(t0, e);
    issue_fence();
    prefetch_span(nxp, ub);
    issue_fence();
    accumulate(e);
  }

  // the token groups' parts of c_h, and the lanes' parts of l
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hm >> h) & 1u)) continue;
    ls[h] = wave_sum(ls[h]);
#pragma unroll
    for (int k = 0; k < 4; ++k) cacc[h][k] = group_sum<GL>(cacc[h][k]);
  }

  // (D) a_h[dim] = sum_i V_V[i][dim] (sigma_V c_h)[i]; rows past rV hold a
  // clamped copy of row rV - 1 and get weight 0 (so do components of c past
  // rV, which the clamped U_V pieces leave arbitrary)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hm >> h) & 1u)) continue;
    const float cs[4] = {cacc[h][0] * svg.x, cacc[h][1] * svg.y, cacc[h][2] * svg.z,
                         cacc[h][3] * svg.w};
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < VK; ++k) {
      const int i0 = 2 * k, i1 = 2 * k + 1;
      if (i0 >= rv) continue;
      const float w0 = readlane(cs[i0 & 3], GL * (i0 >> 2));
      const float w1 = i1 < rv ? readlane(cs[i1 & 3], GL * (i1 >> 2)) : 0.f;
      const float w = half ? w1 : w0;
      a[0] += w * vd[k].x;
      a[1] += w * vd[k].y;
      a[2] += w * vd[k].z;
      a[3] += w * vd[k].w;
    }
    // the swaps read the other half of the wave: every lane runs them
    const float4 sum = make_float4(xor32_sum(a[0]), xor32_sum(a[1]), xor32_sum(a[2]), xor32_sum(a[3]));
    if (half == 0) *(float4*)&scr[h][4 * dq] = sum;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hm >> h) & 1u)) continue;
    const float2 ah = *(const float2*)&scr[h][2 * lane];
    float w1, w2;
    const float M = merge_w(zm[h], ms[h], w1, w2);
    za[h][0] = za[h][0] * w1 + ah.x * w2;
    za[h][1] = za[h][1] * w1 + ah.y * w2;
    zl[h] = zl[h] * w1 + ls[h] * w2;
    zm[h] = M;
  }
  __builtin_amdgcn_wave_barrier();
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele within each row of 16
// lanes by DPP row shifts (lanes shifted in from outside the row add 0), then
// the totals of the rows below each row.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

// ---------------------------------------------------------------------------
// the layer kernel
// ---------------------------------------------------------------------------
static_assert(kChunk * kMaxGroup <= kThreads, "one gate per thread");
template <int G> constexpr bool smem_fits() {
  return sizeof(Smem<G>) <= 40 * 1024 &&                          // layer kernel
         sizeof(ZSmem<G>) + sizeof(Stage<G>) <= 80 * 1024 &&       // zoom kernel: two per CU
         sizeof(Smem<G>::rt) <= sizeof(Smem<G>::w) &&
         sizeof(ZoomScratchAny<G>) <= sizeof(float) * stage_floats<stage_rows<G>()>() &&
         stage_rows<G>() % 2 == 0 && stage_rows<G>() <= 32;
}
static_assert(smem_fits<1>() && smem_fits<2>() && smem_fits<3>() && smem_fits<4>() &&
              smem_fits<5>() && smem_fits<6>() && smem_fits<7>() && smem_fits<8>(),
              "LDS layout of the layer and zoom kernels");
static_assert(kChunk <= 64, "a chunk's zoom sets are one wave ballot");

// The ascending zoom lists of a KV head's query heads and its union, from the
// chunks' zoom bit masks: a block scan of the popcounts, and each thread
// writes its chunk's ids.
template <int G>
__device__ __attribute__((always_inline)) void tail_lists(const LayerGeom& geo, const LayerArgs& a,
                                                          int g, int (*wc)[kWaves]) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int W = geo.n_work, sc = geo.n_compressed, h0 = g * G, nc = geo.n_chunks;
  auto list_pass = [&](int c, const uint32_t (&word)[kListWords], int (&base)[kListWords]) {
    int incl[kListWords];
#pragma unroll
    for (int li = 0; li <= G; ++li) {
      incl[li] = wave_incl_scan(__popc(word[li]));
      if (lane == 63) wc[li][wid] = incl[li];
    }
    __syncthreads();
#pragma unroll
    for (int li = 0; li <= G; ++li) {
      int off = base[li], tot = 0;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        off += (wv < wid) ? wc[li][wv] : 0;
        tot += wc[li][wv];
      }
      off += incl[li] - __popc(word[li]);
      int32_t* dst = li < G ? a.list + (size_t)(h0 + li) * sc : a.ulist + (size_t)g * sc;
      uint32_t bits = word[li];
      while (bits) {
        const int bb = __ffs(bits) - 1;
        bits &= bits - 1;
        dst[off++] = c * kChunk + bb;
      }
      base[li] += tot;
    }
    __syncthreads();
  };
  int base[kListWords];
#pragma unroll
  for (int li = 0; li < kListWords; ++li) base[li] = 0;
  for (int c0 = 0; c0 < nc; c0 += kThreads) {
    const int c = c0 + tid;
    uint32_t word[kListWords];
#pragma unroll
    for (int li = 0; li < kListWords; ++li)
      word[li] = (li <= G && c < nc) ? a.chunk_bits[((size_t)g * W + c) * kListWords + li] : 0u;
    list_pass(c, word, base);
  }
  if (tid <= G) {
    int v = 0;
#pragma unroll
    for (int li = 0; li <= G; ++li)
      if (li == tid) v = base[li];
    if (tid < G) a.count[h0 + tid] = v;
    else a.ucount[g] = v;
  }
}

// The merge of query head h's partial softmax states (one per slot) into o:
// an online pass per thread over its stripe of slots, B slots' loads in
// flight at a time, then the stripes combined by log-sum-exp through LDS.
template <int G>
__device__ __attribute__((always_inline)) void tail_merge(const LayerGeom& geo, const LayerArgs& a,
                                                          int mode, int h, MergeScratch& mg) {
  const int tid = threadIdx.x;
  const int g = h / G, hl = h % G;
  // the layer kernel's slots, then those of the zoom workgroups this KV head got
  const int ns = geo.n_work + ((mode & kZoomSplit) ? a.zcount[g] : 0);
  const float* pg = a.part + (size_t)g * geo.n_slots() * G * kPartStride;
  constexpr int B = 16;
  const int dq = tid % kMergeQuads, stripe = tid / kMergeQuads;
  float M = -INFINITY, Ls = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sl0 = stripe; sl0 < ns; sl0 += B * kMergeStripes) {
    float m[B], l[B];
    float4 x[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int sl = sl0 + u * kMergeStripes;
      m[u] = -INFINITY;
      l[u] = 0.f;
      x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (sl < ns) {
        const float* p = pg + ((size_t)sl * G + hl) * kPartStride;
        const float2 ml = *(const float2*)p;
        m[u] = ml.x;
        l[u] = ml.y;
        x[u] = *(const float4*)(p + 4 + 4 * dq);
      }
    }
    float bm = m[0];
#pragma unroll
    for (int u = 1; u < B; ++u) bm = fmaxf(bm, m[u]);
    if (bm == -INFINITY) continue;
    const float Mn = fmaxf(M, bm);
    const float wo = (M == -INFINITY) ? 0.f : __expf(M - Mn);
    acc.x *= wo;
    acc.y *= wo;
    acc.z *= wo;
    acc.w *= wo;
    Ls *= wo;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float wt = (m[u] == -INFINITY) ? 0.f : __expf(m[u] - Mn);
      acc.x += wt * x[u].x;
      acc.y += wt * x[u].y;
      acc.z += wt * x[u].z;
      acc.w += wt * x[u].w;
      Ls += wt * l[u];
    }
    M = Mn;
  }
  mg.red[stripe * kMergeQuads + dq] = acc;
  if (dq == 0) {
    mg.m[stripe] = M;
    mg.l[stripe] = Ls;
  }
  __syncthreads();
  if (tid < kMergeQuads) {
    float Mx = -INFINITY;
    for (int st = 0; st < kMergeStripes; ++st) Mx = fmaxf(Mx, mg.m[st]);
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (Mx != -INFINITY) {
      for (int st = 0; st < kMergeStripes; ++st) {
        const float ms_ = mg.m[st];
        if (ms_ == -INFINITY) continue;
        const float wt = __expf(ms_ - Mx);
        const float4 y = mg.red[st * kMergeQuads + tid];
        t.x += wt * y.x;
        t.y += wt * y.y;
        t.z += wt * y.z;
        t.w += wt * y.w;
        L += wt * mg.l[st];
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *(float4*)(a.o + (size_t)h * kHeadDim + 4 * dq) =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

// ---------------------------------------------------------------------------
// The zoom kernel: every zoomed span of a layer, dealt to geo.z_total
// workgroups in proportion to each KV head's union size, so a KV head whose
// heads zoom many spans gets as many workgroups as its share of the work.
//
// Every workgroup reads the chunks' union bit masks of all KV heads (written by
// the layer launch), counts each union U_g and takes the same decision: a KV
// head with U_g > 0 gets Z_g = 1 + (its share of the z_total - n_nonempty
// others, by cumulative integer rounding, so the shares add up exactly);
// workgroup z belongs to the KV head g with B_g <= z < B_g + Z_g, B_g the sum
// of the Z of the heads before it, and takes the spans [U_g i / Z_g,
// U_g (i + 1) / Z_g) of g's ascending union, i = z - B_g.  Workgroup 0 also
// records each Z_g for the tail's merge.  z_total is at least
// Hkv S_c / kZoomBatch + Hkv, so a share never exceeds kZoomBatch spans and
// their metadata fit LDS at once.  The 4 waves each run the software
// pipeline of zoom_span32 over spans wid, wid + 4, ... of the share (spans
// above rank 32 afterwards, through zoom_span), and the 4 wave states merge
// into one partial per head of g, in slot n_work + i.
// ---------------------------------------------------------------------------
template <int G>
__device__ __attribute__((always_inline)) void zoom_body(const LayerGeom& geo, const LayerArgs& a,
                                                         int z, ZSmem<G>& s, Stage<G>& stg) {
  constexpr int SR = stage_rows<G>();
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  float* const stage = stg.v[uniform(wid)];
  const int hkv = geo.n_kv_heads, W = geo.n_work, nc = geo.n_chunks, scs = geo.sc_stride;
  const int zt = geo.z_total;

  // ---- union sizes of every KV head, and this workgroup's share -------------
  for (int g = tid; g < hkv; g += kThreads) s.cnt[g] = 0;
  __syncthreads();
  for (int p = tid; p < hkv * nc; p += kThreads) {
    const int g = p / nc, c = p % nc;
    const int n = __popc(a.chunk_bits[((size_t)g * W + c) * kListWords + G]);
    if (n) atomicAdd(&s.cnt[g], n);
  }
  if (tid == 0) s.g = -1;
  __syncthreads();
  if (wid == 0) {
    // lane = KV head (64 at a time): totals, then each head's share of the
    // workgroups by cumulative rounding (exact in float64: every product is
    // far below 2^53 and the quotients far from the next integer)
    int U = 0, nne = 0;
    for (int g0 = 0; g0 < hkv; g0 += 64) {
      const int c = g0 + lane < hkv ? s.cnt[g0 + lane] : 0;
      U += __builtin_amdgcn_readlane(wave_incl_scan(c), 63);
      nne += __popcll(__ballot(c > 0));
    }
    const double extra = (double)(zt - nne);   // z_total >= Hkv >= nne
    int cum = 0, base = 0;
    for (int g0 = 0; g0 < hkv; g0 += 64) {
      const int g = g0 + lane;
      const int c = g < hkv ? s.cnt[g] : 0;
      const int incl = wave_incl_scan(c);
      const double e0 = U ? floor(extra * (double)(cum + incl - c) / (double)U) : 0.0;
      const double e1 = U ? floor(extra * (double)(cum + incl) / (double)U) : 0.0;
      const int zg = (c > 0 ? 1 : 0) + (int)(e1 - e0);
      const int zincl = wave_incl_scan(zg);
      const int b = base + zincl - zg;   // first workgroup of head g
      if (g < hkv) {
        if (z == 0) a.zcount[g] = zg;
        if (z >= b && z < b + zg) {
          const int i = z - b;
          s.g = g;
          s.i = i;
          s.zg = zg;
          s.lo = (int)((long long)c * i / zg);
          s.hi = (int)((long long)c * (i + 1) / zg);
        }
      }
      cum += __builtin_amdgcn_readlane(incl, 63);
      base += __builtin_amdgcn_readlane(zincl, 63);
    }
  }
  __syncthreads();
  SEKV_TL(g_tl_attend, 3, SEKV_NOW());
  const int g = s.g;
  SEKV_TL(g_tl_attend, 10, g + 1);
  if (g < 0) return;   // uniform: no span for this workgroup
  // z_total >= Hkv S_c / kZoomBatch + Hkv, so a share never exceeds one batch
  const int lo = s.lo, nb = min(s.hi - s.lo, kZoomBatch), slot = W + s.i;

  // ---- the group's queries, scaled by 1/sqrt(d) -----------------------------
  const float scale = rsqrtf((float)kHeadDim);
  for (int o = tid; o < G * kHeadDim; o += kThreads)
    s.qs[o / kHeadDim][o % kHeadDim] = a.q[(size_t)g * G * kHeadDim + o] * scale;

  // ---- spans lo .. lo + nb - 1 of g's union: wave 0 scans the chunks'
  // popcounts, each lane writes its chunk's spans that fall in the range
  if (wid == 0) {
    int run = 0;
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const int c = c0 + lane;
      uint32_t word[kListWords];
#pragma unroll
      for (int li = 0; li <= G; ++li)
        word[li] = c < nc ? a.chunk_bits[((size_t)g * W + c) * kListWords + li] : 0u;
      const int pop = __popc(word[G]);
      const int incl = wave_incl_scan(pop);
      int k = run + incl - pop;   // rank of this chunk's first span in the union
      if (k < lo + nb && k + pop > lo) {
        uint32_t bits = word[G];
        while (bits) {
          const int bb = __ffs(bits) - 1;
          bits &= bits - 1;
          if (k >= lo && k < lo + nb) {
            unsigned hm = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) hm |= ((word[h] >> bb) & 1u) << h;
            s.m_n[k - lo] = c * kChunk + bb;   // the span id for now
            s.bits[k - lo] = (int)hm;
          }
          ++k;
        }
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  __syncthreads();
  SEKV_TL(g_tl_attend, 4, SEKV_NOW());
  SEKV_TL(g_tl_attend, 11, nb);
  if (tid < nb) {
    const int j = s.m_n[tid];
    const size_t gj = (size_t)g * scs + j;
    s.m_off[tid] = a.fac_off[gj] - a.off_base;
    s.m_r[tid] = a.rank[gj];
    s.m_n[tid] = a.clen[j];
  }
  __syncthreads();
  SEKV_TL(g_tl_attend, 5, SEKV_NOW());

  float zm[G], zl[G], za[G][2];   // the wave's state (lane: dims 2 lane, 2 lane + 1)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    zm[h] = -INFINITY;
    zl[h] = 0.f;
    za[h][0] = za[h][1] = 0.f;
  }
  const SpanRef zero{a.zero_block, 1, 1, 1, 0u};
  // ---- the wave's spans u = wid, wid + kWaves, ... of rank <= 32, pipelined
  auto next_small = [&](int u) {
    while (u < nb && rank_max(s.m_r[u]) > 32) u += kWaves;
    return uniform(u);
  };
  int u = next_small(wid);
  if (u < nb) {
    SpanRef cu = span_ref(s, a.pool, u);
    stage_vk<SR>(cu.rk <= SR ? cu : zero, stage);
    float4 ub[8];
    prefetch_span(cu, ub);
    for (;;) {
      const int un = next_small(u + kWaves);
      const bool has_nx = un < nb;
      const SpanRef nx = span_ref(s, a.pool, min(un, nb - 1));
      // stand-ins when there is no next span: this one again (its V_K only if
      // it is staged, else the zeros)
      const SpanRef nxp = has_nx ? nx : cu;
      const SpanRef nxs = has_nx && nx.rk <= SR ? nx : (cu.rk <= SR ? cu : zero);
      float (*scr)[kHeadDim] = s.w[wid].st.acc;
      if (cu.rk <= 16 && cu.rv <= 16)
        zoom_span32<G, SR, 16>(cu, nxp, nxs, ub, stage, scr, s.qs, zm, zl, za);
      else
        zoom_span32<G, SR, 32>(cu, nxp, nxs, ub, stage, scr, s.qs, zm, zl, za);
      if (!has_nx) break;
      cu = nx;
      u = un;
    }
  }
  // ---- then those of rank > 32, with the stage as scratch once its DMA is done
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  SEKV_TL_WAVE(g_tl_attend, 6, SEKV_NOW());
  for (u = wid; u < nb; u += kWaves) {
    if (rank_max(s.m_r[u]) <= 32) continue;
    const SpanRef sp = span_ref(s, a.pool, u);
    zoom_span<G>(sp.blk, sp.n, sp.rk, sp.rv, sp.hm, s.qs,
                 *reinterpret_cast<ZoomScratchAny<G>*>(stage), zm, zl, za);
  }
  __syncthreads();   // every wave is done with its span scratch

  // ---- the 4 wave states into one partial per head, slot n_work + i ---------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.w[wid].st.acc[h][2 * lane] = za[h][0];
    s.w[wid].st.acc[h][2 * lane + 1] = za[h][1];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s.w[wid].st.m[h] = zm[h];
      s.w[wid].st.l[h] = zl[h];
    }
  }
  __syncthreads();
  float* dst = a.part + ((size_t)g * geo.n_slots() + slot) * G * kPartStride;
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, s.w[wv].st.m[h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        const float m1 = s.w[wv].st.m[h];
        if (m1 != -INFINITY) {
          const float wt = __expf(m1 - M);
          L += s.w[wv].st.l[h] * wt;
          A += s.w[wv].st.acc[h][d] * wt;
        }
      }
    }
    dst[(size_t)h * kPartStride + 4 + d] = A;
    if (d == 0) {
      dst[(size_t)h * kPartStride] = M;
      dst[(size_t)h * kPartStride + 1] = L;
    }
  }
}

// One workgroup of a tail launch: x < Hq merges query head x, the others
// write KV head x - Hq's lists.
template <int G>
__device__ __attribute__((always_inline)) void layer_tail(const LayerGeom& geo, const LayerArgs& a,
                                                          int mode, int x, int (*wc)[kWaves],
                                                          MergeScratch& mg) {
  const int hq = geo.n_kv_heads * G;
  if (x < hq) {
    if (mode & kMerge) tail_merge<G>(geo, a, mode, x, mg);
  } else if (x < hq + geo.n_kv_heads) {
    if (mode & kLists) tail_lists<G>(geo, a, x - hq, wc);
  }
}

// The full-resolution rows and coarse entries of one layer of one sequence
// (mode kDense): workgroup `block` of its Hkv x n_work grid attends its slice
// of the rows and its chunk's coarse entries (those its heads did not zoom,
// read from the route's mask), one partial per head into slot w; it also
// writes the chunk's zoom masks from the mask unless kKeepBits.  Mode
// kMaskBits alone only writes those masks.
template <typename T, int G>
__device__ __attribute__((always_inline)) void layer_body(const LayerGeom& geo,
                                                          const LayerArgs& a, int mode,
                                                          int block, Smem<G>& s) {
  using Ln = Lanes<T>;
  constexpr int CLOADS = (kChunk / kWaves) / Ln::RPW;     // coarse entries: loads per wave
  constexpr int DLOADS = kRowBlock / Ln::RPW;             // full-resolution rows: loads per pass

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int W = geo.n_work;
  const int g = block / W, w = block % W;
  const int sc = geo.n_compressed, D = geo.n_dense;
  const int scs = geo.sc_stride;   // the span arrays' stride (route buffers use sc)
  const int h0 = g * G;
  const int j0 = w * kChunk, nj = w < geo.n_chunks ? min(kChunk, sc - j0) : 0;
  const int d0 = w * geo.dense_rows, d1 = min(D, d0 + geo.dense_rows);
  const bool dense = (mode & kDense) != 0;
  const float scale = rsqrtf((float)kHeadDim);

  // ---- everything this workgroup reads, issued up front: query, the
  // full-resolution rows (first pass) and the coarse entries.  The query goes
  // to LDS only after every load is out, so the prologue is one round trip.
  constexpr int QPT = (G * kHeadDim + kThreads - 1) / kThreads;   // query floats per thread
  float qx[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int o = tid + i * kThreads;
    qx[i] = o < G * kHeadDim ? a.q[(size_t)h0 * kHeadDim + o] : 0.f;
  }
  const T* DK = (const T*)a.dense_k + (size_t)g * geo.dense_stride * kHeadDim;
  const T* DV = (const T*)a.dense_v + (size_t)g * geo.dense_stride * kHeadDim;
  uint4 dk[DLOADS], dv[DLOADS];
  const int dr0 = d0 + wid * kRowBlock;
  if (dense) rows_load<T, DLOADS>(DK, DV, dr0, min(d1, dr0 + kRowBlock), dk, dv);
  const int cr0 = j0 + wid * (kChunk / kWaves);
  const int cr1 = min(j0 + nj, cr0 + kChunk / kWaves);
  uint4 kr[CLOADS], vr[CLOADS];
  float cbias[CLOADS];   // ln n of each coarse entry (loaded with it)
  if (dense && nj > 0) {
    const T* K = (const T*)a.kbar + (size_t)g * scs * kHeadDim;
    const T* V = (const T*)a.vbar + (size_t)g * scs * kHeadDim;
    rows_load<T, CLOADS>(K, V, cr0, cr1, kr, vr);
#pragma unroll
    for (int u = 0; u < CLOADS; ++u)
      cbias[u] = a.lnn32[min(cr0 + u * Ln::RPW + lane / Ln::LPR, j0 + nj - 1)];
  }
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int o = tid + i * kThreads;
    if (o < G * kHeadDim) s.qs[o / kHeadDim][o % kHeadDim] = qx[i] * scale;
  }
  if (tid < kChunk) s.bits[tid] = 0;
  __syncthreads();

  // ---- the heads of the group that zoom each span of the chunk (from the mask)
  if (nj > 0) {
    for (int idx = tid; idx < nj * G; idx += kThreads) {
      const int jl = idx / G, hl = idx % G;
      if (a.mask[(size_t)(h0 + hl) * sc + j0 + jl]) atomicOr(&s.bits[jl], 1 << hl);
    }
  }
  __syncthreads();
  if (mode & kKeepBits) SEKV_TL(g_tl_attend, 3, SEKV_NOW());

  // ---- zoom sets of the chunk: one wave ballot per list (per head, then the
  // union), read by the zoom kernel and by the tail's lists -----------------
  if (wid == 0 && nj > 0 && !(mode & kKeepBits)) {
    const int b = lane < nj ? s.bits[lane] : 0;
#pragma unroll
    for (int li = 0; li <= G; ++li) {
      const bool z = li < G ? ((b >> li) & 1) != 0 : b != 0;
      const unsigned long long bal = __ballot(z);
      if (lane == 0) a.chunk_bits[((size_t)g * W + w) * kListWords + li] = (uint32_t)bal;
    }
  }
  if (!dense) return;

  // ---- full-resolution rows and coarse entries: each wave's state ----------
  {
    QSlice<T, G> qv;
    qv.load(s.qs);
    RowState<T, G> rs;
    rs.init();
    const float nob[DLOADS] = {};
    rows_accumulate<T, G, DLOADS>(dk, dv, dr0, min(d1, dr0 + kRowBlock), qv, nob, nullptr, 0, rs);
    for (int p0 = d0 + kWaves * kRowBlock; p0 < d1; p0 += kWaves * kRowBlock) {
      const int r0 = p0 + wid * kRowBlock, r1 = min(d1, r0 + kRowBlock);
      rows_load<T, DLOADS>(DK, DV, r0, r1, dk, dv);
      rows_accumulate<T, G, DLOADS>(dk, dv, r0, r1, qv, nob, nullptr, 0, rs);
    }
    if (nj > 0) rows_accumulate<T, G, CLOADS>(kr, vr, cr0, cr1, qv, cbias, s.bits, j0, rs);
    rows_finish<T, G>(rs);
    rows_store<T, G>(rs, s.w[wid].st.acc, s.w[wid].st.m, s.w[wid].st.l);
  }
  __syncthreads();
  if (mode & kKeepBits) SEKV_TL(g_tl_attend, 4, SEKV_NOW());

  // ---- this workgroup's partial: slot w -------------------------------------
  float* dst = a.part + ((size_t)g * geo.n_slots() + w) * G * kPartStride;
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, s.w[wv].st.m[h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        const float m1 = s.w[wv].st.m[h];
        if (m1 != -INFINITY) {
          const float wt = __expf(m1 - M);
          L += s.w[wv].st.l[h] * wt;
          A += s.w[wv].st.acc[h][d] * wt;
        }
      }
    }
    dst[(size_t)h * kPartStride + 4 + d] = A;
    if (d == 0) {
      dst[(size_t)h * kPartStride] = M;
      dst[(size_t)h * kPartStride + 1] = L;
    }
  }
}

// The route of one layer on its own (sekv_route, and the first launch of
// sekv_route_attn): workgroup b of KV head g = b mod Hkv gates the spans of
// chunks RC r .. RC (r + 1) - 1, r = b / Hkv.  With RC chunks per workgroup
// the group's projected queries (G x dr outputs over P's 64 KB at G = 4,
// dr = 32) are formed once per RC chunks; launch_route takes RC = 1 for grids
// up to one workgroup per CU, 2 up to two, kRouteChunks beyond (batches of
// long contexts), where fewer, fuller workgroups pay.  Per chunk: mask and gate values of every (head, span), then one
// ballot per list into the chunk's zoom masks, as the layer kernel writes them.
template <typename T, int G, int RC>
__device__ __attribute__((always_inline)) void route_body(const LayerGeom& geo, const LayerArgs& a,
                                                          int block, Smem<G>& s) {
  using Ln = Lanes<T>;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int W = geo.n_work, nc = geo.n_chunks, sc = geo.n_compressed, dr = geo.route_dim;
  const int scs = geo.sc_stride;
  // consecutive workgroups take consecutive KV heads: the dispatcher deals
  // workgroups to the XCDs round robin, so with Hkv a multiple of the XCD
  // count each XCD's L2 fetches the projections of its own KV heads only
  const int g = block % geo.n_kv_heads, c0 = (block / geo.n_kv_heads) * RC;
  const int h0 = g * G;

  // ---- all loads up front: query, projections, each chunk's summaries, ln n
  constexpr int QPT = (G * kHeadDim + kThreads - 1) / kThreads;
  float qx[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int o = tid + i * kThreads;
    qx[i] = o < G * kHeadDim ? a.q[(size_t)h0 * kHeadDim + o] : 0.f;
  }
  const int nout = G * dr, part = tid & 7, orow = tid >> 3;
  float4 pv[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int o = min(orow + 32 * k, nout - 1);   // rows past nout are never used
    const float* pr = a.proj + ((size_t)h0 * dr + o) * kHeadDim + part * 4;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) pv[k][c4] = *(const float4*)(pr + 32 * c4);
  }
  constexpr int kSumVec = 4;
  const int svec = (dr * (int)sizeof(T)) % 16 == 0 ? dr * (int)sizeof(T) / 16 : 0;
  const bool sfast = svec > 0 && svec <= kSumVec;
  const int jl = tid / G, hl = tid % G, h = h0 + hl;   // this thread's (span, head) of a chunk
  uint4 sum[RC][kSumVec];
  double lnn[RC];
  int nj[RC];
#pragma unroll
  for (int cc = 0; cc < RC; ++cc) {
    const int c = c0 + cc, j = c * kChunk + jl;
    nj[cc] = c < nc ? min(kChunk, sc - c * kChunk) : 0;
    lnn[cc] = 0.0;
    if (tid < nj[cc] * G) {
      if (sfast) {
        const uint4* sr = (const uint4*)((const T*)a.summ + ((size_t)h * scs + j) * dr);
#pragma unroll
        for (int v = 0; v < kSumVec; ++v) sum[cc][v] = sr[min(v, svec - 1)];
      }
      lnn[cc] = a.lnn64[j];
    }
  }
  float tau_f = tid < kChunk * G ? a.tau[h] : 0.f;
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int o = tid + i * kThreads;
    if (o < G * kHeadDim) s.rt.qu[o / kHeadDim][o % kHeadDim] = qx[i];
  }
  if (tid < kChunk) s.bits[tid] = 0;
  __syncthreads();
  SEKV_TL(g_tl_route, 4, SEKV_NOW());

  // ---- q~_h = P_h q_h (float64), as the layer kernel forms it
  for (int k0 = 0; k0 < nout; k0 += 128) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int o = k0 + orow + 32 * k;
      if (k0 > 0 && o < nout) {
        const float* pr = a.proj + ((size_t)h0 * dr + o) * kHeadDim + part * 4;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) pv[k][c4] = *(const float4*)(pr + 32 * c4);
      }
      double acc = 0.0;
      if (o < nout) {
        const float* qh = &s.rt.qu[o / dr][part * 4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const float4 x = pv[k][c4];
          const float* qc = qh + 32 * c4;
          acc += (double)x.x * (double)qc[0] + (double)x.y * (double)qc[1] +
                 (double)x.z * (double)qc[2] + (double)x.w * (double)qc[3];
        }
      }
      acc = group_sum<8>(acc);
      if (part == 0 && o < nout) s.rt.qt[o / dr][o % dr] = acc;
    }
  }
  __syncthreads();

  SEKV_TL(g_tl_route, 2, SEKV_NOW());
  // ---- each chunk: gates, then its zoom masks (one ballot per list)
  asm volatile("" : "+v"(tau_f));   // its widening stays here, not next to its load
  const double tau_d = (double)tau_f;
#pragma unroll
  for (int cc = 0; cc < RC; ++cc) {
    const int c = c0 + cc;
    if (c >= nc) break;   // uniform
    if (tid < nj[cc] * G) {
      const int j = c * kChunk + jl;
      double x = 0.0;
      if (sfast) {
#pragma unroll
        for (int v = 0; v < kSumVec; ++v) {
          if (v < svec) {
            float f[Ln::EPL];
            unpack16(sum[cc][v], f, T());
#pragma unroll
            for (int e = 0; e < Ln::EPL; ++e) x += s.rt.qt[hl][v * Ln::EPL + e] * (double)f[e];
          }
        }
      } else {
        const T* sr = (const T*)a.summ + ((size_t)h * scs + j) * dr;
        for (int i = 0; i < dr; ++i) x += s.rt.qt[hl][i] * (double)Store<T>::load(sr + i);
      }
      x += a.gamma * lnn[cc];
      const double p = 1.0 / (1.0 + exp(-x));
      const bool z = p > tau_d;
      a.mask[(size_t)h * sc + j] = (uint8_t)z;
      if (a.prob) a.prob[(size_t)h * sc + j] = p;
      if (z) atomicOr(&s.bits[jl], 1 << hl);
    }
    __syncthreads();
    if (cc == 0) SEKV_TL(g_tl_route, 3, SEKV_NOW());
    if (wid == 0) {
      const int b = lane < nj[cc] ? s.bits[lane] : 0;
#pragma unroll
      for (int li = 0; li <= G; ++li) {
        const bool z = li < G ? ((b >> li) & 1) != 0 : b != 0;
        const unsigned long long bal = __ballot(z);
        if (lane == 0) a.chunk_bits[((size_t)g * W + c) * kListWords + li] = (uint32_t)bal;
      }
      if (lane < kChunk) s.bits[lane] = 0;   // wave 0 alone reads and clears them
    }
    __syncthreads();
  }
}

template <typename T, int G, int RC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void route_kernel(LayerGeom geo, LayerArgs a) {
  __shared__ Smem<G> s;
  SEKV_TL(g_tl_route, 0, SEKV_NOW());
  route_body<T, G, RC>(geo, a, blockIdx.x, s);
  SEKV_TL(g_tl_route, 1, SEKV_NOW());
}

template <typename T, int G, int RC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void route_batch_kernel(BatchLayerArgs b) {
  const int i = blockIdx.y;
  const int nc = b.geo[i].n_chunks;
  if ((int)blockIdx.x >= b.geo[i].n_kv_heads * ((nc + RC - 1) / RC)) return;
  __shared__ Smem<G> s;
  route_body<T, G, RC>(b.geo[i], b.arg[i], blockIdx.x, s);
}

// chunks per route workgroup for a launch of `wgs1` workgroups at one chunk each
inline int route_chunks(long long wgs1) { return wgs1 <= 256 ? 1 : (wgs1 <= 512 ? 2 : kRouteChunks); }

template <typename T, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void layer_kernel(LayerGeom geo, LayerArgs a, int mode) {
  __shared__ Smem<G> s;
  layer_body<T, G>(geo, a, mode, blockIdx.x, s);
}

// A batch of sequences, one cache each: blockIdx.y is the sequence; each runs
// its own Hkv x n_work workgroups and the rest of grid.x returns at once.
template <typename T, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void layer_batch_kernel(BatchLayerArgs b, int mode) {
  const int i = blockIdx.y;
  if ((int)blockIdx.x >= b.geo[i].n_kv_heads * b.geo[i].n_work) return;
  __shared__ Smem<G> s;
  layer_body<T, G>(b.geo[i], b.arg[i], mode, blockIdx.x, s);
}

// The merge and lists of one layer in a launch of their own: one workgroup
// per query head merges, one per KV head writes the lists (grid.x =
// Hkv (G + 1); grid.y: the sequence of a batch).  The layer launch before it
// wrote the partial states and chunk masks; the kernel boundary makes them
// visible here, so the layer kernel needs no ticket and no agent-scope fence.
template <int G>
__global__ __launch_bounds__(kThreads) void layer_tail_kernel(LayerGeom geo, LayerArgs a,
                                                              int mode) {
  __shared__ int wc[kListWords][kWaves];
  __shared__ MergeScratch mg;
  SEKV_TL(g_tl_tail, 0, SEKV_NOW());
  layer_tail<G>(geo, a, mode, blockIdx.x, wc, mg);
  SEKV_TL(g_tl_tail, 1, SEKV_NOW());
}

template <int G>
__global__ __launch_bounds__(kThreads) void layer_tail_batch_kernel(BatchLayerArgs b, int mode) {
  __shared__ int wc[kListWords][kWaves];
  __shared__ MergeScratch mg;
  const int i = blockIdx.y;
  layer_tail<G>(b.geo[i], b.arg[i], mode, blockIdx.x, wc, mg);
}

// The zoomed spans of one layer on their own (geo.z_total workgroups): the
// host tier's, after its rows launch and the factor fetch.
template <int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void zoom_kernel(LayerGeom geo, LayerArgs a) {
  __shared__ ZSmem<G> s;
  __shared__ Stage<G> stg;
  zoom_body<G>(geo, a, blockIdx.x, s, stg);
}

// The full-resolution rows, coarse entries and zoomed spans of a layer whose
// route is already out (chunk masks written by a route-only layer launch):
// the first geo.z_total workgroups (launch_attend passes z_attend there)
// attend the zoomed spans, the next Hkv x n_work rows and coarse entries (the
// chunk masks stay as the route wrote them).  Neither kind waits for the
// other, so the zoomed spans are attended while the rows are, not after them;
// the zoom workgroups, the longer ones, are dispatched first.
template <int G>
struct ZoomLds {
  ZSmem<G> z;
  Stage<G> st;
};
template <int G>
union AttendLds {
  Smem<G> l;
  ZoomLds<G> zz;
  int wc[kListWords][kWaves];
};
template <typename T, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attend_kernel(LayerGeom geo, LayerArgs a, int mode) {
  __shared__ AttendLds<G> u;
  SEKV_TL(g_tl_attend, 0, SEKV_NOW());
  const int nz = geo.n_compressed ? geo.z_total : 0;
  const int nr = geo.n_kv_heads * geo.n_work;
  const int x = blockIdx.x;
  SEKV_TL(g_tl_attend, 1, x < nz ? 0 : (x < nz + nr ? 1 : 2));
  if (x < nz)
    zoom_body<G>(geo, a, x, u.zz.z, u.zz.st);
  else if (x < nz + nr)
    layer_body<T, G>(geo, a, (mode & ~kLists) | kKeepBits, x - nz, u.l);
  else if (mode & kLists)   // the lists need only the route's chunk masks
    tail_lists<G>(geo, a, x - nz - nr, u.wc);
  SEKV_TL(g_tl_attend, 2, SEKV_NOW());
}
static_assert(sizeof(AttendLds<4>) <= 80 * 1024 && sizeof(AttendLds<5>) <= 80 * 1024,
              "two attend workgroups per CU");

// A batch of sequences (grid.y), each with its own z_attend zoom workgroups
// and Hkv x n_work row workgroups; the rest of grid.x returns at once.
template <typename T, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attend_batch_kernel(BatchLayerArgs b, int mode) {
  __shared__ AttendLds<G> u;
  const int i = blockIdx.y;
  LayerGeom geo = b.geo[i];
  const int nz = geo.n_compressed ? geo.z_attend : 0;
  const int nr = geo.n_kv_heads * geo.n_work;
  const int x = blockIdx.x;
  const int nl = (mode & kLists) ? geo.n_kv_heads : 0;
  if (x >= nz + nr + nl) return;
  geo.z_total = geo.z_attend;
  if (x < nz)
    zoom_body<G>(geo, b.arg[i], x, u.zz.z, u.zz.st);
  else if (x < nz + nr)
    layer_body<T, G>(geo, b.arg[i], (mode & ~kLists) | kKeepBits, x - nz, u.l);
  else
    tail_lists<G>(geo, b.arg[i], x - nz - nr, u.wc);
}

hipError_t launch_zoom(const LayerGeom& g, const LayerArgs& a, hipStream_t st) {
  if (g.n_compressed == 0) return hipSuccess;
  const dim3 grid(g.z_total);
#define SEKV_ZOOM(GG)                                                                       \
  case GG:                                                                                  \
    hipLaunchKernelGGL((zoom_kernel<GG>), grid, dim3(kThreads), 0, st, g, a);               \
    break;
  switch (g.group) {
    SEKV_ZOOM(1) SEKV_ZOOM(2) SEKV_ZOOM(3) SEKV_ZOOM(4) SEKV_ZOOM(5) SEKV_ZOOM(6) SEKV_ZOOM(7)
    SEKV_ZOOM(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ZOOM
  return hipGetLastError();
}

hipError_t launch_layer_tail(int mode, const LayerGeom& g, const LayerArgs& a, hipStream_t st) {
  const dim3 grid(g.n_kv_heads * g.group + ((mode & kLists) ? g.n_kv_heads : 0));
#define SEKV_TAIL(GG)                                                                          \
  case GG:                                                                                     \
    hipLaunchKernelGGL((layer_tail_kernel<GG>), grid, dim3(kThreads), 0, st, g, a, mode);     \
    break;
  switch (g.group) {
    SEKV_TAIL(1) SEKV_TAIL(2) SEKV_TAIL(3) SEKV_TAIL(4) SEKV_TAIL(5) SEKV_TAIL(6) SEKV_TAIL(7)
    SEKV_TAIL(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_TAIL
  return hipGetLastError();
}

hipError_t launch_layer_tail_batch(int mode, int group, const BatchLayerArgs& b, int batch,
                                   hipStream_t st) {
  if (batch < 1 || batch > kMaxBatch) return hipErrorInvalidValue;
  int nx = 0;
  for (int i = 0; i < batch; ++i)
    nx = max(nx, b.geo[i].n_kv_heads * group + ((mode & kLists) ? b.geo[i].n_kv_heads : 0));
  const dim3 grid(nx, batch);
#define SEKV_TAIL(GG)                                                                          \
  case GG:                                                                                     \
    hipLaunchKernelGGL((layer_tail_batch_kernel<GG>), grid, dim3(kThreads), 0, st, b, mode);  \
    break;
  switch (group) {
    SEKV_TAIL(1) SEKV_TAIL(2) SEKV_TAIL(3) SEKV_TAIL(4) SEKV_TAIL(5) SEKV_TAIL(6) SEKV_TAIL(7)
    SEKV_TAIL(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_TAIL
  return hipGetLastError();
}

hipError_t launch_layer_batch(int bf16, int mode, int group, const BatchLayerArgs& b, int batch,
                              hipStream_t st) {
  if (batch < 1 || batch > kMaxBatch) return hipErrorInvalidValue;
  int nx = 0;
  for (int i = 0; i < batch; ++i) nx = max(nx, b.geo[i].n_kv_heads * b.geo[i].n_work);
  const dim3 grid(nx, batch);
#define SEKV_LAYER(GG)                                                                       \
  case GG:                                                                                   \
    if (bf16)                                                                                \
      hipLaunchKernelGGL((layer_batch_kernel<uint16_t, GG>), grid, dim3(kThreads), 0, st, b, \
                         mode);                                                              \
    else                                                                                     \
      hipLaunchKernelGGL((layer_batch_kernel<float, GG>), grid, dim3(kThreads), 0, st, b,    \
                         mode);                                                              \
    break;
  switch (group) {
    SEKV_LAYER(1) SEKV_LAYER(2) SEKV_LAYER(3) SEKV_LAYER(4) SEKV_LAYER(5) SEKV_LAYER(6)
    SEKV_LAYER(7) SEKV_LAYER(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_LAYER
  return hipGetLastError();
}

hipError_t launch_attend(int bf16, int mode, const LayerGeom& g, const LayerArgs& a,
                         hipStream_t st) {
  if ((mode & ~kLists) != kDense) return hipErrorInvalidValue;
  LayerGeom ga = g;   // the zoom shares over z_attend workgroups (their count is
  ga.z_total = g.z_attend;   // recorded for the merge, within the z_total slots)
  const dim3 grid(ga.n_work * ga.n_kv_heads + (ga.n_compressed ? ga.z_total : 0) +
                  ((mode & kLists) ? ga.n_kv_heads : 0));
#define SEKV_ATTEND(GG)                                                                      \
  case GG:                                                                                   \
    if (bf16)                                                                                \
      hipLaunchKernelGGL((attend_kernel<uint16_t, GG>), grid, dim3(kThreads), 0, st, ga, a,  \
                         mode);                                                              \
    else                                                                                     \
      hipLaunchKernelGGL((attend_kernel<float, GG>), grid, dim3(kThreads), 0, st, ga, a,     \
                         mode);                                                              \
    break;
  switch (g.group) {
    SEKV_ATTEND(1) SEKV_ATTEND(2) SEKV_ATTEND(3) SEKV_ATTEND(4) SEKV_ATTEND(5) SEKV_ATTEND(6)
    SEKV_ATTEND(7) SEKV_ATTEND(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ATTEND
  return hipGetLastError();
}

hipError_t launch_attend_batch(int bf16, int mode, int group, const BatchLayerArgs& b, int batch,
                               hipStream_t st) {
  if ((mode & ~kLists) != kDense || batch < 1 || batch > kMaxBatch) return hipErrorInvalidValue;
  int nx = 0;
  for (int i = 0; i < batch; ++i)
    nx = max(nx, b.geo[i].n_kv_heads * b.geo[i].n_work +
                     (b.geo[i].n_compressed ? b.geo[i].z_attend : 0) +
                     ((mode & kLists) ? b.geo[i].n_kv_heads : 0));
  const dim3 grid(nx, batch);
#define SEKV_ATTEND(GG)                                                                      \
  case GG:                                                                                   \
    if (bf16)                                                                                \
      hipLaunchKernelGGL((attend_batch_kernel<uint16_t, GG>), grid, dim3(kThreads), 0, st, b, \
                         mode);                                                              \
    else                                                                                     \
      hipLaunchKernelGGL((attend_batch_kernel<float, GG>), grid, dim3(kThreads), 0, st, b,   \
                         mode);                                                              \
    break;
  switch (group) {
    SEKV_ATTEND(1) SEKV_ATTEND(2) SEKV_ATTEND(3) SEKV_ATTEND(4) SEKV_ATTEND(5) SEKV_ATTEND(6)
    SEKV_ATTEND(7) SEKV_ATTEND(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ATTEND
  return hipGetLastError();
}

hipError_t launch_route(int bf16, const LayerGeom& g, const LayerArgs& a, hipStream_t st) {
  if (g.n_compressed == 0) return hipSuccess;
  const int rc = route_chunks((long long)g.n_kv_heads * g.n_chunks);
  const dim3 grid(g.n_kv_heads * ((g.n_chunks + rc - 1) / rc));
#define SEKV_ROUTE_RC(TT, GG)                                                                \
  if (rc == 1)                                                                               \
    hipLaunchKernelGGL((route_kernel<TT, GG, 1>), grid, dim3(kThreads), 0, st, g, a);        \
  else if (rc == 2)                                                                          \
    hipLaunchKernelGGL((route_kernel<TT, GG, 2>), grid, dim3(kThreads), 0, st, g, a);        \
  else                                                                                       \
    hipLaunchKernelGGL((route_kernel<TT, GG, kRouteChunks>), grid, dim3(kThreads), 0, st, g, a);
#define SEKV_ROUTE(GG)                                                                       \
  case GG:                                                                                   \
    if (bf16) {                                                                              \
      SEKV_ROUTE_RC(uint16_t, GG)                                                            \
    } else {                                                                                 \
      SEKV_ROUTE_RC(float, GG)                                                               \
    }                                                                                        \
    break;
  switch (g.group) {
    SEKV_ROUTE(1) SEKV_ROUTE(2) SEKV_ROUTE(3) SEKV_ROUTE(4) SEKV_ROUTE(5) SEKV_ROUTE(6)
    SEKV_ROUTE(7) SEKV_ROUTE(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ROUTE
#undef SEKV_ROUTE_RC
  return hipGetLastError();
}

hipError_t launch_route_batch(int bf16, int group, const BatchLayerArgs& b, int batch,
                              hipStream_t st) {
  if (batch < 1 || batch > kMaxBatch) return hipErrorInvalidValue;
  long long wgs1 = 0;
  for (int i = 0; i < batch; ++i) wgs1 += (long long)b.geo[i].n_kv_heads * b.geo[i].n_chunks;
  const int rc = route_chunks(wgs1);
  int nx = 0;
  for (int i = 0; i < batch; ++i)
    nx = max(nx, b.geo[i].n_kv_heads * ((b.geo[i].n_chunks + rc - 1) / rc));
  if (nx == 0) return hipSuccess;
  const dim3 grid(nx, batch);
#define SEKV_ROUTE_RC(TT, GG)                                                                \
  if (rc == 1)                                                                               \
    hipLaunchKernelGGL((route_batch_kernel<TT, GG, 1>), grid, dim3(kThreads), 0, st, b);     \
  else if (rc == 2)                                                                          \
    hipLaunchKernelGGL((route_batch_kernel<TT, GG, 2>), grid, dim3(kThreads), 0, st, b);     \
  else                                                                                       \
    hipLaunchKernelGGL((route_batch_kernel<TT, GG, kRouteChunks>), grid, dim3(kThreads), 0, st, b);
#define SEKV_ROUTE(GG)                                                                       \
  case GG:                                                                                   \
    if (bf16) {                                                                              \
      SEKV_ROUTE_RC(uint16_t, GG)                                                            \
    } else {                                                                                 \
      SEKV_ROUTE_RC(float, GG)                                                               \
    }                                                                                        \
    break;
  switch (group) {
    SEKV_ROUTE(1) SEKV_ROUTE(2) SEKV_ROUTE(3) SEKV_ROUTE(4) SEKV_ROUTE(5) SEKV_ROUTE(6)
    SEKV_ROUTE(7) SEKV_ROUTE(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ROUTE
#undef SEKV_ROUTE_RC
  return hipGetLastError();
}

hipError_t launch_layer(int bf16, int mode, const LayerGeom& g, const LayerArgs& a,
                        hipStream_t st) {
  dim3 grid(g.n_work * g.n_kv_heads);
#define SEKV_LAYER(GG)                                                                      \
  case GG:                                                                                  \
    if (bf16)                                                                               \
      hipLaunchKernelGGL((layer_kernel<uint16_t, GG>), grid, dim3(kThreads), 0, st, g, a,   \
                         mode);                                                             \
    else                                                                                    \
      hipLaunchKernelGGL((layer_kernel<float, GG>), grid, dim3(kThreads), 0, st, g, a, mode); \
    break;
  switch (g.group) {
    SEKV_LAYER(1) SEKV_LAYER(2) SEKV_LAYER(3) SEKV_LAYER(4) SEKV_LAYER(5) SEKV_LAYER(6)
    SEKV_LAYER(7) SEKV_LAYER(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_LAYER
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// small fill (used instead of a memset so the calls can be graph-captured)
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host tier: copy the factor blocks of a layer's union spans from mapped
// pinned host memory into device staging at the same layer-relative offsets
// (16-byte loads over the host link).
// ---------------------------------------------------------------------------
constexpr int kFetchSlots = 64;

__global__ __launch_bounds__(256) void fetch_gather_kernel(
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ rank,
    const uint64_t* __restrict__ fac_off, uint64_t layer_base, int sc, int scs,
    const float* __restrict__ host, float* __restrict__ stage) {
  const int zs = blockIdx.x, g = blockIdx.y;
  const int nu = ucount[g];
  for (int u = zs; u < nu; u += kFetchSlots) {
    const int j = ulist[(size_t)g * sc + u];
    const FactorView fv = FactorView::packed(rank[(size_t)g * scs + j], clen[j]);
    const uint64_t off = fac_off[(size_t)g * scs + j];
    const uint4* src = (const uint4*)(host + off);
    uint4* dst = (uint4*)(stage + (off - layer_base));
    const int nvec = (int)(fv.block_floats() / 4);
    for (int k = threadIdx.x; k < nvec; k += 256) dst[k] = src[k];
  }
}

hipError_t launch_fetch_gather(const LayerGeom& g, const int32_t* ulist, const int32_t* ucount,
                               const int32_t* clen, const int32_t* rank,
                               const uint64_t* fac_off, uint64_t layer_base,
                               const float* host_pool_mapped, float* stage, hipStream_t st) {
  if (g.n_compressed == 0) return hipSuccess;
  hipLaunchKernelGGL(fetch_gather_kernel, dim3(kFetchSlots, g.n_kv_heads), dim3(256), 0, st,
                     ulist, ucount, clen, rank, fac_off, layer_base, g.n_compressed,
                     g.sc_stride, host_pool_mapped, stage);
  return hipGetLastError();
}

}  // namespace sekv

#ifdef SEKV_TIMELINE
// The diagnostic build's stamp tables (each kTlWgs x kTlSlots entries of
// 64 bits, in workgroup order) copied to host memory, or zeroed.  Returns a
// hipError_t.  Not part of the product library's ABI.
extern "C" int sekv_timeline_read(unsigned long long* route, unsigned long long* attend,
                                  unsigned long long* tail) {
  hipError_t e = hipMemcpyFromSymbol(route, HIP_SYMBOL(sekv::g_tl_route), sizeof(sekv::g_tl_route));
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(attend, HIP_SYMBOL(sekv::g_tl_attend), sizeof(sekv::g_tl_attend));
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(tail, HIP_SYMBOL(sekv::g_tl_tail), sizeof(sekv::g_tl_tail));
  return (int)e;
}
extern "C" int sekv_timeline_clear() {
  static unsigned long long zeros[sekv::kTlWgs * sekv::kTlSlots];
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(sekv::g_tl_route), zeros, sizeof(zeros));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(sekv::g_tl_attend), zeros, sizeof(zeros));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(sekv::g_tl_tail), zeros, sizeof(zeros));
  return (int)e;
}
#endif
