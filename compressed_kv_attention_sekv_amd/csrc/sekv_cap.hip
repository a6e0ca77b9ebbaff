// Matched-budget cap of one layer's zoom decisions (gfx950).
//
// SeKV paper Sec. 3.3 (zoom-in decoding): when the spans the router selects
// would exceed the GPU KV budget, spans are kept in decreasing order of their
// gate value until the budget is filled.  Per KV head, the candidates are the
// spans of the group's union; a candidate's key is the largest gate value p
// among the group's heads that zoomed it, ties going to the lower span id; a
// candidate stays zoomed iff the total length of the candidates up to and
// including it in that order is at most the budget (lengths are >= 1, so the
// kept set is the longest prefix that fits).  A dropped span reverts to its
// coarse entry for every head of the group.
//
// A second reading takes one budget for the whole layer: one order over the
// candidates of every KV head (ties to the lower KV head, then the lower span
// id), whose kept prefix bounds the total the layer reconstructs.
//
// One workgroup of 512 threads per KV head (the layer scope's decisions: up
// to 8 per KV head, each taking a share of its candidates).  The order is
// never materialised: each candidate's inclusive prefix length is a sum over
// the candidates that precede it, counted against LDS tiles of (key, id,
// length); when the candidates fit one tile, each candidate's sum is split
// over several threads so that every thread counts.  The sums are integers,
// so the decisions do not depend on any sort or order and are deterministic.  Then one pass over the
// union clears the dropped spans from the masks and compacts the union and
// every head's list at once (a head's new list is the kept union filtered by
// its mask bit), in place and stably, with ballot scans.  Every gather is
// issued without waiting on another, so each phase is one or two round trips.
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

constexpr int kCapThreads = 512;
constexpr int kCapWaves = kCapThreads / 64;
constexpr int kCapTile = 4096;

// largest gate value among the heads [h0, h0 + G) that zoomed span j (gate
// values are probabilities, so -1 marks "none"); all 2 G loads go out at once
template <int G>
__device__ __forceinline__ double cap_key(const uint8_t* __restrict__ mask,
                                          const double* __restrict__ prob, int sc, int h0,
                                          int j) {
  uint8_t mb[G];
  double pb[G];
#pragma unroll
  for (int hl = 0; hl < G; ++hl) {
    const size_t o = (size_t)(h0 + hl) * sc + j;
    mb[hl] = mask[o];
    pb[hl] = prob[o];
  }
  double k = -1.0;
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
    if (mb[hl] && pb[hl] > k) k = pb[hl];
  return k;
}

// exclusive prefix counts of NF flags at once over the workgroup, in thread
// order; tot[f] receives the workgroup's count of flag f.  Every thread must
// call it.
template <int NF>
__device__ __forceinline__ void cap_scan(const int (&flag)[NF], int (&pos)[NF], int (&tot)[NF],
                                         int (*s_wave)[kCapWaves]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  int before[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const unsigned long long b = __ballot(flag[f]);
    before[f] = __popcll(b & below);
    if (lane == 0) s_wave[f][wave] = __popcll(b);
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int base = 0, t = 0;
    for (int w = 0; w < kCapWaves; ++w) {
      const int c = s_wave[f][w];
      base += w < wave ? c : 0;
      t += c;
    }
    pos[f] = base + before[f];
    tot[f] = t;
  }
  __syncthreads();
}

// one candidate in LDS: a single 16-byte read per comparison
struct alignas(16) CapEnt {
  double key;
  int id;   // span id; in the layer-wide single tile, KV head x S_c + span id
  int len;
};

// Which phases a launch runs: both, for one KV head's own budget; or, for one
// budget over the whole layer, the decisions (counted against every KV head's
// candidates, written as one byte per union position) and then, in a launch
// of its own, their application (the decisions read other heads' masks and
// unions, which the application rewrites).
enum CapPhase : int { kCapBoth = 0, kCapDecide = 1, kCapApply = 2 };

template <int G, int PHASE>
__global__ __launch_bounds__(kCapThreads) void cap_budget_kernel(
    int sc, int hkv, long long budget, const int32_t* __restrict__ clen,
    const double* __restrict__ prob, uint8_t* mask, int32_t* list, int32_t* count, int32_t* ulist,
    int32_t* ucount, uint8_t* __restrict__ drop) {
  __shared__ CapEnt s_ent[kCapTile];
  __shared__ int s_wave[G + 1][kCapWaves];
  __shared__ int s_upre[kMaxKvHeads + 1];   // layer scope: candidates of the KV heads before
  __shared__ long long s_part[kCapThreads]; // layer scope: parts of the candidates' sums
  extern __shared__ uint32_t s_drop[];  // one bit per union position

  const int g = blockIdx.x, tid = threadIdx.x;
  const int h0 = g * G;
  int32_t* ul = ulist + (size_t)g * sc;
  const int U = ucount[g];
  for (int w = tid; w < (U + 31) / 32; w += kCapThreads) s_drop[w] = 0u;

  // 1. inclusive prefix length of every candidate in (key desc, KV head asc,
  //    id asc) order, over this KV head's candidates or over every KV head's
  //    (layer scope); with a single tile of its own candidates a candidate's
  //    own key comes from it
  if (PHASE == kCapDecide) {
    // layer scope: the KV heads' candidate counts and their running sum
    if (tid < 64) {
      int run = 0;
      for (int g0 = 0; g0 < hkv; g0 += 64) {
        int v = g0 + tid < hkv ? ucount[g0 + tid] : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(v, o, 64);
          if (tid >= o) v += u;
        }
        if (g0 + tid < hkv) s_upre[g0 + tid + 1] = run + v;
        run += __shfl(v, 63, 64);
      }
      if (tid == 0) s_upre[0] = 0;
    }
    __syncthreads();
  }
  // layer scope with every KV head's candidates in one tile: they are
  // gathered in one pass (two round trips in all, instead of two per KV
  // head), and a candidate's place among equal keys is its KV head x S_c + id
  if (PHASE == kCapDecide && s_upre[hkv] <= kCapTile && (long long)hkv * sc < (1ll << 31)) {
    const int Ut = s_upre[hkv];
    for (int k = tid; k < Ut; k += kCapThreads) {
      int lo = 0, hi = hkv;   // the KV head of candidate k: s_upre[go] <= k < s_upre[go + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_upre[mid] <= k) lo = mid; else hi = mid;
      }
      const int j = ulist[(size_t)lo * sc + (k - s_upre[lo])];
      CapEnt e;
      e.key = cap_key<G>(mask, prob, sc, lo * G, j);
      e.id = lo * sc + j;
      e.len = clen[j];
      s_ent[k] = e;
    }
    __syncthreads();
    // workgroup y of the KV head decides its candidates [i0, i1); each
    // candidate's sum over the tile is split into P parts, one per thread,
    // so that every thread counts
    const int i0 = (int)((long long)U * blockIdx.y / gridDim.y);
    const int i1 = (int)((long long)U * (blockIdx.y + 1) / gridDim.y);
    const int nloc = i1 - i0;
    const int cpb = min(kCapThreads, max(64, (nloc + 63) & ~63));   // candidates per pass
    const int P = kCapThreads / cpb;                                 // parts per candidate
    const int p = tid / cpb, il = tid % cpb;
    const int k0 = (int)((long long)Ut * p / P), k1 = (int)((long long)Ut * (p + 1) / P);
    for (int b0 = 0; b0 < nloc; b0 += cpb) {
      const bool mine = p < P && b0 + il < nloc;
      long long S = 0;
      if (mine) {
        const CapEnt me = s_ent[s_upre[g] + i0 + b0 + il];
#pragma unroll 8
        for (int k = k0; k < k1; ++k) {
          const CapEnt e = s_ent[k];
          const bool before = (e.key > me.key) | ((e.key == me.key) & (e.id <= me.id));
          S += before ? e.len : 0;
        }
      }
      s_part[tid] = S;
      __syncthreads();
      if (mine && p == 0) {
        for (int q = 1; q < P; ++q) S += s_part[q * cpb + il];
        drop[(size_t)g * sc + i0 + b0 + il] = S > budget;
      }
      __syncthreads();
    }
    return;
  }
  if (PHASE == kCapDecide && blockIdx.y > 0) return;   // the tiled path runs in y = 0
  if (PHASE == kCapBoth && U <= kCapTile) {
    // one KV head's candidates in one tile: each candidate's sum over it split
    // into P parts, one per thread, so that every thread counts
    for (int k = tid; k < U; k += kCapThreads) {
      const int j = ul[k];
      CapEnt e;
      e.key = cap_key<G>(mask, prob, sc, h0, j);
      e.id = j;
      e.len = clen[j];
      s_ent[k] = e;
    }
    __syncthreads();
    const int cpb = min(kCapThreads, max(64, (U + 63) & ~63));   // candidates per pass
    const int P = kCapThreads / cpb;                              // parts per candidate
    const int p = tid / cpb, il = tid % cpb;
    const int k0 = (int)((long long)U * p / P), k1 = (int)((long long)U * (p + 1) / P);
    for (int b0 = 0; b0 < U; b0 += cpb) {
      const bool mine = p < P && b0 + il < U;
      long long S = 0;
      if (mine) {
        const CapEnt me = s_ent[b0 + il];
#pragma unroll 8
        for (int k = k0; k < k1; ++k) {
          const CapEnt e = s_ent[k];
          const bool before = (e.key > me.key) | ((e.key == me.key) & (e.id <= me.id));
          S += before ? e.len : 0;
        }
      }
      s_part[tid] = S;
      __syncthreads();
      if (mine && p == 0) {
        for (int q = 1; q < P; ++q) S += s_part[q * cpb + il];
        const int i = b0 + il;
        if (S > budget) atomicOr(&s_drop[i >> 5], 1u << (i & 31));
      }
      __syncthreads();
    }
  } else if (PHASE != kCapApply) {
    const int ga = PHASE == kCapDecide ? 0 : g, gb = PHASE == kCapDecide ? hkv : g + 1;
    for (int base = 0; base < U; base += kCapThreads) {
      const int i = base + tid;
      const bool have = i < U;
      int ji = 0;
      double ki = 0.0;
      if (have) {
        ji = ul[i];
        ki = cap_key<G>(mask, prob, sc, h0, ji);
      }
      long long S = 0;
      for (int go = ga; go < gb; ++go) {
        const int32_t* ulo = ulist + (size_t)go * sc;
        const int Uo = ucount[go];
        for (int t0 = 0; t0 < Uo; t0 += kCapTile) {
          const int tn = min(kCapTile, Uo - t0);
          __syncthreads();
          for (int k = tid; k < tn; k += kCapThreads) {
            const int j = ulo[t0 + k];
            CapEnt e;
            e.key = cap_key<G>(mask, prob, sc, go * G, j);
            e.id = j;
            e.len = clen[j];
            s_ent[k] = e;
          }
          __syncthreads();
          if (have) {
            // branch-free: every entry is read (one broadcast 16-byte LDS
            // read) and counted with a select, so the reads of an unrolled
            // group are all in flight together; candidates of a lower KV
            // head win key ties, of a higher one lose them
            const bool lower = go < g, same = go == g;
#pragma unroll 8
            for (int k = 0; k < tn; ++k) {
              const CapEnt e = s_ent[k];
              const bool before = (e.key > ki) |
                                  ((e.key == ki) & (lower | (same & (e.id <= ji))));
              S += before ? e.len : 0;
            }
          }
        }
      }
      if (PHASE == kCapDecide) {
        if (have) drop[(size_t)g * sc + i] = S > budget;
      } else if (have && S > budget) {
        atomicOr(&s_drop[i >> 5], 1u << (i & 31));
      }
    }
    if (PHASE == kCapDecide) return;
  } else {
    __syncthreads();
    for (int i = tid; i < U; i += kCapThreads)
      if (drop[(size_t)g * sc + i]) atomicOr(&s_drop[i >> 5], 1u << (i & 31));
  }
  __syncthreads();

  // 2. one pass over the union: a dropped span leaves every head's mask; the
  //    union keeps its kept spans and head h's list the kept spans in h's mask,
  //    ascending.  In place: each block of positions is read before any of it
  //    is written, and writes never pass the position being read.
  int out[G + 1];
#pragma unroll
  for (int f = 0; f <= G; ++f) out[f] = 0;
  for (int base = 0; base < U; base += kCapThreads) {
    const int i = base + tid;
    int flag[G + 1];
    int j = 0;
    uint8_t mb[G];
#pragma unroll
    for (int f = 0; f <= G; ++f) flag[f] = 0;
    if (i < U) {
      j = ul[i];
#pragma unroll
      for (int hl = 0; hl < G; ++hl) mb[hl] = mask[(size_t)(h0 + hl) * sc + j];
      const bool keep = !((s_drop[i >> 5] >> (i & 31)) & 1u);
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        flag[hl] = keep && mb[hl] != 0;
        if (!keep && mb[hl]) mask[(size_t)(h0 + hl) * sc + j] = 0;
      }
      flag[G] = keep;
    }
    int pos[G + 1], tot[G + 1];
    cap_scan<G + 1>(flag, pos, tot, s_wave);
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
      if (flag[hl]) list[(size_t)(h0 + hl) * sc + out[hl] + pos[hl]] = j;
    if (flag[G]) ul[out[G] + pos[G]] = j;
#pragma unroll
    for (int f = 0; f <= G; ++f) out[f] += tot[f];
  }
  if (tid < G) {
    int v = 0;
#pragma unroll
    for (int hl = 0; hl < G; ++hl) v = hl == tid ? out[hl] : v;
    count[h0 + tid] = v;
  }
  if (tid == G) ucount[g] = out[G];
}

}  // namespace

size_t cap_budget_lds_bytes(int sc) { return (size_t)((sc + 31) / 32) * sizeof(uint32_t); }

hipError_t launch_cap_budget(int sc, int hkv, int group, long long budget, const int32_t* clen,
                             const double* prob, uint8_t* mask, int32_t* list, int32_t* count,
                             int32_t* ulist, int32_t* ucount, uint8_t* drop, hipStream_t st) {
  if (sc <= 0 || hkv <= 0) return hipSuccess;
  const size_t lds = cap_budget_lds_bytes(sc);
  // layer scope: each KV head's decisions over qd workgroups (about 256 in all)
  const int qd = max(1, min(8, 256 / hkv));
  // drop == NULL: each KV head's own budget (one launch); else one budget for
  // the layer: the decisions, then their application
#define SEKV_CAP(GG)                                                                           \
  case GG:                                                                                     \
    if (!drop) {                                                                               \
      hipLaunchKernelGGL((cap_budget_kernel<GG, kCapBoth>), dim3(hkv), dim3(kCapThreads), lds, \
                         st, sc, hkv, budget, clen, prob, mask, list, count, ulist, ucount,    \
                         drop);                                                                \
    } else {                                                                                   \
      hipLaunchKernelGGL((cap_budget_kernel<GG, kCapDecide>), dim3(hkv, qd), dim3(kCapThreads), \
                         lds, st, sc, hkv, budget, clen, prob, mask, list, count, ulist,       \
                         ucount, drop);                                                        \
      hipLaunchKernelGGL((cap_budget_kernel<GG, kCapApply>), dim3(hkv), dim3(kCapThreads),     \
                         lds, st, sc, hkv, budget, clen, prob, mask, list, count, ulist,       \
                         ucount, drop);                                                        \
    }                                                                                          \
    break;
  switch (group) {
    SEKV_CAP(1) SEKV_CAP(2) SEKV_CAP(3) SEKV_CAP(4) SEKV_CAP(5) SEKV_CAP(6) SEKV_CAP(7)
    SEKV_CAP(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_CAP
  return hipGetLastError();
}

}  // namespace sekv
