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
// One workgroup of 1024 threads per KV head.  The order is never materialised:
// each candidate's inclusive prefix length is a sum over the candidates that
// precede it, counted against LDS tiles of (key, id, length), so the decisions
// do not depend on any sort and are deterministic.  Masks, the per-head lists
// and the union are then compacted in place, stably, with ballot scans.
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

constexpr int kCapThreads = 1024;
constexpr int kCapWaves = kCapThreads / 64;
constexpr int kCapTile = 2048;

// largest gate value among the heads [h0, h0 + G) that zoomed span j (gate
// values are probabilities, so -1 marks "none")
__device__ __forceinline__ double cap_key(const uint8_t* __restrict__ mask,
                                          const double* __restrict__ prob, int sc, int h0, int G,
                                          int j) {
  double k = -1.0;
  for (int hl = 0; hl < G; ++hl) {
    const size_t o = (size_t)(h0 + hl) * sc + j;
    if (mask[o] && prob[o] > k) k = prob[o];
  }
  return k;
}

// exclusive prefix count of `flag` over the workgroup, in thread order;
// *total receives the workgroup's count.  Every thread must call it.
__device__ __forceinline__ int cap_scan(int flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long b = __ballot(flag);
  const int before = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(b);
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kCapWaves; ++w) {
    const int c = s_wave[w];
    base += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + before;
}

__global__ __launch_bounds__(kCapThreads) void cap_budget_kernel(
    int sc, int G, long long budget, const int32_t* __restrict__ clen,
    const double* __restrict__ prob, uint8_t* mask, int32_t* list, int32_t* count,
    int32_t* ulist, int32_t* ucount) {
  __shared__ double s_key[kCapTile];
  __shared__ int s_id[kCapTile];
  __shared__ int s_len[kCapTile];
  __shared__ int s_wave[kCapWaves];
  extern __shared__ uint32_t s_drop[];  // one bit per union position

  const int g = blockIdx.x, tid = threadIdx.x;
  const int h0 = g * G;
  int32_t* ul = ulist + (size_t)g * sc;
  const int U = ucount[g];
  for (int w = tid; w < (U + 31) / 32; w += kCapThreads) s_drop[w] = 0u;

  // 1. inclusive prefix length of every candidate in (key desc, id asc) order
  for (int base = 0; base < U; base += kCapThreads) {
    const int i = base + tid;
    const bool have = i < U;
    int ji = 0;
    double ki = 0.0;
    if (have) {
      ji = ul[i];
      ki = cap_key(mask, prob, sc, h0, G, ji);
    }
    long long S = 0;
    for (int t0 = 0; t0 < U; t0 += kCapTile) {
      const int tn = min(kCapTile, U - t0);
      __syncthreads();
      for (int k = tid; k < tn; k += kCapThreads) {
        const int j = ul[t0 + k];
        s_id[k] = j;
        s_len[k] = clen[j];
        s_key[k] = cap_key(mask, prob, sc, h0, G, j);
      }
      __syncthreads();
      if (have) {
        for (int k = 0; k < tn; ++k) {
          const double kk = s_key[k];
          if (kk > ki || (kk == ki && s_id[k] <= ji)) S += s_len[k];
        }
      }
    }
    if (have && S > budget) atomicOr(&s_drop[i >> 5], 1u << (i & 31));
  }
  __syncthreads();

  // 2. a dropped span leaves the mask of every head of the group
  for (int i = tid; i < U; i += kCapThreads) {
    if ((s_drop[i >> 5] >> (i & 31)) & 1u) {
      const int j = ul[i];
      for (int hl = 0; hl < G; ++hl) mask[(size_t)(h0 + hl) * sc + j] = 0;
    }
  }
  __syncthreads();

  // 3. the union keeps its kept candidates, in ascending order (in place:
  //    every tile is read before any of its entries is written, and writes
  //    never pass the position being read)
  int out = 0;
  for (int base = 0; base < U; base += kCapThreads) {
    const int i = base + tid;
    int j = 0, keep = 0;
    if (i < U) {
      j = ul[i];
      keep = !((s_drop[i >> 5] >> (i & 31)) & 1u);
    }
    int tot;
    const int pos = cap_scan(keep, s_wave, &tot);
    if (keep) ul[out + pos] = j;
    out += tot;
  }
  if (tid == 0) ucount[g] = out;

  // 4. each head's ascending list keeps the spans still in its mask
  for (int hl = 0; hl < G; ++hl) {
    const int h = h0 + hl;
    int32_t* lst = list + (size_t)h * sc;
    const uint8_t* m = mask + (size_t)h * sc;
    const int n = count[h];
    int o = 0;
    for (int base = 0; base < n; base += kCapThreads) {
      const int i = base + tid;
      int j = 0, keep = 0;
      if (i < n) {
        j = lst[i];
        keep = m[j] != 0;
      }
      int tot;
      const int pos = cap_scan(keep, s_wave, &tot);
      if (keep) lst[o + pos] = j;
      o += tot;
    }
    if (tid == 0) count[h] = o;
  }
}

}  // namespace

size_t cap_budget_lds_bytes(int sc) { return (size_t)((sc + 31) / 32) * sizeof(uint32_t); }

hipError_t launch_cap_budget(int sc, int hkv, int group, long long budget, const int32_t* clen,
                             const double* prob, uint8_t* mask, int32_t* list, int32_t* count,
                             int32_t* ulist, int32_t* ucount, hipStream_t st) {
  if (sc <= 0 || hkv <= 0) return hipSuccess;
  hipLaunchKernelGGL(cap_budget_kernel, dim3(hkv), dim3(kCapThreads), cap_budget_lds_bytes(sc),
                     st, sc, group, budget, clen, prob, mask, list, count, ulist, ucount);
  return hipGetLastError();
}

}  // namespace sekv
