// HBM residency cache of host-tier span factors (gfx950).
//
// With factors in pinned host memory, every zoomed span's block crosses the
// host link each time it is zoomed (SeKV paper Sec. 3.2: bases on the CPU,
// fetched for the selected spans; the paper's limitation section names that
// transfer as the cost of the CPU tier).  Decoding tends to zoom the same
// spans again, so blocks stay in an HBM cache between calls.
//
// Placement is two-choice: block (layer, KV head, span) may live in set
// h1(key) or h2(key) (two hashes mod n_sets), one fixed-size slot per set,
// each set tagged with the block it holds.  One call (one layer) runs two
// kernels on the fetch stream:
//   claim: every union span whose block fits a slot bids for both its sets
//          with a 64-bit atomicMax of (epoch, holds, inverted key): bids of
//          older calls always lose (no reset pass), a set's current holder
//          beats any newcomer, and otherwise the lowest key wins;
//   fetch: a span reads its block from a set it won that holds it (a hit, no
//          copy); else it copies the block from host memory into a set it won
//          (the first) and takes the tag; a span that won neither set, or
//          whose block is larger than a slot, is copied into the layer's
//          staging area at its layer-relative offset, as without the cache.
//          Each union span's block offset goes to an offset table that the
//          attention reads instead of the pool's own offsets.
// Each set is written by at most its winner in a call and a span reads only a
// set it won, so no block a call reads is overwritten during it; results do
// not depend on where a block was read from.
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

constexpr int kResSlotsPerHead = 64;   // workgroups per KV head in the fetch

__device__ __forceinline__ uint64_t res_mix(uint64_t x) {
  // splitmix64 finalizer (Steele, Lea and Flood, 2014)
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

__device__ __forceinline__ uint64_t res_bid(uint64_t epoch, bool holds, uint64_t key) {
  return (epoch << (kResKeyBits + 1)) | ((uint64_t)holds << kResKeyBits) | (kResKeyMask - key);
}

// the two candidate sets of a block (distinct when there are two sets or more)
__device__ __forceinline__ void res_sets(uint64_t key, uint64_t n_sets, uint64_t& s1,
                                         uint64_t& s2) {
  const uint64_t h = res_mix(key);
  s1 = h % n_sets;
  s2 = n_sets > 1 ? (s1 + 1 + (res_mix(h) % (n_sets - 1))) % n_sets : s1;
}

__global__ __launch_bounds__(256) void res_claim_kernel(
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ rank, int sc, int scs,
    int layer, int hkv, uint64_t slot_floats, uint64_t n_sets, uint64_t epoch,
    const long long* __restrict__ tag, unsigned long long* __restrict__ claim) {
  const int g = blockIdx.y;
  const int nu = ucount[g];
  for (int u = blockIdx.x * 256 + threadIdx.x; u < nu; u += gridDim.x * 256) {
    const int j = ulist[(size_t)g * sc + u];
    const FactorView fv = FactorView::packed(rank[(size_t)g * scs + j], clen[j]);
    if (fv.block_floats() > slot_floats) continue;
    const uint64_t key = ((uint64_t)layer * hkv + g) * (uint64_t)sc + j;
    uint64_t s1, s2;
    res_sets(key, n_sets, s1, s2);
    atomicMax(&claim[s1], (unsigned long long)res_bid(epoch, tag[s1] == (long long)key, key));
    if (s2 != s1)
      atomicMax(&claim[s2], (unsigned long long)res_bid(epoch, tag[s2] == (long long)key, key));
  }
}

__global__ __launch_bounds__(256) void res_fetch_kernel(
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ rank,
    const uint64_t* __restrict__ fac_off, uint64_t layer_base, int sc, int scs, int layer,
    int hkv,
    uint64_t slot_floats, uint64_t n_sets, uint64_t epoch,
    const unsigned long long* __restrict__ claim, long long* __restrict__ tag,
    const float* __restrict__ host, float* __restrict__ arena, uint64_t slots_off,
    uint64_t* __restrict__ off_out, unsigned long long* __restrict__ stats) {
  const int g = blockIdx.y;
  const int nu = ucount[g];
  for (int u = blockIdx.x; u < nu; u += kResSlotsPerHead) {
    const int j = ulist[(size_t)g * sc + u];
    const FactorView fv = FactorView::packed(rank[(size_t)g * scs + j], clen[j]);
    const uint64_t nfl = fv.block_floats();
    const uint64_t hoff = fac_off[(size_t)g * scs + j];
    const uint64_t key = ((uint64_t)layer * hkv + g) * (uint64_t)sc + j;
    uint64_t dst_off = hoff - layer_base;   // the layer's staging (arena start)
    bool copy = true, hit = false, cached = false;
    uint64_t set = 0;
    if (nfl <= slot_floats) {
      uint64_t s1, s2;
      res_sets(key, n_sets, s1, s2);
      const bool h1 = tag[s1] == (long long)key, h2 = tag[s2] == (long long)key;
      const bool w1 = claim[s1] == res_bid(epoch, h1, key);
      const bool w2 = s2 != s1 && claim[s2] == res_bid(epoch, h2, key);
      if ((w1 && h1) || (w2 && h2)) {
        set = (w1 && h1) ? s1 : s2;
        hit = true;
      } else if (w1 || w2) {
        set = w1 ? s1 : s2;
      }
      if (w1 || w2) {
        cached = true;
        dst_off = slots_off + set * slot_floats;
        copy = !hit;
      }
    }
    if (copy) {
      const uint4* src = (const uint4*)(host + hoff);
      uint4* dst = (uint4*)(arena + dst_off);
      const int nvec = (int)(nfl / 4);
      for (int k = threadIdx.x; k < nvec; k += 256) dst[k] = src[k];
    }
    // every lane has read the tag before it changes
    __syncthreads();
    if (threadIdx.x == 0) {
      off_out[(size_t)g * scs + j] = dst_off;
      if (cached && !hit) tag[set] = (long long)key;
      const unsigned long long bytes = (unsigned long long)fv.alg_bytes();
      atomicAdd(&stats[hit ? 0 : 1], 1ull);
      atomicAdd(&stats[hit ? 2 : 3], bytes);
    }
  }
}

}  // namespace

hipError_t launch_resident_fetch(const LayerGeom& g, int layer, const int32_t* ulist,
                                 const int32_t* ucount, const int32_t* clen, const int32_t* rank,
                                 const uint64_t* fac_off, uint64_t layer_base,
                                 const float* host_pool_mapped, const ResidencyView& rv,
                                 uint64_t epoch, hipStream_t st) {
  if (g.n_compressed == 0) return hipSuccess;
  const int sc = g.n_compressed, hkv = g.n_kv_heads;
  const int cx = (sc + 255) / 256;
  hipLaunchKernelGGL(res_claim_kernel, dim3(cx < 64 ? cx : 64, hkv), dim3(256), 0, st, ulist,
                     ucount, clen, rank, sc, g.sc_stride, layer, hkv, rv.slot_floats, rv.n_sets,
                     epoch, rv.tag, rv.claim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(res_fetch_kernel, dim3(kResSlotsPerHead, hkv), dim3(256), 0, st, ulist,
                     ucount, clen, rank, fac_off, layer_base, sc, g.sc_stride, layer, hkv,
                     rv.slot_floats,
                     rv.n_sets, epoch, rv.claim, rv.tag, host_pool_mapped, rv.arena,
                     rv.slots_off, rv.off, rv.stats);
  return hipGetLastError();
}

}  // namespace sekv
