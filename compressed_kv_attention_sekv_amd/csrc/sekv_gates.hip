// Soft-gated span factors (gfx950): the gated reconstruction of Eq. 8,
// K^ = U diag(g * sigma) V^T, applied to a built cache's factor pool.
//
// SeKV paper Sec. 3.2 (low-rank paragraph) and Eq. 8: every singular
// component of a span carries a gate in [0, 1]; components with negligible
// gates are not stored.  The key and the value matrix of a span have gates of
// their own, so each keeps its own rank.  The host decides, per (layer, KV
// head, span) and per matrix, which of the stored components stay (gate >=
// eps, at least one: the largest gate) and lays out a new pool; this kernel
// repacks each block into it: rows of V^T and columns of U of the kept
// components, in their order, and sigma scaled by the gate.  Padding stays
// zero.
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

constexpr int kGateThreads = 256;

__global__ __launch_bounds__(kGateThreads) void gate_repack_kernel(
    const float* __restrict__ old_pool, const uint64_t* __restrict__ old_off,
    const int32_t* __restrict__ old_rank, float* __restrict__ new_pool,
    const uint64_t* __restrict__ new_off, const int32_t* __restrict__ new_rank,
    const uint8_t* __restrict__ kept, const float* __restrict__ key_gates,
    const float* __restrict__ value_gates, const int32_t* __restrict__ clen, int sc, int scs,
    int max_rank, uint64_t n_blocks) {
  // block b = lg * scs + j of the tables; the gates are laid out [lg][sc][R]
  const uint64_t b = blockIdx.x;
  if (b >= n_blocks) return;
  const uint64_t lg = b / (uint64_t)scs;
  const int j = (int)(b % (uint64_t)scs);
  if (j >= sc) return;
  const uint64_t gi = lg * (uint64_t)sc + j;
  const int n = clen[j];
  const FactorView fo = FactorView::packed(old_rank[b], n);
  const FactorView fn = FactorView::packed(new_rank[b], n);
  const float* src = old_pool + old_off[b];
  float* dst = new_pool + new_off[b];
  for (int kv = 0; kv < 2; ++kv) {
    const uint8_t* kp = kept + (b * 2 + kv) * (uint64_t)max_rank;
    const float* gb = (kv ? value_gates : key_gates) + gi * (uint64_t)max_rank;
    const int nr = fn.r(kv), nr4 = fn.r4(kv), or4 = fo.r4(kv);
    // V^T rows of the kept components
    for (int e = threadIdx.x; e < nr * kHeadDim; e += kGateThreads) {
      const int i = e / kHeadDim, c = e % kHeadDim;
      dst[fn.vt(kv) + e] = src[fo.vt(kv) + (size_t)kp[i] * kHeadDim + c];
    }
    // U, token-major: row t holds the kept components' coefficients
    for (int e = threadIdx.x; e < n * nr; e += kGateThreads) {
      const int t = e / nr, i = e % nr;
      dst[fn.u(kv) + (size_t)t * nr4 + i] = src[fo.u(kv) + (size_t)t * or4 + kp[i]];
    }
    // sigma scaled by the gate
    for (int i = threadIdx.x; i < nr; i += kGateThreads)
      dst[fn.sigma(kv) + i] = gb[kp[i]] * src[fo.sigma(kv) + kp[i]];
  }
}

}  // namespace

hipError_t launch_gate_repack(const float* old_pool, const uint64_t* old_off,
                              const int32_t* old_rank, float* new_pool, const uint64_t* new_off,
                              const int32_t* new_rank, const uint8_t* kept, const float* key_gates,
                              const float* value_gates, const int32_t* clen, int sc, int scs,
                              int max_rank, uint64_t n_blocks, hipStream_t st) {
  if (n_blocks == 0 || sc == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_repack_kernel, dim3((unsigned)n_blocks), dim3(kGateThreads), 0, st,
                     old_pool, old_off, old_rank, new_pool, new_off, new_rank, kept, key_gates,
                     value_gates, clen, sc, scs, max_rank, n_blocks);
  return hipGetLastError();
}

}  // namespace sekv
