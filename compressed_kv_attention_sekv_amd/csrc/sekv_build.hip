// Build-side kernels of the SeKV cache (gfx950): surprisal statistics and
// span table, full-resolution gather, span means and routing summaries, and
// the per-span truncated SVD of keys and values.
//
// SeKV paper Sec. 3.1 (segmentation) and Sec. 3.2 (dual-resolution store).
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {

// ---------------------------------------------------------------------------
// block-wide exclusive scan of one int per thread (wave64 shuffles + LDS)
// ---------------------------------------------------------------------------
template <int NT>
__device__ int block_exclusive_scan(int v, int* total, int* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = (lane < NT / 64) ? lds[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < NT / 64) lds[lane] = w;
  }
  __syncthreads();
  const int base = wid ? lds[wid - 1] : 0;
  *total = lds[NT / 64 - 1];
  __syncthreads();
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Segmentation (Sec. 3.1): one workgroup of 1024 threads, each owning a
// contiguous chunk of positions, so every list comes out ascending.
// mean and population std in float64 (two passes, fixed tree order);
// anchor(t) = t < N - window && s_t > mean + alpha * std.
// ---------------------------------------------------------------------------
constexpr int kSegThreads = 1024;

__global__ __launch_bounds__(kSegThreads) void segment_kernel(const float* __restrict__ s, int n,
                                                              int window, double alpha,
                                                              int min_len, SegOut o) {
  __shared__ double red[kSegThreads];
  __shared__ int scan_lds[kSegThreads / 64];
  const int tid = threadIdx.x;

  const int chunk = (n + kSegThreads - 1) / kSegThreads;
  const int t0 = min(n, tid * chunk), t1 = min(n, t0 + chunk);

  double acc = 0.0;
  for (int t = t0; t < t1; ++t) acc += (double)s[t];
  red[tid] = acc;
  __syncthreads();
  for (int w = kSegThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double mu = red[0] / (double)n;
  __syncthreads();
  acc = 0.0;
  for (int t = t0; t < t1; ++t) {
    const double dv = (double)s[t] - mu;
    acc += dv * dv;
  }
  red[tid] = acc;
  __syncthreads();
  for (int w = kSegThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double sigma = sqrt(red[0] / (double)n);
  const double thr = mu + alpha * sigma;
  const int limit = max(n - window, 0);

  auto anchor = [&](int t) -> bool { return t < limit && (double)s[t] > thr; };

  // anchors, run starts and run ends, each ascending
  // a run may start in one thread's chunk and end in another's, so starts
  // and ends get separate offsets
  int na = 0, ns = 0, ne = 0;
  for (int t = t0; t < t1; ++t) {
    if (t >= limit) break;
    const bool a = anchor(t);
    na += a;
    if (!a && (t == 0 || anchor(t - 1))) ns++;
    if (!a && (t == limit - 1 || anchor(t + 1))) ne++;
  }
  int tot_a, tot_s, tot_e;
  const int off_a = block_exclusive_scan<kSegThreads>(na, &tot_a, scan_lds);
  const int off_s = block_exclusive_scan<kSegThreads>(ns, &tot_s, scan_lds);
  const int off_e = block_exclusive_scan<kSegThreads>(ne, &tot_e, scan_lds);
  {
    int ia = off_a, is = off_s, ie = off_e;
    for (int t = t0; t < t1; ++t) {
      if (t >= limit) break;
      const bool a = anchor(t);
      if (a) {
        o.anchors[ia++] = t;
        continue;
      }
      if (t == 0 || anchor(t - 1)) o.span_start[is++] = t;
      if (t == limit - 1 || anchor(t + 1)) o.span_len[ie++] = t;  // end position for now
    }
  }
  __syncthreads();
  const int n_spans = tot_s;
  const int schunk = (n_spans + kSegThreads - 1) / kSegThreads;
  const int j0 = min(n_spans, tid * schunk), j1 = min(n_spans, j0 + schunk);
  int nc = 0;
  for (int j = j0; j < j1; ++j) {
    const int len = o.span_len[j] - o.span_start[j] + 1;
    o.span_len[j] = len;
    const int k = len >= min_len ? 0 : 1;
    o.kind[j] = (uint8_t)k;
    nc += (k == 0);
  }
  int tot_c;
  const int off_c = block_exclusive_scan<kSegThreads>(nc, &tot_c, scan_lds);
  {
    int ic = off_c;
    for (int j = j0; j < j1; ++j) {
      if (o.kind[j] == 0) {
        o.cspan[ic] = j;
        o.cstart[ic] = o.span_start[j];
        o.clen[ic] = o.span_len[j];
        ++ic;
      }
    }
  }
  // full-resolution set: window, anchors and the tokens of short spans
  for (int t = t0; t < t1; ++t) o.flag[t] = (uint8_t)(t >= limit || anchor(t));
  __syncthreads();
  for (int j = j0; j < j1; ++j) {
    if (o.kind[j] == 1) {
      const int b = o.span_start[j], len = o.span_len[j];
      for (int t = b; t < b + len; ++t) o.flag[t] = 1;
    }
  }
  __syncthreads();
  int nd = 0;
  for (int t = t0; t < t1; ++t) nd += o.flag[t];
  int tot_d;
  const int off_d = block_exclusive_scan<kSegThreads>(nd, &tot_d, scan_lds);
  {
    int id = off_d;
    for (int t = t0; t < t1; ++t)
      if (o.flag[t]) o.dense_pos[id++] = t;
  }
  if (tid == 0) {
    o.stats[0] = mu;
    o.stats[1] = sigma;
    o.stats[2] = thr;
    o.counts[0] = tot_a;
    o.counts[1] = n_spans;
    o.counts[2] = tot_c;
    o.counts[3] = tot_d;
  }
}

hipError_t launch_segment(const float* s, int n, int window, double alpha, int min_len,
                          const SegOut& o, hipStream_t st) {
  hipLaunchKernelGGL(segment_kernel, dim3(1), dim3(kSegThreads), 0, st, s, n, window, alpha,
                     min_len, o);
  return hipGetLastError();
}

// ln n_j of each compressed span: float64 for the router, float32 for attention
__global__ void log_len_kernel(const int32_t* clen, int sc, double* lnn64, float* lnn32) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= sc) return;
  const double v = log((double)clen[j]);
  lnn64[j] = v;
  lnn32[j] = (float)v;
}

hipError_t launch_log_len(const int32_t* clen, int sc, double* lnn64, float* lnn32,
                          hipStream_t st) {
  if (sc == 0) return hipSuccess;
  hipLaunchKernelGGL(log_len_kernel, dim3((sc + 255) / 256), dim3(256), 0, st, clen, sc, lnn64,
                     lnn32);
  return hipGetLastError();
}

// retained rank r_j = min(max(requested, 1), n_j, d, R) of spans j0 .. j0 + n - 1
// (the request is that of the span's first row of rank_by_pos)
__global__ void span_rank_kernel(const int32_t* rank_by_pos, const int32_t* cstart,
                                 const int32_t* clen, int n_tokens, int j0, int n, int stride,
                                 int max_rank, int32_t* rank) {
  const int j = j0 + (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int lg = blockIdx.y;
  if (j >= j0 + n) return;
  int r = rank_by_pos ? rank_by_pos[(size_t)lg * n_tokens + cstart[j]] : max_rank;
  r = max(r, 1);
  r = min(r, clen[j]);
  r = min(r, kHeadDim);
  r = min(r, max_rank);
  rank[(size_t)lg * stride + j] = pack_ranks(r, r);   // keys and values alike
}

hipError_t launch_span_rank(const int32_t* rank_by_pos, const int32_t* cstart,
                            const int32_t* clen, int n_tokens, int j0, int n, int stride,
                            int n_lg, int max_rank, int32_t* rank, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(span_rank_kernel, dim3((n + 255) / 256, n_lg), dim3(256), 0, st,
                     rank_by_pos, cstart, clen, n_tokens, j0, n, stride, max_rank, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Full-resolution gather: rows of the window, anchors and short spans into a
// contiguous [L][Hkv][D][d] block, 16-byte vectors.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          int n_tokens, const int32_t* pos,
                                                          int n_rows, int dst_stride,
                                                          int vec_per_row,
                                                          uint4* __restrict__ dst) {
  const int lg = blockIdx.y;
  const int rows_per_block = 256 / vec_per_row;
  const int r = blockIdx.x * rows_per_block + threadIdx.x / vec_per_row;
  const int c = threadIdx.x % vec_per_row;
  if (r >= n_rows || threadIdx.x >= rows_per_block * vec_per_row) return;
  const size_t s_off = ((size_t)lg * n_tokens + pos[r]) * vec_per_row + c;
  const size_t d_off = ((size_t)lg * dst_stride + r) * vec_per_row + c;
  dst[d_off] = src[s_off];
}

hipError_t launch_gather_dense(int bf16, const void* src, int n_tokens, const int32_t* pos,
                               int n_dense, int dst_stride, int n_lg, void* dst, hipStream_t st) {
  if (n_dense == 0) return hipSuccess;
  const int vec = bf16 ? kHeadDim * 2 / 16 : kHeadDim * 4 / 16;
  const int rows = 256 / vec;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((n_dense + rows - 1) / rows, n_lg), dim3(256), 0,
                     st, (const uint4*)src, n_tokens, pos, n_dense, dst_stride, vec, (uint4*)dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Span means and summaries (Sec. 3.2): one workgroup per (compressed span,
// layer x KV head), one thread per head dimension.  Weights, means and the
// projections are float64; each stored value is rounded once.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kHeadDim) void span_summarize_kernel(
    const float* __restrict__ s, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ w_route, int n_tokens, const int32_t* __restrict__ cstart,
    const int32_t* __restrict__ clen, int j0, int sc, int hkv, int group, int dr,
    T* __restrict__ kbar,
    T* __restrict__ vbar, T* __restrict__ summ) {
  __shared__ double km_sh[kHeadDim];
  const int j = j0 + (int)blockIdx.x, lg = blockIdx.y;
  const int layer = lg / hkv, g = lg % hkv;
  const int dim = threadIdx.x;
  const int b = cstart[j], n = clen[j];

  double tot = 0.0;
  for (int t = 0; t < n; ++t) tot += (double)s[b + t];
  const T* kr = k + ((size_t)lg * n_tokens + b) * kHeadDim + dim;
  const T* vr = v + ((size_t)lg * n_tokens + b) * kHeadDim + dim;
  double km = 0.0, vm = 0.0;
  for (int t = 0; t < n; ++t) {
    const double w = (tot == 0.0) ? 1.0 / (double)n : (double)s[b + t] / tot;
    km += w * (double)Store<T>::load(kr + (size_t)t * kHeadDim);
    vm += w * (double)Store<T>::load(vr + (size_t)t * kHeadDim);
  }
  const size_t m_off = ((size_t)lg * sc + j) * kHeadDim + dim;
  kbar[m_off] = Store<T>::from_f64(km);
  vbar[m_off] = Store<T>::from_f64(vm);
  km_sh[dim] = km;
  __syncthreads();
  const int hq = hkv * group;
  for (int o = dim; o < group * dr; o += kHeadDim) {
    const int hl = o / dr, i = o % dr;
    const int h = g * group + hl;
    const float* wr = w_route + (((size_t)layer * hq + h) * dr + i) * kHeadDim;
    double acc = 0.0;
    for (int c = 0; c < kHeadDim; ++c) acc += (double)wr[c] * km_sh[c];
    summ[(((size_t)layer * hq + h) * sc + j) * dr + i] = Store<T>::from_f64(acc);
  }
}

hipError_t launch_span_summarize(int bf16, const float* s, const void* k, const void* v,
                                 const float* w_route, int n_tokens, const int32_t* cstart,
                                 const int32_t* clen, int j0, int n, int sc, int n_layers,
                                 int hkv, int group, int dr, void* kbar, void* vbar, void* summ,
                                 hipStream_t st) {
  if (n == 0) return hipSuccess;
  dim3 grid(n, n_layers * hkv);
  if (bf16)
    hipLaunchKernelGGL(span_summarize_kernel<uint16_t>, grid, dim3(kHeadDim), 0, st, s,
                       (const uint16_t*)k, (const uint16_t*)v, w_route, n_tokens, cstart, clen,
                       j0, sc, hkv, group, dr, (uint16_t*)kbar, (uint16_t*)vbar, (uint16_t*)summ);
  else
    hipLaunchKernelGGL(span_summarize_kernel<float>, grid, dim3(kHeadDim), 0, st, s,
                       (const float*)k, (const float*)v, w_route, n_tokens, cstart, clen, j0,
                       sc, hkv, group, dr, (float*)kbar, (float*)vbar, (float*)summ);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Window append support.
//
// gather_words: dst[lg][r] = src[lg][pos[r]] for 32-bit words (surprisal or
// requested rank of each full-resolution row).
// compact_rows: remove sorted, disjoint row ranges [a_i, a_i + n_i) from rows
// [0, n_rows) of every (layer, KV head) block (one workgroup each), moving the
// rows after them down.  Rows only move to lower indices, so a workgroup that
// reads a chunk of rows, waits, then writes it never overwrites a row of a
// later chunk before reading it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_words_kernel(const uint32_t* __restrict__ src,
                                                           int src_stride, const int32_t* pos,
                                                           int n, int dst_stride,
                                                           uint32_t* __restrict__ dst) {
  const int lg = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < n) dst[(size_t)lg * dst_stride + r] = src[(size_t)lg * src_stride + pos[r]];
}

hipError_t launch_gather_words(const uint32_t* src, int src_stride, const int32_t* pos, int n,
                               int dst_stride, int n_lg, uint32_t* dst, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_words_kernel, dim3((n + 255) / 256, n_lg), dim3(256), 0, st, src,
                     src_stride, pos, n, dst_stride, dst);
  return hipGetLastError();
}

template <typename E>
__global__ __launch_bounds__(256) void compact_rows_kernel(E* __restrict__ base, int stride,
                                                           int elems_per_row, int n_rows,
                                                           const int32_t* __restrict__ ranges,
                                                           int n_ranges) {
  constexpr int kUnroll = 4;
  E* rows = base + (size_t)blockIdx.x * stride * elems_per_row;
  const int rows_per_pass = 256 / elems_per_row;
  const int first = ranges[0];
  for (int r0 = first; r0 < n_rows; r0 += rows_per_pass * kUnroll) {
    E val[kUnroll];
    int dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = threadIdx.x;
      const int r = r0 + (u * rows_per_pass) + t / elems_per_row;
      const int e = t % elems_per_row;
      dst[u] = -1;
      if (t < rows_per_pass * elems_per_row && r < n_rows) {
        int removed = 0;
        bool gone = false;
        for (int i = 0; i < n_ranges; ++i) {
          const int a = ranges[2 * i], len = ranges[2 * i + 1];
          if (r >= a + len) removed += len;
          else if (r >= a) gone = true;
        }
        if (!gone) {
          val[u] = rows[(size_t)r * elems_per_row + e];
          dst[u] = (r - removed) * elems_per_row + e;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) rows[dst[u]] = val[u];
    __syncthreads();
  }
}

hipError_t launch_compact_rows(void* base, int elem_bytes, int stride, int elems_per_row,
                               int n_rows, int n_lg, const int32_t* ranges, int n_ranges,
                               hipStream_t st) {
  if (n_ranges == 0 || n_lg == 0) return hipSuccess;
  if (elems_per_row < 1 || elems_per_row > 256) return hipErrorInvalidValue;
  if (elem_bytes == 16)
    hipLaunchKernelGGL(compact_rows_kernel<uint4>, dim3(n_lg), dim3(256), 0, st, (uint4*)base,
                       stride, elems_per_row, n_rows, ranges, n_ranges);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(compact_rows_kernel<uint32_t>, dim3(n_lg), dim3(256), 0, st,
                       (uint32_t*)base, stride, elems_per_row, n_rows, ranges, n_ranges);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-span truncated SVD (Sec. 3.2 low-rank paragraph; hard gates on Eq. 8).
//
// One workgroup per (span, layer x KV head).  With X the span's n x d token
// matrix and m = min(n, d), the m x m Gram matrix (X X^T if n <= d, else
// X^T X) is formed in float64 and diagonalised by one-sided Jacobi
// (Hestenes): column pairs are rotated until every pair is orthogonal to
// working precision, pairs scheduled by the round-robin (circle) method so
// the m/2 rotations of a round are independent.  The converged columns are
// lambda_i e_i with lambda_i = sigma_i^2; the top r by norm are kept and the
// other singular vectors come from X itself (v = X^T u / sigma or
// u = X v / sigma).
// ---------------------------------------------------------------------------
constexpr int kSvdThreads = 256;
constexpr int kSvdMaxSweeps = 30;
constexpr double kSvdTol = 1e-14;

__device__ __forceinline__ float load_as_float(const float* p) { return *p; }
__device__ __forceinline__ float load_as_float(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ int rr_player(int pos, int round, int me) {
  return pos == 0 ? 0 : ((pos - 1 + round) % (me - 1)) + 1;
}

template <typename T, int MAXM>
__global__ __launch_bounds__(kSvdThreads) void span_svd_kernel(
    const T* __restrict__ x, int n_tokens, const int32_t* __restrict__ cstart,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ span_ids, int sc,
    const int32_t* __restrict__ rank, const uint64_t* __restrict__ fac_off,
    float* __restrict__ pool, int which) {
  constexpr int TPP = 512 / MAXM;             // threads per column pair
  constexpr int KPT = (MAXM + TPP - 1) / TPP;  // column entries per thread
  constexpr int NT4 = MAXM / 4;                // Gram register tiles per side
  constexpr int TILES = (NT4 * NT4 + kSvdThreads - 1) / kSvdThreads;
  constexpr int KC = 32;                       // staged summation chunk
  extern __shared__ double smem[];
  __shared__ double sh_lmax;

  const int tid = threadIdx.x;
  const int j = span_ids[blockIdx.x];
  const int lg = blockIdx.y;
  const int b = cstart[j], n = clen[j];
  const int32_t ranks = rank[(size_t)lg * sc + j];
  const int r = rank_of(ranks, which);
  const bool small = n <= kHeadDim;
  const int m = small ? n : kHeadDim;
  const int me = m + (m & 1);
  const int ld = me + 1;
  double* A = smem;                           // column c at A + c * ld
  double* nrm = smem + (size_t)me * ld;
  int* order = (int*)(nrm + me);
  float* Y = (float*)smem;                    // staging [KC][MAXM], aliases A during the Gram
  const T* X = x + ((size_t)lg * n_tokens + b) * kHeadDim;

  // ---- Gram matrix, float64 accumulation in registers -------------------
  double acc[TILES][16];
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[tt][e] = 0.0;
  const int ksum = small ? kHeadDim : n;      // summation length
  const int nt4 = (me + 3) / 4;
  for (int k0 = 0; k0 < ksum; k0 += KC) {
    const int kc = min(KC, ksum - k0);
    __syncthreads();
    for (int idx = tid; idx < KC * MAXM; idx += kSvdThreads) {
      const int kk = idx / MAXM, c = idx % MAXM;
      float val = 0.f;
      if (kk < kc && c < m)
        val = small ? load_as_float(X + (size_t)c * kHeadDim + k0 + kk)
                    : load_as_float(X + (size_t)(k0 + kk) * kHeadDim + c);
      Y[kk * MAXM + c] = val;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      const int tile = tid + tt * kSvdThreads;
      if (tile >= nt4 * nt4) continue;
      const int p0 = (tile / nt4) * 4, q0 = (tile % nt4) * 4;
      for (int kk = 0; kk < kc; ++kk) {
        const float4 yp = *(const float4*)(Y + kk * MAXM + p0);
        const float4 yq = *(const float4*)(Y + kk * MAXM + q0);
        const double pv[4] = {yp.x, yp.y, yp.z, yp.w};
        const double qv[4] = {yq.x, yq.y, yq.z, yq.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[tt][a * 4 + c] += pv[a] * qv[c];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) {
    const int tile = tid + tt * kSvdThreads;
    if (tile >= nt4 * nt4) continue;
    const int p0 = (tile / nt4) * 4, q0 = (tile % nt4) * 4;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = p0 + a, q = q0 + c;
        if (p < me && q < me) A[(size_t)q * ld + p] = (p < m && q < m) ? acc[tt][a * 4 + c] : 0.0;
      }
  }
  __syncthreads();

  // ---- one-sided Jacobi sweeps ------------------------------------------
  const int npairs = me / 2;
  const int pid = tid / TPP, sub = tid % TPP;
  const bool active = pid < npairs;
  for (int sweep = 0; sweep < kSvdMaxSweeps; ++sweep) {
    int rotated = 0;
    for (int round = 0; round < me - 1; ++round) {
      if (active) {
        const int p = rr_player(pid, round, me);
        const int q = rr_player(me - 1 - pid, round, me);
        double* ap = A + (size_t)p * ld;
        double* aq = A + (size_t)q * ld;
        double xp[KPT], xq[KPT];
        double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const int kk = sub + i * TPP;
          xp[i] = kk < m ? ap[kk] : 0.0;
          xq[i] = kk < m ? aq[kk] : 0.0;
          al += xp[i] * xp[i];
          be += xq[i] * xq[i];
          ga += xp[i] * xq[i];
        }
#pragma unroll
        for (int o = 1; o < TPP; o <<= 1) {
          al += __shfl_xor(al, o, 64);
          be += __shfl_xor(be, o, 64);
          ga += __shfl_xor(ga, o, 64);
        }
        if (fabs(ga) > kSvdTol * sqrt(al) * sqrt(be)) {
          const double zeta = (be - al) / (2.0 * ga);
          const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          const double c = 1.0 / sqrt(1.0 + t * t);
          const double sn = c * t;
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            const int kk = sub + i * TPP;
            if (kk < m) {
              ap[kk] = c * xp[i] - sn * xq[i];
              aq[kk] = sn * xp[i] + c * xq[i];
            }
          }
          rotated = 1;
        }
      }
      __syncthreads();
    }
    if (!__syncthreads_or(rotated)) break;
  }

  // ---- order the components by lambda = column norm ----------------------
  for (int c = tid; c < me; c += kSvdThreads) {
    double s2 = 0.0;
    const double* ac = A + (size_t)c * ld;
    for (int kk = 0; kk < m; ++kk) s2 += ac[kk] * ac[kk];
    nrm[c] = sqrt(s2);
  }
  __syncthreads();
  for (int c = tid; c < me; c += kSvdThreads) {
    int pos = 0;
    const double v = nrm[c];
    for (int o = 0; o < me; ++o) pos += (nrm[o] > v) || (nrm[o] == v && o < c);
    order[pos] = c;
  }
  __syncthreads();
  if (tid == 0) sh_lmax = nrm[order[0]];
  __syncthreads();
  const double lmax = sh_lmax;

  // ---- write the factors ---------------------------------------------------
  const FactorView fv = FactorView::packed(ranks, n);
  const int r4 = fv.r4(which);
  float* blk = pool + fac_off[(size_t)lg * sc + j];
  float* vt = blk + fv.vt(which);
  float* u = blk + fv.u(which);
  float* sg = blk + fv.sigma(which);
  auto live = [&](int i) -> bool {
    const double lam = nrm[order[i]];
    return lam > 0.0 && lam > lmax * 1e-24;
  };
  for (int i = tid; i < r4; i += kSvdThreads)
    sg[i] = (i < r && live(i)) ? (float)sqrt(nrm[order[i]]) : 0.f;
  if (small) {
    // u_i = A[:,p] / lambda (token space); v_i = X^T u_i / sigma
    for (int idx = tid; idx < n * r4; idx += kSvdThreads) {
      const int t = idx / r4, i = idx % r4;
      float val = 0.f;
      if (i < r && live(i)) val = (float)(A[(size_t)order[i] * ld + t] / nrm[order[i]]);
      u[idx] = val;
    }
    for (int idx = tid; idx < r * kHeadDim; idx += kSvdThreads) {
      const int i = idx / kHeadDim, c = idx % kHeadDim;
      float val = 0.f;
      if (live(i)) {
        const double lam = nrm[order[i]];
        const double* ac = A + (size_t)order[i] * ld;
        double sacc = 0.0;
        for (int t = 0; t < n; ++t) sacc += (double)load_as_float(X + (size_t)t * kHeadDim + c) * ac[t];
        val = (float)(sacc / (lam * sqrt(lam)));
      }
      vt[idx] = val;
    }
  } else {
    // v_i = A[:,p] / lambda (head-dim space); u_i = X v_i / sigma
    for (int idx = tid; idx < r * kHeadDim; idx += kSvdThreads) {
      const int i = idx / kHeadDim, c = idx % kHeadDim;
      float val = 0.f;
      if (live(i)) val = (float)(A[(size_t)order[i] * ld + c] / nrm[order[i]]);
      vt[idx] = val;
    }
    for (int idx = tid; idx < n * r4; idx += kSvdThreads) {
      const int t = idx / r4, i = idx % r4;
      float val = 0.f;
      if (i < r && live(i)) {
        const double lam = nrm[order[i]];
        const double* ac = A + (size_t)order[i] * ld;
        const T* xr = X + (size_t)t * kHeadDim;
        double sacc = 0.0;
        for (int c = 0; c < kHeadDim; ++c) sacc += (double)load_as_float(xr + c) * ac[c];
        val = (float)(sacc / (lam * sqrt(lam)));
      }
      u[idx] = val;
    }
  }
}

template <int MAXM>
static size_t svd_lds_bytes() {
  const int me = MAXM;
  const size_t a = (size_t)me * (me + 1) * sizeof(double);
  const size_t y = (size_t)32 * MAXM * sizeof(float);
  return (a > y ? a : y) + (size_t)me * sizeof(double) + (size_t)me * sizeof(int);
}

template <typename T, int MAXM>
static hipError_t launch_svd_t(const T* x, int n_tokens, const int32_t* cstart,
                               const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                               int n_lg, const int32_t* rank, const uint64_t* fac_off,
                               float* pool, int which, hipStream_t st) {
  const size_t lds = svd_lds_bytes<MAXM>();
  hipError_t e = hipFuncSetAttribute((const void*)span_svd_kernel<T, MAXM>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((span_svd_kernel<T, MAXM>), dim3(n_ids, n_lg), dim3(kSvdThreads), lds, st,
                     x, n_tokens, cstart, clen, span_ids, sc, rank, fac_off, pool, which);
  return hipGetLastError();
}

hipError_t launch_span_svd(int bf16, const void* x, int n_tokens, const int32_t* cstart,
                           const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                           int n_lg, const int32_t* rank, const uint64_t* fac_off, float* pool,
                           int which, int max_m, hipStream_t st) {
  if (n_ids == 0) return hipSuccess;
#define SEKV_SVD_DISPATCH(M)                                                                   \
  return bf16 ? launch_svd_t<uint16_t, M>((const uint16_t*)x, n_tokens, cstart, clen, span_ids, \
                                          n_ids, sc, n_lg, rank, fac_off, pool, which, st)     \
              : launch_svd_t<float, M>((const float*)x, n_tokens, cstart, clen, span_ids,      \
                                       n_ids, sc, n_lg, rank, fac_off, pool, which, st)
  if (max_m <= 32) { SEKV_SVD_DISPATCH(32); }
  if (max_m <= 64) { SEKV_SVD_DISPATCH(64); }
  SEKV_SVD_DISPATCH(128);
#undef SEKV_SVD_DISPATCH
}

}  // namespace sekv
