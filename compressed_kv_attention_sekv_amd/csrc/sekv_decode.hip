// Decode-step kernels of the SeKV cache (gfx950): router with ordered
// compaction, split-K attention over full-resolution rows and coarse span
// entries, factored attention over zoomed spans, and the log-sum-exp merge.
//
// SeKV paper Sec. 3.2 (gate) and Sec. 3.3 (Eq. 9 zoom decision; one softmax
// over anchors, window, reconstructed zoomed tokens and coarse entries with a
// length correction).
#include <hip/hip_runtime.h>
#include <math.h>

#include "sekv_internal.h"

namespace sekv {

constexpr int kPartStride = 132;  // per (head, slot): m, l, -, -, acc[128]
constexpr int kTileRows = 256;    // rows (or coarse entries) per attention tile

// ---------------------------------------------------------------------------
// Router.  Grid (chunks of 256 spans, KV heads); each workgroup projects the
// queries of its group's heads (float64), gates its chunk of spans, and
// compacts each head's zoom set and the group union in chunk order into
// scratch.  The last workgroup of a group to finish (ticket counter) copies
// the chunk lists into the ascending output lists and resets the ticket, so
// no launch leaves state behind and no workgroup ever waits.
// ---------------------------------------------------------------------------
constexpr int kRouteChunk = 256;

template <typename T>
__global__ __launch_bounds__(kRouteChunk) void route_kernel(
    const float* __restrict__ q, const float* __restrict__ proj, const float* __restrict__ tau,
    const T* __restrict__ summ, const double* __restrict__ lnn64, double gamma, int sc,
    int group, int dr, int nchunks, uint8_t* __restrict__ mask, double* __restrict__ prob,
    int32_t* __restrict__ list, int32_t* __restrict__ count, int32_t* __restrict__ ulist,
    int32_t* __restrict__ ucount, int32_t* __restrict__ scratch, uint32_t* __restrict__ tickets) {
  __shared__ double qt[kMaxGroup * kMaxRouteDim];
  __shared__ int wcnt[kMaxGroup + 1][kRouteChunk / 64];
  __shared__ int sh_last;
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nl = group + 1;  // lists per group: heads, then the union
  int32_t* scr_list = scratch + (size_t)g * nl * (nchunks * kRouteChunk + nchunks);
  int32_t* scr_cnt = scr_list + (size_t)nl * nchunks * kRouteChunk;

  for (int o = wid; o < group * dr; o += kRouteChunk / 64) {
    const int hl = o / dr, i = o % dr, h = g * group + hl;
    const float* pr = proj + ((size_t)h * dr + i) * kHeadDim;
    const float* qr = q + (size_t)h * kHeadDim;
    double a = (double)pr[lane] * (double)qr[lane] + (double)pr[lane + 64] * (double)qr[lane + 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == 0) qt[hl * dr + i] = a;
  }
  __syncthreads();

  const int j = c * kRouteChunk + tid;
  unsigned bits = 0;
  if (j < sc) {
    const double prior = gamma * lnn64[j];
    for (int hl = 0; hl < group; ++hl) {
      const int h = g * group + hl;
      const T* sr = summ + ((size_t)h * sc + j) * dr;
      double x = 0.0;
      for (int i = 0; i < dr; ++i) x += qt[hl * dr + i] * (double)Store<T>::load(sr + i);
      x += prior;
      const double p = 1.0 / (1.0 + exp(-x));
      const bool z = p > (double)tau[h];
      bits |= (unsigned)z << hl;
      mask[(size_t)h * sc + j] = (uint8_t)z;
      if (prob) prob[(size_t)h * sc + j] = p;
    }
  }
  for (int li = 0; li < nl; ++li) {
    const bool z = (j < sc) && (li < group ? ((bits >> li) & 1u) != 0 : bits != 0);
    const unsigned long long bal = __ballot(z);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[li][wid] = __popcll(bal);
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRouteChunk / 64; ++w) {
      base += (w < wid) ? wcnt[li][w] : 0;
      total += wcnt[li][w];
    }
    if (z) scr_list[((size_t)li * nchunks + c) * kRouteChunk + base + before] = j;
    if (tid == 0) scr_cnt[c * nl + li] = total;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&tickets[g], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = (prev == (unsigned)(nchunks - 1));
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  for (int li = 0; li < nl; ++li) {
    int32_t* dst = li < group ? list + (size_t)(g * group + li) * sc : ulist + (size_t)g * sc;
    int base = 0;
    for (int cc = 0; cc < nchunks; ++cc) {
      const int cnt = __hip_atomic_load(&scr_cnt[cc * nl + li], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      const int32_t* src = scr_list + ((size_t)li * nchunks + cc) * kRouteChunk;
      for (int k = tid; k < cnt; k += kRouteChunk) dst[base + k] = src[k];
      base += cnt;
    }
    if (tid == 0) {
      if (li < group) count[g * group + li] = base;
      else ucount[g] = base;
    }
  }
  if (tid == 0) __hip_atomic_store(&tickets[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_route(int bf16, const DecodeGeom& g, const float* q, const float* proj,
                        const float* tau, const void* summ, const double* lnn64, double gamma,
                        uint8_t* mask, double* prob, int32_t* list, int32_t* count,
                        int32_t* ulist, int32_t* ucount, int32_t* scratch, uint32_t* tickets,
                        hipStream_t st) {
  const int nchunks = (g.n_compressed + kRouteChunk - 1) / kRouteChunk;
  if (nchunks == 0) return hipSuccess;
  dim3 grid(nchunks, g.n_kv_heads);
  if (bf16)
    hipLaunchKernelGGL(route_kernel<uint16_t>, grid, dim3(kRouteChunk), 0, st, q, proj, tau,
                       (const uint16_t*)summ, lnn64, gamma, g.n_compressed, g.group, g.route_dim,
                       nchunks, mask, prob, list, count, ulist, ucount, scratch, tickets);
  else
    hipLaunchKernelGGL(route_kernel<float>, grid, dim3(kRouteChunk), 0, st, q, proj, tau,
                       (const float*)summ, lnn64, gamma, g.n_compressed, g.group, g.route_dim,
                       nchunks, mask, prob, list, count, ulist, ucount, scratch, tickets);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Full-resolution rows and coarse entries.  Grid (tiles, KV heads).  Each
// 16-byte lane load carries EPL elements of one row; LPR lanes cover a row,
// so one wave instruction reads RPW whole rows (1 KB, coalesced).  All G query
// heads of the group share every K/V load.  Each row slot keeps its own
// online-softmax state; slots are combined through LDS at the end.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& raw, float* out);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& raw, float* out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& raw, float* out) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

template <typename T, int G>
__global__ __launch_bounds__(256) void attn_tiles_kernel(
    const float* __restrict__ q, const T* __restrict__ dense_k, const T* __restrict__ dense_v,
    const T* __restrict__ kbar, const T* __restrict__ vbar, const float* __restrict__ lnn32,
    const uint8_t* __restrict__ mask, int n_dense, int sc, int dense_tiles, int n_slots,
    float* __restrict__ part) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPR = kHeadDim / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int UNR = 4;
  constexpr int NSLOT = 4 * RPW;
  __shared__ float red[G][NSLOT][kPartStride];

  const int tile = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sub = lane / LPR, sl = lane % LPR;
  const bool coarse = tile >= dense_tiles;
  int r0, r1;
  const T* K;
  const T* V;
  if (!coarse) {
    r0 = tile * kTileRows;
    r1 = min(n_dense, r0 + kTileRows);
    K = dense_k + (size_t)g * n_dense * kHeadDim;
    V = dense_v + (size_t)g * n_dense * kHeadDim;
  } else {
    r0 = (tile - dense_tiles) * kTileRows;
    r1 = min(sc, r0 + kTileRows);
    K = kbar + (size_t)g * sc * kHeadDim;
    V = vbar + (size_t)g * sc * kHeadDim;
  }
  const float scale = rsqrtf((float)kHeadDim);
  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[h][e] = q[(size_t)(g * G + h) * kHeadDim + sl * EPL + e] * scale;
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  for (int base = r0 + wid * RPW; base < r1; base += 4 * RPW * UNR) {
    uint4 kr[UNR], vr[UNR];
    int row[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      row[u] = base + u * 4 * RPW + sub;
      const int rr = row[u] < r1 ? row[u] : r0;
      kr[u] = *(const uint4*)(K + (size_t)rr * kHeadDim + sl * EPL);
      vr[u] = *(const uint4*)(V + (size_t)rr * kHeadDim + sl * EPL);
    }
    float s[UNR][G];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[EPL];
      unpack16<T>(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d += qv[h][e] * kf[e];
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o, 64);
        s[u][h] = d;
      }
      const bool valid = row[u] < r1;
      float bias = 0.f;
      if (coarse && valid) bias = lnn32[row[u]];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        bool keep = valid;
        if (coarse && valid) keep = mask[(size_t)(g * G + h) * sc + row[u]] == 0;
        s[u][h] = keep ? s[u][h] + bias : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = s[0][h];
#pragma unroll
      for (int u = 1; u < UNR; ++u) bm = fmaxf(bm, s[u][h]);
      const float mn = fmaxf(m[h], bm);
      if (mn == -INFINITY) continue;
      const float corr = __expf(m[h] - mn);
      l[h] *= corr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= corr;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float p = __expf(s[u][h] - mn);
        float vf[EPL];
        unpack16<T>(vr[u], vf);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[e];
      }
      m[h] = mn;
    }
  }

  const int slot = wid * RPW + sub;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[h][slot][4 + sl * EPL + e] = acc[h][e];
    if (sl == 0) {
      red[h][slot][0] = m[h];
      red[h][slot][1] = l[h];
    }
  }
  __syncthreads();
  for (int o = tid; o < G * kHeadDim; o += 256) {
    const int h = o / kHeadDim, dim = o % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int sidx = 0; sidx < NSLOT; ++sidx) M = fmaxf(M, red[h][sidx][0]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int sidx = 0; sidx < NSLOT; ++sidx) {
        const float ms = red[h][sidx][0];
        const float w = ms == -INFINITY ? 0.f : __expf(ms - M);
        L += red[h][sidx][1] * w;
        A += red[h][sidx][4 + dim] * w;
      }
    }
    float* dst = part + ((size_t)(g * G + h) * n_slots + tile) * kPartStride;
    dst[4 + dim] = A;
    if (dim == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

template <typename T>
static hipError_t launch_tiles_t(const DecodeGeom& g, const float* q, const T* dk, const T* dv,
                                 const T* kb, const T* vb, const float* lnn32,
                                 const uint8_t* mask, float* part, hipStream_t st) {
  const int tiles = g.dense_tiles + g.coarse_tiles;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, g.n_kv_heads);
#define SEKV_TILES(GG)                                                                        \
  case GG:                                                                                    \
    hipLaunchKernelGGL((attn_tiles_kernel<T, GG>), grid, dim3(256), 0, st, q, dk, dv, kb, vb, \
                       lnn32, mask, g.n_dense, g.n_compressed, g.dense_tiles, g.n_slots,      \
                       part);                                                                 \
    break;
  switch (g.group) {
    SEKV_TILES(1) SEKV_TILES(2) SEKV_TILES(3) SEKV_TILES(4) SEKV_TILES(5) SEKV_TILES(6)
    SEKV_TILES(7) SEKV_TILES(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_TILES
  return hipGetLastError();
}

hipError_t launch_attn_tiles(int bf16, const DecodeGeom& g, const float* q, const void* dense_k,
                             const void* dense_v, const void* kbar, const void* vbar,
                             const float* lnn32, const uint8_t* mask, float* part,
                             hipStream_t st) {
  if (bf16)
    return launch_tiles_t<uint16_t>(g, q, (const uint16_t*)dense_k, (const uint16_t*)dense_v,
                                    (const uint16_t*)kbar, (const uint16_t*)vbar, lnn32, mask,
                                    part, st);
  return launch_tiles_t<float>(g, q, (const float*)dense_k, (const float*)dense_v,
                               (const float*)kbar, (const float*)vbar, lnn32, mask, part, st);
}

// ---------------------------------------------------------------------------
// Zoomed spans, factored (Eq. 8 with hard gates).  Grid (zoom slots, KV
// heads); slot z of group g takes union entries z, z + slots, ...  For a span
// with factors U, sigma, V of keys and of values and the heads H that zoomed
// it:  b_h = sigma_K * (V_K^T q_h) / sqrt(d);  e_{h,t} = U_K[t] . b_h;
// p = exp(e - m);  c_h = U_V^T p;  acc_h += V_V (sigma_V * c_h).
// Reconstructed rows are never formed: per head the work is 2 r (n + d)
// multiply-adds against 8 r (n + d + 1) bytes of factors read once for all
// heads of the group.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void block_max_sum(float* v, bool is_max, float (*red)[G]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = v[h];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float y = __shfl_xor(x, o, 64);
      x = is_max ? fmaxf(x, y) : x + y;
    }
    if (lane == 0) red[wid][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = red[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) x = is_max ? fmaxf(x, red[w][h]) : x + red[w][h];
    v[h] = x;
  }
  __syncthreads();
}

template <int G>
__global__ __launch_bounds__(256) void attn_zoom_kernel(
    const float* __restrict__ q, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ rank,
    const uint64_t* __restrict__ fac_off, uint64_t off_base, const float* __restrict__ pool,
    int sc, int slot0, int n_slots, int zslots, float* __restrict__ part) {
  constexpr int HPT = (G + 1) / 2;  // output heads per thread
  __shared__ float qs[G][kHeadDim];
  __shared__ float bsh[G][kHeadDim];
  __shared__ float csh[G][kHeadDim];
  __shared__ float psh[G][256];
  __shared__ float red[4][G];
  const int zs = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x;
  const float scale = rsqrtf((float)kHeadDim);
  for (int o = tid; o < G * kHeadDim; o += 256)
    qs[o / kHeadDim][o % kHeadDim] = q[(size_t)g * G * kHeadDim + o] * scale;
  const int dim = tid & (kHeadDim - 1), hsel = tid >> 7;
  float m_run[G], l_run[G], acc_run[HPT];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }
#pragma unroll
  for (int k = 0; k < HPT; ++k) acc_run[k] = 0.f;
  __syncthreads();

  const int nu = ucount[g];
  const int rsub = tid >> 3, part8 = tid & 7;
  for (int u = zs; u < nu; u += zslots) {
    const int j = ulist[(size_t)g * sc + u];
    unsigned hm = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) hm |= (unsigned)(mask[(size_t)(g * G + h) * sc + j] != 0) << h;
    const int n = clen[j];
    const int r = rank[(size_t)g * sc + j];
    const FactorView fv(r, n);
    const float* blk = pool + (fac_off[(size_t)g * sc + j] - off_base);
    const float* vk = blk + fv.vt(0);
    const float* uk = blk + fv.u(0);
    const float* sk = blk + fv.sigma(0);
    const float* vv = blk + fv.vt(1);
    const float* uv = blk + fv.u(1);
    const float* sv = blk + fv.sigma(1);

    // b_h = sigma_K * (V_K^T q_h), scale folded into q
    for (int i0 = 0; i0 < r; i0 += 32) {
      const int i = i0 + rsub;
      float pa[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pa[h] = 0.f;
      if (i < r) {
        const float4* row = (const float4*)(vk + (size_t)i * kHeadDim + part8 * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const float4 x = row[c4];
          const int d0 = part8 * 16 + c4 * 4;
#pragma unroll
          for (int h = 0; h < G; ++h)
            pa[h] += x.x * qs[h][d0] + x.y * qs[h][d0 + 1] + x.z * qs[h][d0 + 2] + x.w * qs[h][d0 + 3];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pa[h] += __shfl_xor(pa[h], 1, 64);
        pa[h] += __shfl_xor(pa[h], 2, 64);
        pa[h] += __shfl_xor(pa[h], 4, 64);
      }
      if (part8 == 0 && i < r) {
        const float sg = sk[i];
#pragma unroll
        for (int h = 0; h < G; ++h) bsh[h][i] = pa[h] * sg;
      }
    }
    for (int o = tid; o < G * kHeadDim; o += 256) csh[o / kHeadDim][o % kHeadDim] = 0.f;
    __syncthreads();

    float ms[G], ls[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ms[h] = -INFINITY;
      ls[h] = 0.f;
    }
    for (int t0 = 0; t0 < n; t0 += 256) {
      const int t = t0 + tid;
      float e[G];
#pragma unroll
      for (int h = 0; h < G; ++h) e[h] = 0.f;
      if (t < n) {
        for (int i = 0; i < r; ++i) {
          const float x = uk[(size_t)i * fv.n4 + t];
#pragma unroll
          for (int h = 0; h < G; ++h) e[h] += x * bsh[h][i];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (t >= n || !((hm >> h) & 1u)) e[h] = -INFINITY;
      float cm[G];
#pragma unroll
      for (int h = 0; h < G; ++h) cm[h] = e[h];
      block_max_sum<G>(cm, true, red);
      float corr[G], p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(ms[h], cm[h]);
        corr[h] = (ms[h] == -INFINITY) ? 0.f : __expf(ms[h] - mn);
        p[h] = (e[h] == -INFINITY) ? 0.f : __expf(e[h] - mn);
        psh[h][tid] = p[h];
        ms[h] = mn;
      }
      block_max_sum<G>(p, false, red);  // also orders the psh writes before use
#pragma unroll
      for (int h = 0; h < G; ++h) ls[h] = ls[h] * corr[h] + p[h];
      const int tn = min(256, n - t0);
      for (int i0 = 0; i0 < r; i0 += 32) {
        const int i = i0 + rsub;
        float pc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pc[h] = 0.f;
        if (i < r) {
          const float* ur = uv + (size_t)i * fv.n4 + t0;
          for (int k = part8; k < tn; k += 8) {
            const float x = ur[k];
#pragma unroll
            for (int h = 0; h < G; ++h) pc[h] += psh[h][k] * x;
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          pc[h] += __shfl_xor(pc[h], 1, 64);
          pc[h] += __shfl_xor(pc[h], 2, 64);
          pc[h] += __shfl_xor(pc[h], 4, 64);
        }
        if (part8 == 0 && i < r) {
#pragma unroll
          for (int h = 0; h < G; ++h) csh[h][i] = csh[h][i] * corr[h] + pc[h];
        }
      }
      __syncthreads();
    }

    // acc_h[dim] += sum_i V_V[i][dim] sigma_V[i] c_h[i], merged into the running state
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
      const int h = hsel + 2 * k;
      if (h >= G || !((hm >> h) & 1u)) continue;
      float a = 0.f;
      for (int i = 0; i < r; ++i) a += vv[(size_t)i * kHeadDim + dim] * sv[i] * csh[h][i];
      const float M = fmaxf(m_run[h], ms[h]);
      const float wr = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - M);
      const float wsp = __expf(ms[h] - M);
      acc_run[k] = acc_run[k] * wr + a * wsp;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((hm >> h) & 1u)) continue;
      const float M = fmaxf(m_run[h], ms[h]);
      const float wr = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - M);
      l_run[h] = l_run[h] * wr + ls[h] * __expf(ms[h] - M);
      m_run[h] = M;
    }
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int h = hsel + 2 * k;
    if (h >= G) continue;
    float* dst = part + ((size_t)(g * G + h) * n_slots + slot0 + zs) * kPartStride;
    dst[4 + dim] = acc_run[k];
    if (dim == 0) {
      dst[0] = m_run[h];
      dst[1] = l_run[h];
    }
  }
}

hipError_t launch_attn_zoom(const DecodeGeom& g, const float* q, const uint8_t* mask,
                            const int32_t* ulist, const int32_t* ucount, const int32_t* clen,
                            const int32_t* rank, const uint64_t* fac_off, const float* pool,
                            uint64_t off_base, float* part, hipStream_t st) {
  if (g.zoom_slots == 0) return hipSuccess;
  dim3 grid(g.zoom_slots, g.n_kv_heads);
  const int slot0 = g.dense_tiles + g.coarse_tiles;
#define SEKV_ZOOM(GG)                                                                           \
  case GG:                                                                                      \
    hipLaunchKernelGGL((attn_zoom_kernel<GG>), grid, dim3(256), 0, st, q, mask, ulist, ucount,  \
                       clen, rank, fac_off, off_base, pool, g.n_compressed, slot0, g.n_slots,   \
                       g.zoom_slots, part);                                                     \
    break;
  switch (g.group) {
    SEKV_ZOOM(1) SEKV_ZOOM(2) SEKV_ZOOM(3) SEKV_ZOOM(4) SEKV_ZOOM(5) SEKV_ZOOM(6) SEKV_ZOOM(7)
    SEKV_ZOOM(8)
    default: return hipErrorInvalidValue;
  }
#undef SEKV_ZOOM
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of the split-K partials: o = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kHeadDim) void attn_merge_kernel(const float* __restrict__ part,
                                                              int n_slots, float* __restrict__ o) {
  const int h = blockIdx.x, dim = threadIdx.x;
  const float* ph = part + (size_t)h * n_slots * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < n_slots; ++s) M = fmaxf(M, ph[(size_t)s * kPartStride]);
  float L = 0.f, A = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_slots; ++s) {
      const float ms = ph[(size_t)s * kPartStride];
      if (ms == -INFINITY) continue;
      const float w = __expf(ms - M);
      L += ph[(size_t)s * kPartStride + 1] * w;
      A += ph[(size_t)s * kPartStride + 4 + dim] * w;
    }
  }
  o[(size_t)h * kHeadDim + dim] = L > 0.f ? A / L : 0.f;
}

hipError_t launch_attn_merge(const DecodeGeom& g, const float* part, float* o, hipStream_t st) {
  hipLaunchKernelGGL(attn_merge_kernel, dim3(g.n_q_heads), dim3(kHeadDim), 0, st, part,
                     g.n_slots, o);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host tier: copy the factor blocks of a layer's union spans from mapped
// pinned host memory into device staging at the same layer-relative offsets
// (16-byte loads over the host link).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fetch_gather_kernel(
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ rank,
    const uint64_t* __restrict__ fac_off, uint64_t layer_base, int sc, int zslots,
    const float* __restrict__ host, float* __restrict__ stage) {
  const int zs = blockIdx.x, g = blockIdx.y;
  const int nu = ucount[g];
  for (int u = zs; u < nu; u += zslots) {
    const int j = ulist[(size_t)g * sc + u];
    const FactorView fv(rank[(size_t)g * sc + j], clen[j]);
    const uint64_t off = fac_off[(size_t)g * sc + j];
    const uint4* src = (const uint4*)(host + off);
    uint4* dst = (uint4*)(stage + (off - layer_base));
    const int nvec = (int)(fv.block_floats() / 4);
    for (int k = threadIdx.x; k < nvec; k += 256) dst[k] = src[k];
  }
}

hipError_t launch_fetch_gather(const DecodeGeom& g, const int32_t* ulist, const int32_t* ucount,
                               const int32_t* clen, const int32_t* rank,
                               const uint64_t* fac_off, uint64_t layer_base,
                               const float* host_pool_mapped, float* stage, hipStream_t st) {
  if (g.zoom_slots == 0) return hipSuccess;
  hipLaunchKernelGGL(fetch_gather_kernel, dim3(g.zoom_slots, g.n_kv_heads), dim3(256), 0, st,
                     ulist, ucount, clen, rank, fac_off, layer_base, g.n_compressed,
                     g.zoom_slots, host_pool_mapped, stage);
  return hipGetLastError();
}

}  // namespace sekv
