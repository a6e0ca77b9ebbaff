// Randomized truncated SVD of span keys and values (gfx950).
//
// SeKV paper Sec. 3.2 (low-rank paragraph): each span's key and value
// matrices are factored by a truncated SVD, computed with a randomized method.
// This is the range-finder scheme of Halko, Martinsson and Tropp (2011,
// Algorithms 4.3/4.4 with 5.1): for a span's n x d matrix X and target rank r,
//   Y = X Omega with a d x k random sign matrix, k = r + 8 (rounded up to
//   even); q = 2 power iterations Z = X^T Q, Y = X Z, each factor
//   re-orthonormalised; Q = orth(Y); B = Q^T X (k x d); the eigenpairs
//   (lambda_i, w_i) of the k x k matrix B B^T by one-sided Jacobi; then
//   sigma_i = sqrt(lambda_i), u_i = Q w_i, v_i = B^T w_i / sigma_i.
// Orthonormalisation is Cholesky QR applied twice (G = M^T M = R^T R in
// float64, M <- M R^-1); a pivot below 1e-10 of the largest diagonal marks a
// numerically dependent column, which is zeroed and carries no component.
//
// One workgroup of 256 threads per (span, layer x KV head), spans of
// 40 < n <= 640 tokens and ranks up to 32; everything but X sits in LDS, sized
// for up to 128, 256 or 640 rows (one launch each), so that spans of up to 128
// tokens fit two workgroups per CU.
#include <hip/hip_runtime.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

constexpr int kRsThreads = 256;
constexpr int kRsMaxK = kRsvdMaxRank + 8;
constexpr int kRsPower = 2;
constexpr int kRsMaxSweeps = 30;
constexpr double kRsTol = 1e-14;
constexpr double kRsDep = 1e-10;

template <int ROWS>
struct RsSmem {
  float y[ROWS][kRsMaxK];          // sketch, then the orthonormal basis Q (n x k)
  float z[kHeadDim][kRsMaxK];      // test matrix, then X^T Q (d x k)
  double g[kRsMaxK][kRsMaxK];      // Gram matrix, Cholesky work, then B B^T
  double rc[kRsMaxK][kRsMaxK];     // Cholesky factor R (upper triangle, row-major)
  double nrm[kRsMaxK];
  double diag_max;
  int order[kRsMaxK];
  int dep[kRsMaxK];
};

__device__ __forceinline__ float rs_load(const float* p) { return *p; }
__device__ __forceinline__ float rs_load(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ uint64_t rs_hash(uint64_t x) {
  // splitmix64 (Steele, Lea and Flood, 2014)
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// out[t][i] = sum_c X[t][c] in[c][i] for t < n, i < k (in: d x k in LDS)
template <typename T>
__device__ void rs_x_times(const T* X, int n, int k, const float (*in)[kRsMaxK],
                           float (*out)[kRsMaxK]) {
  for (int t = threadIdx.x; t < n; t += kRsThreads) {
    float acc[kRsMaxK];
#pragma unroll
    for (int i = 0; i < kRsMaxK; ++i) acc[i] = 0.f;
    const T* xr = X + (size_t)t * kHeadDim;
    for (int c = 0; c < kHeadDim; ++c) {
      const float xv = rs_load(xr + c);
#pragma unroll
      for (int i = 0; i < kRsMaxK; ++i)
        if (i < k) acc[i] += xv * in[c][i];
    }
#pragma unroll
    for (int i = 0; i < kRsMaxK; ++i)
      if (i < k) out[t][i] = acc[i];
  }
}

// out[c][i] = sum_t X[t][c] in[t][i] for c < d, i < k (in: n x k in LDS)
template <typename T>
__device__ void rs_xt_times(const T* X, int n, int k, const float (*in)[kRsMaxK],
                            float (*out)[kRsMaxK]) {
  const int c = threadIdx.x;
  if (c >= kHeadDim) return;
  double acc[kRsMaxK];
#pragma unroll
  for (int i = 0; i < kRsMaxK; ++i) acc[i] = 0.0;
  for (int t = 0; t < n; ++t) {
    const double xv = rs_load(X + (size_t)t * kHeadDim + c);
#pragma unroll
    for (int i = 0; i < kRsMaxK; ++i)
      if (i < k) acc[i] += xv * (double)in[t][i];
  }
#pragma unroll
  for (int i = 0; i < kRsMaxK; ++i)
    if (i < k) out[c][i] = (float)acc[i];
}

// M (rows x k, in LDS) <- M R^-1 with M^T M = R^T R: one Cholesky QR pass.
// Dependent columns (pivot <= kRsDep x the largest diagonal) become zero.
template <int ROWS>
__device__ void rs_cholqr(RsSmem<ROWS>& s, float (*M)[kRsMaxK], int rows, int k) {
  const int tid = threadIdx.x;
  for (int p = tid; p < k * k; p += kRsThreads) {
    const int i = p / k, j = p % k;
    if (i > j) continue;
    double a = 0.0;
    for (int t = 0; t < rows; ++t) a += (double)M[t][i] * (double)M[t][j];
    s.g[i][j] = a;
    s.g[j][i] = a;
  }
  __syncthreads();
  if (tid == 0) {
    double dm = 0.0;
    for (int i = 0; i < k; ++i) dm = fmax(dm, s.g[i][i]);
    s.diag_max = dm;
  }
  __syncthreads();
  const double thr = kRsDep * s.diag_max;
  // right-looking Cholesky, one column per step
  for (int j = 0; j < k; ++j) {
    const double d = s.g[j][j];
    const bool dep = !(d > thr);
    const double rjj = dep ? 0.0 : sqrt(d);
    for (int l = tid; l < k; l += kRsThreads)
      s.rc[j][l] = l < j ? 0.0 : (l == j ? rjj : (dep ? 0.0 : s.g[j][l] / rjj));
    if (tid == 0) s.dep[j] = dep ? 1 : 0;
    __syncthreads();
    for (int p = tid; p < k * k; p += kRsThreads) {
      const int l = p / k, m = p % k;
      if (l > j && m > j) s.g[l][m] -= s.rc[j][l] * s.rc[j][m];
    }
    __syncthreads();
  }
  // R^-1 (upper triangular) into g, one column per thread, by back
  // substitution; rows and columns of dependent components are zero
  for (int jc = tid; jc < k; jc += kRsThreads) {
    for (int p = k - 1; p >= 0; --p) {
      double v = 0.0;
      if (p <= jc && !s.dep[p]) {
        if (p == jc) {
          v = 1.0 / s.rc[p][p];
        } else {
          double a = 0.0;
          for (int l = p + 1; l <= jc; ++l) a += s.rc[p][l] * s.g[l][jc];
          v = -a / s.rc[p][p];
        }
      }
      s.g[p][jc] = v;
    }
  }
  __syncthreads();
  // M <- M R^-1, one row per thread, the row held in registers
  for (int t = tid; t < rows; t += kRsThreads) {
    float m[kRsMaxK];
#pragma unroll
    for (int p = 0; p < kRsMaxK; ++p) m[p] = p < k ? M[t][p] : 0.f;
    for (int j = 0; j < k; ++j) {
      double a = 0.0;
#pragma unroll
      for (int p = 0; p < kRsMaxK; ++p)
        if (p <= j) a += (double)m[p] * s.g[p][j];
      M[t][j] = (float)a;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int rs_player(int pos, int round, int k) {
  return pos == 0 ? 0 : ((pos - 1 + round) % (k - 1)) + 1;
}

template <typename T, int ROWS>
__global__ __launch_bounds__(kRsThreads) void span_rsvd_kernel(
    const T* __restrict__ x, int n_tokens, const int32_t* __restrict__ cstart,
    const int32_t* __restrict__ clen, const int32_t* __restrict__ span_ids, int sc,
    const int32_t* __restrict__ rank, const uint64_t* __restrict__ fac_off,
    float* __restrict__ pool, int which) {
  extern __shared__ double smem_raw[];
  RsSmem<ROWS>& s = *reinterpret_cast<RsSmem<ROWS>*>(smem_raw);
  const int tid = threadIdx.x;
  const int j = span_ids[blockIdx.x];
  const int lg = blockIdx.y;
  const int b = cstart[j], n = clen[j];
  const int32_t ranks = rank[(size_t)lg * sc + j];
  const int r = rank_of(ranks, which);
  const int k = min(kRsMaxK, (r + 8 + 1) & ~1);
  const T* X = x + ((size_t)lg * n_tokens + b) * kHeadDim;

  // ---- random sign test matrix, then the sketch and its power iterations ---
  const uint64_t seed = (((uint64_t)lg * sc + j) << 1) | (uint64_t)which;
  for (int p = tid; p < kHeadDim * k; p += kRsThreads) {
    const int c = p / k, i = p % k;
    s.z[c][i] = (rs_hash(seed * 0x100000001b3ull + (uint64_t)p) >> 63) ? 1.f : -1.f;
  }
  __syncthreads();
  rs_x_times(X, n, k, s.z, s.y);
  __syncthreads();
  // intermediate bases need only stay well conditioned (one pass); the
  // final Q is orthonormalised twice
  rs_cholqr(s, s.y, n, k);
  for (int it = 0; it < kRsPower; ++it) {
    rs_xt_times(X, n, k, s.y, s.z);
    __syncthreads();
    rs_cholqr(s, s.z, kHeadDim, k);
    rs_x_times(X, n, k, s.z, s.y);
    __syncthreads();
    rs_cholqr(s, s.y, n, k);
  }
  rs_cholqr(s, s.y, n, k);
  // ---- B^T = X^T Q (d x k) and H = B B^T (k x k) ----------------------------
  rs_xt_times(X, n, k, s.y, s.z);
  __syncthreads();
  for (int p = tid; p < k * k; p += kRsThreads) {
    const int i = p / k, jj = p % k;
    if (i > jj) continue;
    double a = 0.0;
    for (int c = 0; c < kHeadDim; ++c) a += (double)s.z[c][i] * (double)s.z[c][jj];
    s.g[i][jj] = a;
    s.g[jj][i] = a;
  }
  __syncthreads();

  // ---- eigenpairs of H by one-sided Jacobi on its columns (g[c][.]) --------
  constexpr int TPP = 8;
  const int npairs = k / 2;
  const int pid = tid / TPP, sub = tid % TPP;
  const bool active = pid < npairs;
  for (int sweep = 0; sweep < kRsMaxSweeps; ++sweep) {
    int rotated = 0;
    for (int round = 0; round < k - 1; ++round) {
      if (active) {
        const int p = rs_player(pid, round, k);
        const int q = rs_player(k - 1 - pid, round, k);
        double* ap = s.g[p];
        double* aq = s.g[q];
        constexpr int KPT = kRsMaxK / TPP;
        double xp[KPT], xq[KPT];
        double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const int kk = sub + i * TPP;
          xp[i] = kk < k ? ap[kk] : 0.0;
          xq[i] = kk < k ? aq[kk] : 0.0;
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
        if (fabs(ga) > kRsTol * sqrt(al) * sqrt(be)) {
          const double zeta = (be - al) / (2.0 * ga);
          const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          const double c = 1.0 / sqrt(1.0 + t * t);
          const double sn = c * t;
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            const int kk = sub + i * TPP;
            if (kk < k) {
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

  // ---- order by lambda = column norm; w_i = column / lambda ----------------
  for (int c = tid; c < k; c += kRsThreads) {
    double s2 = 0.0;
    for (int kk = 0; kk < k; ++kk) s2 += s.g[c][kk] * s.g[c][kk];
    s.nrm[c] = sqrt(s2);
  }
  __syncthreads();
  for (int c = tid; c < k; c += kRsThreads) {
    int pos = 0;
    const double v = s.nrm[c];
    for (int o = 0; o < k; ++o) pos += (s.nrm[o] > v) || (s.nrm[o] == v && o < c);
    s.order[pos] = c;
  }
  __syncthreads();
  const double lmax = s.nrm[s.order[0]];
  auto live = [&](int i) -> bool {
    const double lam = s.nrm[s.order[i]];
    return lam > 0.0 && lam > lmax * 1e-24;
  };

  // ---- factors: sigma, u_i = Q w_i (token-major), v_i = B^T w_i / sigma -----
  const FactorView fv = FactorView::packed(ranks, n);
  const int r4 = fv.r4(which);
  float* blk = pool + fac_off[(size_t)lg * sc + j];
  float* vt = blk + fv.vt(which);
  float* u = blk + fv.u(which);
  float* sg = blk + fv.sigma(which);
  for (int i = tid; i < r4; i += kRsThreads)
    sg[i] = (i < r && live(i)) ? (float)sqrt(s.nrm[s.order[i]]) : 0.f;
  for (int idx = tid; idx < n * r4; idx += kRsThreads) {
    const int t = idx / r4, i = idx % r4;
    float val = 0.f;
    if (i < r && live(i)) {
      const double* w = s.g[s.order[i]];
      const double lam = s.nrm[s.order[i]];
      double a = 0.0;
      for (int p = 0; p < k; ++p) a += (double)s.y[t][p] * w[p];
      val = (float)(a / lam);
    }
    u[idx] = val;
  }
  for (int idx = tid; idx < r * kHeadDim; idx += kRsThreads) {
    const int i = idx / kHeadDim, c = idx % kHeadDim;
    float val = 0.f;
    if (live(i)) {
      const double* w = s.g[s.order[i]];
      const double lam = s.nrm[s.order[i]];
      double a = 0.0;
      for (int p = 0; p < k; ++p) a += (double)s.z[c][p] * w[p];
      val = (float)(a / (lam * sqrt(lam)));
    }
    vt[idx] = val;
  }
}

template <typename T, int ROWS>
hipError_t launch_rsvd_t(const T* x, int n_tokens, const int32_t* cstart, const int32_t* clen,
                         const int32_t* span_ids, int n_ids, int sc, int n_lg,
                         const int32_t* rank, const uint64_t* fac_off, float* pool, int which,
                         hipStream_t st) {
  const size_t lds = sizeof(RsSmem<ROWS>);
  hipError_t e = hipFuncSetAttribute((const void*)span_rsvd_kernel<T, ROWS>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((span_rsvd_kernel<T, ROWS>), dim3(n_ids, n_lg), dim3(kRsThreads), lds, st,
                     x, n_tokens, cstart, clen, span_ids, sc, rank, fac_off, pool, which);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_span_rsvd(int bf16, const void* x, int n_tokens, const int32_t* cstart,
                            const int32_t* clen, const int32_t* span_ids, int n_ids, int sc,
                            int n_lg, const int32_t* rank, const uint64_t* fac_off, float* pool,
                            int which, int max_rows, hipStream_t st) {
  if (n_ids == 0) return hipSuccess;
#define SEKV_RSVD(ROWS)                                                                         \
  return bf16 ? launch_rsvd_t<uint16_t, ROWS>((const uint16_t*)x, n_tokens, cstart, clen,       \
                                              span_ids, n_ids, sc, n_lg, rank, fac_off, pool,   \
                                              which, st)                                        \
              : launch_rsvd_t<float, ROWS>((const float*)x, n_tokens, cstart, clen, span_ids,   \
                                           n_ids, sc, n_lg, rank, fac_off, pool, which, st)
  if (max_rows <= 128) { SEKV_RSVD(128); }
  if (max_rows <= 256) { SEKV_RSVD(256); }
  SEKV_RSVD(kRsvdMaxRows);
#undef SEKV_RSVD
}

}  // namespace sekv
