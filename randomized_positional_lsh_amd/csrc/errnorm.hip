// The error of the sampled mask mean against the ALiBi bias matrix,
// E = L* - M~ with L*[r, j] = exp(-|r - j| / sigma) and M~ = c / s
// (explainer of arXiv 2605.09472, Methodology 1 and Theorem 2.1), at
// sequence lengths where E itself cannot be formed: its row maxima and its
// product with a vector, from the per-tile plan records of one head.
//
// Row maxima.  For j <= r the count is c(j) = #{i : st_i(r) <= j}, for
// j >= r it is #{i : en_i(r) > j}; both are step functions and L*(r, j) is
// monotone on each side of r, so on every step |L* - c/s| peaks at an end
// of the step.  The candidates are st_i, st_i - 1, en_i - 1 and en_i, each
// scored with its own count: O(s^2) per row instead of O(n s).
//
// Products.  L* x = F + G - x with the one-sided sums
// F[r] = sum_{j<=r} a^(r-j) x_j and G[r] = sum_{j>=r} a^(j-r) x_j,
// a = exp(-1/sigma): first-order recurrences, scanned in 1024-element tiles
// with carries between tiles.  (M(h_i) x)[r] is the sum of x over r's block,
// a difference of prefix sums, which the same scan yields (a = 1).
#include <algorithm>
#include <cmath>

#include "../../include/plpsh.h"
#include "internal.h"

namespace plpsh {
namespace {

constexpr int kRowsPerBlock = 64;
constexpr int kScanThreads = 256;
constexpr int kScanPer = 4;
constexpr int kScanTile = kScanThreads * kScanPer;  // 1024

// block [st, en) of the row at position p of the 128-row tile starting at r0
__device__ __forceinline__ void row_block(const PlanRec& rec, int r0, int p, int& st, int& en) {
  const uint64_t lo64 = rec.bits[0] | (static_cast<uint64_t>(rec.bits[1]) << 32);
  const uint64_t hi64 = rec.bits[2] | (static_cast<uint64_t>(rec.bits[3]) << 32);
  const int q = p & 63;
  const uint64_t le = q == 63 ? ~0ull : ((2ull << q) - 1);  // bits <= q
  const uint64_t half = p < 64 ? lo64 : hi64;
  const uint64_t m = half & le, gt = half & ~le;
  const int sp = m ? (p & 64) + 63 - __builtin_clzll(m) : ((p >= 64 && lo64) ? 63 - __builtin_clzll(lo64) : 0);
  const int ep = gt ? (p & 64) + __builtin_ctzll(gt) : ((p < 64 && hi64) ? 64 + __builtin_ctzll(hi64) : kPlanTile);
  st = sp ? r0 + sp : rec.a;
  en = ep < kPlanTile ? r0 + ep : rec.e2;
}

__global__ __launch_bounds__(kRowsPerBlock) void rowmax_kernel(const PlanRec* __restrict__ plan, int n, int s,
                                                               double sigma, double* __restrict__ rowmax) {
  extern __shared__ int sh[];  // st[s][64], en[s][64]: each thread reads its own column only
  int* sst = sh;
  int* sen = sh + s * kRowsPerBlock;
  const int lane = threadIdx.x;
  const int r = blockIdx.x * kRowsPerBlock + lane;
  const int rr = min(r, n - 1);
  const int q = rr >> 7, r0 = q << 7, p = rr & 127;
  const PlanRec* rec = plan + static_cast<size_t>(q) * s;
  for (int i = 0; i < s; ++i) {
    int st, en;
    row_block(rec[i], r0, p, st, en);
    sst[i * kRowsPerBlock + lane] = st;
    sen[i * kRowsPerBlock + lane] = en;
  }
  const double ds = static_cast<double>(s);
  double best = 0.0;  // j = r: L* = 1 = s / s
  for (int i = 0; i < s; ++i) {
    const int st = sst[i * kRowsPerBlock + lane];
    const int en = sen[i * kRowsPerBlock + lane];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int j = st - k2;
      if (j >= 0 && j < rr) {
        int c = 0;
        for (int k = 0; k < s; ++k) c += sst[k * kRowsPerBlock + lane] <= j;
        const double f = exp(-static_cast<double>(rr - j) / sigma) - static_cast<double>(c) / ds;
        best = fmax(best, fabs(f));
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int j = en - 1 + k2;
      if (j > rr && j < n) {
        int c = 0;
        for (int k = 0; k < s; ++k) c += sen[k * kRowsPerBlock + lane] > j;
        const double f = exp(-static_cast<double>(j - rr) / sigma) - static_cast<double>(c) / ds;
        best = fmax(best, fabs(f));
      }
    }
  }
  if (r < n) rowmax[r] = best;
}

// Local scans of one 1024-element tile: prefix sums P, forward decayed sums
// F and backward decayed sums G; tile aggregates for the carries.
__global__ __launch_bounds__(kScanThreads) void scan_local_kernel(const double* __restrict__ x, int n, double alpha,
                                                                  double* __restrict__ pl, double* __restrict__ fl,
                                                                  double* __restrict__ gl,
                                                                  double* __restrict__ agg) {
  __shared__ double sp[kScanThreads], sf[kScanThreads], sg[kScanThreads];
  const int t = threadIdx.x;
  const size_t base = static_cast<size_t>(blockIdx.x) * kScanTile + t * kScanPer;
  double xv[kScanPer], p[kScanPer], f[kScanPer], g[kScanPer];
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) xv[k] = base + k < static_cast<size_t>(n) ? x[base + k] : 0.0;
  p[0] = xv[0];
  f[0] = xv[0];
#pragma unroll
  for (int k = 1; k < kScanPer; ++k) {
    p[k] = p[k - 1] + xv[k];
    f[k] = alpha * f[k - 1] + xv[k];
  }
  g[kScanPer - 1] = xv[kScanPer - 1];
#pragma unroll
  for (int k = kScanPer - 2; k >= 0; --k) g[k] = alpha * g[k + 1] + xv[k];
  double ap[kScanPer + 1];  // alpha^k
  ap[0] = 1.0;
#pragma unroll
  for (int k = 1; k <= kScanPer; ++k) ap[k] = ap[k - 1] * alpha;
  sp[t] = p[kScanPer - 1];
  sf[t] = f[kScanPer - 1];
  sg[t] = g[0];
  __syncthreads();
  double mul = ap[kScanPer];  // decay across d threads: alpha^(4 d)
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const double vp = sp[t] + (t >= d ? sp[t - d] : 0.0);
    const double vf = sf[t] + (t >= d ? mul * sf[t - d] : 0.0);
    const double vg = sg[t] + (t + d < kScanThreads ? mul * sg[t + d] : 0.0);
    __syncthreads();
    sp[t] = vp;
    sf[t] = vf;
    sg[t] = vg;
    __syncthreads();
    mul *= mul;
  }
  const double pbefore = t > 0 ? sp[t - 1] : 0.0;
  const double fbefore = t > 0 ? sf[t - 1] : 0.0;
  const double gafter = t + 1 < kScanThreads ? sg[t + 1] : 0.0;
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) {
    if (base + k < static_cast<size_t>(n)) {
      pl[base + k] = p[k] + pbefore;
      fl[base + k] = f[k] + ap[k + 1] * fbefore;
      gl[base + k] = g[k] + ap[kScanPer - k] * gafter;
    }
  }
  if (t == 0) {
    agg[3 * blockIdx.x + 0] = sp[kScanThreads - 1];
    agg[3 * blockIdx.x + 1] = sf[kScanThreads - 1];
    agg[3 * blockIdx.x + 2] = sg[0];
  }
}

// Carries between tiles: car[3b] = P before tile b, car[3b+1] = F at the
// element before tile b, car[3b+2] = G at the element after tile b.  The
// aggregates (at most 512 tiles) are staged in LDS by the whole block, then
// chained by one thread.
constexpr int kMaxScanTiles = PLPSH_MAX_N / kScanTile;
__global__ __launch_bounds__(256) void scan_carry_kernel(const double* __restrict__ agg, int nb, double alpha_tile,
                                                         double* __restrict__ car) {
  __shared__ double sa[3 * kMaxScanTiles];
  for (int i = threadIdx.x; i < 3 * nb; i += 256) sa[i] = agg[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    double cp = 0.0, cf = 0.0;
    for (int b = 0; b < nb; ++b) {
      const double ap = sa[3 * b + 0], af = sa[3 * b + 1];
      sa[3 * b + 0] = cp;
      sa[3 * b + 1] = cf;
      cp += ap;
      cf = af + alpha_tile * cf;
    }
    double cg = 0.0;
    for (int b = nb - 1; b >= 0; --b) {
      const double ag = sa[3 * b + 2];
      sa[3 * b + 2] = cg;
      cg = ag + alpha_tile * cg;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 3 * nb; i += 256) car[i] = sa[i];
}

__device__ __forceinline__ double prefix_incl(const double* pl, const double* car, int m) {
  return pl[m] + car[3 * (m / kScanTile)];
}

// y = L* x - (1/s) sum_i M(h_i) x
__global__ __launch_bounds__(256) void combine_kernel(const double* __restrict__ x, const PlanRec* __restrict__ plan,
                                                      int n, int s, double sigma, const double* __restrict__ pl,
                                                      const double* __restrict__ fl, const double* __restrict__ gl,
                                                      const double* __restrict__ car, double* __restrict__ y) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  const int b = r / kScanTile, k = r % kScanTile;
  const double fwd = fl[r] + exp(-static_cast<double>(k + 1) / sigma) * car[3 * b + 1];
  const double bwd = gl[r] + exp(-static_cast<double>(kScanTile - k) / sigma) * car[3 * b + 2];
  const double lx = fwd + bwd - x[r];
  const int q = r >> 7, r0 = q << 7, p = r & 127;
  const PlanRec* rec = plan + static_cast<size_t>(q) * s;
  double mx = 0.0;
  for (int i = 0; i < s; ++i) {
    int st, en;
    row_block(rec[i], r0, p, st, en);
    mx += prefix_incl(pl, car, en - 1) - (st > 0 ? prefix_incl(pl, car, st - 1) : 0.0);
  }
  y[r] = lx - mx / static_cast<double>(s);
}

// <V_j, w> for the m vectors V_j = V + j * ld: workgroup (j, k) sums rows
// k, k + kDotSplit * 256, ... into part[j * kDotSplit + k]; a second pass adds
// the parts of each j in a fixed order.
constexpr int kDotSplit = 32;
__global__ __launch_bounds__(256) void dots_kernel(const double* __restrict__ V, size_t ld, const double* __restrict__ w,
                                                   int n, double* __restrict__ part) {
  __shared__ double red[256];
  const double* v = V + static_cast<size_t>(blockIdx.x) * ld;
  double acc = 0.0;
  for (int r = blockIdx.y * 256 + threadIdx.x; r < n; r += 256 * kDotSplit) acc += v[r] * w[r];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x * kDotSplit + blockIdx.y] = red[0];
}
__global__ __launch_bounds__(256) void dots_sum_kernel(const double* __restrict__ part, int m,
                                                       double* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= m) return;
  double acc = 0.0;
  for (int k = 0; k < kDotSplit; ++k) acc += part[j * kDotSplit + k];
  out[j] = acc;
}

// w -= sum_{j<m} h[j] V_j
__global__ __launch_bounds__(256) void sub_proj_kernel(const double* __restrict__ V, size_t ld,
                                                       const double* __restrict__ h, int m, int n,
                                                       double* __restrict__ w) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  double acc = 0.0;
  for (int j = 0; j < m; ++j) acc += h[j] * V[static_cast<size_t>(j) * ld + r];
  w[r] -= acc;
}

__global__ __launch_bounds__(256) void scale_kernel(const double* __restrict__ w, double c, int n,
                                                    double* __restrict__ v) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n) v[r] = w[r] * c;
}

// largest entry and its first index: per-block partials, then one block
__global__ __launch_bounds__(256) void argmax_kernel(const double* __restrict__ a, const int* __restrict__ ia, int n,
                                                     double* __restrict__ ov, int* __restrict__ oi) {
  __shared__ double sv[256];
  __shared__ int si[256];
  double bv = -1.0;
  int bi = 0;
  for (int r = blockIdx.x * 256 + threadIdx.x; r < n; r += 256 * gridDim.x) {
    const double v = a[r];
    const int i = ia ? ia[r] : r;
    if (v > bv || (v == bv && i < bi)) {
      bv = v;
      bi = i;
    }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const double v = sv[threadIdx.x + o];
      const int i = si[threadIdx.x + o];
      if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && i < si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ov[blockIdx.x] = sv[0];
    oi[blockIdx.x] = si[0];
  }
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace

size_t err_scan_bytes(int n) {
  const size_t nb = static_cast<size_t>(cdiv(n, kScanTile));
  return (3 * static_cast<size_t>(n) + 6 * nb) * sizeof(double);
}

size_t err_dots_bytes(int m) { return static_cast<size_t>(m) * kDotSplit * sizeof(double); }

hipError_t launch_err_rowmax(const PlanRec* plan, int n, int s, double sigma, double* rowmax, hipStream_t st) {
  const size_t lds = 2 * static_cast<size_t>(s) * kRowsPerBlock * sizeof(int);
  static LdsOptIn opt;
  if (hipError_t e = opt.ensure(reinterpret_cast<const void*>(rowmax_kernel), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(rowmax_kernel, dim3(cdiv(n, kRowsPerBlock)), dim3(kRowsPerBlock), lds, st, plan, n, s, sigma,
                     rowmax);
  return hipGetLastError();
}

hipError_t launch_err_matvec(const PlanRec* plan, int n, int s, double sigma, const double* x, double* y, void* scratch,
                             hipStream_t st) {
  const int nb = cdiv(n, kScanTile);
  double* pl = static_cast<double*>(scratch);
  double* fl = pl + n;
  double* gl = fl + n;
  double* agg = gl + n;
  double* car = agg + 3 * static_cast<size_t>(nb);
  const double alpha = std::exp(-1.0 / sigma);
  const double alpha_tile = std::exp(-static_cast<double>(kScanTile) / sigma);
  hipLaunchKernelGGL(scan_local_kernel, dim3(nb), dim3(kScanThreads), 0, st, x, n, alpha, pl, fl, gl, agg);
  hipLaunchKernelGGL(scan_carry_kernel, dim3(1), dim3(256), 0, st, agg, nb, alpha_tile, car);
  hipLaunchKernelGGL(combine_kernel, dim3(cdiv(n, 256)), dim3(256), 0, st, x, plan, n, s, sigma, pl, fl, gl, car, y);
  return hipGetLastError();
}

hipError_t launch_err_dots(const double* V, size_t ld, int m, const double* w, int n, double* out, double* part,
                           hipStream_t st) {
  hipLaunchKernelGGL(dots_kernel, dim3(m, kDotSplit), dim3(256), 0, st, V, ld, w, n, part);
  hipLaunchKernelGGL(dots_sum_kernel, dim3(cdiv(m, 256)), dim3(256), 0, st, part, m, out);
  return hipGetLastError();
}

hipError_t launch_err_sub_proj(const double* V, size_t ld, const double* h, int m, int n, double* w, hipStream_t st) {
  hipLaunchKernelGGL(sub_proj_kernel, dim3(cdiv(n, 256)), dim3(256), 0, st, V, ld, h, m, n, w);
  return hipGetLastError();
}

hipError_t launch_err_scale(const double* w, double c, int n, double* v, hipStream_t st) {
  hipLaunchKernelGGL(scale_kernel, dim3(cdiv(n, 256)), dim3(256), 0, st, w, c, n, v);
  return hipGetLastError();
}

hipError_t launch_err_argmax(const double* a, int n, double* pv, int* pi, double* out_v, int* out_i, hipStream_t st) {
  const int nb = std::min(256, cdiv(n, 256));
  hipLaunchKernelGGL(argmax_kernel, dim3(nb), dim3(256), 0, st, a, nullptr, n, pv, pi);
  hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(256), 0, st, pv, pi, nb, out_v, out_i);
  return hipGetLastError();
}

}  // namespace plpsh
