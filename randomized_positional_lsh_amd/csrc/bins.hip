// Bin-boundary kernel: from the hashes (delta, u) to the blocks they cut the
// positions into.
//
// Positional LSH (explainer of arXiv 2605.09472, Methodology 1): random
// binning of the integer positions places x in bin floor((x - u) / delta);
// the bins are contiguous and non-overlapping, so a hash is fully described
// by the positions where a new block starts.  Here each hash gets one
// workgroup that builds a bitmap of block starts in LDS, turns it into int32
// prefix offsets (the start of every block) by a popcount scan, and writes a
// 32-byte record per 128-row query tile for the attention kernel.
//
// Bit-exactness: every bin value is floor of the IEEE binary64 quotient of
// the binary64 difference (x - u) by delta, as in the definition; this file
// is compiled with -ffp-contract=off.  Each position is evaluated (a product
// with the reciprocal settles the floor unless the quotient is within a few
// ulp of an integer, where the division itself is taken) and compared with
// its predecessor; position 0 always starts a block.
#include <climits>

#include "internal.h"

namespace plpsh {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Start flags of the 32 positions x0 .. x0 + 31 (bit b: bin(x0 + b) differs
// from bin(x0 + b - 1)), bins evaluated in binary64 as floor((x - u) / delta).
// First from the product with a rounded reciprocal, which is within 2.2 ulp
// of the quotient: where no integer lies within 2^-50 |q| of it the floor
// equals that of the correctly rounded quotient.  If any of the 33 positions
// misses that margin (rare) the word is redone with the division itself.
// The fast pass is fully unrolled so that the evaluations overlap.
__device__ __forceinline__ uint32_t start_flags(int x0, double u, double delta, double rinv) {
  double f[33];
  bool exact = false;
#pragma unroll
  for (int k = 0; k < 33; ++k) {
    const double d = static_cast<double>(x0 - 1 + k) - u;
    const double q = d * rinv;
    const double fl = floor(q);
    const double fr = q - fl;  // exact for |q| < 2^52
    const double margin = fabs(q) * 0x1p-50;
    f[k] = fl;
    exact = exact || !(fr > margin && fr < 1.0 - margin);
  }
  uint32_t m = 0u;
  if (!exact) {
#pragma unroll
    for (int b = 0; b < 32; ++b) m |= static_cast<uint32_t>(f[b + 1] != f[b]) << b;
  } else {
    double prev = floor((static_cast<double>(x0 - 1) - u) / delta);
    for (int b = 0; b < 32; ++b) {
      const double bb = floor((static_cast<double>(x0 + b) - u) / delta);
      m |= static_cast<uint32_t>(bb != prev) << b;
      prev = bb;
    }
  }
  return m;
}

// Exclusive scan of one int per thread over the workgroup.
__device__ int wg_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) base += k < w ? wsum[k] : 0;
  int tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) tot += wsum[k];
  *total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kThreads) void bins_kernel(const double* __restrict__ du, int n, int s,
                                                        int ntile, int nwords,
                                                        int32_t* __restrict__ nblk,
                                                        int32_t* __restrict__ starts,
                                                        PlanRec* __restrict__ plan) {
  extern __shared__ uint32_t lds[];
  uint32_t* bits = lds;                                   // [nwords] start bitmap
  int32_t* pre = reinterpret_cast<int32_t*>(lds + nwords);  // [nwords] starts before word
  __shared__ int wsum[kWaves];

  const int hid = blockIdx.x;  // hash index h * s + i
  const int h = hid / s, i = hid - h * s;
  const int tid = threadIdx.x;
  const double delta = du[2 * hid], u = du[2 * hid + 1];
  const double rinv = 1.0 / delta;

  // block starts: bit x of the map is set iff x = 0 or bin(x) != bin(x - 1)
  // (one 32-position word per thread and step; words past n stay zero)
  const int nused = (n + 31) >> 5;
  for (int w = tid; w < nwords; w += kThreads) {
    uint32_t m = 0u;
    if (w < nused) {
      const int x0 = 32 * w;
      m = start_flags(x0, u, delta, rinv);
      if (x0 == 0) m |= 1u;
      if (n - x0 < 32) m &= (1u << (n - x0)) - 1u;
    }
    bits[w] = m;
  }
  __syncthreads();

  // popcount prefix over words: each thread a contiguous run of words
  const int per = (nwords + kThreads - 1) / kThreads;
  const int w0 = tid * per, w1 = min(w0 + per, nwords);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(bits[w]);
  int total;
  int base = wg_exclusive_scan(local, wsum, &total);
  for (int w = w0; w < w1; ++w) {
    pre[w] = base;
    base += __popc(bits[w]);
  }
  __syncthreads();

  int32_t* st = starts + static_cast<size_t>(hid) * (n + 1);
  if (delta < 4.0) {
    // dense: one position per thread, consecutive threads write consecutive starts
#pragma unroll 4
    for (int x = tid; x < n; x += kThreads) {
      const uint32_t m = bits[x >> 5];  // both reads unconditional, so unrolled steps overlap
      const int o = pre[x >> 5] + __popc(m & ((1u << (x & 31)) - 1u));
      if ((m >> (x & 31)) & 1u) st[o] = x;
    }
  } else {
    for (int w = tid; w < nused; w += kThreads) {
      uint32_t m = bits[w];
      int b = pre[w];
      while (m) {
        st[b++] = (w << 5) + (__ffs(m) - 1);
        m &= m - 1;
      }
    }
  }
  if (tid == 0) {
    nblk[hid] = total;
    st[total] = n;
  }
  __threadfence_block();
  __syncthreads();

  // plan records: tile q covers rows [128 q, 128 q + 128)
  PlanRec* pl = plan + static_cast<size_t>(h) * ntile * s + i;
  for (int q = tid; q < ntile; q += kThreads) {
    const int r0 = q * kPlanTile;
    const int rl = min(r0 + kPlanTile - 1, n - 1);
    const int x0w = r0 >> 5, xlw = rl >> 5;
    const int kb0 = pre[x0w] + __popc(bits[x0w] & (0xFFFFFFFFu >> (31 - (r0 & 31)))) - 1;
    const int kbl = pre[xlw] + __popc(bits[xlw] & (0xFFFFFFFFu >> (31 - (rl & 31)))) - 1;
    PlanRec rec;
    rec.a = st[kb0];
    rec.e = st[kb0 + 1];
    rec.a2 = st[kbl];
    rec.e2 = st[kbl + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) rec.bits[j] = bits[x0w + j];
    rec.bits[0] &= ~1u;
    if (n - r0 < kPlanTile) {
      const int p = n - r0;
#pragma unroll
      for (int j = 0; j < 4; ++j) rec.bits[j] |= (p >> 5) == j ? 1u << (p & 31) : 0u;
    }
    pl[static_cast<size_t>(q) * s] = rec;
  }
}

}  // namespace

BinsLayout bins_layout(int heads, int s, int n) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t hs = static_cast<size_t>(heads) * s;
  const size_t ntile = (static_cast<size_t>(n) + kPlanTile - 1) / kPlanTile;
  BinsLayout L;
  L.off_nblk = 0;
  L.off_starts = up(hs * sizeof(int32_t));
  L.off_plan = L.off_starts + up(hs * (static_cast<size_t>(n) + 1) * sizeof(int32_t));
  L.total = L.off_plan + up(static_cast<size_t>(heads) * ntile * s * sizeof(PlanRec));
  return L;
}

hipError_t launch_bins(const double* du, int heads, int s, int n, void* bins, hipStream_t stream) {
  const BinsLayout L = bins_layout(heads, s, n);
  char* base = static_cast<char*>(bins);
  const int ntile = (n + kPlanTile - 1) / kPlanTile;
  const int nwords = 4 * ntile + 4;  // covers positions < 128 (ntile + 1)
  const size_t lds = static_cast<size_t>(nwords) * 2 * sizeof(uint32_t);
  // opt in to the dynamic LDS this launch needs (the largest request so far)
  static size_t attr_bytes = 0;  // benign race: the attribute only grows
  if (lds > 64 * 1024 && lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bins_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  hipLaunchKernelGGL(bins_kernel, dim3(heads * s), dim3(kThreads), lds, stream, du, n, s, ntile, nwords,
                     reinterpret_cast<int32_t*>(base + L.off_nblk),
                     reinterpret_cast<int32_t*>(base + L.off_starts),
                     reinterpret_cast<PlanRec*>(base + L.off_plan));
  return hipGetLastError();
}

}  // namespace plpsh
