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
// Most hashes take a second kernel with more parallelism: the positions are
// cut into parts of 8192, one 256-thread workgroup each.  A part needs the
// number of block starts before it, which has a closed form unless delta is
// within 2^-30 of 1 (the bound is derived at bins_part_kernel); a launch in
// which some hash is that close to 1 takes the per-hash kernel.
//
// Bit-exactness: every bin value is floor of the IEEE binary64 quotient of
// the binary64 difference (x - u) by delta, as in the definition; this file
// is compiled with -ffp-contract=off.  Each position is evaluated (a product
// with the reciprocal settles the floor unless the quotient is within a few
// ulp of an integer, where the division itself is taken) and compared with
// its predecessor; position 0 always starts a block.
#include <climits>

#include "bins_device.h"
#include "internal.h"

namespace plpsh {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

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
  // per 32-position word: its start bitmap (x) and the number of block
  // starts before it (y), side by side so that one 8-byte read gets both
  extern __shared__ uint2 wd[];
  __shared__ int wsum[kWaves];

  const int hid = blockIdx.x;  // hash index h * s + i
  const int h = hid / s, i = hid - h * s;
  const int tid = threadIdx.x;
  const double delta = du[2 * hid], u = du[2 * hid + 1];
  const double rinv = 1.0 / delta;
  const bool wide = delta >= 32.0;

  // block starts: bit x of the map is set iff x = 0 or bin(x) != bin(x - 1)
  // (one 32-position word per thread and step; words past n stay zero)
  const int nused = (n + 31) >> 5;
  for (int w = tid; w < nwords; w += kThreads) {
    uint32_t m = 0u;
    if (w < nused) {
      const int x0 = 32 * w;
      double prev;
      m = start_flags(x0, u, delta, rinv, wide, &prev);
      if (x0 == 0) m |= 1u;
      if (n - x0 < 32) m &= (1u << (n - x0)) - 1u;
    }
    wd[w].x = m;
  }
  __syncthreads();

  // popcount prefix over words: each thread a contiguous run of words
  const int per = (nwords + kThreads - 1) / kThreads;
  const int w0 = tid * per, w1 = min(w0 + per, nwords);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(wd[w].x);
  int total;
  int base = wg_exclusive_scan(local, wsum, &total);
  for (int w = w0; w < w1; ++w) {
    const uint32_t m = wd[w].x;
    wd[w].y = static_cast<uint32_t>(base);
    base += __popc(m);
  }
  __syncthreads();

  int32_t* st = starts + static_cast<size_t>(hid) * (n + 1);
  if (delta < 4.0) {
    // dense: one position per thread, consecutive threads write consecutive
    // starts.  Four positions per thread and step: the four words (bitmap and
    // offset in one read each; indices clamped into the array, the stores
    // guarded) are read before any store, and the offsets are pinned in
    // registers there, so the compiler cannot move the reads into the store
    // branches, which would serialise one LDS round trip per position.
    const int last = nwords - 1;
    for (int x0 = tid; x0 < n; x0 += 4 * kThreads) {
      uint2 e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = wd[min((x0 + k * kThreads) >> 5, last)];
      int o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int x = x0 + k * kThreads;
        o[k] = static_cast<int>(e[k].y) + __popc(e[k].x & ((1u << (x & 31)) - 1u));
        asm volatile("" : "+v"(o[k]));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int x = x0 + k * kThreads;
        if (x < n && ((e[k].x >> (x & 31)) & 1u)) st[o[k]] = x;
      }
    }
  } else {
    for (int w = tid; w < nused; w += kThreads) {
      const uint2 e = wd[w];
      uint32_t m = e.x;
      int b = static_cast<int>(e.y);
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
    const uint2 e0 = wd[x0w], el = wd[xlw];
    const int kb0 = static_cast<int>(e0.y) + __popc(e0.x & (0xFFFFFFFFu >> (31 - (r0 & 31)))) - 1;
    const int kbl = static_cast<int>(el.y) + __popc(el.x & (0xFFFFFFFFu >> (31 - (rl & 31)))) - 1;
    PlanRec rec;
    rec.a = st[kb0];
    rec.e = st[kb0 + 1];
    rec.a2 = st[kbl];
    rec.e2 = st[kbl + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) rec.bits[j] = wd[x0w + j].x;
    rec.bits[0] &= ~1u;
    if (n - r0 < kPlanTile) {
      const int p = n - r0;
#pragma unroll
      for (int j = 0; j < 4; ++j) rec.bits[j] |= (p >> 5) == j ? 1u << (p & 31) : 0u;
    }
    pl[static_cast<size_t>(q) * s] = rec;
  }
}

// ---- part kernel

constexpr int kPartThreads = 256;
constexpr int kPartWords = 256;  // 32-position words per part, one per thread; a multiple of 4, so
                                 // that the four words of a 128-row tile lie in one part

// Exclusive scan of one int per thread over a kPartThreads workgroup.
__device__ int part_exclusive_scan(int v, int* wsum, int* total) {
  constexpr int kW = kPartThreads / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kW; ++k) {
    base += k < w ? wsum[k] : 0;
    tot += wsum[k];
  }
  *total = tot;
  return base + x - v;
}

// One part (blockIdx.y) of one hash (blockIdx.x).
//
// Closed form of the start count.  With n <= 2^19 and u <= delta, the
// computed difference x - u of consecutive positions is 1 within 2^-32 when
// delta < 2^19 (larger delta: within 2^-51 delta), and the rounded quotient
// adds at most 2^-34 / delta each.  So consecutive computed quotients differ
// by more than 1 when delta <= 1 - 2^-30 (every position starts a block) and
// by less than 1 when delta >= 1 + 2^-30: bins then rise by 0 or 1 per
// position, every bin value between bin(0) and bin(n - 1) holds a block, and
// the starts in [0, x] number bin(x) - bin(0) + 1.
__global__ __launch_bounds__(kPartThreads) void bins_part_kernel(const double* __restrict__ du, int n, int s,
                                                                 int ntile, int32_t* __restrict__ nblk,
                                                                 int32_t* __restrict__ starts,
                                                                 PlanRec* __restrict__ plan) {
  __shared__ uint2 wd[kPartWords];  // per word: start bitmap, starts before it within the part
  __shared__ int wsum[kPartThreads / 64];
  const int hid = blockIdx.x;
  const int h = hid / s, i = hid - h * s;
  const int tid = threadIdx.x;
  const double delta = du[2 * hid], u = du[2 * hid + 1];
  const bool every = delta <= 1.0 - 0x1p-30;  // else delta >= 1 + 2^-30 (checked by the launcher)
  const bool wide = delta >= 32.0;
  const double rinv = 1.0 / delta;
  const int nused = (n + 31) >> 5;
  const int w0 = blockIdx.y * kPartWords;
  const int w = w0 + tid;

  uint32_t m = 0u;
  if (w < nused) {
    const int x0 = 32 * w;
    double prev;
    m = every ? ~0u : start_flags(x0, u, delta, rinv, wide, &prev);
    if (x0 == 0) m |= 1u;
    if (n - x0 < 32) m &= (1u << (n - x0)) - 1u;
  }
  int total;
  const int local = part_exclusive_scan(__popc(m), wsum, &total);
  wd[tid] = make_uint2(m, static_cast<uint32_t>(local));

  // starts before the part, and in all
  const double b0 = every ? 0.0 : exact_bin(0, u, delta);
  const int x0p = 32 * w0;
  const int before = every ? x0p : (x0p == 0 ? 0 : static_cast<int>(exact_bin(x0p - 1, u, delta) - b0) + 1);
  int32_t* st = starts + static_cast<size_t>(hid) * (n + 1);
  if (every) {
    for (int x = x0p + tid; x < min(x0p + 32 * kPartWords, n); x += kPartThreads) st[x] = x;
  } else {
    int o = before + local;
    while (m) {
      st[o++] = 32 * w + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
  if (blockIdx.y == gridDim.y - 1 && tid == 0) {
    const int nb = every ? n : static_cast<int>(exact_bin(n - 1, u, delta) - b0) + 1;
    nblk[hid] = nb;
    st[nb] = n;
  }
  __syncthreads();

  // plan records of the part's tiles
  const int q = w0 / 4 + tid;
  if (tid < kPartWords / 4 && q < ntile) {
    const int r0 = q * kPlanTile;
    const int rl = min(r0 + kPlanTile - 1, n - 1);
    PlanRec rec;
    if (every) {
      rec.a = r0;
      rec.e = r0 + 1;
      rec.a2 = rl;
      rec.e2 = rl + 1;
    } else {
      const double k0 = exact_bin(r0, u, delta), k1 = exact_bin(rl, u, delta);
      rec.a = first_at_least(k0, u, delta, rinv, n);
      rec.e = first_at_least(k0 + 1.0, u, delta, rinv, n);
      rec.a2 = first_at_least(k1, u, delta, rinv, n);
      rec.e2 = first_at_least(k1 + 1.0, u, delta, rinv, n);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) rec.bits[j] = wd[4 * tid + j].x;
    rec.bits[0] &= ~1u;
    if (n - r0 < kPlanTile) {
      const int p = n - r0;
#pragma unroll
      for (int j = 0; j < 4; ++j) rec.bits[j] |= (p >> 5) == j ? 1u << (p & 31) : 0u;
    }
    plan[(static_cast<size_t>(h) * ntile + q) * s + i] = rec;
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

bool bins_near_one(const double* delta, long long count) {
  for (long long t = 0; t < count; ++t)
    if (delta[t] > 1.0 - 0x1p-30 && delta[t] < 1.0 + 0x1p-30) return true;
  return false;
}

hipError_t launch_bins(const double* du, int heads, int s, int n, void* bins, bool near_one, hipStream_t stream) {
  const BinsLayout L = bins_layout(heads, s, n);
  char* base = static_cast<char*>(bins);
  const int ntile = (n + kPlanTile - 1) / kPlanTile;
  if (!near_one) {
    const int parts = (4 * ntile + kPartWords - 1) / kPartWords;
    hipLaunchKernelGGL(bins_part_kernel, dim3(heads * s, parts), dim3(kPartThreads), 0, stream, du, n, s, ntile,
                       reinterpret_cast<int32_t*>(base + L.off_nblk),
                       reinterpret_cast<int32_t*>(base + L.off_starts),
                       reinterpret_cast<PlanRec*>(base + L.off_plan));
    return hipGetLastError();
  }
  const int nwords = 4 * ntile + 4;  // covers positions < 128 (ntile + 1)
  const size_t lds = static_cast<size_t>(nwords) * 2 * sizeof(uint32_t);
  // opt in to the dynamic LDS this launch needs (the largest request so far)
  static LdsOptIn opt;
  if (hipError_t e = opt.ensure(reinterpret_cast<const void*>(&bins_kernel), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(bins_kernel, dim3(heads * s), dim3(kThreads), lds, stream, du, n, s, ntile, nwords,
                     reinterpret_cast<int32_t*>(base + L.off_nblk),
                     reinterpret_cast<int32_t*>(base + L.off_starts),
                     reinterpret_cast<PlanRec*>(base + L.off_plan));
  return hipGetLastError();
}

}  // namespace plpsh
