// Device evaluation of the bins of a hash, shared by the bin kernels
// (bins.hip) and the attention kernel's own plan of its query tile
// (attn.hip).
//
// Positional LSH (explainer of arXiv 2605.09472, Methodology 1) places the
// integer position x in bin floor((x - u) / delta).  Every function here
// returns exactly what that definition gives in IEEE binary64: the binary64
// difference x - u, its binary64 quotient by delta, and the floor.  A
// product with a rounded reciprocal stands in for the division wherever it
// provably yields the same floor; elsewhere the division itself is taken.
// Contraction of multiplies and adds into fused operations is switched off
// in every function, whatever the including file's flags.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace plpsh {
namespace {

// The bin of x by its definition (binary64 difference, quotient, floor).
__device__ __forceinline__ double exact_bin(int x, double u, double delta) {
#pragma clang fp contract(off)
  return floor((static_cast<double>(x) - u) / delta);
}

// Bin of position x from the product with a rounded reciprocal, which is
// within 2.2 ulp of the quotient: where no integer lies within 2^-50 |q| of
// it the floor equals that of the correctly rounded quotient, and the
// function returns true (certified).
__device__ __forceinline__ bool certified_bin(int x, double u, double rinv, double* f) {
#pragma clang fp contract(off)
  const double q = (static_cast<double>(x) - u) * rinv;
  const double fl = floor(q);
  const double fr = q - fl;  // exact for |q| < 2^52
  const double margin = fabs(q) * 0x1p-50;
  *f = fl;
  return fr > margin && fr < 1.0 - margin;
}

// The bin of x: the certified product, else the division.
__device__ __forceinline__ double bin_at(int x, double u, double delta, double rinv) {
  double f;
  return certified_bin(x, u, rinv, &f) ? f : exact_bin(x, u, delta);
}

// Start flags of the 32 positions x0 .. x0 + 31 (bit b: bin(x0 + b) differs
// from bin(x0 + b - 1)), bins evaluated in binary64 as floor((x - u) / delta);
// *prev receives bin(x0 - 1).
//
// Wide hashes (delta >= 32, the same for the whole workgroup, so the branch
// does not diverge): computed bins never decrease with x (the rounded
// subtraction and division are monotone), and the bins of x0 - 1 and
// x0 + 31 differ by at most one.  Equal bins mean no start in the word;
// bins one apart mean exactly one start, found by bisection (5 more
// evaluations).  Everything else, and any evaluation that is not
// certified, takes the general pass: all 33 bins by certified products,
// and if one of them misses the margin (rare), the division itself.
// The general pass is fully unrolled so that the evaluations overlap.
__device__ __forceinline__ uint32_t start_flags(int x0, double u, double delta, double rinv, bool wide,
                                                double* prev) {
#pragma clang fp contract(off)
  if (wide) {
    double fa, fb;
    bool ok = certified_bin(x0 - 1, u, rinv, &fa);
    ok = certified_bin(x0 + 31, u, rinv, &fb) && ok;
    if (ok && fa == fb) {
      *prev = fa;
      return 0u;
    }
    if (ok && fb == fa + 1.0) {
      int lo = -1, hi = 31;  // bin(x0 + lo) = fa, bin(x0 + hi) = fb
#pragma unroll
      for (int it = 0; it < 5; ++it) {
        const int mid = (lo + hi) >> 1;
        double fm;
        ok = certified_bin(x0 + mid, u, rinv, &fm) && ok;
        if (fm == fb) hi = mid; else lo = mid;
      }
      if (ok) {
        *prev = fa;
        return 1u << hi;
      }
    }
  }
  // The 33 bins from one product and then one fused multiply-add each:
  // q_k = k rinv + q_0 lies within 36 2^-53 max(|q_0|, |q_k|, 32 / delta) of
  // the exact quotient (q_0's three roundings, k times the reciprocal's, the
  // fma's own), and the binary64 quotient of the definition within 2^-52 |q|
  // of it, so a fractional part farther than 2^-47 max(|q_0|, |q_32|,
  // 32 rinv) from an integer settles the floor.
  const double q0 = (static_cast<double>(x0 - 1) - u) * rinv;
  const double margin = 0x1p-47 * fmax(fmax(fabs(q0), fabs(fma(32.0, rinv, q0))), 32.0 * rinv);
  double f[33];
  bool exact = false;
#pragma unroll
  for (int k = 0; k < 33; ++k) {
    const double q = fma(static_cast<double>(k), rinv, q0);
    const double fl = floor(q);
    const double fr = q - fl;  // exact for |q| < 2^52
    f[k] = fl;
    exact = exact || !(fr > margin && fr < 1.0 - margin);
  }
  uint32_t m = 0u;
  if (!exact) {
    *prev = f[0];
#pragma unroll
    for (int b = 0; b < 32; ++b) m |= static_cast<uint32_t>(f[b + 1] != f[b]) << b;
  } else {
    double pv = exact_bin(x0 - 1, u, delta);
    *prev = pv;
    for (int b = 0; b < 32; ++b) {
      const double bb = exact_bin(x0 + b, u, delta);
      m |= static_cast<uint32_t>(bb != pv) << b;
      pv = bb;
    }
  }
  return m;
}

// Smallest x in [0, n] with bin(x) >= k (n if there is none).  Bins never
// decrease with x; the real-number answer ceil(k delta + u) is taken as the
// first guess, rounding moves the answer by at most a position or two, and a
// bisection settles anything further.
__device__ __forceinline__ int first_at_least(double k, double u, double delta, double rinv, int n) {
#pragma clang fp contract(off)
  const double gd = ceil(fma(k, delta, u));
  int g = gd <= 0.0 ? 0 : (gd >= static_cast<double>(n) ? n : static_cast<int>(gd));
  for (int it = 0; it < 4; ++it) {
    if (g > 0 && bin_at(g - 1, u, delta, rinv) >= k) {
      --g;
    } else if (g < n && bin_at(g, u, delta, rinv) < k) {
      ++g;
    } else {
      return g;
    }
  }
  int lo = 0, hi = n;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (bin_at(mid, u, delta, rinv) >= k) hi = mid; else lo = mid + 1;
  }
  return lo;
}

}  // namespace
}  // namespace plpsh
