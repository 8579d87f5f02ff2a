// Host draw of the random-binning hashes: SplitMix64 in counter mode mapped
// to delta ~ Gamma(2, sigma) (sum of two unit exponentials, scaled) and
// u ~ U[0, delta).  The exact recipe is specified in plpsh.h.
#include <cmath>
#include <cstdint>

#include "internal.h"

namespace plpsh {
namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Open-interval uniform from the top 52 bits: ((z >> 12) + 0.5) * 2^-52.
inline double unit_open(uint64_t z) {
  return (static_cast<double>(z >> 12) + 0.5) * 0x1p-52;
}

}  // namespace

void draw_hash(uint64_t seed, int h, int i, double sigma, double* delta, double* u) {
  double U[3];
  for (int k = 0; k < 3; ++k) {
    const uint64_t c = (static_cast<uint64_t>(h) << 32) | (static_cast<uint64_t>(i) << 2) | static_cast<uint64_t>(k);
    U[k] = unit_open(mix64(seed + (c + 1) * kGamma));
  }
  const double t = (-std::log(U[0])) - std::log(U[1]);
  const double dl = sigma * t;
  *delta = dl;
  *u = dl * U[2];
}

void draw_hashes(uint64_t seed, int heads, int s, const double* sigma, double* delta, double* u) {
  for (int h = 0; h < heads; ++h)
    for (int i = 0; i < s; ++i) draw_hash(seed, h, i, sigma[h], &delta[h * s + i], &u[h * s + i]);
}

}  // namespace plpsh
