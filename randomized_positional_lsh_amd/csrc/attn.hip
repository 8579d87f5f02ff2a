// Count-weighted windowed attention on gfx950 matrix cores.
//
// Computes, for every query row r (explainer of arXiv 2605.09472,
// Theorem 2.1 and Theorem 2.2 with the mask mean M~ in place of the ALiBi
// matrix L*):
//
//   O_r = sum_j c[r,j] C[r,j] e^{S[r,j]} v_j / sum_j c[r,j] C[r,j] e^{S[r,j]},
//   c[r,j] = #{i : bin_i(r) == bin_i(j)},  S = Q K^T / sqrt(d).
//
// All s hashes share one pass over the keys: the logits and the exponentials
// are computed once per (query, key) pair and weighted by the integer count
// c, which is itself produced by the matrix cores in the layout of S.
//
// Work decomposition.  One workgroup (4 waves) owns 128 query rows of one
// (batch, head); wave w owns rows 32w..32w+31 as two 16-row blocks.  Keys
// are streamed in 64-key tiles through LDS (double buffered): first the two
// "near" tiles covering the query rows themselves, then the tiles to the
// left down to the smallest block start of the tile's first row, then (when
// not causal) the tiles to the right up to the largest block end of its last
// row.  Nothing outside that window can have c > 0.
//
// Counts as a matrix product (exact small integers in bf16, fp32 result):
//  * keys left of the tile (j < r0): hash i contributes to (r, j) iff its
//    block [a_i, e_i) containing r0 also contains r and j, i.e.
//    [r < e_i] [j >= a_i].  So c = U V^T over a K dimension of one slot per
//    hash, with U[r,i] = [r < e_i] (fixed per query tile) and
//    V[j,i] = [j >= a_i], a prefix of ones once the hashes are sorted by a_i.
//  * keys right of the tile: symmetric with the block containing the last row.
//  * keys among the tile's own rows: c[r,j] = sum_{p <= j} H[r,p] where
//    H[r,p] counts hashes whose block of r starts at p (clamped to r0) minus
//    those whose block of r ends at p; the sum over p <= j is a product with
//    the constant lower-triangular matrix [p <= j] (K = 128 positions).
//
// Softmax: running row maximum shared by all hashes, rescaled only when a
// tile's maximum exceeds it by more than 2^8 in the exponential (so the
// rescale is rare); masked entries (c = 0, or j > r when causal) enter as
// -inf; the first tile processed contains the diagonal, where c = s > 0.
//
// The dense exact-ALiBi variant (MODE_ALIBI) uses the same skeleton with the
// weight e^{S - |r-j|/sigma} over every key.
#include <climits>
#include <type_traits>

#include "internal.h"

namespace plpsh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;   // threads per workgroup
constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int MAXS = 128; // hashes per head
constexpr float kLog2e = 1.4426950408889634f;

enum { MODE_PLSH = 0, MODE_ALIBI = 1 };
enum { KIND_NEAR = 0, KIND_LEFT = 1, KIND_RIGHT = 2 };

struct HeadOrder { uint16_t h[1024]; };  // heads, most expensive first
struct HeadScale { float beta[256]; };   // log2(e) / sigma_h (dense ALiBi)

struct FwdArgs {
  const void* q; const void* k; const void* v; void* o;
  const PlanRec* plan;
  int B, Hq, Hkv, n, s, ntile, cs;
};

template <int D, bool BF, int MODE>
struct Cfg {
  using T = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr int EPC = 16 / sizeof(T);           // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per key row
  static constexpr int KSTR = D + EPC;                 // K row stride (elements), +16 bytes
  static constexpr int VSTR = BN + 4;                  // transposed V row stride (keys)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int KV_BYTES = 2 * (K_ELEMS + V_ELEMS) * static_cast<int>(sizeof(T));
  static constexpr int HSTR = BM + 8;                  // H row stride (bf16)
  static constexpr int H_BYTES = MODE == MODE_PLSH ? BM * HSTR * 2 : 0;
  static constexpr int BIG = ((KV_BYTES > H_BYTES ? KV_BYTES : H_BYTES) + 15) / 16 * 16;
  static constexpr int SMALL = MODE == MODE_PLSH ? MAXS * 32 + 4 * MAXS * 4 + 9 * 16 + 64 : 64;
  static constexpr int LDS = BIG + SMALL;
  static constexpr int KLD = BN * CPR / NT;            // 16-byte K loads per thread
  static constexpr int UNITS = (BN / 4) * CPR;         // 4-key x 16-byte V units
  static constexpr int VIT = (UNITS + NT - 1) / NT;    // V units per thread
  static constexpr int KS = BF ? D / 32 : D / 4;       // k-steps of the logit product
  static constexpr int DB = D / 16;                    // 16-wide output column blocks
};

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_exact(float x) {  // x is a small integer
  return static_cast<uint16_t>(__float_as_uint(x) >> 16);
}
__device__ __forceinline__ float xmax16(float x) {  // max over the 4 lanes sharing lane & 15
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float xsum16(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}
__device__ __forceinline__ int clamp08(int x) { return x < 0 ? 0 : (x > 8 ? 8 : x); }

template <int D, bool BF, int MODE>
struct Tile {
  using C = Cfg<D, BF, MODE>;
  using T = typename C::T;
  u32x4 k[C::KLD];
  u32x4 v[C::VIT][4];

  __device__ __forceinline__ void load(const T* __restrict__ Kp, const T* __restrict__ Vp, int j0, int n,
                                       int tid) {
#pragma unroll
    for (int it = 0; it < C::KLD; ++it) {
      const int idx = tid + NT * it;
      const int key = idx / C::CPR, ch = idx % C::CPR;
      const int j = j0 + key;
      k[it] = (j >= 0 && j < n) ? *reinterpret_cast<const u32x4*>(Kp + static_cast<size_t>(j) * D + ch * C::EPC)
                                : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = tid + NT * it;
      const int ch = u % C::CPR, kq = u / C::CPR;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = j0 + 4 * kq + t;
        v[it][t] = (u < C::UNITS && j >= 0 && j < n)
                       ? *reinterpret_cast<const u32x4*>(Vp + static_cast<size_t>(j) * D + ch * C::EPC)
                       : u32x4{0, 0, 0, 0};
      }
    }
  }

  // K row-major [key][dim]; V transposed [dim][key].
  __device__ __forceinline__ void store(T* __restrict__ sK, T* __restrict__ sV, int tid) const {
#pragma unroll
    for (int it = 0; it < C::KLD; ++it) {
      const int idx = tid + NT * it;
      const int key = idx / C::CPR, ch = idx % C::CPR;
      *reinterpret_cast<u32x4*>(sK + key * C::KSTR + ch * C::EPC) = k[it];
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int u = tid + NT * it;
      if (u >= C::UNITS) continue;
      const int ch = u % C::CPR, kq = u / C::CPR;
      if constexpr (BF) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t r0 = v[it][0][m], r1 = v[it][1][m], r2 = v[it][2][m], r3 = v[it][3][m];
          const u32x2 lo = {(r0 & 0xFFFFu) | (r1 << 16), (r2 & 0xFFFFu) | (r3 << 16)};
          const u32x2 hi = {(r0 >> 16) | (r1 & 0xFFFF0000u), (r2 >> 16) | (r3 & 0xFFFF0000u)};
          const int dim = ch * 8 + 2 * m;
          *reinterpret_cast<u32x2*>(sV + dim * C::VSTR + 4 * kq) = lo;
          *reinterpret_cast<u32x2*>(sV + (dim + 1) * C::VSTR + 4 * kq) = hi;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4 col = {v[it][0][m], v[it][1][m], v[it][2][m], v[it][3][m]};
          *reinterpret_cast<u32x4*>(sV + (ch * 4 + m) * C::VSTR + 4 * kq) = col;
        }
      }
    }
  }
};

template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
__global__ __launch_bounds__(NT, (Cfg<D, BF, MODE>::LDS > 80 * 1024 ? 1 : 2)) void fwd_kernel(FwdArgs A, HeadOrder ord,
                                                                                     HeadScale hsc) {
  using C = Cfg<D, BF, MODE>;
  using T = typename C::T;
  constexpr bool PL = MODE == MODE_PLSH;
  constexpr int KS = C::KS, DB = C::DB;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sKb = reinterpret_cast<T*>(smem);
  T* sVb = sKb + 2 * C::K_ELEMS;
  uint16_t* sH = reinterpret_cast<uint16_t*>(smem);
  unsigned char* sm = smem + C::BIG;
  PlanRec* sRec = reinterpret_cast<PlanRec*>(sm);
  int* sAa = reinterpret_cast<int*>(sm + MAXS * 32);  // a_i sorted ascending
  int* sAe = sAa + MAXS;                             // e_i in that order
  int* sEe = sAe + MAXS;                             // e2_i sorted descending
  int* sEa = sEe + MAXS;                             // a2_i in that order
  u32x4* sTh = reinterpret_cast<u32x4*>(sEa + MAXS); // thermometer patterns
  int* sSc = reinterpret_cast<int*>(sTh + 9);         // window scalars

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- work item: XCD-aware order (consecutive tiles of a head share an XCD)
  const int gid = blockIdx.x;
  const int xcd = gid & 7, kk = gid >> 3;
  const int inst = kk / A.cs;
  const int qt = xcd * A.cs + kk % A.cs;
  if (qt >= A.ntile) return;
  const int b = inst % A.B;
  const int h = ord.h[inst / A.B];
  const int kvh = h / (A.Hq / A.Hkv);
  const int n = A.n, s = A.s;
  const int r0 = qt * BM;
  const int nrows = min(BM, n - r0);
  const int rlast = r0 + nrows - 1;
  const T* __restrict__ Qp = static_cast<const T*>(A.q) + static_cast<size_t>(b * A.Hq + h) * n * D;
  const T* __restrict__ Kp = static_cast<const T*>(A.k) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
  const T* __restrict__ Vp = static_cast<const T*>(A.v) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
  T* __restrict__ Op = static_cast<T*>(A.o) + static_cast<size_t>(b * A.Hq + h) * n * D;

  // rows of this lane: R[rb] = r0 + 32 w + 16 rb + l16 (relative: rr[rb])
  int rr[2], R[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    rr[rb] = 32 * w + 16 * rb + l16;
    R[rb] = r0 + rr[rb];
  }

  // ---- Q fragments (operand B of S^T = K Q^T)
  u32x4 qb[2][BF ? KS : 1];
  float qf[2][BF ? 1 : KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const bool ok = R[rb] < n;
    const T* qrow = Qp + static_cast<size_t>(ok ? R[rb] : 0) * D;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[rb][ks] = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int c4 = 0; c4 < KS / 4; ++c4) {
        const u32x4 x = ok ? *reinterpret_cast<const u32x4*>(qrow + KS * g + 4 * c4) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[rb][4 * c4 + e] = __uint_as_float(x[e]);
      }
    }
  }

  // ---- window of keys that can carry weight
  int lo, hi, afull = INT_MAX, efull = INT_MIN, cntA = 0;
  u32x4 hf[2][PL ? 4 : 1];          // near counts H (operand B), [rb][position chunk]
  u32x4 ufl[2][PL ? NCH : 1];       // left:  [r < e_slot]
  u32x4 ufr[2][PL && !CAUSAL ? NCH : 1];  // right: [r >= a2_slot]
  if constexpr (PL) {
    if (tid < s) sRec[tid] = A.plan[(static_cast<size_t>(h) * A.ntile + qt) * s + tid];
    if (tid < 9) {
      u32x4 p;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        p[q] = (tid >= 2 * q + 2) ? 0x3F803F80u : (tid == 2 * q + 1 ? 0x00003F80u : 0u);
      sTh[tid] = p;
    }
    for (int x = tid; x < C::H_BYTES / 16; x += NT) reinterpret_cast<u32x4*>(sH)[x] = u32x4{0, 0, 0, 0};
    __syncthreads();
    if (tid < s) {
      const PlanRec me = sRec[tid];
      int rk = 0, rk2 = 0;
      for (int k2 = 0; k2 < s; ++k2) {
        const int ak = sRec[k2].a, ek = sRec[k2].e2;
        rk += (ak < me.a) || (ak == me.a && k2 < tid);
        rk2 += (ek > me.e2) || (ek == me.e2 && k2 < tid);
      }
      sAa[rk] = me.a;
      sAe[rk] = me.e;
      sEe[rk2] = me.e2;
      sEa[rk2] = me.a2;
    }
    if (w == 0) {
      int vlo = INT_MAX, vhi = INT_MIN, vaf = INT_MAX, vef = INT_MIN, vca = 0;
      for (int i = lane; i < s; i += 64) {
        const PlanRec& Rr = sRec[i];
        vlo = min(vlo, Rr.a);
        vhi = max(vhi, Rr.e2);
        if (Rr.e > rlast) vaf = min(vaf, Rr.a);
        if (Rr.a2 <= r0) vef = max(vef, Rr.e2);
        vca += Rr.a < r0;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        vlo = min(vlo, __shfl_xor(vlo, o, 64));
        vhi = max(vhi, __shfl_xor(vhi, o, 64));
        vaf = min(vaf, __shfl_xor(vaf, o, 64));
        vef = max(vef, __shfl_xor(vef, o, 64));
        vca += __shfl_xor(vca, o, 64);
      }
      if (lane == 0) {
        sSc[0] = vlo; sSc[1] = vhi; sSc[2] = vaf; sSc[3] = vef; sSc[4] = vca;
      }
    }
    // near counts: thread p owns row r0 + p of H
    if (tid < BM) {
      const int p = tid, wp = p >> 5, bp = p & 31;
      uint16_t* Hrow = sH + p * C::HSTR;
      for (int i = 0; i < s; ++i) {
        const u32x4 bw = *reinterpret_cast<const u32x4*>(sRec[i].bits);
        int st = 0, en = BM;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t le = q < wp ? 0xFFFFFFFFu : (q == wp ? (0xFFFFFFFFu >> (31 - bp)) : 0u);
          const uint32_t m = bw[q] & le;
          if (m) st = 32 * q + 31 - __clz(m);
        }
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          const uint32_t gt = q > wp ? 0xFFFFFFFFu : (q == wp ? (bp == 31 ? 0u : (0xFFFFFFFEu << bp)) : 0u);
          const uint32_t m = bw[q] & gt;
          if (m) en = 32 * q + __ffs(m) - 1;
        }
        Hrow[st] = f32_to_bf16_exact(bf16_bits_to_f32(Hrow[st]) + 1.0f);
        if (en < BM) Hrow[en] = f32_to_bf16_exact(bf16_bits_to_f32(Hrow[en]) - 1.0f);
      }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        hf[rb][ch] = *reinterpret_cast<const u32x4*>(sH + rr[rb] * C::HSTR + 32 * ch + 8 * g);
    // count operands for the side tiles
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        u32x4 f = {0, 0, 0, 0}, f2 = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int slot = 32 * ch + 8 * g + t;
          const bool in = slot < s;
          const uint32_t one = 0x3F80u << (16 * (t & 1));
          if (in && R[rb] < sAe[slot]) f[t >> 1] |= one;
          if (!CAUSAL && in && R[rb] >= sEa[slot]) f2[t >> 1] |= one;
        }
        ufl[rb][ch] = f;
        if constexpr (!CAUSAL) ufr[rb][ch] = f2;
      }
    }
    lo = sSc[0];
    hi = sSc[1];
    afull = sSc[2];
    efull = sSc[3];
    cntA = sSc[4];
    __syncthreads();  // H region is reused for K/V from here on
  } else {
    lo = 0;
    hi = n;
  }

  // ---- tile list
  const int nnear = nrows > BN ? 2 : 1;
  const int nleft = lo < r0 ? (r0 - lo + BN - 1) / BN : 0;
  const int nright = (!CAUSAL && hi > r0 + BM) ? (hi - (r0 + BM) + BN - 1) / BN : 0;
  const int ntl = nnear + nleft + nright;
  auto tile_j0 = [&](int t) {
    return t < nnear ? r0 + BN * t
                     : (t < nnear + nleft ? r0 - BN * (t - nnear + 1) : r0 + BM + BN * (t - nnear - nleft));
  };

  // ---- softmax state
  const float sc = rsqrtf(static_cast<float>(D)) * kLog2e;   // logit -> log2 units
  const float scp = MODE == MODE_PLSH ? sc : 1.0f;            // scale applied at exp time
  const float thr = 8.0f / scp;                               // rescale threshold (logit units)
  const float beta = MODE == MODE_ALIBI ? hsc.beta[h] : 0.0f;
  float Mrow[2] = {-INFINITY, -INFINITY}, Msc[2] = {0.f, 0.f}, lsum[2] = {0.f, 0.f};
  f32x4 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // side-tile count state (uniform)
  int lcnt_hi = cntA, rA = s, rB = s;

  Tile<D, BF, MODE> tl;
  tl.load(Kp, Vp, tile_j0(0), n, tid);
  tl.store(sKb, sVb, tid);
  __syncthreads();

  for (int t = 0; t < ntl; ++t) {
    const int buf = t & 1;
    const T* sK = sKb + buf * C::K_ELEMS;
    const T* sV = sVb + buf * C::V_ELEMS;
    const int j0 = tile_j0(t);
    const int kind = t < nnear ? KIND_NEAR : (t < nnear + nleft ? KIND_LEFT : KIND_RIGHT);
    if (t + 1 < ntl) tl.load(Kp, Vp, tile_j0(t + 1), n, tid);

    // per-lane count of sorted hashes active at this lane's key of each 16-key block
    int mkey[4] = {0, 0, 0, 0};
    if constexpr (PL) {
      if (kind == KIND_LEFT) {
        int clo = lcnt_hi;
        while (clo > 0 && sAa[clo - 1] >= j0) --clo;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mkey[kb] = clo;
        for (int x = clo; x < lcnt_hi; ++x) {
          const int av = sAa[x];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mkey[kb] += (j0 + 16 * kb + l16 >= av);
        }
        lcnt_hi = clo;
      } else if (!CAUSAL && kind == KIND_RIGHT) {
        while (rA > 0 && sEe[rA - 1] < j0 + BN) --rA;
        while (rB > 0 && sEe[rB - 1] <= j0) --rB;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mkey[kb] = rA;
        for (int x = rA; x < rB; ++x) {
          const int ev = sEe[x];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mkey[kb] += (ev > j0 + 16 * kb + l16);
        }
      }
    }
    bool need_mask;
    if constexpr (PL)
      need_mask = kind == KIND_NEAR || (kind == KIND_LEFT && j0 < afull) || (kind == KIND_RIGHT && j0 + BN > efull);
    else
      need_mask = kind == KIND_NEAR || j0 < 0 || j0 + BN > n;

#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int jc = j0 + 32 * kc;
      // causal: skip key chunks entirely above this wave's last row
      if (CAUSAL && kind == KIND_NEAR && jc > r0 + 32 * w + 31) continue;

      f32x4 sacc[2][2], cacc[2][2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sacc[x][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          cacc[x][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      // S^T = K Q^T
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int kb = 2 * kc + kb2;
        const T* krow = sK + (16 * kb + l16) * C::KSTR;
        if constexpr (BF) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 32 * ks + 8 * g);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sacc[kb2][rb] = mfma_bf16(a, qb[rb][ks], sacc[kb2][rb]);
          }
        } else {
#pragma unroll
          for (int c4 = 0; c4 < KS / 4; ++c4) {
            const u32x4 a4 = *reinterpret_cast<const u32x4*>(krow + KS * g + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                sacc[kb2][rb] = mfma_f32(__uint_as_float(a4[e]), qf[rb][4 * c4 + e], sacc[kb2][rb]);
          }
        }
      }
      // counts c^T in the layout of S^T
      if constexpr (PL) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int kb = 2 * kc + kb2;
          if (kind == KIND_NEAR) {
            const int jrel0 = j0 - r0 + 16 * kb;          // first key of the block, relative to r0
            const int jrel = jrel0 + l16;
            int chmax = (jrel0 + 15) >> 5;
            if (CAUSAL) chmax = min(chmax, w);
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
              if (ch > chmax) break;
              const u32x4 th = sTh[clamp08(jrel - 32 * ch - 8 * g + 1)];
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) cacc[kb2][rb] = mfma_bf16(th, hf[rb][ch], cacc[kb2][rb]);
            }
          } else if (kind == KIND_LEFT) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
              const u32x4 th = sTh[clamp08(mkey[kb] - 32 * ch - 8 * g)];
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) cacc[kb2][rb] = mfma_bf16(th, ufl[rb][ch], cacc[kb2][rb]);
            }
          } else if constexpr (!CAUSAL) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
              const u32x4 th = sTh[clamp08(mkey[kb] - 32 * ch - 8 * g)];
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) cacc[kb2][rb] = mfma_bf16(th, ufr[rb][ch], cacc[kb2][rb]);
            }
          }
        }
      }
      // masking and the tile's row maxima
      float tmx[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int J = jc + 16 * kb2 + 4 * g + e;
            float x = sacc[kb2][rb][e];
            if constexpr (MODE == MODE_ALIBI) {
              const float dist = fabsf(static_cast<float>(R[rb] - J));
              x = fmaf(x, sc, -beta * dist);
            }
            if (need_mask) {
              bool ok;
              if constexpr (PL)
                ok = cacc[kb2][rb][e] > 0.5f;
              else
                ok = J >= 0 && J < n;
              if (CAUSAL && kind == KIND_NEAR) ok = ok && (J <= R[rb]);
              x = ok ? x : -INFINITY;
            }
            sacc[kb2][rb][e] = x;
            mx = fmaxf(mx, x);
          }
        }
        tmx[rb] = xmax16(mx);
      }
      const bool grow = tmx[0] > Mrow[0] + thr || tmx[1] > Mrow[1] + thr;
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float mn = fmaxf(Mrow[rb], tmx[rb]);
          const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((Mrow[rb] - mn) * scp);
          Mrow[rb] = mn;
          Msc[rb] = mn == -INFINITY ? 0.0f : mn * scp;
          lsum[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][rb] *= alpha;
        }
      }
      // weights and the value product O^T += V^T P^T
      if constexpr (BF) {
        u32x4 pf[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float p[2][4];
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][rb][e], scp, -Msc[rb]));
              if constexpr (PL) x *= cacc[kb2][rb][e];
              p[kb2][e] = x;
              lsum[rb] += x;
            }
          pf[rb] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                         pack_bf16(p[1][2], p[1][3])};
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const T* vrow = sV + (16 * db + l16) * C::VSTR + 32 * kc + 4 * g;
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 16);
          const u32x4 a = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[db][rb] = mfma_bf16(a, pf[rb], acc[db][rb]);
        }
      } else {
        float p[2][2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][rb][e], scp, -Msc[rb]));
              if constexpr (PL) x *= cacc[kb2][rb][e];
              p[rb][kb2][e] = x;
              lsum[rb] += x;
            }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const u32x4 a4 =
                *reinterpret_cast<const u32x4*>(sV + (16 * db + l16) * C::VSTR + 32 * kc + 16 * kb2 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                acc[db][rb] = mfma_f32(__uint_as_float(a4[e]), p[rb][kb2][e], acc[db][rb]);
          }
        }
      }
    }

    if (t + 1 < ntl) {
      // buf ^ 1 was last read in the previous iteration, which every wave left
      // through the barrier below; one barrier per tile publishes the store.
      tl.store(sKb + (buf ^ 1) * C::K_ELEMS, sVb + (buf ^ 1) * C::V_ELEMS, tid);
      __syncthreads();
    }
  }

  // ---- epilogue: O_r = acc / l
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = xsum16(lsum[rb]);
    const float inv = 1.0f / l;
    if (R[rb] >= n) continue;
    T* orow = Op + static_cast<size_t>(R[rb]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o = acc[db][rb] * inv;
      if constexpr (BF) {
        *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g) = u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
      } else {
        *reinterpret_cast<f32x4*>(orow + 16 * db + 4 * g) = o;
      }
    }
  }
}

template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
hipError_t launch_one(const FwdArgs& a, const HeadOrder& ord, const HeadScale& hs, int grid, hipStream_t st) {
  using C = Cfg<D, BF, MODE>;
  auto kfn = fwd_kernel<D, BF, CAUSAL, NCH, MODE>;
  static bool attr_done = false;  // benign race: idempotent
  if (C::LDS > 64 * 1024 && !attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(NT), C::LDS, st, a, ord, hs);
  return hipGetLastError();
}

template <int D, bool BF, bool CAUSAL, int MODE>
hipError_t dispatch_nch(const FwdArgs& a, const HeadOrder& o, const HeadScale& hs, int grid, hipStream_t st) {
  if constexpr (MODE == MODE_ALIBI) {
    return launch_one<D, BF, CAUSAL, 1, MODE>(a, o, hs, grid, st);
  } else {
    if (a.s <= 32) return launch_one<D, BF, CAUSAL, 1, MODE>(a, o, hs, grid, st);
    if (a.s <= 64) return launch_one<D, BF, CAUSAL, 2, MODE>(a, o, hs, grid, st);
    return launch_one<D, BF, CAUSAL, 4, MODE>(a, o, hs, grid, st);
  }
}

template <int MODE>
hipError_t dispatch(const FwdArgs& a, const HeadOrder& o, const HeadScale& hs, int d, int dtype, int causal,
                    int grid, hipStream_t st) {
  const bool bf = dtype == 1;
#define PLPSH_CASE(DD, BB, CC) \
  if (d == DD && bf == BB && (causal != 0) == CC) return dispatch_nch<DD, BB, CC, MODE>(a, o, hs, grid, st);
  PLPSH_CASE(64, true, false)
  PLPSH_CASE(64, true, true)
  PLPSH_CASE(128, true, false)
  PLPSH_CASE(128, true, true)
  PLPSH_CASE(64, false, false)
  PLPSH_CASE(64, false, true)
  PLPSH_CASE(128, false, false)
  PLPSH_CASE(128, false, true)
#undef PLPSH_CASE
  return hipErrorInvalidValue;
}

int grid_size(int ntile, int instances, int* cs) {
  *cs = (ntile + 7) / 8;
  return 8 * *cs * instances;
}

}  // namespace

hipError_t launch_plsh_fwd(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                           int n, int d, int dtype, int s, int causal, const void* bins, const uint16_t* order,
                           hipStream_t st) {
  const BinsLayout L = bins_layout(hq, s, n);
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.plan = reinterpret_cast<const PlanRec*>(static_cast<const char*>(bins) + L.off_plan);
  a.B = batch; a.Hq = hq; a.Hkv = hkv; a.n = n; a.s = s;
  a.ntile = (n + BM - 1) / BM;
  const int grid = grid_size(a.ntile, batch * hq, &a.cs);
  HeadOrder ord;
  for (int i = 0; i < hq; ++i) ord.h[i] = order[i];
  HeadScale hs{};
  return dispatch<MODE_PLSH>(a, ord, hs, d, dtype, causal, grid, st);
}

hipError_t launch_alibi_fwd(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                            int n, int d, int dtype, const float* beta, int causal, hipStream_t st) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.plan = nullptr;
  a.B = batch; a.Hq = hq; a.Hkv = hkv; a.n = n; a.s = 1;
  a.ntile = (n + BM - 1) / BM;
  const int grid = grid_size(a.ntile, batch * hq, &a.cs);
  HeadOrder ord;
  for (int i = 0; i < hq; ++i) ord.h[i] = static_cast<uint16_t>(i);
  HeadScale hs{};
  for (int i = 0; i < hq; ++i) hs.beta[i] = beta[i];
  return dispatch<MODE_ALIBI>(a, ord, hs, d, dtype, causal, grid, st);
}

}  // namespace plpsh
