// Count-weighted windowed attention on gfx950 matrix cores.
//
// Computes, for every query row r (explainer of arXiv 2605.09472,
// Theorem 2.1 and Theorem 2.2 with the mask mean M~ in place of the ALiBi
// matrix L*):
//
//   O_r = sum_j c[r,j] C[r,j] e^{S[r,j]} v_j / sum_j c[r,j] C[r,j] e^{S[r,j]},
//   c[r,j] = #{i : bin_i(r) == bin_i(j)},  S = Q K^T / sqrt(d).
//
// All s hashes share one pass over the keys: the logits and exponentials are
// computed once per (query, key) pair and weighted by the integer count c,
// which the matrix cores produce in the layout of S.
//
// Work decomposition.  One workgroup (NW waves) owns 128 query rows of one
// (batch, head); wave w owns rows WR w .. WR w + WR - 1 as 16-row blocks.  Keys
// stream through LDS in 64-key tiles, two stages deep, loaded straight from
// HBM into LDS by buffer loads (rows past the sequence end read as zero).
// Order: the two "near" tiles holding the query rows themselves, then tiles
// to the left down to the smallest block start of the first row, then (not
// causal) tiles to the right up to the largest block end of the last row;
// nothing outside that window has c > 0.
//
// LDS layouts.  K and V tiles are row-major (one key per row) with their
// 16-byte chunks XOR-swizzled by key so that the logit operand reads (one
// 16-byte chunk per lane) and the transposing value-operand reads
// (ds_read_b64_tr_b16: lane 4a+b of each 16-lane group receives element b
// of lanes a, a+4, a+8, a+12) are free of bank conflicts.
//
// Counts as matrix products (exact small integers in bf16, fp32 result):
//  * keys left of the tile (j < r0): hash i adds 1 to (r, j) iff its block
//    [a_i, e_i) containing r0 also contains r and j, i.e. [r < e_i][j >= a_i].
//    So c = U V^T with one K-slot per hash: U[r,i] = [r < e_i] is fixed per
//    query tile and V[j,i] = [j >= a_i] is a prefix of ones once the hashes
//    are sorted by a_i (taken from a 9-entry table of bf16 prefixes).
//  * keys right of the tile: the same with the block containing the last row.
//  * keys among the tile's own rows: c[r,j] = sum_{p <= j} H[r,p] where H
//    counts hashes whose block of r starts at position p (clamped to r0)
//    minus those whose block of r ends at p; summing over p <= j is a
//    product with the constant matrix [p <= j] (K = 128 positions).  With
//    the causal cut every block of r ends at r + 1, so H holds -s there and
//    the product gives c = 0 past the row.
//
// Masking: c is exactly 0 off a row's support (and, causal, past the row)
// and at least 1 on it, so chunks that straddle a support edge mask on c.
//
// Softmax: one running row maximum shared by all hashes.  It is raised only
// when a tile exceeds it by more than 2^8 in the exponential, so rescaling
// is rare; masked entries (c = 0, or j > r when causal) enter as -inf; the
// first tile holds the diagonal, where c = s > 0.
//
// MODE_ALIBI computes exact dense ALiBi attention, weight e^{S - |r-j|/sigma},
// over every key with the same pipeline.
#include <climits>
#include <type_traits>

#include "internal.h"

namespace plpsh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) unsigned char lds_uchar_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;    // query rows per workgroup
constexpr int NRB = 1;     // 16-row blocks per wave
constexpr int WR = 16 * NRB;  // query rows per wave
constexpr int NW = BM / WR;   // waves per workgroup
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr int BN = 64;     // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

enum { MODE_PLSH = 0, MODE_ALIBI = 1, MODE_LITERAL = 2 };
enum { KIND_NEAR = 0, KIND_LEFT = 1, KIND_RIGHT = 2 };

// heads, most expensive first, two 16-bit entries per word (dword elements
// keep the lookup a scalar load)
struct HeadOrder {
  uint32_t w[512];
  __host__ __device__ int get(int i) const { return static_cast<int>((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu); }
  void set(int i, int h) { w[i >> 1] |= static_cast<uint32_t>(h) << (16 * (i & 1)); }
};
struct HeadScale { float beta[256]; };   // log2(e) / sigma_h (dense ALiBi)

struct FwdArgs {
  const void* q; const void* k; const void* v; void* o;
  const PlanRec* plan;
  float* lse;  // optional: log of each row's normaliser, [B, Hq, n]
  int B, Hq, Hkv, n, s, ntile, cs;
};

template <int D, bool BF>
struct Geo {
  using T = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr int ES = sizeof(T);
  static constexpr int RB = D * ES;                  // bytes per key row
  static constexpr int CPR = RB / 16;                // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;              // rows per 1 KB load instruction
  static constexpr int TILE = BN * RB;               // bytes of one K or V tile
  static constexpr int NI = TILE / 1024 / NW;        // load instructions per wave per matrix
  static_assert(TILE % (1024 * NW) == 0, "tile loads split evenly over the waves");
  static constexpr int STAGE = 2 * TILE;             // K tile + V tile
  static constexpr int HC = (BM + 1) * BM * 2;       // near counts, bf16 [p][r], p <= 128
  static constexpr int BIG = 2 * STAGE > STAGE + HC ? 2 * STAGE : STAGE + HC;
  static constexpr int KS = BF ? D / 32 : D / 4;     // k-steps of the logit product
  static constexpr int DB = D / 16;                  // 16-wide output column blocks
  __device__ static int swk(int key) { return key & 15 & (CPR - 1); }
  __device__ static int swv(int key) { return CPR >= 16 ? 2 * (key & 7) : 2 * (key & 3); }
};

// small-LDS region: the 9 x 16-byte bf16 prefixes of ones; per-row support
// bounds [lo, hi) of the workgroup's rows
constexpr int SM_TH = 0;
constexpr int SM_LO = 256;
constexpr int SM_HI = SM_LO + 4 * BM;
constexpr int SM_SORT = SM_HI + 4 * BM;      // 4 x 128 ints: a, e in a order; e2, a2 in e2 order
constexpr int SMALL = SM_SORT + 4 * 4 * 128;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float xmax16(float x) {  // max over the 4 lanes sharing lane & 15
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float xsum16(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}
__device__ __forceinline__ int clamp08(int x) { return min(max(x, 0), 8); }
// Near counts are accumulated as 16-bit integers biased by 2^15 (two per
// dword, integer LDS atomics: far cheaper here than packed bf16 atomics) and
// turned into bf16 after they are read.
constexpr uint32_t kBias2 = 0x80008000u;
__device__ __forceinline__ void lds_add(unsigned char* p, uint32_t v) {
  __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_sub(unsigned char* p, uint32_t v) {
  __hip_atomic_fetch_sub(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// two biased 16-bit counts -> two bf16 (exact: |count| <= 256); 2^23 + x
// assembled in the mantissa, then 2^23 + 2^15 subtracted
__device__ __forceinline__ uint32_t biased_to_bf16x2(uint32_t x) {
  const float lo = __uint_as_float(0x4B000000u | (x & 0xFFFFu)) - 8421376.0f;
  const float hi = __uint_as_float(0x4B000000u | (x >> 16)) - 8421376.0f;
  return pack_bf16(lo, hi);
}
// Workgroup barrier that orders LDS only: global loads stay in flight (an
// LDS DMA still in flight is waited for, as its data lands in LDS).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ u32x4 lds128(const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p); }
// 32-bit LDS address of a pointer into the workgroup's LDS, and back
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_uchar_t*)(p)));
}
__device__ __forceinline__ u32x4 lds128_at(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ u32x2 lds_tr16_at(uint32_t a) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(static_cast<uintptr_t>(a)));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<unsigned char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

template <int D, bool BF>
struct TileLoader {
  using G = Geo<D, BF>;
  int koff[G::NI], voff[G::NI];  // per-lane byte offsets inside a tile (constant)

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int I = w * G::NI + i;
      const int key = I * G::RPI + lane / G::CPR;
      const int pc = lane % G::CPR;
      koff[i] = key * G::RB + 16 * (pc ^ G::swk(key));
      voff[i] = key * G::RB + 16 * (pc ^ G::swv(key));
    }
  }
  // K/V rows j0 .. j0 + 63 into one stage; rows at or past n read as zero.
  //
  // The loads are written as inline assembly on purpose: the compiler treats
  // every later LDS access as possibly aliasing an LDS load in flight and
  // would wait for it, serialising compute on tile t with the load of tile
  // t + 1.  The data is consumed only after the full wait of the tile
  // barrier, which is therefore the one synchronisation these loads need.
  __device__ __forceinline__ void issue(const void* Kh, const void* Vh, int j0, int n, unsigned char* stage,
                                        int w) const {
    const int rows = n - j0;
    const int nrec = rows > 0 ? rows * G::RB : 0;
    const size_t off = static_cast<size_t>(j0) * G::RB;
    const uint64_t kb = reinterpret_cast<uint64_t>(Kh) + off;
    const uint64_t vb = reinterpret_cast<uint64_t>(Vh) + off;
    // buffer resources: base, 32-bit data format, num_records = bytes left
    const i32x4 rk = {static_cast<int>(kb), static_cast<int>((kb >> 32) & 0xFFFF), nrec, 0x00020000};
    const i32x4 rv = {static_cast<int>(vb), static_cast<int>((vb >> 32) & 0xFFFF), nrec, 0x00020000};
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uchar_t*)(stage)));
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int I = w * G::NI + i;
      // lane L's 16 bytes land at M0 + 16 L; s_nop covers the SGPR and M0
      // write-to-use hazards, which the compiler does not look for in asm
      asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(koff[i]), "s"(rk), "{m0}"(lds0 + I * 1024)
                   : "memory");
      asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff[i]), "s"(rv), "{m0}"(lds0 + G::TILE + I * 1024)
                   : "memory");
    }
  }
};

template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
struct Fwd {
  using G = Geo<D, BF>;
  using T = typename G::T;
  static constexpr bool PL = MODE == MODE_PLSH;
  static constexpr int KS = G::KS, DB = G::DB;

  // per-lane state
  int lane, l16, g, w;
  int rr[NRB], R[NRB];
  int lo_r[NRB], hi_r[NRB];  // support of the row: keys [lo, hi) carry weight (causal cut included)
  int loF, loL, hiF, hiL;    // wave-uniform: bounds of the wave's first and last row
  float nbase[NRB][4];       // near counts at the key before each 32-position chunk of the tile
  float sc, scp, thr, beta;
  float Mrow[NRB], Msc[NRB], lsum[NRB];
  bool started;               // wave-uniform: the running maximum has been raised once
  f32x4 acc[DB][NRB];
  u32x4 qb[NRB][BF ? KS : 1];
  float qf[NRB][BF ? 1 : KS];
  int koff[BF ? 1 : KS / 4];   // fp32: logit-operand chunk offsets within a row block
  uint32_t kbase;              // bf16: logit-operand offset of k-step 0; k-step ks: ^ 64 ks
  uint32_t ka[BF ? KS : 1];    // bf16: LDS addresses of the current tile's logit operand, per k-step
  int vtr0;                    // value-operand (transposing read) offset of block 0; block db: ^ 32 db
  const unsigned char* sTh;

  __device__ __forceinline__ void init_offsets() {
    // K operand: key = 16 kb + l16; logical chunk c = 4 ks + g (bf16) or (KS/4) g + c4 (fp32)
    if constexpr (BF) {
      // l16 RB | 16 ((4 ks + g) ^ swk(l16)): the k-step bits 6-7 enter only
      // through the XOR, so k-step ks is kbase ^ 64 ks
      kbase = l16 * G::RB + 16 * (g ^ G::swk(l16));
      koff[0] = 0;
    } else {
#pragma unroll
      for (int c4 = 0; c4 < KS / 4; ++c4) koff[c4] = l16 * G::RB + 16 * (((KS / 4) * g + c4) ^ G::swk(l16));
    }
    // V operand
    if constexpr (BF) {
      const int a = l16 & 3, t = l16 >> 2;
      const int key = 4 * g + t;  // + 32 kc + 16 hh: multiples of 8, swizzle unchanged
      // bits: key * RB | 32 (db ^ swv(key) / 2) | 16 (a >> 1) | 8 (a & 1), disjoint fields,
      // so block db's offset is vtr0 ^ 32 db (stage and chunk bases are multiples of 256)
      vtr0 = key * G::RB + 16 * ((a >> 1) ^ G::swv(key)) + 8 * (a & 1);
      static_assert(G::RB % 256 == 0 || G::RB == 128, "V row layout");
    } else {
      vtr0 = 0;
    }
  }

  // per tile: the logit-operand addresses of its stage (stage bases are
  // multiples of 256, so adding one commutes with the k-step XOR)
  __device__ __forceinline__ void begin_k(const unsigned char* sK) {
    if constexpr (BF) {
      const uint32_t b = lds_addr(sK) + kbase;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = b ^ (64 * ks);
    }
  }

  // ---- one 32-key chunk of a tile: logits, counts, softmax, value product
  // TI: index of the near tile (its keys start at r0 + 64 TI), 0 otherwise
  template <int KIND, int TI>
  __device__ __forceinline__ void chunk(const unsigned char* sK, const unsigned char* sV, int j0, int r0, int n,
                                        int kc, const int (&mkey)[4], const u32x4 (&cnt_b)[NRB][4]) {
    const int jc = j0 + 32 * kc;
    // Row supports are single intervals whose ends grow with the row, so the
    // chunk misses every row of the wave, lies inside every row's support,
    // or needs an elementwise mask.
    if (jc + 32 <= loF || jc >= hiL) return;
    const bool inside = jc >= loL && jc + 32 <= hiF;
    f32x4 sacc[2][NRB], cacc[2][NRB];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        sacc[x][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        cacc[x][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // S^T = K Q^T
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const unsigned char* kr = sK + (16 * (2 * kc + kb2)) * G::RB;
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 a = lds128_at(ka[ks] + (16 * (2 * kc + kb2)) * G::RB);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) sacc[kb2][rb] = mfma_bf16(a, qb[rb][ks], sacc[kb2][rb]);
        }
      } else {
#pragma unroll
        for (int c4 = 0; c4 < KS / 4; ++c4) {
          const u32x4 a4 = lds128(kr + koff[c4]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
              sacc[kb2][rb] = mfma_f32(__uint_as_float(a4[e]), qf[rb][4 * c4 + e], sacc[kb2][rb]);
        }
      }
    }
    // counts in the layout of S^T
    if constexpr (PL) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int kb = 2 * kc + kb2;
        if constexpr (KIND == KIND_NEAR) {
          // c[r, j] = nbase[r][ch] + sum over positions p of chunk ch with p <= j of H[r, p]
          const int jrel0 = 64 * TI + 16 * kb;
          const int ch = jrel0 >> 5;
          const u32x4 th = lds128(sTh + 16 * clamp08(jrel0 + l16 - 32 * ch - 8 * g + 1));
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const float b0 = nbase[rb][ch];
            cacc[kb2][rb] = mfma_bf16(th, cnt_b[rb][ch], f32x4{b0, b0, b0, b0});
          }
        } else {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) {
            const u32x4 th = lds128(sTh + 16 * clamp08(mkey[kb] - 32 * ch - 8 * g));
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) cacc[kb2][rb] = mfma_bf16(th, cnt_b[rb][ch], cacc[kb2][rb]);
          }
        }
      }
    }
    // weights in log2 units (ALiBi) or logits (PLSH); masking; local maxima
    float lmx[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) lmx[rb] = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int J = jc + 16 * kb2 + 4 * g + e;
          float x = sacc[kb2][rb][e];
          if constexpr (MODE == MODE_ALIBI) x = fmaf(x, sc, -beta * fabsf(static_cast<float>(R[rb] - J)));
          sacc[kb2][rb][e] = x;
        }
    if (!inside) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bool ok;
            if constexpr (PL) {
              // the count is exactly 0 off the row's support and (causal)
              // past the row itself, and at least 1 on it
              ok = cacc[kb2][rb][e] > 0.5f;
            } else {
              const int J = jc + 16 * kb2 + 4 * g + e;
              ok = J >= lo_r[rb] && J < hi_r[rb];
            }
            sacc[kb2][rb][e] = ok ? sacc[kb2][rb][e] : -INFINITY;
          }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) lmx[rb] = fmaxf(lmx[rb], sacc[kb2][rb][e]);
    // raise the running maximum only when some row outgrows it by the margin
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) grow = grow || lmx[rb] > Mrow[rb] + thr;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // until the wave's first raise every maximum is -inf and every sum
      // zero: that raise rescales nothing
      const bool rescale = started;
      started = true;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mn = fmaxf(Mrow[rb], xmax16(lmx[rb]));
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((Mrow[rb] - mn) * scp);
        Mrow[rb] = mn;
        Msc[rb] = mn == -INFINITY ? 0.0f : mn * scp;
        if (rescale) {
          lsum[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][rb] *= alpha;
        }
      }
    }
    // weights and the value product O^T += V^T P^T
    if constexpr (BF) {
      u32x4 pf[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
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
      const unsigned char* vb = sV + (32 * kc) * G::RB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t va = (lds_addr(vb) + vtr0) ^ (32 * db);
        const u32x2 v0 = lds_tr16_at(va);
        const u32x2 v1 = lds_tr16_at(va + 16 * G::RB);
        const u32x4 a = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[db][rb] = mfma_bf16(a, pf[rb], acc[db][rb]);
      }
    } else {
      float p[NRB][2][4];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
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
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 32 * kc + 16 * kb2 + 4 * g + e;
          const unsigned char* vrow = sV + key * G::RB + 4 * (l16 & 3);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int c = (4 * db + (l16 >> 2)) ^ G::swv(key);
            const float va = *reinterpret_cast<const float*>(vrow + 16 * c);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) acc[db][rb] = mfma_f32(va, p[rb][kb2][e], acc[db][rb]);
          }
        }
    }
  }
};

template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
// second bound: waves per SIMD, from the workgroups that fit a CU's LDS
__global__ __launch_bounds__(NT, (Geo<D, BF>::BIG + SMALL > 80 * 1024 ? 1 : 2) * NW / 4) void fwd_kernel(FwdArgs A,
                                                                                              HeadOrder ord,
                                                                                              HeadScale hsc) {
  using G = Geo<D, BF>;
  using T = typename G::T;
  using F = Fwd<D, BF, CAUSAL, NCH, MODE>;
  constexpr bool PL = MODE == MODE_PLSH;
  constexpr bool LIT = MODE == MODE_LITERAL;
  constexpr int KS = G::KS, DB = G::DB;

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  unsigned char* stage0 = smem;
  unsigned char* stage1 = smem + G::STAGE;
  unsigned char* hc = stage1;  // near counts live in stage 1 until the prologue ends
  unsigned char* sm = smem + G::BIG;

  F f;
  const int tid = threadIdx.x;
  f.lane = tid & 63;
  f.l16 = f.lane & 15;
  f.g = f.lane >> 4;
  f.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = f.lane, l16 = f.l16, g = f.g, w = f.w;
  f.sTh = sm + SM_TH;

  // ---- work item: consecutive tiles of a head stay on one XCD
  const int gid = blockIdx.x;
  const int xcd = gid & 7, kk = gid >> 3;
  const int inst = kk / A.cs;
  const int qt = xcd * A.cs + kk % A.cs;
  if (qt >= A.ntile) return;
  const int b = inst % A.B;
  const int h = ord.get(inst / A.B);
  const int kvh = h / (A.Hq / A.Hkv);
  const int n = A.n, s = A.s;
  const int r0 = qt * BM;
  const int nrows = min(BM, n - r0);
  const T* Qp = static_cast<const T*>(A.q) + static_cast<size_t>(b * A.Hq + h) * n * D;
  const T* Kh = static_cast<const T*>(A.k) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
  const T* Vh = static_cast<const T*>(A.v) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
  T* Op = static_cast<T*>(A.o) + static_cast<size_t>(b * A.Hq + h) * n * D;

  // ---- plan records of the tile's hashes (issued before the key tiles, so
  // that waiting for them never waits for a tile): lane l holds hashes l and
  // l + 64
  constexpr int SP = 32 * NCH;                 // slots per sorted array
  int va0 = INT_MAX, va1 = INT_MAX;            // a_i sorted (lane k: k-th, k+64-th)
  int ve0 = INT_MIN, ve1 = INT_MIN;            // e2_i sorted descending
  u32x4 aeL[PL ? NCH : 1][2];                  // e_i of slots 32 ch + 8 g .. + 7 (a order)
  u32x4 eaL[(PL && !CAUSAL) ? NCH : 1][2];     // a2_i of those slots (e2 order)
  u32x4 pb[2];                                 // boundary bits
  u32x4 pr[2];                                 // a, e, a2, e2
  int lo = 0, hi = n, cntA = 0;
  if constexpr (PL || LIT) {
    const size_t tix = static_cast<size_t>(h) * A.ntile + qt;
    const PlanRec* rec = A.plan + tix * s;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int i = lane + 64 * x;
      const bool ok = (x == 0 || NCH == 4) && i < s;
      const PlanRec* ri = rec + (i < s ? i : 0);
      pb[x] = ok ? *reinterpret_cast<const u32x4*>(ri->bits) : u32x4{0, 0, 0, 0};
      // absent hashes: a = +inf, e = -inf, a2 = +inf, e2 = -inf (never count)
      if constexpr (CAUSAL && PL) {
        // a and e only: the last row's block (a2, e2) bounds keys right of
        // the tile, which causal rows never see.  (Loading the unused half
        // lets the compiler reuse its registers, which then waits for the
        // load before the query loads are issued.)
        const u32x2 v = *reinterpret_cast<const u32x2*>(ri);
        pr[x] = ok ? u32x4{v[0], v[1], 0x7FFFFFFFu, 0x80000000u}
                   : u32x4{0x7FFFFFFFu, 0x80000000u, 0x7FFFFFFFu, 0x80000000u};
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(ri);
        pr[x] = ok ? v : u32x4{0x7FFFFFFFu, 0x80000000u, 0x7FFFFFFFu, 0x80000000u};
      }
    }
  }

  // first tile (the query rows' own keys): loaded right away, or (PLSH)
  // right after the first barrier of the count set-up, which would wait for it
  TileLoader<D, BF> ld;
  ld.init(w, lane);
  if constexpr (MODE == MODE_ALIBI) ld.issue(Kh, Vh, r0, n, stage0, w);

#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    f.rr[rb] = WR * w + 16 * rb + l16;
    f.R[rb] = r0 + f.rr[rb];
  }
  // Q fragments (operand B of S^T = K Q^T).  Rows past n read row n - 1: their
  // results are never stored and rows do not mix, and an unconditional load
  // is waited for only where it is first used.
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const T* qrow = Qp + static_cast<size_t>(min(f.R[rb], n - 1)) * D;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) f.qb[rb][ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int c4 = 0; c4 < KS / 4; ++c4) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + KS * g + 4 * c4);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.qf[rb][4 * c4 + e] = __uint_as_float(x[e]);
      }
    }
  }
  f.init_offsets();

  // ---- count operands
  u32x4 hf[NRB][4];                          // near: H (operand B) per position chunk
  u32x4 ufl[NRB][PL ? NCH : 1];              // left:  [r < e_slot]
  u32x4 ufr[NRB][(PL && !CAUSAL) ? NCH : 1]; // right: [r >= a2_slot]
  if constexpr (PL) {
    // clear the near-count matrix (stage 1, not yet in use; row 128 is spare)
    for (int x = tid; x < G::HC / 16; x += NT) reinterpret_cast<u32x4*>(hc)[x] = u32x4{kBias2, kBias2, kBias2, kBias2};
    if (tid < 9) {
      u32x4 p;
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = (tid >= 2 * q + 2) ? 0x3F803F80u : (tid == 2 * q + 1 ? 0x00003F80u : 0u);
      *reinterpret_cast<u32x4*>(sm + SM_TH + 16 * tid) = p;
    }
    if (tid < BM) {
      reinterpret_cast<int*>(sm + SM_LO)[tid] = INT_MAX;
      reinterpret_cast<int*>(sm + SM_HI)[tid] = INT_MIN;
    }
    lds_barrier();
    ld.issue(Kh, Vh, r0, n, stage0, w);
    {
      // H[r][p] (stored [p][r], biased int16) by atomic adds: wave w takes the
      // hashes i = w mod NW for all 128 rows, rows lane and 64 + lane.  For
      // row r and hash i, +1 at the start of the block of r (0 when it starts
      // before the tile) and, not causal, -1 at its end (the spare row 128
      // when past the tile).  The boundary bits are wave-uniform, so every
      // branch here is scalar.  The same pass gives each row its support
      // [lo, hi): the least block start and the greatest block end over the
      // hashes (causal: the row itself ends it).
      const uint64_t le = lane == 63 ? ~0ull : ((2ull << lane) - 1);  // bits <= lane
      unsigned char* col0 = hc + 2 * (lane - (lane & 1));
      unsigned char* col1 = col0 + 2 * 64;
      const uint32_t onev = 1u << (16 * (lane & 1));
      int lo0 = INT_MAX, hi0 = INT_MIN, lo1 = INT_MAX, hi1 = INT_MIN;
      int nfull = 0, flo = INT_MAX, fhi = INT_MIN;  // hashes with one block over the tile
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x == 1 && NCH != 4) break;
        const int iend = min(s, 64 * x + 64);
        for (int i = 64 * x + w; i < iend; i += NW) {
          const uint32_t b0 = __builtin_amdgcn_readlane(pb[x][0], i & 63);
          const uint32_t b1 = __builtin_amdgcn_readlane(pb[x][1], i & 63);
          const uint32_t b2 = __builtin_amdgcn_readlane(pb[x][2], i & 63);
          const uint32_t b3 = __builtin_amdgcn_readlane(pb[x][3], i & 63);
          const int ai = __builtin_amdgcn_readlane(static_cast<int>(pr[x][0]), i & 63);
          const int ei = __builtin_amdgcn_readlane(static_cast<int>(pr[x][3]), i & 63);
          const uint64_t lo64 = b0 | (static_cast<uint64_t>(b1) << 32);
          const uint64_t hi64 = b2 | (static_cast<uint64_t>(b3) << 32);
          if ((lo64 | hi64) == 0) {  // one block over the whole tile
            ++nfull;
            flo = min(flo, ai);
            fhi = max(fhi, ei);
            continue;
          }
          // row lane (first half), row 64 + lane (second half)
          const uint64_t m0 = lo64 & le, m1 = hi64 & le;
          const int st0 = m0 ? 63 - __builtin_clzll(m0) : 0;
          const int st1 = m1 ? 127 - __builtin_clzll(m1) : (lo64 ? 63 - __builtin_clzll(lo64) : 0);
          lds_add(col0 + st0 * (2 * BM), onev);
          lds_add(col1 + st1 * (2 * BM), onev);
          lo0 = min(lo0, st0 ? r0 + st0 : ai);   // st = 0: the block of row r0
          lo1 = min(lo1, st1 ? r0 + st1 : ai);
          if constexpr (!CAUSAL) {
            // the -1 at each block's end; causal rows instead end every
            // block at the row itself (below), since keys past it are cut
            const uint64_t g0 = lo64 & ~le, g1 = hi64 & ~le;
            const int en0 = g0 ? __builtin_ctzll(g0) : (hi64 ? 64 + __builtin_ctzll(hi64) : BM);
            const int en1 = g1 ? 64 + __builtin_ctzll(g1) : BM;
            lds_sub(col0 + en0 * (2 * BM), onev);
            lds_sub(col1 + en1 * (2 * BM), onev);
            hi0 = max(hi0, en0 < BM ? r0 + en0 : ei);  // en = BM: the block of the last row
            hi1 = max(hi1, en1 < BM ? r0 + en1 : ei);
          }
        }
      }
      if (nfull > 0) {
        lds_add(col0, static_cast<uint32_t>(nfull) * onev);
        lds_add(col1, static_cast<uint32_t>(nfull) * onev);
      }
      if constexpr (CAUSAL) {
        // every block of row r ends after r, so with the keys past r cut the
        // s blocks all end at r + 1 (row 127: the spare position 128)
        if (w == NW - 1) {
          lds_sub(col0 + (lane + 1) * (2 * BM), static_cast<uint32_t>(s) * onev);
          lds_sub(col1 + (lane + 65) * (2 * BM), static_cast<uint32_t>(s) * onev);
        }
      }
      lo0 = min(lo0, flo);
      lo1 = min(lo1, flo);
      int* sLo = reinterpret_cast<int*>(sm + SM_LO);
      __hip_atomic_fetch_min(sLo + lane, lo0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_min(sLo + 64 + lane, lo1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if constexpr (!CAUSAL) {
        hi0 = max(hi0, fhi);
        hi1 = max(hi1, fhi);
        int* sHi = reinterpret_cast<int*>(sm + SM_HI);
        __hip_atomic_fetch_max(sHi + lane, hi0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_max(sHi + 64 + lane, hi1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    // the hashes in two orders for the far tiles (waves with the fewest
    // hashes above): by the start a of the first row's block ascending, and
    // (not causal) by the end e2 of the last row's block descending; ties by
    // hash index.  Slots s .. SP-1 get sentinels that never count.
    if (w == NW - 4 || (!CAUSAL && w == NW - 3)) {
      const bool by_a = w == NW - 4;
      int* sk = reinterpret_cast<int*>(sm + SM_SORT) + (by_a ? 0 : 2 * 128);
      int* sv = sk + 128;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x == 1 && NCH != 4) break;
        const int i = lane + 64 * x;
        // (-e2 is safe: e2 >= 1 for the hashes that take part)
        const int key = by_a ? static_cast<int>(pr[x][0]) : (i < s ? -static_cast<int>(pr[x][3]) : 0);
        int rank = 0;
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          if (y == 1 && NCH != 4) break;
          const int kend = min(s, 64 * y + 64);
          const int kv = by_a ? static_cast<int>(pr[y][0]) : (lane + 64 * y < s ? -static_cast<int>(pr[y][3]) : 0);
          for (int k = 64 * y; k < kend; ++k) {
            const int kk = __builtin_amdgcn_readlane(kv, k & 63);
            rank += (kk < key) || (kk == key && k < i);
          }
        }
        if (i < s) {
          sk[rank] = by_a ? static_cast<int>(pr[x][0]) : static_cast<int>(pr[x][3]);
          sv[rank] = by_a ? static_cast<int>(pr[x][1]) : static_cast<int>(pr[x][2]);
        } else if (i < SP) {
          sk[i] = by_a ? INT_MAX : INT_MIN;
          sv[i] = by_a ? INT_MIN : INT_MAX;
        }
      }
    }
    // window of keys with weight, and the hashes whose first-row block starts
    // left of the tile (every wave, from its registers)
    {
      int vlo = static_cast<int>(pr[0][0]), vhi = static_cast<int>(pr[0][3]);
      int vca = static_cast<int>(pr[0][0]) < r0;
      if constexpr (NCH == 4) {
        vlo = min(vlo, static_cast<int>(pr[1][0]));
        vhi = max(vhi, static_cast<int>(pr[1][3]));
        vca += static_cast<int>(pr[1][0]) < r0;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        vlo = min(vlo, __shfl_xor(vlo, o, 64));
        vhi = max(vhi, __shfl_xor(vhi, o, 64));
        vca += __shfl_xor(vca, o, 64);
      }
      lo = __builtin_amdgcn_readfirstlane(vlo);
      hi = __builtin_amdgcn_readfirstlane(vhi);
      cntA = __builtin_amdgcn_readfirstlane(vca);
    }
    lds_barrier();
    // H operand through transposing reads of the [position][row] matrix:
    // source lane a + 4t of a 16-lane group reads rows 4a..4a+3 at position p0 + t
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int p0 = 32 * ch + 8 * g;
        const unsigned char* base = hc + (p0 + (l16 >> 2)) * (2 * BM) + 2 * (WR * w + 16 * rb + 4 * (l16 & 3));
        const u32x2 x0 = lds_tr16(base);
        const u32x2 x1 = lds_tr16(base + 4 * (2 * BM));
        hf[rb][ch] = u32x4{biased_to_bf16x2(x0[0]), biased_to_bf16x2(x0[1]), biased_to_bf16x2(x1[0]),
                           biased_to_bf16x2(x1[1])};
        // this lane's 8 positions of chunk ch, then the chunk's sum over the 4 lane groups
        int cs = -8 * 32768;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          cs += static_cast<int>((x0[q] & 0xFFFFu) + (x0[q] >> 16) + (x1[q] & 0xFFFFu) + (x1[q] >> 16));
        cs += __shfl_xor(cs, 16, 64);
        cs += __shfl_xor(cs, 32, 64);
        f.nbase[rb][ch] = static_cast<float>(cs);  // chunk sum for now; prefix below
      }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float run = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const float sum = f.nbase[rb][ch];
        f.nbase[rb][ch] = run;
        run += sum;
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f.lo_r[rb] = reinterpret_cast<const int*>(sm + SM_LO)[f.rr[rb]];
      // causal: every block of the row ends after it, so the cut at the row
      // is the support's end
      f.hi_r[rb] = CAUSAL ? min(f.R[rb] + 1, n) : reinterpret_cast<const int*>(sm + SM_HI)[f.rr[rb]];
    }
    {
      const int* sAa = reinterpret_cast<const int*>(sm + SM_SORT);
      const int* sAe = sAa + 128;
      const int* sEe = sAa + 256;
      const int* sEa = sAa + 384;
      va0 = sAa[lane];
      if constexpr (NCH == 4) va1 = sAa[64 + lane];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int x = 0; x < 2; ++x) aeL[ch][x] = *reinterpret_cast<const u32x4*>(sAe + 32 * ch + 8 * g + 4 * x);
      if constexpr (!CAUSAL) {
        ve0 = sEe[lane];
        if constexpr (NCH == 4) ve1 = sEe[64 + lane];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
          for (int x = 0; x < 2; ++x) eaL[ch][x] = *reinterpret_cast<const u32x4*>(sEa + 32 * ch + 8 * g + 4 * x);
      }
    }
    // far operands: slot k of the a order counts for row r iff r < e_k; slot
    // k of the e2 order iff r >= a2_k (sentinel slots never count)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        u32x4 fl, fr;
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const int e0 = static_cast<int>(aeL[ch][u2 >> 1][2 * (u2 & 1)]);
          const int e1 = static_cast<int>(aeL[ch][u2 >> 1][2 * (u2 & 1) + 1]);
          fl[u2] = (f.R[rb] < e0 ? 0x3F80u : 0u) | (f.R[rb] < e1 ? 0x3F800000u : 0u);
          if constexpr (!CAUSAL) {
            const int a0 = static_cast<int>(eaL[ch][u2 >> 1][2 * (u2 & 1)]);
            const int a1 = static_cast<int>(eaL[ch][u2 >> 1][2 * (u2 & 1) + 1]);
            fr[u2] = (f.R[rb] >= a0 ? 0x3F80u : 0u) | (f.R[rb] >= a1 ? 0x3F800000u : 0u);
          }
        }
        ufl[rb][ch] = fl;
        if constexpr (!CAUSAL) ufr[rb][ch] = fr;
      }
    }
  }

  if constexpr (MODE == MODE_ALIBI) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f.lo_r[rb] = 0;
      f.hi_r[rb] = CAUSAL ? min(f.R[rb] + 1, n) : n;
    }
  }
  f.loF = __builtin_amdgcn_readlane(f.lo_r[0], 0);
  f.hiF = __builtin_amdgcn_readlane(f.hi_r[0], 0);
  f.loL = __builtin_amdgcn_readlane(f.lo_r[NRB - 1], 15);
  f.hiL = __builtin_amdgcn_readlane(f.hi_r[NRB - 1], 15);

  // ---- tile schedule
  const int nnear = nrows > BN ? 2 : 1;
  const int nleft = lo < r0 ? (r0 - lo + BN - 1) / BN : 0;
  const int nright = (!CAUSAL && hi > r0 + BM) ? (hi - (r0 + BM) + BN - 1) / BN : 0;
  const int ntl = nnear + nleft + nright;
  auto tile_j0 = [&](int t) {
    return t < nnear ? r0 + BN * t
                     : (t < nnear + nleft ? r0 - BN * (t - nnear + 1) : r0 + BM + BN * (t - nnear - nleft));
  };

  // ---- softmax state
  f.sc = rsqrtf(static_cast<float>(D)) * kLog2e;  // logit -> log2 units
  f.scp = MODE == MODE_ALIBI ? 1.0f : f.sc;        // scale applied at exp time
  f.thr = 8.0f / f.scp;                            // rescale margin (units of x)
  f.beta = MODE == MODE_ALIBI ? hsc.beta[h] : 0.0f;
  f.started = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    f.Mrow[rb] = -INFINITY;
    f.Msc[rb] = 0.f;
    f.lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) f.acc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tile loop, in three phases so that each phase's count operands die
  // with it.  Tile t has landed when iteration t starts (issued one
  // iteration earlier); after the barrier every wave is done with tile t-1,
  // whose stage then receives tile t+1.
  auto begin_tile = [&](int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntl) ld.issue(Kh, Vh, tile_j0(t + 1), n, (t & 1) ? stage0 : stage1, w);
  };
  if constexpr (LIT) {
    // One short attention per hash, as in the reduction of Theorem 2.2: for
    // hash i, row r attends to the keys of its own block of hash i.  The
    // partial sums of all hashes share one running maximum, so they add up
    // to the count-weighted sums with no merge step; the logits of a key
    // tile are recomputed for every hash whose blocks reach it.
    auto recv = [&](int i, int c) {
      return __builtin_amdgcn_readlane(static_cast<int>(i < 64 ? pr[0][c] : pr[1][c]), i & 63);
    };
    // keys of hash i that some row of the tile attends to: [a_i, e2_i)
    auto span = [&](int i, int& ja, int& je) {
      ja = recv(i, 0);
      je = recv(i, 3);
      if constexpr (CAUSAL) je = min(je, r0 + nrows);
    };
    // each row's block of hash i: the last boundary at or before the row
    // (else a_i) and the first boundary after it (else e2_i)
    auto set_hash = [&](int i) {
      const uint32_t b0 = __builtin_amdgcn_readlane(i < 64 ? pb[0][0] : pb[1][0], i & 63);
      const uint32_t b1 = __builtin_amdgcn_readlane(i < 64 ? pb[0][1] : pb[1][1], i & 63);
      const uint32_t b2 = __builtin_amdgcn_readlane(i < 64 ? pb[0][2] : pb[1][2], i & 63);
      const uint32_t b3 = __builtin_amdgcn_readlane(i < 64 ? pb[0][3] : pb[1][3], i & 63);
      const int ai = recv(i, 0), ei = recv(i, 3);
      const uint64_t lo64 = b0 | (static_cast<uint64_t>(b1) << 32);
      const uint64_t hi64 = b2 | (static_cast<uint64_t>(b3) << 32);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int p = f.rr[rb];
        const int q = p & 63;
        const uint64_t le = q == 63 ? ~0ull : ((2ull << q) - 1);
        const uint64_t half = p < 64 ? lo64 : hi64;
        const uint64_t m = half & le, gt = half & ~le;
        int st = m ? (p & 64) + 63 - __builtin_clzll(m) : ((p >= 64 && lo64) ? 63 - __builtin_clzll(lo64) : 0);
        int en = gt ? (p & 64) + __builtin_ctzll(gt) : ((p < 64 && hi64) ? 64 + __builtin_ctzll(hi64) : BM);
        f.lo_r[rb] = st ? r0 + st : ai;
        f.hi_r[rb] = en < BM ? r0 + en : ei;
        if constexpr (CAUSAL) f.hi_r[rb] = min(f.hi_r[rb], f.R[rb] + 1);
      }
      f.loF = __builtin_amdgcn_readlane(f.lo_r[0], 0);
      f.hiF = __builtin_amdgcn_readlane(f.hi_r[0], 0);
      f.loL = __builtin_amdgcn_readlane(f.lo_r[NRB - 1], 15);
      f.hiL = __builtin_amdgcn_readlane(f.hi_r[NRB - 1], 15);
    };
    const int mkey0[4] = {0, 0, 0, 0};
    int i = 0, j0, jend;
    span(0, j0, jend);
    ld.issue(Kh, Vh, j0, n, stage0, w);
    set_hash(0);
    for (int t = 0;; ++t) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // the next (hash, tile) goes to the other stage, which every wave is done with
      int ni = i, nj = j0 + BN, nje = jend;
      if (nj >= jend) {
        ni = i + 1;
        if (ni < s) span(ni, nj, nje);
      }
      if (ni < s) ld.issue(Kh, Vh, nj, n, (t & 1) ? stage0 : stage1, w);
      const unsigned char* st = (t & 1) ? stage1 : stage0;
      f.begin_k(st);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) f.template chunk<KIND_NEAR, 0>(st, st + G::TILE, j0, r0, n, kc, mkey0, hf);
      if (ni >= s) break;
      if (ni != i) set_hash(ni);
      i = ni;
      j0 = nj;
      jend = nje;
    }
  } else {
  int t = 0;
  {
    // the near tiles: keys r0 .. r0 + 63 in stage 0, r0 + 64 .. r0 + 127 in stage 1
    const int mkey0[4] = {0, 0, 0, 0};
    begin_tile(0);
    f.begin_k(stage0);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) f.template chunk<KIND_NEAR, 0>(stage0, stage0 + G::TILE, r0, r0, n, kc, mkey0, hf);
    if (nnear > 1) {
      begin_tile(1);
      f.begin_k(stage1);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        f.template chunk<KIND_NEAR, 1>(stage1, stage1 + G::TILE, r0 + BN, r0, n, kc, mkey0, hf);
    }
    t = nnear;
  }
  {
    u32x4 cb[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) cb[rb][ch] = PL && ch < NCH ? ufl[rb][ch < NCH ? ch : 0] : u32x4{0, 0, 0, 0};
    int lcnt_hi = cntA;
    for (; t < nnear + nleft; ++t) {
      begin_tile(t);
      const int j0 = tile_j0(t);
      const unsigned char* st = (t & 1) ? stage1 : stage0;
      int mkey[4] = {0, 0, 0, 0};
      if constexpr (PL) {
        // hashes whose block start a lies in this tile: a in [j0, j0 + 64)
        int clo = lcnt_hi;
        while (clo > 0) {
          const int x = clo - 1;
          const int av = __builtin_amdgcn_readlane(x < 64 ? va0 : va1, x & 63);
          if (av < j0) break;
          clo = x;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mkey[kb] = clo;
        for (int x = clo; x < lcnt_hi; ++x) {
          const int av = __builtin_amdgcn_readlane(x < 64 ? va0 : va1, x & 63);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mkey[kb] += (j0 + 16 * kb + l16 >= av);
        }
        lcnt_hi = clo;
      }
      f.begin_k(st);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) f.template chunk<KIND_LEFT, 0>(st, st + G::TILE, j0, r0, n, kc, mkey, cb);
    }
  }
  if constexpr (!CAUSAL) {
    u32x4 cb[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) cb[rb][ch] = PL && ch < NCH ? ufr[rb][ch < NCH ? ch : 0] : u32x4{0, 0, 0, 0};
    int rA = s, rB = s;
    for (; t < ntl; ++t) {
      begin_tile(t);
      const int j0 = tile_j0(t);
      const unsigned char* st = (t & 1) ? stage1 : stage0;
      int mkey[4] = {0, 0, 0, 0};
      if constexpr (PL) {
        while (rA > 0 && __builtin_amdgcn_readlane(rA - 1 < 64 ? ve0 : ve1, (rA - 1) & 63) < j0 + BN) --rA;
        while (rB > 0 && __builtin_amdgcn_readlane(rB - 1 < 64 ? ve0 : ve1, (rB - 1) & 63) <= j0) --rB;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mkey[kb] = rA;
        for (int x = rA; x < rB; ++x) {
          const int ev = __builtin_amdgcn_readlane(x < 64 ? ve0 : ve1, x & 63);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mkey[kb] += (ev > j0 + 16 * kb + l16);
        }
      }
      f.begin_k(st);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) f.template chunk<KIND_RIGHT, 0>(st, st + G::TILE, j0, r0, n, kc, mkey, cb);
    }
  }
  }

  // ---- epilogue: O_r = acc / l
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float l = xsum16(f.lsum[rb]);
    const float inv = 1.0f / l;
    if (f.R[rb] >= n) continue;
    if constexpr (MODE != MODE_ALIBI) {
      // log sum_j c C e^S = ln 2 (Msc + log2 l): the weights were e^{S - Msc ln 2}
      if (A.lse != nullptr && g == 0)
        A.lse[static_cast<size_t>(b * A.Hq + h) * n + f.R[rb]] = 0.6931471805599453f * (f.Msc[rb] + log2f(l));
    }
    T* orow = Op + static_cast<size_t>(f.R[rb]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o = f.acc[db][rb] * inv;
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
  constexpr int lds = Geo<D, BF>::BIG + SMALL;
  auto kfn = fwd_kernel<D, BF, CAUSAL, NCH, MODE>;
  static LdsOptIn opt;
  if (hipError_t e = opt.ensure(reinterpret_cast<const void*>(kfn), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(NT), lds, st, a, ord, hs);
  return hipGetLastError();
}

template <int D, bool BF, bool CAUSAL, int MODE>
hipError_t dispatch_nch(const FwdArgs& a, const HeadOrder& o, const HeadScale& hs, int grid, hipStream_t st) {
  if constexpr (MODE == MODE_ALIBI) {
    return launch_one<D, BF, CAUSAL, 1, MODE>(a, o, hs, grid, st);
  } else if constexpr (MODE == MODE_LITERAL) {
    return launch_one<D, BF, CAUSAL, 4, MODE>(a, o, hs, grid, st);  // both plan-record registers loaded
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
                           bool literal, float* lse, hipStream_t st) {
  const BinsLayout L = bins_layout(hq, s, n);
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.lse = lse;
  a.plan = reinterpret_cast<const PlanRec*>(static_cast<const char*>(bins) + L.off_plan);
  a.B = batch; a.Hq = hq; a.Hkv = hkv; a.n = n; a.s = s;
  a.ntile = (n + BM - 1) / BM;
  const int grid = grid_size(a.ntile, batch * hq, &a.cs);
  HeadOrder ord{};
  for (int i = 0; i < hq; ++i) ord.set(i, order[i]);
  HeadScale hs{};
  if (literal) return dispatch<MODE_LITERAL>(a, ord, hs, d, dtype, causal, grid, st);
  return dispatch<MODE_PLSH>(a, ord, hs, d, dtype, causal, grid, st);
}

hipError_t launch_alibi_fwd(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                            int n, int d, int dtype, const float* beta, int causal, hipStream_t st) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.lse = nullptr;
  a.plan = nullptr;
  a.B = batch; a.Hq = hq; a.Hkv = hkv; a.n = n; a.s = 1;
  a.ntile = (n + BM - 1) / BM;
  const int grid = grid_size(a.ntile, batch * hq, &a.cs);
  HeadOrder ord{};
  for (int i = 0; i < hq; ++i) ord.set(i, i);
  HeadScale hs{};
  for (int i = 0; i < hq; ++i) hs.beta[i] = beta[i];
  return dispatch<MODE_ALIBI>(a, ord, hs, d, dtype, causal, grid, st);
}

}  // namespace plpsh
