// Device code of the attention kernels (attn.hip): tile
// geometry, LDS helpers, the K/V tile loader and the per-chunk computation of
// the count-weighted attention (logits, counts, softmax, value product).
//
// Computes, for every query row r (explainer of arXiv 2605.09472,
// Theorem 2.1 and Theorem 2.2 with the mask mean M~ in place of the ALiBi
// matrix L*):
//
//   O_r = sum_j c[r,j] C[r,j] e^{S[r,j]} v_j / sum_j c[r,j] C[r,j] e^{S[r,j]},
//   c[r,j] = #{i : bin_i(r) == bin_i(j)},  S = Q K^T / sqrt(d).
#pragma once
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
  // Plan in the kernel (count-weighted mode, when du is not null): each
  // workgroup evaluates the bins of its query tile from the (delta, u)
  // pairs du[2 (h s + i)], du[2 (h s + i) + 1] instead of reading `plan`,
  // and the workgroups of batch row 0 write the bin buffer's block counts,
  // block starts and plan records (the bin kernel's output, bit for bit).
  const double* du;
  int32_t* nblk;
  int32_t* starts;
  PlanRec* plan_out;
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
constexpr int SM_KEYS = SM_SORT + 4 * 4 * 128;  // 2 x 128 ints: the sort keys (a; -e2)
constexpr int SM_REC = SM_KEYS + 2 * 4 * 128;  // 128 x 32 bytes: plan records evaluated in the kernel
constexpr int SM_BASE = SM_REC + 32 * 128;  // 128 ints: block index of row r0's block, per hash
constexpr int SMALL = SM_BASE + 4 * 128;

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

// K/V tile loader: NL waves share the DMA of each 64-key tile.
template <int D, bool BF, int NL = NW>
struct TileLoader {
  using G = Geo<D, BF>;
  static constexpr int NI = G::TILE / 1024 / NL;  // 1 KB load instructions per wave per matrix
  static_assert(G::TILE % (1024 * NL) == 0, "tile loads split evenly over the loading waves");
  int koff[NI], voff[NI];  // per-lane byte offsets inside a tile (constant)

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int I = w * NI + i;
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
    for (int i = 0; i < NI; ++i) {
      const int I = w * NI + i;
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
  uint32_t vbase;              // bf16: LDS address of the current tile's value operand (this lane, block 0)
  int vtr0;                    // value-operand (transposing read) offset of block 0; block db: ^ 32 db
  uint32_t sTh;                // LDS address of the table of bf16 prefixes of ones

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
      vbase = lds_addr(sK + G::TILE) + vtr0;
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
          const u32x4 th = lds128_at(sTh + 16 * clamp08(jrel0 + l16 - 32 * ch - 8 * g + 1));
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const float b0 = nbase[rb][ch];
            cacc[kb2][rb] = mfma_bf16(th, cnt_b[rb][ch], f32x4{b0, b0, b0, b0});
          }
        } else {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) {
            const u32x4 th = lds128_at(sTh + 16 * clamp08(mkey[kb] - 32 * ch - 8 * g));
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) cacc[kb2][rb] = mfma_bf16(th, cnt_b[rb][ch], cacc[kb2][rb]);
          }
        }
      }
    }
    // weights in log2 units (ALiBi) or logits (PLSH); masking; local maxima
    float lmx[NRB];
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
    auto mask = [&]() {
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
    };
    auto row_max = [&]() {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        lmx[rb] = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 4; ++e) lmx[rb] = fmaxf(lmx[rb], sacc[kb2][rb][e]);
      }
    };
    // Far tiles come after the near tiles, where every row met its own key
    // (c = s > 0), so their rows' maxima are finite.  There the mask can wait
    // for the raise below: if no entry, counted or not, outgrows its row's
    // maximum by the margin, every exponent is at most 8 and an uncounted
    // entry weighs 2^t * 0 = 0; only a chunk that triggers the raise is
    // masked first.
    constexpr bool DEFER = PL && KIND != KIND_NEAR;
    if (!inside && !DEFER) mask();
    row_max();
    // raise the running maximum only when some row outgrows it by the margin
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) grow = grow || lmx[rb] > Mrow[rb] + thr;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      if constexpr (DEFER) {
        if (!inside) {
          mask();
          row_max();
        }
      }
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
      (void)sV;  // (its LDS address is vbase, set by begin_k)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // key offsets 32 kc RB are multiples of 256, so adding them commutes
        // with the block XOR
        const uint32_t va = (vbase + (32 * kc) * G::RB) ^ (32 * db);
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

}  // namespace
}  // namespace plpsh
