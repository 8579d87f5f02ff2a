// Backward pass of Positional-LSH attention, for training with the
// approximation in place of exact ALiBi (explainer of arXiv 2605.09472, Key
// results, experimental validation: Qwen3 trained from scratch, Mistral
// fine-tuned with it).
//
// With W = c o C o exp(S), S = Q K^T / sqrt(d), P = W / (W 1) and the row
// log-normaliser LSE saved by the forward pass (P = c o C o exp(S - LSE)):
//   dV = P^T dO,  dP = dO V^T,  D_r = <dO_r, O_r>,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// The counts c do not depend on Q, K, V; they are recomputed from the same
// bins as the forward pass.
//
// One kernel template serves both directions.  A workgroup owns 128
// consecutive positions ("own": query rows for dQ, keys for dK/dV; 8 waves of
// 16) and walks 64-position tiles of the other side ("other": keys for dQ,
// query rows for dK/dV) over the window where c can be non-zero.  In both
// directions the products are laid out [other x own]:
//   T1 = Ya Xa^T (S),  T2 = Yb Xb^T (dP),  Acc1 += Ya^T dS,  Acc2 += Yb^T P
// with (Xa, Xb, Ya, Yb) = (Q, dO, K, V) for dQ and (K, V, Q, dO) for dK/dV;
// Acc1 is dQ^T or dK^T, Acc2 (dK/dV only) dV^T.  The counts in the same
// layout: far tiles as a product of an own-side and an other-side 0/1 factor
// over the hashes (a block shared across a tile edge must contain that
// edge), the tiles overlapping the own positions hash by hash.  c is
// symmetric, so both directions use the same formulas.  With GQA the dK/dV
// workgroup sums over the query heads of its KV head.
#include <climits>
#include <mutex>
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) unsigned char lds_uchar_t;

constexpr int BM = 128;      // own positions per workgroup
constexpr int NW = 8;        // waves, 16 own positions each
constexpr int NT = 64 * NW;
constexpr int BN = 64;       // other positions per tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BG {
  static constexpr int RB = 2 * D;              // bytes per row (bf16)
  static constexpr int CPR = RB / 16;           // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;         // rows per 1 KB load instruction
  static constexpr int TILE = BN * RB;
  static constexpr int NI = TILE / 1024 / NW;   // load instructions per wave per matrix
  static_assert(TILE % (1024 * NW) == 0, "tile loads split evenly over the waves");
  static constexpr int STAGE = 2 * TILE + 512;  // Ya, Yb, then (dK/dV) LSE and D of the tile's rows
  static constexpr int KS = D / 32;
  static constexpr int DB = D / 16;
  // near-count matrix H[p][own] (biased int16, p <= 128): in stage 1 while
  // the counts are set up when it fits, else a region of its own
  static constexpr int HC = (BM + 1) * BM * 2;
  static constexpr int HOFF = HC <= STAGE ? STAGE : 2 * STAGE;
  static constexpr int BIG = HC <= STAGE ? 2 * STAGE : 2 * STAGE + HC;
  __device__ static int sw(int row) { return CPR >= 16 ? 2 * (row & 7) : 2 * (row & 3); }
};
// small-LDS region
constexpr int SM_HASH = 0;                   // per hash slot: a, e, a2, e2 of the own tile (16 bytes)
constexpr int SM_TH = SM_HASH + 128 * 16;    // 9 x 16-byte bf16 prefixes of ones
constexpr int SM_LO = SM_TH + 256;           // per own position: support [lo, hi)
constexpr int SM_HI = SM_LO + 4 * BM;
constexpr int SMALL = SM_HI + 4 * BM;

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dout;
  const float* lse; const float* dd;   // [B, Hq, n]
  void* dq; void* dk; void* dv;
  const PlanRec* plan;
  int B, Hq, Hkv, n, s, ntile, cs;
};
struct BwdOrder { uint32_t w[512]; };  // instances (heads or KV groups), most expensive first, 16-bit entries

__device__ __forceinline__ int order_get(const BwdOrder& o, int i) {
  return static_cast<int>((o.w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
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
__device__ __forceinline__ float lds_f32_at(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ u32x2 lds_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<unsigned char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 lds128(const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ int clamp08(int x) { return min(max(x, 0), 8); }
// near counts: 16-bit integers biased by 2^15, two per dword, integer LDS atomics
constexpr uint32_t kBias2 = 0x80008000u;
__device__ __forceinline__ void lds_add(unsigned char* p, uint32_t v) {
  __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_sub(unsigned char* p, uint32_t v) {
  __hip_atomic_fetch_sub(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// two biased 16-bit counts -> two bf16 (exact for |count| <= 256)
__device__ __forceinline__ uint32_t biased_to_bf16x2(uint32_t x) {
  const float lo = __uint_as_float(0x4B000000u | (x & 0xFFFFu)) - 8421376.0f;
  const float hi = __uint_as_float(0x4B000000u | (x >> 16)) - 8421376.0f;
  return pack_bf16(lo, hi);
}

// block [st, en) of own position r0 + p for one hash, from its plan record
// fields (uniform): boundary bits, a (block of r0) and e2 (block of the
// tile's last row)
__device__ __forceinline__ void own_block(uint64_t lo64, uint64_t hi64, int a, int e2, int r0, int p, int& st,
                                          int& en) {
  const int q = p & 63;
  const uint64_t le = q == 63 ? ~0ull : ((2ull << q) - 1);
  const uint64_t half = p < 64 ? lo64 : hi64;
  const uint64_t m = half & le, gt = half & ~le;
  const int sp = m ? (p & 64) + 63 - __builtin_clzll(m) : ((p >= 64 && lo64) ? 63 - __builtin_clzll(lo64) : 0);
  const int ep = gt ? (p & 64) + __builtin_ctzll(gt) : ((p < 64 && hi64) ? 64 + __builtin_ctzll(hi64) : BM);
  st = sp ? r0 + sp : a;
  en = ep < BM ? r0 + ep : e2;
}

template <int D, bool CAUSAL, int NCH, bool KEYSIDE>
__global__ __launch_bounds__(NT, 2) void bwd_kernel(BwdArgs A, BwdOrder ord) {
  using G = BG<D>;
  using T = uint16_t;
  constexpr int KS = G::KS, DB = G::DB;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  auto stage = [&](int i) { return smem + i * G::STAGE; };
  unsigned char* hc = smem + G::HOFF;
  unsigned char* sm = smem + G::BIG;

  const int tid = threadIdx.x;
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = A.n, s = A.s;
  const int grp = A.Hq / A.Hkv;

  // ---- work item: consecutive own tiles of an instance stay on one XCD
  const int gid = blockIdx.x;
  const int xcd = gid & 7, kk = gid >> 3;
  const int inst = kk / A.cs;
  const int ot = xcd * A.cs + kk % A.cs;
  if (ot >= A.ntile) return;
  const int b = inst % A.B;
  const int hsel = order_get(ord, inst / A.B);   // query head (dQ) or KV head (dK/dV)
  const int o0 = ot * BM;
  const int own = o0 + 16 * w + l16;             // this lane's own position
  const int ownc = min(own, n - 1);

  // ---- own-side operands (B of T1 and T2): 16 rows of Xa and Xb per wave
  const T* Xa;
  const T* Xb;
  if constexpr (KEYSIDE) {
    Xa = static_cast<const T*>(A.k) + static_cast<size_t>(b * A.Hkv + hsel) * n * D;
    Xb = static_cast<const T*>(A.v) + static_cast<size_t>(b * A.Hkv + hsel) * n * D;
  } else {
    Xa = static_cast<const T*>(A.q) + static_cast<size_t>(b * A.Hq + hsel) * n * D;
    Xb = static_cast<const T*>(A.dout) + static_cast<size_t>(b * A.Hq + hsel) * n * D;
  }
  u32x4 xa[KS], xb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    xa[ks] = *reinterpret_cast<const u32x4*>(Xa + static_cast<size_t>(ownc) * D + 32 * ks + 8 * g);
    xb[ks] = *reinterpret_cast<const u32x4*>(Xb + static_cast<size_t>(ownc) * D + 32 * ks + 8 * g);
  }

  // per-lane LDS offsets: tile loads, row-wise reads (T1, T2), transposed reads (Acc)
  int loff[G::NI];
#pragma unroll
  for (int i = 0; i < G::NI; ++i) {
    const int I = w * G::NI + i;
    const int row = I * G::RPI + lane / G::CPR;
    const int pc = lane % G::CPR;
    loff[i] = row * G::RB + 16 * (pc ^ G::sw(row));  // global byte offset landing at LDS slot (row, pc)
  }
  const uint32_t rbase = l16 * G::RB + 16 * (g ^ G::sw(l16));  // row l16, chunk g; k-step ks: ^ 64 ks
  int trbase;  // transposed read: rows 4g + (l16 >> 2) (+16), 8 bytes of column pair (l16 & 3)
  {
    const int a = l16 & 3, t = l16 >> 2;
    const int key = 4 * g + t;
    trbase = key * G::RB + 16 * ((a >> 1) ^ G::sw(key)) + 8 * (a & 1);
  }

  f32x4 acc1[DB], acc2[KEYSIDE ? DB : 1];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc1[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < (KEYSIDE ? DB : 1); ++db) acc2[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = rsqrtf(static_cast<float>(D)) * kLog2e;

  // dK/dV: every query head of the KV group; dQ: the one head
  const int nh = KEYSIDE ? grp : 1;
  for (int hh = 0; hh < nh; ++hh) {
    const int h = KEYSIDE ? hsel * grp + hh : hsel;  // query head (hashes, Q, dO, LSE, D)
    const int kvh = KEYSIDE ? hsel : hsel / grp;
    const T *Ya, *Yb;
    if constexpr (KEYSIDE) {
      Ya = static_cast<const T*>(A.q) + static_cast<size_t>(b * A.Hq + h) * n * D;
      Yb = static_cast<const T*>(A.dout) + static_cast<size_t>(b * A.Hq + h) * n * D;
    } else {
      Ya = static_cast<const T*>(A.k) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
      Yb = static_cast<const T*>(A.v) + static_cast<size_t>(b * A.Hkv + kvh) * n * D;
    }
    const float* lse_h = A.lse + static_cast<size_t>(b * A.Hq + h) * n;
    const float* dd_h = A.dd + static_cast<size_t>(b * A.Hq + h) * n;

    // plan records of the own tile: lane i holds hash i (and i + 64)
    const PlanRec* rec = A.plan + (static_cast<size_t>(h) * A.ntile + ot) * s;
    u32x4 pb[2], pr[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int i = lane + 64 * x;
      const bool ok = (x == 0 || NCH == 4) && i < s;
      const PlanRec* ri = rec + (i < s ? i : 0);
      // both loads unconditional (ri is always a valid record): a load under
      // a lane condition is merged by a wait for every load in flight,
      // including the own-side operands issued just before
      const u32x4 bv = *reinterpret_cast<const u32x4*>(ri->bits);
      pb[x] = ok ? bv : u32x4{0, 0, 0, 0};
      const u32x4 v = *reinterpret_cast<const u32x4*>(ri);
      // absent hashes never count: a = +inf, e = -inf, a2 = +inf, e2 = -inf
      pr[x] = ok ? v : u32x4{0x7FFFFFFFu, 0x80000000u, 0x7FFFFFFFu, 0x80000000u};
    }
    // (a, e, a2, e2) of every hash slot into LDS for the far-count factors;
    // the near-count matrix cleared; supports reset
    __syncthreads();  // previous head's readers are done
    if (w == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int i = lane + 64 * x;
        if (i < 32 * NCH) *reinterpret_cast<u32x4*>(sm + SM_HASH + 16 * i) = pr[x];
      }
    }
    for (int x = tid; x < G::HC / 16; x += NT) reinterpret_cast<u32x4*>(hc)[x] = u32x4{kBias2, kBias2, kBias2, kBias2};
    if (tid < 9) {
      u32x4 pth;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) pth[qq] = (tid >= 2 * qq + 2) ? 0x3F803F80u : (tid == 2 * qq + 1 ? 0x00003F80u : 0u);
      *reinterpret_cast<u32x4*>(sm + SM_TH + 16 * tid) = pth;
    }
    if (tid < BM) {
      reinterpret_cast<int*>(sm + SM_LO)[tid] = INT_MAX;
      reinterpret_cast<int*>(sm + SM_HI)[tid] = INT_MIN;
    }
    // window of other positions with weight: [lo, hi)
    int vlo = static_cast<int>(pr[0][0]), vhi = static_cast<int>(pr[0][3]);
    if constexpr (NCH == 4) {
      vlo = min(vlo, static_cast<int>(pr[1][0]));
      vhi = max(vhi, static_cast<int>(pr[1][3]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      vlo = min(vlo, __shfl_xor(vlo, o, 64));
      vhi = max(vhi, __shfl_xor(vhi, o, 64));
    }
    const int lo = __builtin_amdgcn_readfirstlane(vlo);
    const int hi = __builtin_amdgcn_readfirstlane(vhi);
    lds_barrier();
    {
      // H[own][p] (stored [p][own]) by atomic adds: wave w takes the hashes
      // i = w mod NW for all 128 own positions (lane and 64 + lane): +1 at
      // the start of the position's block (0 when it starts before the
      // tile), -1 at its end (the spare row 128 when past the tile).  The
      // same pass gives each own position its support: the least block
      // start and the greatest block end over the hashes.
      const uint64_t le = lane == 63 ? ~0ull : ((2ull << lane) - 1);
      unsigned char* col0 = hc + 2 * (lane - (lane & 1));
      unsigned char* col1 = col0 + 2 * 64;
      const uint32_t onev = 1u << (16 * (lane & 1));
      int lo0 = INT_MAX, hi0 = INT_MIN, lo1 = INT_MAX, hi1 = INT_MIN;
      int nfull = 0, flo = INT_MAX, fhi = INT_MIN;
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
          const uint64_t m0 = lo64 & le, g0 = lo64 & ~le;
          const int st0 = m0 ? 63 - __builtin_clzll(m0) : 0;
          const int en0 = g0 ? __builtin_ctzll(g0) : (hi64 ? 64 + __builtin_ctzll(hi64) : BM);
          const uint64_t m1 = hi64 & le, g1 = hi64 & ~le;
          const int st1 = m1 ? 127 - __builtin_clzll(m1) : (lo64 ? 63 - __builtin_clzll(lo64) : 0);
          const int en1 = g1 ? 64 + __builtin_ctzll(g1) : BM;
          lds_add(col0 + st0 * (2 * BM), onev);
          lds_sub(col0 + en0 * (2 * BM), onev);
          lds_add(col1 + st1 * (2 * BM), onev);
          lds_sub(col1 + en1 * (2 * BM), onev);
          lo0 = min(lo0, st0 ? o0 + st0 : ai);
          hi0 = max(hi0, en0 < BM ? o0 + en0 : ei);
          lo1 = min(lo1, st1 ? o0 + st1 : ai);
          hi1 = max(hi1, en1 < BM ? o0 + en1 : ei);
        }
      }
      if (nfull > 0) {
        lds_add(col0, static_cast<uint32_t>(nfull) * onev);
        lds_add(col1, static_cast<uint32_t>(nfull) * onev);
      }
      lo0 = min(lo0, flo);
      lo1 = min(lo1, flo);
      hi0 = max(hi0, fhi);
      hi1 = max(hi1, fhi);
      int* sLo = reinterpret_cast<int*>(sm + SM_LO);
      int* sHi = reinterpret_cast<int*>(sm + SM_HI);
      __hip_atomic_fetch_min(sLo + lane, lo0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_max(sHi + lane, hi0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_min(sLo + 64 + lane, lo1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_max(sHi + 64 + lane, hi1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    lds_barrier();
    // H operand of this lane's own position through transposing reads of the
    // [p][own] matrix, and the count before each 32-position chunk
    u32x4 hf[4];
    float nbase[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int p0 = 32 * ch + 8 * g;
      const unsigned char* base = hc + (p0 + (l16 >> 2)) * (2 * BM) + 2 * (16 * w + 4 * (l16 & 3));
      const u32x2 x0 = lds_tr16(base);
      const u32x2 x1 = lds_tr16(base + 4 * (2 * BM));
      hf[ch] = u32x4{biased_to_bf16x2(x0[0]), biased_to_bf16x2(x0[1]), biased_to_bf16x2(x1[0]),
                     biased_to_bf16x2(x1[1])};
      int csum = -8 * 32768;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
        csum += static_cast<int>((x0[qq] & 0xFFFFu) + (x0[qq] >> 16) + (x1[qq] & 0xFFFFu) + (x1[qq] >> 16));
      csum += __shfl_xor(csum, 16, 64);
      csum += __shfl_xor(csum, 32, 64);
      nbase[ch] = static_cast<float>(csum);
    }
    {
      float run = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const float sum = nbase[ch];
        nbase[ch] = run;
        run += sum;
      }
    }
    // support of the own position (causal cut included); wave-uniform
    // bounds of the wave's first and last position
    int lo_own = reinterpret_cast<const int*>(sm + SM_LO)[16 * w + l16];
    int hi_own = reinterpret_cast<const int*>(sm + SM_HI)[16 * w + l16];
    if constexpr (CAUSAL) {
      if constexpr (KEYSIDE) lo_own = max(lo_own, own);
      else hi_own = min(hi_own, own + 1);
    }
    const int loF = __builtin_amdgcn_readlane(lo_own, 0);
    const int hiL = __builtin_amdgcn_readlane(hi_own, 15);

    // own-side count factors over hash slots 32 ch + 8 g .. + 7: left of
    // the own tile [own < e], right of it [own >= a2].  Each is built right
    // before its phase, so that it does not sit beside the near-count
    // operand (or the other factor) in registers.
    u32x4 fl[NCH], fr[NCH];
    // dQ at head_dim 128: the other side's bounds of the lane's slots
    // 32 ch + 8 g + k, read with the own factors: a (left) or e2 (right).
    // The dK/dV kernel has no registers for them and reads them per chunk,
    // as do the head_dim 64 builds (where holding them measured slower).
    constexpr bool HOIST = !KEYSIDE && D == 128;
    int ob[HOIST ? NCH : 1][8];
    auto own_factors = [&](bool right, u32x4 (&f)[NCH]) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const unsigned char* hp = sm + SM_HASH + 16 * (32 * ch + 8 * g);
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const u32x4 r0v = *reinterpret_cast<const u32x4*>(hp + 16 * (2 * u2));
          const u32x4 r1v = *reinterpret_cast<const u32x4*>(hp + 16 * (2 * u2 + 1));
          if constexpr (HOIST) {
            ob[ch][2 * u2] = static_cast<int>(right ? r0v[3] : r0v[0]);
            ob[ch][2 * u2 + 1] = static_cast<int>(right ? r1v[3] : r1v[0]);
          }
          f[ch][u2] = right ? ((own >= static_cast<int>(r0v[2]) ? 0x3F80u : 0u) |
                               (own >= static_cast<int>(r1v[2]) ? 0x3F800000u : 0u))
                            : ((own < static_cast<int>(r0v[1]) ? 0x3F80u : 0u) |
                               (own < static_cast<int>(r1v[1]) ? 0x3F800000u : 0u));
        }
      }
    };
    // dQ: the own row's LSE (log2 units) and D
    float lse2_own = 0.f, dd_own = 0.f;
    if constexpr (!KEYSIDE) {
      lse2_own = lse_h[ownc] * kLog2e;
      dd_own = dd_h[ownc];
    }

    // ---- tile schedule: near tiles (overlapping the own positions), then
    // left (other < own tile) and right (other >= own tile end), as the
    // causal direction allows (dQ: other <= own; dK/dV: other >= own)
    const int nown = min(BM, n - o0);
    const int nnear = nown > BN ? 2 : 1;
    const bool do_left = !CAUSAL || !KEYSIDE;
    const bool do_right = !CAUSAL || KEYSIDE;
    const int nleft = (do_left && lo < o0) ? (o0 - lo + BN - 1) / BN : 0;
    const int nright = (do_right && hi > o0 + BM) ? (hi - (o0 + BM) + BN - 1) / BN : 0;
    const int ntl = nnear + nleft + nright;
    auto tile_j0 = [&](int t) {
      return t < nnear ? o0 + BN * t
                       : (t < nnear + nleft ? o0 - BN * (t - nnear + 1) : o0 + BM + BN * (t - nnear - nleft));
    };
    auto issue = [&](int t, unsigned char* st) {
      const int j0 = tile_j0(t);
      const int rows = n - j0;
      const int nrec = rows > 0 ? rows * G::RB : 0;
      const size_t off = static_cast<size_t>(j0) * G::RB;
      const uint64_t ab = reinterpret_cast<uint64_t>(Ya) + off;
      const uint64_t bb = reinterpret_cast<uint64_t>(Yb) + off;
      const i32x4 ra = {static_cast<int>(ab), static_cast<int>((ab >> 32) & 0xFFFF), nrec, 0x00020000};
      const i32x4 rb = {static_cast<int>(bb), static_cast<int>((bb >> 32) & 0xFFFF), nrec, 0x00020000};
      const uint32_t l0 = lds_addr(st);
#pragma unroll
      for (int i = 0; i < G::NI; ++i) {
        const int I = w * G::NI + i;
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(loff[i]), "s"(ra), "{m0}"(l0 + I * 1024)
                     : "memory");
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(loff[i]), "s"(rb), "{m0}"(l0 + G::TILE + I * 1024)
                     : "memory");
      }
      if constexpr (KEYSIDE) {
        if (w == 0) {  // LSE and D of the tile's 64 rows
          const int frec = rows > 0 ? min(rows, BN) * 4 : 0;
          const uint64_t lb = reinterpret_cast<uint64_t>(lse_h + j0);
          const uint64_t db2 = reinterpret_cast<uint64_t>(dd_h + j0);
          const i32x4 rl = {static_cast<int>(lb), static_cast<int>((lb >> 32) & 0xFFFF), frec, 0x00020000};
          const i32x4 rd = {static_cast<int>(db2), static_cast<int>((db2 >> 32) & 0xFFFF), frec, 0x00020000};
          asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
                       :
                       : "v"(4 * lane), "s"(rl), "{m0}"(l0 + 2 * G::TILE)
                       : "memory");
          asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
                       :
                       : "v"(4 * lane), "s"(rd), "{m0}"(l0 + 2 * G::TILE + 256)
                       : "memory");
        }
      }
    };

    issue(0, stage(0));
    // one tile; the kind (near, left, right) is a compile-time constant so
    // that each phase's count operands die with it
    auto tile = [&](auto kind_c, int t) {
      constexpr int kind = decltype(kind_c)::value;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < ntl) issue(t + 1, stage((t + 1) & 1));
      const unsigned char* st = stage(t & 1);
      const int j0 = tile_j0(t);
      const uint32_t ya = lds_addr(st), yb = lds_addr(st + G::TILE);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int jc = j0 + 32 * kc;
        // chunks outside every own position's support of this wave
        if (jc >= n || jc + 32 <= loF || jc >= hiL) continue;
        // T1 = Ya Xa^T and T2 = Yb Xb^T for other positions jc + 16 kb2 + (row l16 of A)
        f32x4 t1[2], t2[2], cc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          t1[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
          t2[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
          cc[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
          const uint32_t roff = (16 * (2 * kc + kb2)) * G::RB + rbase;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            t1[kb2] = mfma_bf16(lds128_at(ya + (roff ^ (64 * ks))), xa[ks], t1[kb2]);
            t2[kb2] = mfma_bf16(lds128_at(yb + (roff ^ (64 * ks))), xb[ks], t2[kb2]);
          }
        }
        // counts c[other, own] in the same layout
        if constexpr (kind == 0) {
          // near: c = count before the position chunk + prefix of H within
          // it (a product with a table of prefixes of ones), then the causal
          // cut (dQ: other <= own; dK/dV: other >= own)
          // near tile t covers positions o0 + 64 t ..: position chunk 2 t + kc
          const u32x4 hsel = t == 0 ? hf[kc] : hf[2 + kc];
          const float b0 = t == 0 ? nbase[kc] : nbase[2 + kc];
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const u32x4 th = lds128(sm + SM_TH + 16 * clamp08(16 * kb2 + l16 - 8 * g + 1));
            cc[kb2] = mfma_bf16(th, hsel, f32x4{b0, b0, b0, b0});
            if constexpr (CAUSAL) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int j = jc + 16 * kb2 + 4 * g + e;
                const bool ok = KEYSIDE ? j >= own : j <= own;
                cc[kb2][e] = ok ? cc[kb2][e] : 0.0f;
              }
            }
          }
        } else {
          // far: c = sum over hashes of [other factor] [own factor]; the
          // other factor of row l16 of the A operand over slots 8 g .. + 7
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int jo = jc + 16 * kb2 + l16;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
              const unsigned char* hp = sm + SM_HASH + 16 * (32 * ch + 8 * g);
              u32x4 af;
#pragma unroll
              for (int u2 = 0; u2 < 4; ++u2) {
                int b0, b1;
                if constexpr (HOIST) {
                  b0 = ob[ch][2 * u2];
                  b1 = ob[ch][2 * u2 + 1];
                } else {
                  const u32x4 r0v = *reinterpret_cast<const u32x4*>(hp + 16 * (2 * u2));
                  const u32x4 r1v = *reinterpret_cast<const u32x4*>(hp + 16 * (2 * u2 + 1));
                  b0 = static_cast<int>(kind == 1 ? r0v[0] : r0v[3]);
                  b1 = static_cast<int>(kind == 1 ? r1v[0] : r1v[3]);
                }
                if constexpr (kind == 1)  // left: [other >= a]
                  af[u2] = (jo >= b0 ? 0x3F80u : 0u) | (jo >= b1 ? 0x3F800000u : 0u);
                else  // right: [other < e2]
                  af[u2] = (jo < b0 ? 0x3F80u : 0u) | (jo < b1 ? 0x3F800000u : 0u);
              }
              if constexpr (kind == 1) cc[kb2] = mfma_bf16(af, fl[ch], cc[kb2]);
              else cc[kb2] = mfma_bf16(af, fr[ch], cc[kb2]);
            }
          }
        }
        // P and dS; the row of each element is own (dQ) or other (dK/dV).
        // dK/dV: the LSE and D of the tile's rows 16 (2 kc + kb2) + 4 g + e;
        // without the causal cut and at head_dim 128 the four rows of a lane
        // come in one 16-byte read (causal, that read's registers push the
        // build to the limit; at head_dim 64 it measured slower), elsewhere
        // they are read one by one
        constexpr bool WIDE = KEYSIDE && !CAUSAL && D == 128;
        u32x4 lw[WIDE ? 2 : 1], dw[WIDE ? 2 : 1];
        if constexpr (WIDE) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int r4 = 16 * (2 * kc + kb2) + 4 * g;
            lw[kb2] = lds128_at(ya + 2 * G::TILE + 4 * r4);
            dw[kb2] = lds128_at(ya + 2 * G::TILE + 256 + 4 * r4);
          }
        }
        float p[2][4], ds[2][4];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float l2, dr;
            if constexpr (WIDE) {
              l2 = __uint_as_float(lw[kb2][e]) * kLog2e;
              dr = __uint_as_float(dw[kb2][e]);
            } else if constexpr (KEYSIDE) {
              const int rr = 16 * (2 * kc + kb2) + 4 * g + e;  // row within the tile
              l2 = lds_f32_at(ya + 2 * G::TILE + 4 * rr) * kLog2e;
              dr = lds_f32_at(ya + 2 * G::TILE + 256 + 4 * rr);
            } else {
              l2 = lse2_own;
              dr = dd_own;
            }
            // for counted pairs the exponent is <= 0 (c e^(S - LSE) <= 1); the
            // clamp keeps uncounted ones finite so that c = 0 zeroes them
            const float x = fminf(fmaf(t1[kb2][e], sc, -l2), 0.0f);
            const float pv = cc[kb2][e] * __builtin_amdgcn_exp2f(x);
            p[kb2][e] = pv;
            ds[kb2][e] = pv * (t2[kb2][e] - dr);
          }
        const u32x4 sf = {pack_bf16(ds[0][0], ds[0][1]), pack_bf16(ds[0][2], ds[0][3]),
                          pack_bf16(ds[1][0], ds[1][1]), pack_bf16(ds[1][2], ds[1][3])};
        const u32x4 pf = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                          pack_bf16(p[1][2], p[1][3])};
        // Acc1 += Ya^T dS, Acc2 += Yb^T P (transposed reads of the staged tiles)
        const uint32_t tro = (32 * kc) * G::RB + trbase;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t a0 = (ya + tro) ^ (32 * db);
          const u32x2 v0 = lds_tr16_at(a0);
          const u32x2 v1 = lds_tr16_at(a0 + 16 * G::RB);
          acc1[db] = mfma_bf16(u32x4{v0[0], v0[1], v1[0], v1[1]}, sf, acc1[db]);
          if constexpr (KEYSIDE) {
            const uint32_t b0 = (yb + tro) ^ (32 * db);
            const u32x2 w0 = lds_tr16_at(b0);
            const u32x2 w1 = lds_tr16_at(b0 + 16 * G::RB);
            acc2[db] = mfma_bf16(u32x4{w0[0], w0[1], w1[0], w1[1]}, pf, acc2[db]);
          }
        }
        (void)pf;
      }
    };
    int t = 0;
    for (; t < nnear; ++t) tile(std::integral_constant<int, 0>{}, t);
    if constexpr (!CAUSAL || !KEYSIDE) {  // other before own: dQ, or no causal cut
      if (nleft > 0) own_factors(false, fl);
      for (; t < nnear + nleft; ++t) tile(std::integral_constant<int, 1>{}, t);
    }
    if constexpr (!CAUSAL || KEYSIDE) {  // other after own: dK/dV, or no causal cut
      if (nright > 0) own_factors(true, fr);
      for (; t < ntl; ++t) tile(std::integral_constant<int, 2>{}, t);
    }
  }

  // ---- epilogue: Acc1 is dQ^T or dK^T (times sqrt(d) too much), Acc2 dV^T
  if (own >= n) return;
  const float rs = rsqrtf(static_cast<float>(D));
  T* o1;
  if constexpr (KEYSIDE) o1 = static_cast<T*>(A.dk) + (static_cast<size_t>(b * A.Hkv + hsel) * n + own) * D;
  else o1 = static_cast<T*>(A.dq) + (static_cast<size_t>(b * A.Hq + hsel) * n + own) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x4 x = acc1[db] * rs;
    *reinterpret_cast<u32x2*>(o1 + 16 * db + 4 * g) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
  }
  if constexpr (KEYSIDE) {
    T* o2 = static_cast<T*>(A.dv) + (static_cast<size_t>(b * A.Hkv + hsel) * n + own) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 x = acc2[db];
      *reinterpret_cast<u32x2*>(o2 + 16 * db + 4 * g) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    }
  }
}

// D_r = <dO_r, O_r> for every (batch, query head, row): D / 8 lanes per row,
// 16-byte loads
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                     size_t rows, float* __restrict__ dd) {
  constexpr int LPR = D / 8;  // lanes per row
  const size_t r = static_cast<size_t>(blockIdx.x) * (256 / LPR) + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 8;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + r * D + c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + r * D + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(a[k] << 16), __uint_as_float(b[k] << 16), acc);
      acc = fmaf(__uint_as_float(a[k] & 0xFFFF0000u), __uint_as_float(b[k] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < rows && threadIdx.x % LPR == 0) dd[r] = acc;
}

template <int D, bool CAUSAL, int NCH, bool KEYSIDE>
hipError_t launch_bwd_one(const BwdArgs& a, const BwdOrder& ord, int grid, hipStream_t st) {
  constexpr int lds = BG<D>::BIG + SMALL;
  auto kfn = bwd_kernel<D, CAUSAL, NCH, KEYSIDE>;
  static LdsOptIn opt;
  if (hipError_t e = opt.ensure(reinterpret_cast<const void*>(kfn), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(NT), lds, st, a, ord);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool KEYSIDE>
hipError_t launch_bwd_nch(const BwdArgs& a, const BwdOrder& o, int grid, hipStream_t st) {
  if (a.s <= 32) return launch_bwd_one<D, CAUSAL, 1, KEYSIDE>(a, o, grid, st);
  if (a.s <= 64) return launch_bwd_one<D, CAUSAL, 2, KEYSIDE>(a, o, grid, st);
  return launch_bwd_one<D, CAUSAL, 4, KEYSIDE>(a, o, grid, st);
}

template <bool KEYSIDE>
hipError_t launch_bwd_dir(const BwdArgs& a, const BwdOrder& o, int d, int causal, int grid, hipStream_t st) {
  if (d == 64) return causal ? launch_bwd_nch<64, true, KEYSIDE>(a, o, grid, st)
                             : launch_bwd_nch<64, false, KEYSIDE>(a, o, grid, st);
  if (d == 128) return causal ? launch_bwd_nch<128, true, KEYSIDE>(a, o, grid, st)
                              : launch_bwd_nch<128, false, KEYSIDE>(a, o, grid, st);
  return hipErrorInvalidValue;
}

// per device: the second stream of the backward pass and its fork/join events
constexpr int kSideDevices = 64;
struct SideStream {
  std::mutex mu;
  bool ready = false;  // all three created
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[kSideDevices];

}  // namespace

hipError_t launch_plsh_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int n, int d,
                           int s, int causal, const void* bins, const uint16_t* head_order, const uint16_t* kv_order,
                           float* dd, hipStream_t st) {
  const size_t rows = static_cast<size_t>(batch) * hq * n;
  if (d == 64) {
    hipLaunchKernelGGL(rowdot_kernel<64>, dim3(static_cast<unsigned>((rows + 31) / 32)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), rows, dd);
  } else {
    hipLaunchKernelGGL(rowdot_kernel<128>, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), rows, dd);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.lse = lse; a.dd = dd;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.plan = reinterpret_cast<const PlanRec*>(static_cast<const char*>(bins) + bins_layout(hq, s, n).off_plan);
  a.B = batch; a.Hq = hq; a.Hkv = hkv; a.n = n; a.s = s;
  a.ntile = (n + BM - 1) / BM;
  a.cs = (a.ntile + 7) / 8;
  BwdOrder oq{}, okv{};
  for (int i = 0; i < hq; ++i) oq.w[i >> 1] |= static_cast<uint32_t>(head_order[i]) << (16 * (i & 1));
  for (int i = 0; i < hkv; ++i) okv.w[i >> 1] |= static_cast<uint32_t>(kv_order[i]) << (16 * (i & 1));
  // dK/dV and dQ on two streams of the device, the caller's and a second one
  // (both read the same inputs and D, and write different outputs), so that
  // each kernel fills the other's tail; joined back to the caller's stream.
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kSideDevices) return hipErrorInvalidDevice;
  SideStream& side = g_side[dev];
  std::lock_guard<std::mutex> lock(side.mu);
  if (!side.ready) {
    // default priority (the only one used anywhere in this library); a
    // failed creation leaves nothing behind and is retried by the next call
    if (side.s == nullptr && (e = hipStreamCreateWithFlags(&side.s, hipStreamNonBlocking)) != hipSuccess) {
      side.s = nullptr;
      return e;
    }
    if (side.fork == nullptr && (e = hipEventCreateWithFlags(&side.fork, hipEventDisableTiming)) != hipSuccess) {
      side.fork = nullptr;
      return e;
    }
    if (side.join == nullptr && (e = hipEventCreateWithFlags(&side.join, hipEventDisableTiming)) != hipSuccess) {
      side.join = nullptr;
      return e;
    }
    side.ready = true;
  }
  if ((e = hipEventRecord(side.fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(side.s, side.fork, 0)) != hipSuccess) return e;
  // Which kernel goes to the second stream: a dK/dV work item covers the
  // keys of all hq / hkv query heads of its group, so with four or more per
  // group its work items are the heavier ones and go there, otherwise the dQ
  // kernel does (interleaved timing: the Mistral layer, 4 per group, 614
  // against 624 us; the Qwen3 layer, 2 per group, 195 against 224 us; 8
  // heads without groups, 72 against 79 us).  Once forked, the caller's
  // stream always waits for the second stream, also when a launch fails, so
  // that nothing on it outlives the call's order.
  const bool kv_side = hq >= 4 * hkv;
  const int gq = 8 * a.cs * batch * hq, gkv = 8 * a.cs * batch * hkv;
  const hipError_t e1 = kv_side ? launch_bwd_dir<true>(a, okv, d, causal, gkv, side.s)
                                : launch_bwd_dir<false>(a, oq, d, causal, gq, side.s);
  const hipError_t ej = hipEventRecord(side.join, side.s);
  const hipError_t e2 = e1 != hipSuccess ? hipSuccess
                        : kv_side        ? launch_bwd_dir<false>(a, oq, d, causal, gq, st)
                                         : launch_bwd_dir<true>(a, okv, d, causal, gkv, st);
  const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(st, side.join, 0) : ej;
  if (e1 != hipSuccess) return e1;
  if (e2 != hipSuccess) return e2;
  return ew;
}

}  // namespace plpsh
