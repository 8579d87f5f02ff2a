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
// is rare.  In the near tiles masked entries (c = 0, or j > r when causal)
// enter as -inf; they hold the diagonal, where c = s > 0, so every row's
// maximum is finite before the far tiles, where the mask is applied only in
// the (rare) chunks that trigger a raise: otherwise every exponent is at
// most 8 and an uncounted entry weighs 2^t * 0 = 0.
//
// MODE_ALIBI computes exact dense ALiBi attention, weight e^{S - |r-j|/sigma},
// over every key with the same pipeline.
#include "attn_common.h"
#include "bins_device.h"

namespace plpsh {
namespace {

// Tasks of the in-kernel plan: 4 s start-flag tasks (word q = 0..3 of the
// tile, hash i) on waves 0-3 and 4 s bound tasks (a, e, a2, e2 of hash i) on
// waves 4-7, task t = q s + i, lane l of wave w taking t = 64 (w mod 4) + l
// (pass 0) and t + 256 (pass 1, more than 64 hashes).  Packing the tasks into
// whole waves leaves the waves with no task free of the plan's arithmetic
// (at s = 20: two waves of each kind work, not eight).  Returns whether the
// lane has a task in the pass; q and i are then its part and hash.
__device__ __forceinline__ bool plan_task(int w, int lane, int pass, int s, int& q, int& i) {
  const int t = 64 * (w & 3) + lane + 256 * pass;
  q = (t >= s) + (t >= 2 * s) + (t >= 3 * s);
  i = t - q * s;
  return t < 4 * s;
}
// whether wave w has any task in the pass (wave-uniform)
__device__ __forceinline__ bool plan_wave_busy(int w, int pass, int s) { return 64 * (w & 3) + 256 * pass < 4 * s; }

// Plan records of query tile r0 .. r0 + 127 for the hashes of head h,
// evaluated from (delta, u) (bins_device.h), hd/hu holding the pair of the
// lane's task in each pass (plan_task): the record of hash i goes to
// srec + 32 i, in the layout of PlanRec, and the block index of row r0's
// block, bin(r0) - bin(0) (r0 when every position starts a block), to
// sbase[i].  Flag tasks take the start flags of the tile's 32-position word
// q, bound tasks the block bounds a, e (block of row r0; q = 0, 1) or a2, e2
// (block of the last row; q = 2, 3).  In the last tile the workgroup of
// batch row 0 writes the block count and the closing entry n of the bin
// buffer (scatter_starts below writes the starts).  The launcher sends no
// delta within 2^-30 of 1 here (there the start count has no closed form).
template <bool CAUSAL, int NCH>
__device__ __forceinline__ void plan_tile(const FwdArgs& A, const double (&hd)[2], const double (&hu)[2], int h,
                                          int b, int qt, int r0, int n, int s, int w, int lane,
                                          unsigned char* srec, int* sbase) {
  const int rl = min(r0 + BM - 1, n - 1);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1 && NCH != 4) break;
    if (!plan_wave_busy(w, pass, s)) break;
    int q, i;
    if (!plan_task(w, lane, pass, s, q, i)) continue;
    const double delta = hd[pass], u = hu[pass];
    const bool every = delta <= 1.0 - 0x1p-30;
    const double rinv = 1.0 / delta;
    uint32_t* rec = reinterpret_cast<uint32_t*>(srec + 32 * i);
    if (w < 4) {
      const int x0 = r0 + 32 * q;
      uint32_t m = 0u;
      if (x0 < n) {
        double prev;
        m = every ? ~0u : start_flags(x0, u, delta, rinv, delta >= 32.0, &prev);
        if (n - x0 < 32) m &= (1u << (n - x0)) - 1u;
      }
      // bit p: position r0 + p (1 <= p < 128) starts a block, or equals n
      if (q == 0) m &= ~1u;
      const int p = n - r0;
      if (p < BM && (p >> 5) == q) m |= 1u << (p & 31);
      rec[4 + q] = m;
    } else {
      const int r = q < 2 ? r0 : rl;
      const double kr = every ? 0.0 : bin_at(r, u, delta, rinv);
      const int val = every ? r + (q & 1) : first_at_least(kr + static_cast<double>(q & 1), u, delta, rinv, n);
      rec[q] = static_cast<uint32_t>(val);
      if (q == 1) sbase[i] = every ? r0 : static_cast<int>(kr - exact_bin(0, u, delta));
      if (q == 3 && b == 0 && A.starts != nullptr && qt == A.ntile - 1) {
        const int nb = every ? n : static_cast<int>(exact_bin(n - 1, u, delta) - exact_bin(0, u, delta)) + 1;
        A.nblk[h * s + i] = nb;
        A.starts[static_cast<size_t>(h * s + i) * (n + 1) + nb] = n;
      }
    }
  }
}

// The block starts that lie in query tile r0 .. r0 + 127, at their block
// indices in the bin buffer, from the records plan_tile left in LDS: bins
// rise by one at each start, so the tile's starts take consecutive indices,
// the first one that of row r0's block if it starts at r0, else the next.
// The wave takes hashes i0, i0 + di, ...; lane l writes the starts at
// positions r0 + l and r0 + 64 + l, each at the first index plus the number
// of starts before it in the tile (a masked bit count), so that every store
// instruction writes consecutive entries of one hash.
__device__ __forceinline__ void scatter_starts(const FwdArgs& A, int h, int r0, int n, int s, int i0, int di,
                                               int lane, const unsigned char* srec, const int* sbase) {
  const int p = n - r0;  // the closing bit (position n), not a start
  for (int i = i0; i < s; i += di) {
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(srec + 32 * i);
    const bool r0s = __builtin_amdgcn_readfirstlane(static_cast<int>(rec[0])) == r0;  // row r0's block starts at r0
    uint32_t bv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      bv[v] = __builtin_amdgcn_readfirstlane(rec[4 + v]);
      if (p < BM && (p >> 5) == v) bv[v] &= ~(1u << (p & 31));
    }
    if (r0s) bv[0] |= 1u;
    const int o = __builtin_amdgcn_readfirstlane(sbase[i]) + (r0s ? 0 : 1);
    int32_t* st = A.starts + static_cast<size_t>(h * s + i) * (n + 1) + o;
    const int k0 = static_cast<int>(__builtin_amdgcn_mbcnt_hi(bv[1], __builtin_amdgcn_mbcnt_lo(bv[0], 0u)));
    const int k1 = __builtin_popcount(bv[0]) + __builtin_popcount(bv[1]) +
                   static_cast<int>(__builtin_amdgcn_mbcnt_hi(bv[3], __builtin_amdgcn_mbcnt_lo(bv[2], 0u)));
    const uint32_t b0 = lane < 32 ? bv[0] >> lane : bv[1] >> (lane - 32);
    const uint32_t b1 = lane < 32 ? bv[2] >> lane : bv[3] >> (lane - 32);
    if (b0 & 1u) st[k0] = r0 + lane;
    if (b1 & 1u) st[k1] = r0 + 64 + lane;
  }
}

// Workgroups per CU a build is compiled for: two where both fit a CU's LDS
// and the operands fit 128 VGPRs, else one (up to 256 VGPRs): fp32 (its
// operands spilled at d = 64) and the count-weighted d = 128, not causal,
// two- and four-hash-chunk builds (spilled 4 and 26).  One workgroup
// without spills was faster in each case.
template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
constexpr int fwd_wgs_per_cu() {
  if (Geo<D, BF>::BIG + SMALL > 80 * 1024 || !BF) return 1;
  if (MODE == MODE_PLSH && D == 128 && NCH >= 2 && !CAUSAL) return 1;
  return 2;
}

template <int D, bool BF, bool CAUSAL, int NCH, int MODE>
// second bound: waves per SIMD
__global__ __launch_bounds__(NT, (fwd_wgs_per_cu<D, BF, CAUSAL, NCH, MODE>() * NW / 4)) void fwd_kernel(FwdArgs A,
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
  f.sTh = lds_addr(sm + SM_TH);

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
  u32x4 pb[2];                                 // boundary bits
  u32x4 pr[2];                                 // a, e, a2, e2
  int lo = 0, hi = n, cntA = 0;
  // in-kernel plan: (delta, u) of the lane's plan tasks (plan_task), else plan records
  const bool inplan = PL && A.du != nullptr;
  double hd[2] = {1.0, 1.0}, hu[2] = {0.0, 0.0};
  if (inplan) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1 && NCH != 4) break;
      if (!plan_wave_busy(w, pass, s)) break;
      int q, i;
      const bool ok = plan_task(w, lane, pass, s, q, i);
      const double* p = A.du + 2 * (static_cast<size_t>(h) * s + (ok ? i : 0));
      hd[pass] = ok ? p[0] : 1.0;
      hu[pass] = ok ? p[1] : 0.0;
    }
  } else if constexpr (PL || LIT) {
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
    if (inplan) plan_tile<CAUSAL, NCH>(A, hd, hu, h, b, qt, r0, n, s, w, lane, sm + SM_REC,
                                        reinterpret_cast<int*>(sm + SM_BASE));
    lds_barrier();
    if (inplan) {
      const bool out = b == 0 && A.plan_out != nullptr;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int i = lane + 64 * x;
        const bool ok = (x == 0 || NCH == 4) && i < s;
        const u32x4* rec = reinterpret_cast<const u32x4*>(sm + SM_REC + 32 * (i & 127));
        const u32x4 ae = rec[0], bits = rec[1];
        pb[x] = ok ? bits : u32x4{0, 0, 0, 0};
        // causal rows never see the last row's block (a2, e2): sentinels, as
        // when the records are loaded
        pr[x] = ok ? (CAUSAL ? u32x4{ae[0], ae[1], 0x7FFFFFFFu, 0x80000000u} : ae)
                   : u32x4{0x7FFFFFFFu, 0x80000000u, 0x7FFFFFFFu, 0x80000000u};
        if (w == 0 && out && ok) {
          PlanRec* po = A.plan_out + (static_cast<size_t>(h) * A.ntile + qt) * s + i;
          reinterpret_cast<u32x4*>(po)[0] = ae;
          reinterpret_cast<u32x4*>(po)[1] = bits;
        }
      }
    }
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
      // the keys go through LDS, whence every lane reads all of them with
      // broadcast reads, four per read, to count the keys that precede its own
      // (-e2 is safe: e2 >= 1 for the hashes that take part)
      int* kst = reinterpret_cast<int*>(sm + SM_KEYS) + (by_a ? 0 : 128);
      int key[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int i = lane + 64 * x;
        key[x] = by_a ? static_cast<int>(pr[x][0]) : (i < s ? -static_cast<int>(pr[x][3]) : 0);
        if ((x == 0 || NCH == 4) && i < s) kst[i] = key[x];
      }
      // (the wave's own LDS writes come before its reads: LDS operations of
      // a wave take effect in order, and the compiler keeps the order)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x == 1 && NCH != 4) break;
        const int i = lane + 64 * x;
        int rank = 0;
        for (int k0 = 0; k0 < s; k0 += 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = k0 + e, kv = kst[k];
            rank += k < s && ((kv < key[x]) || (kv == key[x] && k < i));
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
    } else if (inplan && b == 0 && A.starts != nullptr) {
      // the tile's block starts in the bin buffer (in-kernel plan, batch row
      // 0), by the waves that do not sort, while the sort runs
      const int nsort = CAUSAL ? 1 : 2;  // waves NW - 4 (and NW - 3) sort
      scatter_starts(A, h, r0, n, s, w < NW - 4 ? w : w - nsort, NW - nsort, lane, sm + SM_REC,
                     reinterpret_cast<const int*>(sm + SM_BASE));
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
      // window of keys with weight: from the least block start of the first
      // row (slot 0 of the a order) to (not causal) the greatest block end of
      // the last row (slot 0 of the e2 order); and the hashes whose first-row
      // block starts left of the tile (slots s and above are not hashes)
      const int* sAa = reinterpret_cast<const int*>(sm + SM_SORT);
      const int a0 = sAa[lane];
      lo = __builtin_amdgcn_readfirstlane(a0);
      cntA = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < s && a0 < r0));
      if constexpr (NCH == 4) cntA += __builtin_popcountll(__builtin_amdgcn_ballot_w64(64 + lane < s && sAa[64 + lane] < r0));
      if constexpr (!CAUSAL) hi = __builtin_amdgcn_readfirstlane(sAa[256]);  // slot 0 of the e2 order
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
  // the sorted orders into registers and the far count operands (after the
  // near tiles, whose near-count operands they would otherwise sit beside):
  // slot k of the a order counts for row r iff r < e_k; slot k of the e2
  // order iff r >= a2_k (sentinel slots never count)
  if constexpr (PL) {
    u32x4 aeL[NCH][2];                  // e_i of slots 32 ch + 8 g .. + 7 (a order)
    u32x4 eaL[CAUSAL ? 1 : NCH][2];     // a2_i of those slots (e2 order)
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
                           bool literal, float* lse, hipStream_t st, const double* du) {
  const BinsLayout L = bins_layout(hq, s, n);
  char* base = const_cast<char*>(static_cast<const char*>(bins));
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.lse = lse;
  a.plan = reinterpret_cast<const PlanRec*>(base + L.off_plan);
  const bool inplan = du != nullptr && !literal;
  a.du = inplan ? du : nullptr;
  a.nblk = inplan ? reinterpret_cast<int32_t*>(base + L.off_nblk) : nullptr;
  a.starts = inplan ? reinterpret_cast<int32_t*>(base + L.off_starts) : nullptr;
  a.plan_out = inplan ? reinterpret_cast<PlanRec*>(base + L.off_plan) : nullptr;
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
  a.du = nullptr;
  a.nblk = nullptr;
  a.starts = nullptr;
  a.plan_out = nullptr;
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
