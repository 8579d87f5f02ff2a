// C ABI of libplpsh (declared in include/plpsh.h): argument validation,
// host hash draws, hash staging and kernel launches.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/plpsh.h"
#include "internal.h"

namespace {

using plpsh::BinsLayout;

thread_local char g_last_hip_error[256] = "";

// Records which HIP call failed; returns true on failure.
bool hip_failed(hipError_t e, const char* what) {
  if (e == hipSuccess) return false;
  std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s (%d)", what, hipGetErrorString(e),
                static_cast<int>(e));
  return true;
}

using plpsh::kMaxDevices;
constexpr int kGroupSlots = 16;  // calls per event
constexpr int kGroups = 2;
constexpr int kSlots = kGroups * kGroupSlots;
constexpr size_t kSlotQuantum = 64 << 10;  // slot sizes: multiples of 64 KB (4096 hashes)

// Per-device ring of pinned host slots holding (delta, u) pairs that the bin
// kernel reads directly (zero copy).  A slot is reused only after an event
// recorded behind the kernel that read it has completed.  An event recorded
// on a stream holds every later launch on it behind the marker, which costs
// the stream several microseconds, so on the null stream one event covers a
// group of up to kGroupSlots consecutive calls: the group closes (its event
// recorded behind its last kernel) when it is full or a call comes on
// another stream.  Calls on other streams, which the caller may destroy
// before a later call, close their group at once.
struct Staging {
  std::mutex mu;
  size_t slot_bytes = 0;  // per slot: the largest request so far, rounded up
  char* host = nullptr;   // kSlots * slot_bytes, pinned
  char* dev = nullptr;    // device view of `host`
  bool events = false;
  hipEvent_t ev[kGroups] = {};
  bool pending[kGroups] = {};  // event recorded and not yet waited for
  int next = 0;                // next slot
  int open_calls = 0;          // calls in the open group (the group of slot next - 1)
  hipStream_t open_stream = nullptr;
};
Staging g_staging[kMaxDevices];

bool staging_close(Staging& S) {
  if (S.open_calls == 0) return true;
  const int g = ((S.next + kSlots - 1) % kSlots) / kGroupSlots;
  if (hip_failed(hipEventRecord(S.ev[g], S.open_stream), "hipEventRecord(staging group)")) return false;
  S.pending[g] = true;
  S.open_calls = 0;
  return true;
}

bool staging_acquire(Staging& S, hipStream_t st, size_t bytes, int* slot) {
  if (!S.events) {
    for (int i = 0; i < kGroups; ++i)
      if (hip_failed(hipEventCreateWithFlags(&S.ev[i], hipEventDisableTiming), "hipEventCreateWithFlags"))
        return false;
    S.events = true;
  }
  if (bytes > S.slot_bytes) {
    // grow the ring: every kernel reading the old one has completed first
    if (!staging_close(S)) return false;
    for (int g = 0; g < kGroups; ++g)
      if (S.pending[g]) {
        if (hip_failed(hipEventSynchronize(S.ev[g]), "hipEventSynchronize(staging group)")) return false;
        S.pending[g] = false;
      }
    if (S.host && hip_failed(hipHostFree(S.host), "hipHostFree(staging)")) return false;
    S.host = S.dev = nullptr;
    S.slot_bytes = 0;
    const size_t sb = (bytes + kSlotQuantum - 1) / kSlotQuantum * kSlotQuantum;
    void* p = nullptr;
    if (hip_failed(hipHostMalloc(&p, kSlots * sb, hipHostMallocMapped | hipHostMallocCoherent),
                   "hipHostMalloc(staging)"))
      return false;
    void* d = nullptr;
    if (hip_failed(hipHostGetDevicePointer(&d, p, 0), "hipHostGetDevicePointer(staging)")) {
      (void)hipHostFree(p);
      return false;
    }
    S.host = static_cast<char*>(p);
    S.dev = static_cast<char*>(d);
    S.slot_bytes = sb;
    S.next = 0;
  }
  // a call on another stream closes the open group and starts the next one,
  // so that every group's event covers all of its calls
  if (S.open_calls > 0 && st != S.open_stream) {
    if (!staging_close(S)) return false;
    S.next = (S.next + kGroupSlots - 1) / kGroupSlots * kGroupSlots % kSlots;
  }
  const int i = S.next;
  const int g = i / kGroupSlots;
  if (i % kGroupSlots == 0 && S.pending[g]) {
    if (hip_failed(hipEventSynchronize(S.ev[g]), "hipEventSynchronize(staging group)")) return false;
    S.pending[g] = false;
  }
  S.next = (i + 1) % kSlots;
  *slot = i;
  return true;
}

bool finite_pos(double x) { return std::isfinite(x) && x > 0.0; }

bool valid_sigma(const double* sigma, int heads) {
  if (!sigma) return false;
  for (int h = 0; h < heads; ++h)
    if (!finite_pos(sigma[h])) return false;
  return true;
}

bool valid_hashes(const double* delta, const double* u, long long count) {
  if (!delta || !u) return false;
  for (long long i = 0; i < count; ++i) {
    if (!finite_pos(delta[i])) return false;
    if (!(u[i] >= 0.0 && u[i] <= delta[i])) return false;
  }
  return true;
}

bool valid_hs(int heads, int s) {
  return heads >= 1 && s >= 1 && s <= PLPSH_MAX_S &&
         static_cast<long long>(heads) * s <= PLPSH_MAX_HASHES;
}

// Upload (delta, u) into a pinned slot and launch(device address of the
// pairs), the one kernel that reads them.
template <class Launch>
plpsh_status with_staged_hashes(int heads, int s, const double* delta, const double* u, hipStream_t st,
                                const char* what, Launch&& launch) {
  int dev = 0;
  if (hip_failed(hipGetDevice(&dev), "hipGetDevice")) return PLPSH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PLPSH_ERR_UNSUPPORTED;
  Staging& S = g_staging[dev];
  std::lock_guard<std::mutex> lock(S.mu);
  const int hs = heads * s;
  int slot = 0;
  if (!staging_acquire(S, st, static_cast<size_t>(hs) * 2 * sizeof(double), &slot)) return PLPSH_ERR_HIP;
  double* du = reinterpret_cast<double*>(S.host + slot * S.slot_bytes);
  for (int t = 0; t < hs; ++t) {
    du[2 * t] = delta[t];
    du[2 * t + 1] = u[t];
  }
  const double* ddu = reinterpret_cast<const double*>(S.dev + slot * S.slot_bytes);
  if (hip_failed(launch(ddu), what)) return PLPSH_ERR_HIP;
  S.open_stream = st;
  ++S.open_calls;
  if (S.next % kGroupSlots == 0 || st != nullptr) {  // group full, or not the null stream
    if (!staging_close(S)) return PLPSH_ERR_HIP;
    S.next = (S.next + kGroupSlots - 1) / kGroupSlots * kGroupSlots % kSlots;
  }
  return PLPSH_OK;
}

// The bin kernel on staged hashes.
plpsh_status run_bins(int heads, int s, int n, const double* delta, const double* u, void* bins,
                      hipStream_t st) {
  const bool near_one = plpsh::bins_near_one(delta, static_cast<long long>(heads) * s);
  return with_staged_hashes(heads, s, delta, u, st, "bin kernel launch", [&](const double* ddu) {
    return plpsh::launch_bins(ddu, heads, s, n, bins, near_one, st);
  });
}

// Common argument checks of the attention entry points (everything except
// sigma / hashes / workspace).
plpsh_status check_qkv(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                       int n, int d, int dtype, int causal) {
  if (batch < 0 || n < 0 || hq < 1 || hkv < 1 || hq % hkv != 0) return PLPSH_ERR_INVALID_ARGUMENT;
  const bool empty = batch == 0 || n == 0;  // empty tensors may have null data
  if (!empty && (!q || !k || !v || !o)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return PLPSH_ERR_INVALID_ARGUMENT;
  if (dtype != PLPSH_DTYPE_F32 && dtype != PLPSH_DTYPE_BF16) return PLPSH_ERR_INVALID_ARGUMENT;
  if (d <= 0) return PLPSH_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return PLPSH_ERR_UNSUPPORTED;
  if (n > PLPSH_MAX_N || hq > 1024 || batch > 65535) return PLPSH_ERR_UNSUPPORTED;
  // the launches index (batch, head, 128-row tile) work items with 32-bit grids
  if ((static_cast<long long>(n + 127) / 128 + 7) * batch * hq >= (1ll << 31)) return PLPSH_ERR_UNSUPPORTED;
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if (al & 15) return PLPSH_ERR_INVALID_ARGUMENT;
  return PLPSH_OK;
}

constexpr int kMaxHeads = 1024;  // check_qkv rejects more query heads

// Query heads by cost, largest first (ties by head index): cost[h] is the
// sum over head h's hashes of min(delta, n), which grows with its key window.
void order_by_cost(int hq, const double* cost, uint16_t* order) {
  for (int h = 0; h < hq; ++h) order[h] = static_cast<uint16_t>(h);
  std::sort(order, order + hq, [&](uint16_t a, uint16_t b) { return cost[a] > cost[b] || (cost[a] == cost[b] && a < b); });
}

// Heads with the widest bins (largest key windows) first when delta is
// known, else the natural order.
void head_order(int hq, int s, int n, const double* delta, uint16_t* order) {
  double cost[kMaxHeads];
  for (int h = 0; h < hq; ++h) {
    cost[h] = 0.0;
    if (delta)
      for (int i = 0; i < s; ++i) cost[h] += std::min(delta[h * s + i], static_cast<double>(n));
  }
  order_by_cost(hq, cost, order);
}

// Launch the attention kernel on a computed bin buffer.
plpsh_status attention_on_bins(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                               int n, int d, int dtype, const double* delta, int s, int causal, const void* bins,
                               hipStream_t st, bool literal = false, float* lse = nullptr) {
  uint16_t order[kMaxHeads];
  head_order(hq, s, n, delta, order);
  if (hip_failed(plpsh::launch_plsh_fwd(q, k, v, o, batch, hq, hkv, n, d, dtype, s, causal, bins, order, literal,
                                        lse, st),
                 "attention kernel launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

plpsh_status attention_common(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                              int n, int d, int dtype, const double* delta, const double* u, int s, int causal,
                              void* ws, void* stream) {
  if (batch == 0 || n == 0) return PLPSH_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (plpsh::bins_near_one(delta, static_cast<long long>(hq) * s)) {
    // some start count without a closed form: the per-hash bin kernel first
    plpsh_status r = run_bins(hq, s, n, delta, u, ws, st);
    if (r != PLPSH_OK) return r;
    return attention_on_bins(q, k, v, o, batch, hq, hkv, n, d, dtype, delta, s, causal, ws, st);
  }
  // one launch: the attention kernel evaluates the bins of its query tiles
  // and writes the bin buffer as the bin kernel would
  uint16_t order[kMaxHeads];
  head_order(hq, s, n, delta, order);
  return with_staged_hashes(hq, s, delta, u, st, "attention kernel launch", [&](const double* ddu) {
    return plpsh::launch_plsh_fwd(q, k, v, o, batch, hq, hkv, n, d, dtype, s, causal, ws, order, false, nullptr,
                                  st, ddu);
  });
}

// ---- error of the mask mean against L* (Theorem 2.1), large n

constexpr int kMaxLanczos = 1000;

bool valid_err(double sigma, int n, int s) {
  return std::isfinite(sigma) && sigma > 0.0 && n >= 1 && n <= PLPSH_MAX_N && s >= 1 && s <= PLPSH_MAX_S;
}

// Number of eigenvalues below x of the symmetric tridiagonal matrix with
// diagonal a[0..k) and off-diagonal b[0..k-1) (Sturm sequence of the LDL^T
// pivots).
int sturm_below(const std::vector<double>& a, const std::vector<double>& b, int k, double x) {
  int cnt = 0;
  double q = 1.0;
  for (int i = 0; i < k; ++i) {
    const double bb = i > 0 ? b[i - 1] * b[i - 1] : 0.0;
    q = a[i] - x - (i > 0 ? bb / q : 0.0);
    if (q == 0.0) q = -1e-300;
    cnt += q < 0.0;
  }
  return cnt;
}

// Largest |eigenvalue| of that matrix, by bisection on the Sturm count.
double tridiag_spectral(const std::vector<double>& a, const std::vector<double>& b, int k) {
  double R = 0.0;
  for (int i = 0; i < k; ++i)
    R = std::max(R, std::fabs(a[i]) + (i > 0 ? std::fabs(b[i - 1]) : 0.0) + (i + 1 < k ? std::fabs(b[i]) : 0.0));
  if (R == 0.0) return 0.0;
  double lo = -R, hi = R;  // largest eigenvalue: count(x) == k for x above it
  for (int it = 0; it < 200 && hi - lo > 1e-15 * R; ++it) {
    const double mid = 0.5 * (lo + hi);
    (sturm_below(a, b, k, mid) < k ? lo : hi) = mid;
  }
  const double lmax = 0.5 * (lo + hi);
  lo = -R;
  hi = R;  // smallest eigenvalue: count(x) >= 1 for x above it
  for (int it = 0; it < 200 && hi - lo > 1e-15 * R; ++it) {
    const double mid = 0.5 * (lo + hi);
    (sturm_below(a, b, k, mid) >= 1 ? hi : lo) = mid;
  }
  const double lmin = 0.5 * (lo + hi);
  return std::max(std::fabs(lmax), std::fabs(lmin));
}

struct ErrWorkspace {
  size_t bins, scan, V, w, rowmax, h, part_v, part_i, scal, dots, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

ErrWorkspace err_workspace(int n, int s, int max_steps) {
  ErrWorkspace L{};
  size_t o = 0;
  L.bins = o;
  o = align256(o + plpsh::bins_layout(1, s, n).total);
  L.scan = o;
  o = align256(o + plpsh::err_scan_bytes(n));
  L.V = o;
  o = align256(o + static_cast<size_t>(max_steps + 1) * n * sizeof(double));
  L.w = o;
  o = align256(o + static_cast<size_t>(n) * sizeof(double));
  L.rowmax = o;
  o = align256(o + static_cast<size_t>(n) * sizeof(double));
  L.h = o;
  o = align256(o + 2 * static_cast<size_t>(max_steps + 1) * sizeof(double));
  L.part_v = o;
  o = align256(o + 256 * sizeof(double));
  L.part_i = o;
  o = align256(o + 256 * sizeof(int));
  L.scal = o;
  o = align256(o + 8 * sizeof(double));
  L.dots = o;
  o = align256(o + plpsh::err_dots_bytes(max_steps + 1));
  L.total = o;
  return L;
}

const plpsh::PlanRec* plan_of(const void* bins, int s, int n) {
  return reinterpret_cast<const plpsh::PlanRec*>(static_cast<const char*>(bins) + plpsh::bins_layout(1, s, n).off_plan);
}

}  // namespace

extern "C" {

const char* plpsh_status_string(int32_t st) {
  switch (st) {
    case PLPSH_OK: return "PLPSH_OK";
    case PLPSH_ERR_INVALID_ARGUMENT: return "PLPSH_ERR_INVALID_ARGUMENT";
    case PLPSH_ERR_UNSUPPORTED: return "PLPSH_ERR_UNSUPPORTED";
    case PLPSH_ERR_WORKSPACE_TOO_SMALL: return "PLPSH_ERR_WORKSPACE_TOO_SMALL";
    case PLPSH_ERR_HIP: return "PLPSH_ERR_HIP";
  }
  return "PLPSH_ERR_UNKNOWN";
}

const char* plpsh_version(void) { return "plpsh 0.1.0 (gfx950)"; }

const char* plpsh_last_hip_error(void) { return g_last_hip_error; }

plpsh_status plpsh_draw_hashes(uint64_t seed, int32_t heads, int32_t s, const double* sigma, double* delta,
                               double* u) {
  if (!valid_hs(heads, s) || !delta || !u || !valid_sigma(sigma, heads)) return PLPSH_ERR_INVALID_ARGUMENT;
  plpsh::draw_hashes(seed, heads, s, sigma, delta, u);
  return PLPSH_OK;
}

size_t plpsh_bins_bytes(int32_t heads, int32_t s, int32_t n) {
  if (!valid_hs(heads, s) || n < 1 || n > PLPSH_MAX_N) return 0;
  return plpsh::bins_layout(heads, s, n).total;
}

plpsh_status plpsh_bins_layout(int32_t heads, int32_t s, int32_t n, size_t* off_nblk, size_t* off_starts,
                               size_t* off_plan) {
  if (!valid_hs(heads, s) || n < 1 || n > PLPSH_MAX_N || !off_nblk || !off_starts || !off_plan)
    return PLPSH_ERR_INVALID_ARGUMENT;
  const BinsLayout L = plpsh::bins_layout(heads, s, n);
  *off_nblk = L.off_nblk;
  *off_starts = L.off_starts;
  *off_plan = L.off_plan;
  return PLPSH_OK;
}

plpsh_status plpsh_bins_from_hashes(int32_t heads, int32_t s, int32_t n, const double* delta, const double* u,
                                    void* bins, size_t bins_bytes, void* stream) {
  if (!valid_hs(heads, s) || n < 1 || !bins) return PLPSH_ERR_INVALID_ARGUMENT;
  if (n > PLPSH_MAX_N) return PLPSH_ERR_UNSUPPORTED;
  if (!valid_hashes(delta, u, static_cast<long long>(heads) * s)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(bins) & 255) return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins_bytes < plpsh::bins_layout(heads, s, n).total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  return run_bins(heads, s, n, delta, u, bins, static_cast<hipStream_t>(stream));
}

plpsh_status plpsh_sample_bins(uint64_t seed, int32_t heads, int32_t s, int32_t n, const double* sigma,
                               double* delta, double* u, void* bins, size_t bins_bytes, void* stream) {
  if (!valid_hs(heads, s) || !valid_sigma(sigma, heads)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins) {
    if (n < 1) return PLPSH_ERR_INVALID_ARGUMENT;
    if (n > PLPSH_MAX_N) return PLPSH_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(bins) & 255) return PLPSH_ERR_INVALID_ARGUMENT;
    if (bins_bytes < plpsh::bins_layout(heads, s, n).total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  }
  const size_t hs = static_cast<size_t>(heads) * s;
  std::vector<double> dl(hs), uu(hs);
  plpsh::draw_hashes(seed, heads, s, sigma, dl.data(), uu.data());
  if (delta) std::memcpy(delta, dl.data(), hs * sizeof(double));
  if (u) std::memcpy(u, uu.data(), hs * sizeof(double));
  if (!bins) return PLPSH_OK;
  return run_bins(heads, s, n, dl.data(), uu.data(), bins, static_cast<hipStream_t>(stream));
}

size_t plpsh_workspace_bytes(int32_t heads_q, int32_t s, int32_t n) {
  if (n == 0) return 256;
  return plpsh_bins_bytes(heads_q, s, n);
}

plpsh_status plpsh_attention_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                 int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim, int32_t dtype,
                                 const double* sigma, int32_t s, uint64_t seed, int32_t causal, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  plpsh_status r = check_qkv(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_hs(heads_q, s) || !valid_sigma(sigma, heads_q)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < plpsh_workspace_bytes(heads_q, s, n)) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  const size_t hs = static_cast<size_t>(heads_q) * s;
  std::vector<double> dl(hs), uu(hs);
  plpsh::draw_hashes(seed, heads_q, s, sigma, dl.data(), uu.data());
  return attention_common(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, dl.data(), uu.data(), s,
                          causal, workspace, stream);
}

plpsh_status plpsh_attention_fwd_hashes(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                        int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                        int32_t dtype, const double* delta, const double* u, int32_t s,
                                        int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  plpsh_status r = check_qkv(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_hs(heads_q, s) || !valid_hashes(delta, u, static_cast<long long>(heads_q) * s))
    return PLPSH_ERR_INVALID_ARGUMENT;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < plpsh_workspace_bytes(heads_q, s, n)) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  return attention_common(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, delta, u, s, causal,
                          workspace, stream);
}

plpsh_status plpsh_fixed_blocks_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                    int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                    int32_t dtype, const int32_t* block, int32_t causal, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!block || heads_q < 1 || heads_q > 1024) return PLPSH_ERR_INVALID_ARGUMENT;
  std::vector<double> delta(heads_q), u(heads_q, 0.0);
  for (int h = 0; h < heads_q; ++h) {
    if (block[h] < 1 || block[h] > PLPSH_MAX_N) return PLPSH_ERR_INVALID_ARGUMENT;
    delta[h] = static_cast<double>(block[h]);
  }
  return plpsh_attention_fwd_hashes(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, delta.data(), u.data(),
                                    1, causal, workspace, workspace_bytes, stream);
}

namespace {
plpsh_status fwd_bins(const void* q, const void* k, const void* v, void* o, int32_t batch, int32_t heads_q,
                      int32_t heads_kv, int32_t n, int32_t head_dim, int32_t dtype, int32_t s, int32_t causal,
                      const void* bins, size_t bins_bytes, const double* delta, void* stream, bool literal,
                      float* lse = nullptr) {
  plpsh_status r = check_qkv(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_hs(heads_q, s)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (batch == 0 || n == 0) return PLPSH_OK;
  if (!bins || (reinterpret_cast<uintptr_t>(bins) & 255)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins_bytes < plpsh::bins_layout(heads_q, s, n).total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  if (delta) {
    for (long long i = 0; i < static_cast<long long>(heads_q) * s; ++i)
      if (!finite_pos(delta[i])) return PLPSH_ERR_INVALID_ARGUMENT;
  }
  return attention_on_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, delta, s, causal, bins,
                           static_cast<hipStream_t>(stream), literal, lse);
}
}  // namespace

plpsh_status plpsh_attention_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int32_t batch,
                                     int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                     int32_t dtype, int32_t s, int32_t causal, const void* bins,
                                     size_t bins_bytes, const double* delta, void* stream) {
  if ((!lse && batch > 0 && n > 0) || (reinterpret_cast<uintptr_t>(lse) & 3)) return PLPSH_ERR_INVALID_ARGUMENT;
  return fwd_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins, bins_bytes, delta,
                  stream, false, lse);
}

plpsh_status plpsh_attention_fwd_bins(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                      int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                      int32_t dtype, int32_t s, int32_t causal, const void* bins,
                                      size_t bins_bytes, const double* delta, void* stream) {
  return fwd_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins, bins_bytes, delta,
                  stream, false);
}

plpsh_status plpsh_attention_fwd_literal(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                         int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                         int32_t dtype, int32_t s, int32_t causal, const void* bins,
                                         size_t bins_bytes, const double* delta, void* stream) {
  return fwd_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins, bins_bytes, delta,
                  stream, true);
}

plpsh_status plpsh_alibi_dense_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                   int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim, int32_t dtype,
                                   const double* sigma, int32_t causal, void* stream) {
  plpsh_status r = check_qkv(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_sigma(sigma, heads_q)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (heads_q > 256) return PLPSH_ERR_UNSUPPORTED;
  if (batch == 0 || n == 0) return PLPSH_OK;
  float beta[256];
  for (int h = 0; h < heads_q; ++h) beta[h] = static_cast<float>(1.4426950408889634 / sigma[h]);
  if (hip_failed(plpsh::launch_alibi_fwd(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, beta, causal,
                                         static_cast<hipStream_t>(stream)),
                 "dense ALiBi kernel launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

size_t plpsh_error_workspace_bytes(int32_t n, int32_t s, int32_t max_steps) {
  if (!valid_err(1.0, n, s) || max_steps < 0 || max_steps > kMaxLanczos) return 0;
  if (max_steps == 0) return plpsh::err_scan_bytes(n);
  return err_workspace(n, s, max_steps).total;
}

plpsh_status plpsh_error_rowmax(double sigma, int32_t n, int32_t s, const void* bins, size_t bins_bytes,
                                double* rowmax, void* stream) {
  if (!valid_err(sigma, n, s) || !bins || !rowmax || (reinterpret_cast<uintptr_t>(bins) & 255))
    return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins_bytes < plpsh::bins_layout(1, s, n).total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  if (hip_failed(plpsh::launch_err_rowmax(plan_of(bins, s, n), n, s, sigma, rowmax, static_cast<hipStream_t>(stream)),
                 "error row-maximum kernel launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

plpsh_status plpsh_error_matvec(double sigma, int32_t n, int32_t s, const void* bins, size_t bins_bytes,
                                const double* x, double* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_err(sigma, n, s) || !bins || !x || !y || !workspace || (reinterpret_cast<uintptr_t>(bins) & 255) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) || x == y)
    return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins_bytes < plpsh::bins_layout(1, s, n).total || workspace_bytes < plpsh::err_scan_bytes(n))
    return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  if (hip_failed(plpsh::launch_err_matvec(plan_of(bins, s, n), n, s, sigma, x, y, workspace,
                                          static_cast<hipStream_t>(stream)),
                 "error product kernels launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

plpsh_status plpsh_error_norms(double sigma, int32_t n, int32_t s, const double* delta, const double* u,
                               int32_t max_steps, double tol, uint64_t seed, void* workspace, size_t workspace_bytes,
                               double* spectral, double* maxnorm, int32_t* argmax_row, int32_t* steps,
                               void* stream) {
  if (!valid_err(sigma, n, s) || !valid_hashes(delta, u, s) || max_steps < 1 || max_steps > kMaxLanczos ||
      !(tol > 0.0) || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || !spectral || !maxnorm)
    return PLPSH_ERR_INVALID_ARGUMENT;
  const ErrWorkspace L = err_workspace(n, s, max_steps);
  if (workspace_bytes < L.total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* bins = ws + L.bins;
  plpsh_status r = run_bins(1, s, n, delta, u, bins, st);
  if (r != PLPSH_OK) return r;
  const plpsh::PlanRec* plan = plan_of(bins, s, n);
  double* V = reinterpret_cast<double*>(ws + L.V);
  double* w = reinterpret_cast<double*>(ws + L.w);
  double* rowmax = reinterpret_cast<double*>(ws + L.rowmax);
  double* h1 = reinterpret_cast<double*>(ws + L.h);
  double* h2 = h1 + (max_steps + 1);
  double* scal = reinterpret_cast<double*>(ws + L.scal);
  double* dpart = reinterpret_cast<double*>(ws + L.dots);
  const size_t ld = static_cast<size_t>(n);

  // max norm: row maxima, then the largest of them
  if (hip_failed(plpsh::launch_err_rowmax(plan, n, s, sigma, rowmax, st), "error row-maximum kernel launch") ||
      hip_failed(plpsh::launch_err_argmax(rowmax, n, reinterpret_cast<double*>(ws + L.part_v),
                                          reinterpret_cast<int*>(ws + L.part_i), scal + 4,
                                          reinterpret_cast<int*>(scal + 5), st),
                 "argmax kernel launch"))
    return PLPSH_ERR_HIP;

  // spectral norm: Lanczos on the symmetric E with full reorthogonalisation
  // (classical Gram-Schmidt, twice); the extreme eigenvalues of the
  // tridiagonal matrix by bisection after every step
  std::vector<double> v0(n);
  {
    uint64_t state = seed;
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) {
      state += 0x9E3779B97F4A7C15ull;
      uint64_t z = state;
      z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
      z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
      z ^= z >> 31;
      v0[i] = static_cast<double>(z >> 11) * 0x1p-53 - 0.5;
      nrm += v0[i] * v0[i];
    }
    nrm = std::sqrt(nrm);
    for (double& x : v0) x /= nrm;
  }
  if (hip_failed(hipMemcpyAsync(V, v0.data(), n * sizeof(double), hipMemcpyHostToDevice, st), "hipMemcpyAsync(v0)") ||
      hip_failed(hipStreamSynchronize(st), "hipStreamSynchronize"))
    return PLPSH_ERR_HIP;
  std::vector<double> alpha, beta;
  double spec = 0.0, prev = -1.0;
  int stable = 0, k = 0;
  double host[8];
  for (k = 0; k < max_steps; ++k) {
    double* vk = V + k * ld;
    bool fail = hip_failed(plpsh::launch_err_matvec(plan, n, s, sigma, vk, w, ws + L.scan, st), "error product");
    fail = fail || hip_failed(plpsh::launch_err_dots(V, ld, k + 1, w, n, h1, dpart, st), "dots") ||
           hip_failed(plpsh::launch_err_sub_proj(V, ld, h1, k + 1, n, w, st), "projection") ||
           hip_failed(plpsh::launch_err_dots(V, ld, k + 1, w, n, h2, dpart, st), "dots") ||
           hip_failed(plpsh::launch_err_sub_proj(V, ld, h2, k + 1, n, w, st), "projection") ||
           hip_failed(plpsh::launch_err_dots(w, ld, 1, w, n, scal + 2, dpart, st), "norm") ||
           hip_failed(hipMemcpyAsync(scal, h1 + k, sizeof(double), hipMemcpyDeviceToDevice, st), "copy") ||
           hip_failed(hipMemcpyAsync(scal + 1, h2 + k, sizeof(double), hipMemcpyDeviceToDevice, st), "copy") ||
           hip_failed(hipMemcpyAsync(host, scal, 8 * sizeof(double), hipMemcpyDeviceToHost, st), "copy") ||
           hip_failed(hipStreamSynchronize(st), "hipStreamSynchronize");
    if (fail) return PLPSH_ERR_HIP;
    alpha.push_back(host[0] + host[1]);
    const double bk = std::sqrt(std::max(host[2], 0.0));
    spec = tridiag_spectral(alpha, beta, k + 1);
    if (k == 0) {
      *maxnorm = host[4];
      int im = 0;
      std::memcpy(&im, &host[5], sizeof(int));
      if (argmax_row) *argmax_row = im;
    }
    stable = (prev >= 0.0 && std::fabs(spec - prev) <= tol * spec) ? stable + 1 : 0;
    prev = spec;
    if (stable >= 3 || bk <= 1e-13 * std::max(spec, 1e-300) || k + 1 == max_steps || k + 1 == n) {
      ++k;
      break;
    }
    beta.push_back(bk);
    if (hip_failed(plpsh::launch_err_scale(w, 1.0 / bk, n, V + (k + 1) * ld, st), "scale")) return PLPSH_ERR_HIP;
  }
  *spectral = spec;
  if (steps) *steps = k;
  return PLPSH_OK;
}

size_t plpsh_attention_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t n) {
  if (batch < 0 || heads_q < 1 || n < 0 || n > PLPSH_MAX_N) return 0;
  return std::max<size_t>(256, (static_cast<size_t>(batch) * heads_q * n * sizeof(float) + 255) & ~size_t{255});
}

plpsh_status plpsh_attention_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q,
                                 int32_t heads_kv, int32_t n, int32_t head_dim, int32_t dtype, int32_t s,
                                 int32_t causal, const void* bins, size_t bins_bytes, const double* delta,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  plpsh_status r = check_qkv(q, k, v, dq, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_hs(heads_q, s)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (batch == 0 || n == 0) return PLPSH_OK;
  if (!o || !dout || !lse || !dk || !dv || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return PLPSH_ERR_INVALID_ARGUMENT;
  for (const void* p : {o, dout, static_cast<const void*>(dk), static_cast<const void*>(dv)})
    if (reinterpret_cast<uintptr_t>(p) & 15) return PLPSH_ERR_INVALID_ARGUMENT;
  if (dtype != PLPSH_DTYPE_BF16) return PLPSH_ERR_UNSUPPORTED;
  if (!bins || (reinterpret_cast<uintptr_t>(bins) & 255)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (bins_bytes < plpsh::bins_layout(heads_q, s, n).total) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  if (workspace_bytes < plpsh_attention_bwd_workspace_bytes(batch, heads_q, n)) return PLPSH_ERR_WORKSPACE_TOO_SMALL;
  if (delta) {
    for (long long i = 0; i < static_cast<long long>(heads_q) * s; ++i)
      if (!finite_pos(delta[i])) return PLPSH_ERR_INVALID_ARGUMENT;
  }
  // heads (dQ) and KV groups (dK, dV) with the widest bins first
  std::vector<double> cost(heads_q, 0.0);
  if (delta)
    for (int h = 0; h < heads_q; ++h)
      for (int i = 0; i < s; ++i) cost[h] += std::min(delta[h * s + i], static_cast<double>(n));
  std::vector<uint16_t> oq(heads_q), okv(heads_kv);
  std::iota(oq.begin(), oq.end(), 0);
  std::iota(okv.begin(), okv.end(), 0);
  std::stable_sort(oq.begin(), oq.end(), [&](uint16_t a, uint16_t b) { return cost[a] > cost[b]; });
  const int grp = heads_q / heads_kv;
  std::vector<double> gcost(heads_kv, 0.0);
  for (int h = 0; h < heads_q; ++h) gcost[h / grp] += cost[h];
  std::stable_sort(okv.begin(), okv.end(), [&](uint16_t a, uint16_t b) { return gcost[a] > gcost[b]; });
  if (hip_failed(plpsh::launch_plsh_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads_q, heads_kv, n, head_dim, s,
                                        causal, bins, oq.data(), okv.data(), static_cast<float*>(workspace),
                                        static_cast<hipStream_t>(stream)),
                 "backward kernels launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

}  // extern "C"

// ---- attention with no allocation: the bin buffer in a static device array

namespace {

// The library's own scratch: (delta, u) pairs, then a bin buffer of up to
// PLPSH_NOALLOC_BINS_BYTES.  Every device holds its own copy at its own
// address from module load until the process ends.  In host code `scratch`
// only names the symbol: its device address comes from hipGetSymbolAddress.
constexpr size_t kNoallocHashBytes = static_cast<size_t>(PLPSH_NOALLOC_MAX_HASHES) * 2 * sizeof(double);
__device__ __align__(256) unsigned char scratch[kNoallocHashBytes + PLPSH_NOALLOC_BINS_BYTES];

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (looked up once per device, with
// that device current).
plpsh_status scratch_ptr(char** out) {
  int dev = 0;
  if (hip_failed(hipGetDevice(&dev), "hipGetDevice")) return PLPSH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PLPSH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hip_failed(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return PLPSH_ERR_HIP;
    if (!p) return PLPSH_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return PLPSH_OK;
}

// (delta, u) pairs reach the device as kernel arguments (copied by the
// runtime at launch), kStagePairs per launch: no host staging memory.
constexpr int kStagePairs = 224;
struct StageArgs {
  int32_t first, count;
  double du[2 * kStagePairs];
};
static_assert(sizeof(StageArgs) <= 3600, "kernel arguments stay under 4 KB");

__global__ __launch_bounds__(2 * kStagePairs) void stage_hashes_kernel(StageArgs a, double* __restrict__ dst) {
  const int t = static_cast<int>(threadIdx.x);
  if (t < 2 * a.count) dst[2 * static_cast<size_t>(a.first) + t] = a.du[t];
}

}  // namespace

extern "C" plpsh_status plpsh_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                                    int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t n,
                                                    int32_t head_dim, int32_t dtype, const double* sigma, int32_t s,
                                                    uint64_t seed, int32_t causal, void* stream) {
  plpsh_status r = check_qkv(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, causal);
  if (r != PLPSH_OK) return r;
  if (!valid_hs(heads_q, s) || !valid_sigma(sigma, heads_q)) return PLPSH_ERR_INVALID_ARGUMENT;
  if (batch == 0 || n == 0) return PLPSH_OK;
  const int hs = heads_q * s;
  if (hs > PLPSH_NOALLOC_MAX_HASHES) return PLPSH_ERR_UNSUPPORTED;
  if (plpsh::bins_layout(heads_q, s, n).total > PLPSH_NOALLOC_BINS_BYTES) return PLPSH_ERR_UNSUPPORTED;
  char* base = nullptr;
  if ((r = scratch_ptr(&base)) != PLPSH_OK) return r;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  double* du = reinterpret_cast<double*>(base);
  void* bins = base + kNoallocHashBytes;

  // hashes drawn straight into the launch arguments; per-head costs on the way
  double cost[kMaxHeads] = {};
  bool near_one = false;
  StageArgs a;
  for (int first = 0; first < hs; first += kStagePairs) {
    a.first = first;
    a.count = std::min(kStagePairs, hs - first);
    for (int t = 0; t < a.count; ++t) {
      const int h = (first + t) / s, i = (first + t) - h * s;
      plpsh::draw_hash(seed, h, i, sigma[h], &a.du[2 * t], &a.du[2 * t + 1]);
      cost[h] += std::min(a.du[2 * t], static_cast<double>(n));
      near_one = near_one || plpsh::bins_near_one(&a.du[2 * t], 1);
    }
    hipLaunchKernelGGL(stage_hashes_kernel, dim3(1), dim3(2 * kStagePairs), 0, st, a, du);
    if (hip_failed(hipGetLastError(), "hash staging kernel launch")) return PLPSH_ERR_HIP;
  }
  // with every start count in closed form the attention kernel evaluates its
  // own plan (one launch), else the per-hash bin kernel runs first
  if (near_one && hip_failed(plpsh::launch_bins(du, heads_q, s, n, bins, true, st), "bin kernel launch"))
    return PLPSH_ERR_HIP;
  uint16_t order[kMaxHeads];
  order_by_cost(heads_q, cost, order);
  if (hip_failed(plpsh::launch_plsh_fwd(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins,
                                        order, false, nullptr, st, near_one ? nullptr : du),
                 "attention kernel launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}
