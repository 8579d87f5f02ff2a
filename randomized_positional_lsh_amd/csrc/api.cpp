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

constexpr int kMaxDevices = 64;
constexpr int kSlots = 8;
constexpr size_t kSlotBytes = static_cast<size_t>(PLPSH_MAX_HASHES) * 2 * sizeof(double);

// Per-device ring of pinned host slots holding (delta, u) pairs that the bin
// kernel reads directly (zero copy).  A slot is reused only after the event
// recorded behind the kernel that read it has completed.
struct Staging {
  std::mutex mu;
  bool ready = false;
  char* host = nullptr;   // kSlots * kSlotBytes, pinned
  char* dev = nullptr;    // device view of `host`
  hipEvent_t ev[kSlots] = {};
  bool used[kSlots] = {};
  int next = 0;
};
Staging g_staging[kMaxDevices];

bool staging_acquire(Staging& S, int* slot) {
  if (!S.ready) {
    void* p = nullptr;
    if (hip_failed(hipHostMalloc(&p, kSlots * kSlotBytes, hipHostMallocMapped | hipHostMallocCoherent),
                   "hipHostMalloc(staging)"))
      return false;
    void* d = nullptr;
    if (hip_failed(hipHostGetDevicePointer(&d, p, 0), "hipHostGetDevicePointer(staging)")) return false;
    for (int i = 0; i < kSlots; ++i)
      if (hip_failed(hipEventCreateWithFlags(&S.ev[i], hipEventDisableTiming), "hipEventCreateWithFlags"))
        return false;
    S.host = static_cast<char*>(p);
    S.dev = static_cast<char*>(d);
    S.ready = true;
  }
  const int i = S.next;
  S.next = (S.next + 1) % kSlots;
  if (S.used[i] && hip_failed(hipEventSynchronize(S.ev[i]), "hipEventSynchronize(staging slot)")) return false;
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

// Upload (delta, u) into a pinned slot and launch the bin kernel on it.
plpsh_status run_bins(int heads, int s, int n, const double* delta, const double* u, void* bins,
                      hipStream_t st) {
  int dev = 0;
  if (hip_failed(hipGetDevice(&dev), "hipGetDevice")) return PLPSH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PLPSH_ERR_UNSUPPORTED;
  Staging& S = g_staging[dev];
  std::lock_guard<std::mutex> lock(S.mu);
  int slot = 0;
  if (!staging_acquire(S, &slot)) return PLPSH_ERR_HIP;
  double* du = reinterpret_cast<double*>(S.host + slot * kSlotBytes);
  const int hs = heads * s;
  for (int t = 0; t < hs; ++t) {
    du[2 * t] = delta[t];
    du[2 * t + 1] = u[t];
  }
  const double* ddu = reinterpret_cast<const double*>(S.dev + slot * kSlotBytes);
  if (hip_failed(plpsh::launch_bins(ddu, heads, s, n, bins, st), "bin kernel launch")) return PLPSH_ERR_HIP;
  if (hip_failed(hipEventRecord(S.ev[slot], st), "hipEventRecord(staging slot)")) return PLPSH_ERR_HIP;
  S.used[slot] = true;
  return PLPSH_OK;
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
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if (al & 15) return PLPSH_ERR_INVALID_ARGUMENT;
  return PLPSH_OK;
}

// Launch the attention kernel on a computed bin buffer.  Heads with the
// widest bins (largest key windows) are scheduled first when delta is known.
plpsh_status attention_on_bins(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                               int n, int d, int dtype, const double* delta, int s, int causal, const void* bins,
                               hipStream_t st, bool literal = false) {
  std::vector<uint16_t> order(hq);
  std::iota(order.begin(), order.end(), 0);
  if (delta) {
    std::vector<double> cost(hq, 0.0);
    for (int h = 0; h < hq; ++h)
      for (int i = 0; i < s; ++i) cost[h] += std::min(delta[h * s + i], static_cast<double>(n));
    std::stable_sort(order.begin(), order.end(), [&](uint16_t a, uint16_t b) { return cost[a] > cost[b]; });
  }
  if (hip_failed(plpsh::launch_plsh_fwd(q, k, v, o, batch, hq, hkv, n, d, dtype, s, causal, bins, order.data(),
                                        literal, st),
                 "attention kernel launch"))
    return PLPSH_ERR_HIP;
  return PLPSH_OK;
}

plpsh_status attention_common(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                              int n, int d, int dtype, const double* delta, const double* u, int s, int causal,
                              void* ws, void* stream) {
  if (batch == 0 || n == 0) return PLPSH_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  plpsh_status r = run_bins(hq, s, n, delta, u, ws, st);
  if (r != PLPSH_OK) return r;
  return attention_on_bins(q, k, v, o, batch, hq, hkv, n, d, dtype, delta, s, causal, ws, st);
}

}  // namespace

extern "C" {

const char* plpsh_status_string(plpsh_status st) {
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
                                 int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim, plpsh_dtype dtype,
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
                                        plpsh_dtype dtype, const double* delta, const double* u, int32_t s,
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
                                    plpsh_dtype dtype, const int32_t* block, int32_t causal, void* workspace,
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
                      int32_t heads_kv, int32_t n, int32_t head_dim, plpsh_dtype dtype, int32_t s, int32_t causal,
                      const void* bins, size_t bins_bytes, const double* delta, void* stream, bool literal) {
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
                           static_cast<hipStream_t>(stream), literal);
}
}  // namespace

plpsh_status plpsh_attention_fwd_bins(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                      int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                      plpsh_dtype dtype, int32_t s, int32_t causal, const void* bins,
                                      size_t bins_bytes, const double* delta, void* stream) {
  return fwd_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins, bins_bytes, delta,
                  stream, false);
}

plpsh_status plpsh_attention_fwd_literal(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                         int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim,
                                         plpsh_dtype dtype, int32_t s, int32_t causal, const void* bins,
                                         size_t bins_bytes, const double* delta, void* stream) {
  return fwd_bins(q, k, v, o, batch, heads_q, heads_kv, n, head_dim, dtype, s, causal, bins, bins_bytes, delta,
                  stream, true);
}

plpsh_status plpsh_alibi_dense_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                   int32_t heads_q, int32_t heads_kv, int32_t n, int32_t head_dim, plpsh_dtype dtype,
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

}  // extern "C"
