// Internal declarations shared by the host API and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <mutex>

namespace plpsh {

// One plan record: the blocks of one hash as seen from one 128-row query
// tile (layout documented in plpsh.h).
struct alignas(16) PlanRec {
  int32_t a, e;      // block containing the tile's first row
  int32_t a2, e2;    // block containing the tile's last row
  uint32_t bits[4];  // bit p: position r0 + p (1 <= p < 128) starts a block or equals n
};
static_assert(sizeof(PlanRec) == 32, "plan record is 32 bytes");

constexpr int kPlanTile = 128;

// Dynamic LDS above the 64 KB default needs an opt-in per kernel, and
// hipFuncSetAttribute applies to the device current at the call.  One
// LdsOptIn per kernel records, per device, the largest size granted there, so
// every device is opted in on its first launch and again whenever a launch
// needs more.
constexpr int kMaxDevices = 64;
struct LdsOptIn {
  std::atomic<size_t> granted[kMaxDevices] = {};
  std::mutex mu;
  hipError_t ensure(const void* fn, size_t need) {
    if (need <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (granted[dev].load(std::memory_order_acquire) >= need) return hipSuccess;
    std::lock_guard<std::mutex> lock(mu);
    if (granted[dev].load(std::memory_order_relaxed) >= need) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(need));
    if (e != hipSuccess) return e;
    granted[dev].store(need, std::memory_order_release);
    return hipSuccess;
  }
};

struct BinsLayout {
  size_t off_nblk, off_starts, off_plan, total;
};
BinsLayout bins_layout(int heads, int s, int n);

// Host draw (SplitMix64 counter mode, see plpsh.h): all heads * s hashes,
// or hash i of head h alone (the same value, the streams are counter-based).
void draw_hashes(uint64_t seed, int heads, int s, const double* sigma, double* delta, double* u);
void draw_hash(uint64_t seed, int h, int i, double sigma, double* delta, double* u);

// Device launches.  `du` points to heads*s interleaved (delta, u) pairs in
// device-readable memory.
// near_one: some delta lies within 2^-30 of 1 (such hashes take the per-hash kernel)
bool bins_near_one(const double* delta, long long count);
hipError_t launch_bins(const double* du, int heads, int s, int n, void* bins, bool near_one, hipStream_t st);

// du (device-readable interleaved (delta, u) pairs, count-weighted mode
// only): the kernel evaluates its own plan records and writes the whole bin
// buffer `bins` (no delta may lie within 2^-30 of 1); null: it reads the
// records of a bin buffer that the bin kernel wrote.
hipError_t launch_plsh_fwd(const void* q, const void* k, const void* v, void* o,
                           int batch, int hq, int hkv, int n, int d, int dtype,
                           int s, int causal, const void* bins, const uint16_t* head_order,
                           bool literal, float* lse, hipStream_t st, const double* du = nullptr);

hipError_t launch_alibi_fwd(const void* q, const void* k, const void* v, void* o,
                            int batch, int hq, int hkv, int n, int d, int dtype,
                            const float* beta_host, int causal, hipStream_t st);

// Backward pass (bwd.hip), bf16: dd receives D_r = <dO_r, O_r>, batch*hq*n floats.
hipError_t launch_plsh_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int n, int d,
                           int s, int causal, const void* bins, const uint16_t* head_order, const uint16_t* kv_order,
                           float* dd, hipStream_t st);

// Error of the mask mean against L* (errnorm.hip).  `plan` is the plan-record
// array of one head; scratch for the products is err_scan_bytes(n) bytes.
size_t err_scan_bytes(int n);
hipError_t launch_err_rowmax(const PlanRec* plan, int n, int s, double sigma, double* rowmax, hipStream_t st);
hipError_t launch_err_matvec(const PlanRec* plan, int n, int s, double sigma, const double* x, double* y,
                             void* scratch, hipStream_t st);
size_t err_dots_bytes(int m);  // scratch of launch_err_dots for m vectors
hipError_t launch_err_dots(const double* V, size_t ld, int m, const double* w, int n, double* out, double* part,
                           hipStream_t st);
hipError_t launch_err_sub_proj(const double* V, size_t ld, const double* h, int m, int n, double* w, hipStream_t st);
hipError_t launch_err_scale(const double* w, double c, int n, double* v, hipStream_t st);
hipError_t launch_err_argmax(const double* a, int n, double* pv, int* pi, double* out_v, int* out_i, hipStream_t st);

}  // namespace plpsh
