/*
 * plpsh.h -- C ABI of the Positional-LSH approximation of ALiBi attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Source of the method.  The explainer pages of arXiv 2605.09472,
 * "Positional LSH: Binary Block Matrix Approximation for Attention with
 * Linear Biases" (D. Wolfson, T. Wagner; gist.science, Dutch / Chinese /
 * Japanese versions with the same sections).  Citations below name the
 * section of those pages: "Methodology 1" (positional LSH framework),
 * "Theorem 2.1" (structural approximation), "Theorem 2.2" (algorithmic
 * reduction), "Key results".
 *
 * What is computed.  ALiBi attention with slope 1/sigma weights key j of
 * query r by L*[r,j] = exp(-|r-j|/sigma), a Laplace kernel over positions
 * (Methodology 1).  A random-binning hash of the integer positions --
 * width delta ~ Gamma(shape 2, scale sigma), offset u ~ U[0, delta),
 * bin(x) = floor((x - u) / delta) -- cuts [0, n) into contiguous,
 * non-overlapping blocks, and E[M(h)] = L* for its block mask M(h)
 * (Methodology 1).  With s i.i.d. hashes the empirical mean
 * M~ = (1/s) sum_i M(h_i) approximates L* (Theorem 2.1), and
 *
 *   O_r = sum_j c[r,j] C[r,j] exp(S[r,j]) v_j / sum_j c[r,j] C[r,j] exp(S[r,j])
 *
 * with c[r,j] = #{i : bin_i(r) == bin_i(j)} = s * M~[r,j],
 * S = Q K^T / sqrt(d) and C[r,j] = [j <= r] when causal (else 1), is the
 * attention with L* replaced by M~ (Theorem 2.1, Theorem 2.2).
 *
 * Conventions shared by every entry point.
 *  - Every function returns a plpsh_status, never throws and never exits.
 *  - Every argument is validated before any HIP call; on a validation error
 *    nothing is launched and no output is touched.
 *  - Device pointers are caller-owned device memory (e.g. PyTorch tensors);
 *    the library allocates no device memory (its one static device array,
 *    used by plpsh_attention_fwd_noalloc, is part of the loaded module).
 *    Host pointers are only read or written during the call.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *    enqueued on it and runs asynchronously; results are valid after the
 *    caller synchronises the stream.  PLPSH_ERR_HIP reports a launch or
 *    runtime error returned by HIP during the call; asynchronous device
 *    faults surface at the caller's next synchronisation.
 *  - Work runs on the calling thread's current HIP device.
 *  - Entry points are reentrant.  The library keeps, per device, a small
 *    pinned host staging ring for hash parameters (allocated on first use,
 *    held until process exit).
 */
#ifndef PLPSH_H
#define PLPSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PLPSH_OK = 0,
    PLPSH_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, bad value */
    PLPSH_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim) */
    PLPSH_ERR_WORKSPACE_TOO_SMALL = 3,
    PLPSH_ERR_HIP = 4                 /* HIP runtime / launch error */
} plpsh_status;

/* Element types.  Entry points take the type as an int32_t `dtype` holding
 * one of these values (any other value is rejected with
 * PLPSH_ERR_INVALID_ARGUMENT). */
typedef enum {
    PLPSH_DTYPE_F32 = 0,    /* float32 Q/K/V/O; fp32 matrix cores, fp32 softmax */
    PLPSH_DTYPE_BF16 = 1    /* bfloat16 Q/K/V/O; bf16 matrix cores, fp32 accumulation */
} plpsh_dtype;

/* Limits of this implementation. */
#define PLPSH_MAX_S 128            /* hashes per head */
#define PLPSH_MAX_N 524288         /* sequence length */
#define PLPSH_MAX_HASHES 65536     /* heads * s per call */
#define PLPSH_PLAN_TILE 128        /* query rows per plan record */

/* Human-readable name of a status code (static storage).  Takes the code as
 * a plain integer so that any value is accepted: codes outside plpsh_status
 * give "PLPSH_ERR_UNKNOWN". */
const char* plpsh_status_string(int32_t status);

/* Library version string (static storage). */
const char* plpsh_version(void);

/* Description of the HIP failure behind the most recent PLPSH_ERR_HIP
 * returned on the calling thread ("" if none): the failing HIP call and
 * hipGetErrorString of its result.  Thread-local storage, valid until the
 * thread's next call into the library. */
const char* plpsh_last_hip_error(void);

/*
 * plpsh_draw_hashes -- draw the random-binning hashes on the host.
 *
 * The hash law is the random binning of Rahimi and Recht for the Laplace
 * kernel exp(-|x-y|/sigma) applied to integer positions (Methodology 1); its
 * width follows a Gamma distribution (Theorem 2.1, tools of the proof):
 * delta ~ Gamma(shape 2, scale sigma_h), u ~ U[0, delta).  Draws are
 * independent per (head h, hash i) and do not depend on Q, K, V, as the
 * uniform guarantee of Theorem 2.2 requires.
 *
 * Generator (exact, bit-reproducible): SplitMix64 (Steele, Lea, Flood,
 * OOPSLA 2014) in counter mode.  For k in {0,1,2}:
 *   c_k   = (h << 32) | (i << 2) | k
 *   z_k   = mix64(seed + (c_k + 1) * 0x9E3779B97F4A7C15)  (mod 2^64)
 *   mix64(z): z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
 *             z = (z ^ z>>27) * 0x94D049BB133111EB;  return z ^ z>>31
 *   U_k   = ((z_k >> 12) + 0.5) * 2^-52                  (0 < U_k < 1, exact)
 *   delta = sigma_h * ((-log U_0) - log U_1)            (binary64, this order)
 *   u     = delta * U_2
 * with log the C library's natural logarithm.
 *
 *   seed   : any 64-bit value.
 *   heads  : >= 1; s: 1..PLPSH_MAX_S; heads * s <= PLPSH_MAX_HASHES.
 *   sigma  : host [heads], finite, > 0 (sigma_h = 1 / ALiBi slope of head h).
 *   delta,u: host out [heads * s], index h * s + i; caller-owned.
 * Errors: INVALID_ARGUMENT for null pointers or out-of-range values.
 */
plpsh_status plpsh_draw_hashes(uint64_t seed, int32_t heads, int32_t s,
                               const double* sigma, double* delta, double* u);

/*
 * Bin buffer: the device-side description of the blocks of every hash,
 * computed from (delta, u) by the bin kernel.  Layout (byte offsets from
 * plpsh_bins_layout, each 256-byte aligned), for H = heads hashes-owners,
 * hash index t = h * s + i, T = ceil(n / PLPSH_PLAN_TILE):
 *
 *   nblk  : int32 [H*s]            number of blocks of hash t
 *   starts: int32 [H*s][n+1]       starts[t][k] = first position of block k
 *                                  (k < nblk[t]); starts[t][nblk[t]] = n.
 *                                  Entries beyond are unspecified.
 *                                  (The "int32 prefix offsets" of the bins.)
 *   plan  : record [H][T][s], 32 bytes each, for query tile
 *           [128 q, 128 q + 128) of head h and hash i:
 *             int32 a, e    block [a, e) containing row 128 q
 *             int32 a2, e2  block containing row min(128 q + 127, n - 1)
 *             uint32 bits[4] bit p set iff position 128 q + p (1 <= p < 128)
 *                            starts a block, or equals n
 *
 * Block k of hash t is the maximal run of positions with equal bin value
 * floor((x - u) / delta) evaluated in IEEE binary64 (Methodology 1: bins of
 * the integer indices are contiguous and non-overlapping).  Block starts are
 * bit-exact functions of (delta, u, n).
 */
size_t plpsh_bins_bytes(int32_t heads, int32_t s, int32_t n);
plpsh_status plpsh_bins_layout(int32_t heads, int32_t s, int32_t n,
                               size_t* off_nblk, size_t* off_starts, size_t* off_plan);

/*
 * plpsh_sample_bins -- draw hashes on the host (as plpsh_draw_hashes) and,
 * if `bins` is not NULL, compute the bin buffer on the device.
 *
 *   delta, u   : host out [heads*s] or NULL.
 *   bins       : device out, plpsh_bins_bytes(heads, s, n) bytes, or NULL.
 *   n          : 1..PLPSH_MAX_N (only used when bins != NULL).
 * Errors: INVALID_ARGUMENT (as above; bins_bytes too small counts as
 * WORKSPACE_TOO_SMALL), HIP.
 */
plpsh_status plpsh_sample_bins(uint64_t seed, int32_t heads, int32_t s, int32_t n,
                               const double* sigma, double* delta, double* u,
                               void* bins, size_t bins_bytes, void* stream);

/*
 * plpsh_bins_from_hashes -- the device bin kernel for explicit hashes.
 *   delta, u : host [heads*s]; delta finite and > 0; 0 <= u <= delta.
 */
plpsh_status plpsh_bins_from_hashes(int32_t heads, int32_t s, int32_t n,
                                    const double* delta, const double* u,
                                    void* bins, size_t bins_bytes, void* stream);

/* Workspace bytes needed by plpsh_attention_fwd[_hashes] (= bin buffer). */
size_t plpsh_workspace_bytes(int32_t heads_q, int32_t s, int32_t n);

/*
 * plpsh_attention_fwd -- Positional-LSH ALiBi attention, forward pass
 * (Theorem 2.2 with M~ of Theorem 2.1).  Draws s hashes per query head from
 * `seed` on the host, computes their blocks on the device, then
 * O = count-weighted attention (formula at the top of this file).  One
 * kernel launch does both (each workgroup evaluates the bins of its own
 * query tile) unless some width lies within 2^-30 of 1, when the bin kernel
 * runs first; either way the workspace receives the bin buffer exactly as
 * plpsh_sample_bins writes it (block counts, block starts, plan records).
 *
 *   q, o     : device [batch, heads_q,  n, head_dim], contiguous, d innermost
 *   k, v     : device [batch, heads_kv, n, head_dim], contiguous
 *              All 16-byte aligned; o must not alias q, k or v.
 *              Query head h reads key/value head h / (heads_q / heads_kv).
 *   dtype    : element type of q, k, v and o.
 *   head_dim : 64 or 128 (else UNSUPPORTED).  Scale 1/sqrt(head_dim).
 *   sigma    : host [heads_q], finite, > 0.
 *   s        : 1..PLPSH_MAX_S hashes per head, shared by all batch rows.
 *   causal   : 0 or 1; 1 multiplies the mask elementwise by [j <= r].
 *   workspace: device, >= plpsh_workspace_bytes(heads_q, s, n) bytes,
 *              256-byte aligned; overwritten.
 * batch == 0 or n == 0 is a valid empty call: nothing is launched and
 * q, k, v, o may then be NULL.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
plpsh_status plpsh_attention_fwd(const void* q, const void* k, const void* v, void* o,
                                 int32_t batch, int32_t heads_q, int32_t heads_kv,
                                 int32_t n, int32_t head_dim, int32_t dtype,
                                 const double* sigma, int32_t s, uint64_t seed,
                                 int32_t causal, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Limits of plpsh_attention_fwd_noalloc. */
#define PLPSH_NOALLOC_MAX_HASHES 4096          /* heads_q * s */
#define PLPSH_NOALLOC_BINS_BYTES (64u << 20)   /* plpsh_workspace_bytes(heads_q, s, n) */

/*
 * plpsh_attention_fwd_noalloc -- plpsh_attention_fwd for callers that cannot
 * allocate memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result and errors as
 * plpsh_attention_fwd (bit-identical output for the same seed), minus the
 * workspace: the bin buffer lives in a static device array of the library
 * (PLPSH_NOALLOC_BINS_BYTES plus 16 bytes per hash), and the hashes reach
 * the device as kernel arguments, so the call makes no device or host
 * allocation (no hipMalloc, no pinned staging ring).
 *   Limits: heads_q * s <= PLPSH_NOALLOC_MAX_HASHES and
 *   plpsh_workspace_bytes(heads_q, s, n) <= PLPSH_NOALLOC_BINS_BYTES (a
 *   32-head layer with s = 20 up to n = 16384 fits); beyond them the call
 *   returns PLPSH_ERR_UNSUPPORTED and launches nothing.
 *   The array is per device, held from library load until the process ends,
 *   and shared by every call on that device: each call rewrites everything
 *   it reads there (nothing needs clearing), and calls that overlap on one
 *   device (concurrent streams, other threads) race on it -- order them.
 */
plpsh_status plpsh_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                         int32_t batch, int32_t heads_q, int32_t heads_kv,
                                         int32_t n, int32_t head_dim, int32_t dtype,
                                         const double* sigma, int32_t s, uint64_t seed,
                                         int32_t causal, void* stream);

/*
 * plpsh_attention_fwd_hashes -- as plpsh_attention_fwd with explicit hashes
 * instead of a seed: delta, u host [heads_q * s] (index h * s + i), delta
 * finite > 0, 0 <= u <= delta.  Lets a caller reuse a draw or force special
 * cases (delta >= n: one block, plain attention; delta < 1: single-position
 * blocks, O = V).
 */
plpsh_status plpsh_attention_fwd_hashes(const void* q, const void* k, const void* v, void* o,
                                        int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t n, int32_t head_dim, int32_t dtype,
                                        const double* delta, const double* u, int32_t s,
                                        int32_t causal, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * plpsh_fixed_blocks_fwd -- the "fixed blocks" baseline of the Mistral
 * fine-tuning comparison (Key results, experimental validation): one
 * deterministic partition of the positions into blocks of block[h] tokens
 * per query head, attention inside each block only.  The same path as
 * plpsh_attention_fwd_hashes with s = 1, delta = block[h], u = 0 (blocks
 * [k b, (k + 1) b)).
 *
 *   block    : host [heads_q], each 1..PLPSH_MAX_N.
 *   workspace: device, >= plpsh_workspace_bytes(heads_q, 1, n) bytes,
 *              256-byte aligned; overwritten.
 * Other arguments and errors as plpsh_attention_fwd.
 */
plpsh_status plpsh_fixed_blocks_fwd(const void* q, const void* k, const void* v, void* o,
                                    int32_t batch, int32_t heads_q, int32_t heads_kv,
                                    int32_t n, int32_t head_dim, int32_t dtype,
                                    const int32_t* block, int32_t causal,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * plpsh_attention_fwd_bins -- the attention step alone, on a bin buffer
 * already computed by plpsh_sample_bins / plpsh_bins_from_hashes for the
 * same (heads_q, s, n).  plpsh_attention_fwd gives exactly the results of
 * plpsh_sample_bins followed by this call (bit for bit: output and bin
 * buffer); splitting them lets one draw serve several calls.
 *
 *   bins   : device, >= plpsh_bins_bytes(heads_q, s, n) bytes, 256-byte
 *            aligned, written by the bin kernel for these sizes (the
 *            library cannot check its contents).
 *   delta  : host [heads_q * s] or NULL.  Only used to schedule heads with
 *            the widest bins first; NULL keeps the natural head order.
 * Other arguments, layouts and errors as plpsh_attention_fwd.
 */
plpsh_status plpsh_attention_fwd_bins(const void* q, const void* k, const void* v, void* o,
                                      int32_t batch, int32_t heads_q, int32_t heads_kv,
                                      int32_t n, int32_t head_dim, int32_t dtype,
                                      int32_t s, int32_t causal, const void* bins,
                                      size_t bins_bytes, const double* delta, void* stream);

/*
 * plpsh_attention_fwd_literal -- the same T~ computed as the reduction of
 * Theorem 2.2 states it: one short, unbiased attention per hash, in which
 * row r attends only to the keys of its own block of that hash, the s
 * results summed with the shared causal mask C:
 *   O_r = sum_i sum_{j in block_i(r)} C[r,j] e^{S[r,j]} v_j
 *         / sum_i sum_{j in block_i(r)} C[r,j] e^{S[r,j]}
 * which equals plpsh_attention_fwd_bins up to rounding order, at s times
 * the logit work of the key tiles the blocks reach instead of one pass
 * weighted by the counts.  An ablation of the fused kernel, not a faster
 * path.  Arguments, layouts and errors exactly as plpsh_attention_fwd_bins.
 */
plpsh_status plpsh_attention_fwd_literal(const void* q, const void* k, const void* v, void* o,
                                         int32_t batch, int32_t heads_q, int32_t heads_kv,
                                         int32_t n, int32_t head_dim, int32_t dtype,
                                         int32_t s, int32_t causal, const void* bins,
                                         size_t bins_bytes, const double* delta, void* stream);

/*
 * plpsh_attention_fwd_lse -- plpsh_attention_fwd_bins that also writes each
 * row's log-normaliser, for the backward pass:
 *   lse[b, h, r] = log sum_j c[r, j] C[r, j] exp(S[r, j])   (natural log)
 * lse: device, float32 [batch, heads_q, n], caller-owned.  The weights of T~
 * are then P[r, j] = c[r, j] C[r, j] exp(S[r, j] - lse[r]).  Other arguments,
 * layouts and errors as plpsh_attention_fwd_bins.
 */
plpsh_status plpsh_attention_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int32_t batch, int32_t heads_q, int32_t heads_kv,
                                     int32_t n, int32_t head_dim, int32_t dtype,
                                     int32_t s, int32_t causal, const void* bins,
                                     size_t bins_bytes, const double* delta, void* stream);

/* Workspace of plpsh_attention_bwd: batch * heads_q * n floats, 256-byte
 * rounded (0 for invalid sizes). */
size_t plpsh_attention_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t n);

/*
 * plpsh_attention_bwd -- gradients of sum(dO o T~) for training with the
 * approximation (the pages train and fine-tune models with it: Key results,
 * experimental validation).  With P as above and the counts c of the same
 * bins (which do not depend on Q, K, V):
 *   dV = P^T dO,  dS = P o (dO V^T - D),  D_r = <dO_r, O_r>,
 *   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
 * with the gradients of the query heads of a KV group summed into its KV
 * head.
 *   q, k, v, o : the forward inputs and output (o from the same bins);
 *   dout       : dO, layout of o;   lse: from plpsh_attention_fwd_lse;
 *   dq         : device out, layout of q;  dk, dv: device out, layout of k
 *                (every element written; no accumulation into them);
 *   bins, delta: as plpsh_attention_fwd_bins (delta only orders the work);
 *   workspace  : device, 256-byte aligned, >=
 *                plpsh_attention_bwd_workspace_bytes(batch, heads_q, n).
 * bf16 only (PLPSH_ERR_UNSUPPORTED for f32); head_dim 64 or 128.  Arithmetic:
 * bf16 products on the matrix cores with fp32 accumulation; P and dS are
 * rounded to bf16 before their products.  Asynchronous on `stream`: the dQ
 * kernel and the dK/dV kernel run side by side on two streams of the device,
 * `stream` and a second one (created on first use, default priority, kept
 * until the process ends), forked from and joined back to `stream` with
 * events, so work issued to `stream` afterwards sees all three gradients.
 * The second stream takes the kernel with the heavier work items: dK/dV
 * (whose work items cover every query head of a KV group) when heads_q >=
 * 4 * heads_kv, dQ otherwise.  Calls from several threads are serialised
 * around that fork and join.
 */
plpsh_status plpsh_attention_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q,
                                 int32_t heads_kv, int32_t n, int32_t head_dim, int32_t dtype, int32_t s,
                                 int32_t causal, const void* bins, size_t bins_bytes, const double* delta,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * plpsh_alibi_dense_fwd -- exact ALiBi attention T* (the quantity the
 * approximation targets, Methodology 1), dense over all keys:
 *   O_r = sum_j C[r,j] exp(S[r,j] - |r-j|/sigma_h) v_j / sum_j (same weights)
 * Same layouts, dtypes, head_dim values and error conventions as
 * plpsh_attention_fwd; needs no workspace.  Provided to locate the sequence
 * length where the approximation overtakes exact attention on the same GPU.
 */
plpsh_status plpsh_alibi_dense_fwd(const void* q, const void* k, const void* v, void* o,
                                   int32_t batch, int32_t heads_q, int32_t heads_kv,
                                   int32_t n, int32_t head_dim, int32_t dtype,
                                   const double* sigma, int32_t causal, void* stream);

/* ------------------------------------------------------------------------
 * Error of the mask mean against the bias matrix at large n.
 *
 * E = L* - M~ for one head, with L*[r, j] = exp(-|r - j| / sigma) (the
 * exponentiated ALiBi bias, Methodology 1) and M~ = c / s the mean of the
 * head's s sampled masks (Theorem 2.1).  The pages state that ||E||_2 and
 * ||E||_max fall like 1/sqrt(s) and that their experiments saw the matrix
 * error go to zero as s grows (Key results, experimental validation); these
 * calls measure both norms without forming E (O(n s) memory and work per
 * product).  All arithmetic is IEEE binary64.
 *
 *   sigma : finite, > 0.   n: 1..PLPSH_MAX_N.   s: 1..PLPSH_MAX_S.
 *   bins  : device bin buffer of ONE head (heads = 1) for these (s, n),
 *           written by plpsh_bins_from_hashes / plpsh_sample_bins,
 *           256-byte aligned, >= plpsh_bins_bytes(1, s, n) bytes.
 * ------------------------------------------------------------------------ */

/* Workspace for plpsh_error_matvec (max_steps = 0) or plpsh_error_norms
 * (max_steps >= 1, at most 1000); 0 for invalid sizes. */
size_t plpsh_error_workspace_bytes(int32_t n, int32_t s, int32_t max_steps);

/*
 * plpsh_error_rowmax -- rowmax[r] = max_j |L*[r, j] - c[r, j] / s|, for
 * r in [0, n).  rowmax: device, n doubles (caller-owned).  Asynchronous on
 * `stream`.
 */
plpsh_status plpsh_error_rowmax(double sigma, int32_t n, int32_t s, const void* bins, size_t bins_bytes,
                                double* rowmax, void* stream);

/*
 * plpsh_error_matvec -- y = E x for device vectors x, y of n doubles (no
 * overlap).  workspace: device, 256-byte aligned, >=
 * plpsh_error_workspace_bytes(n, s, 0) bytes.  Asynchronous on `stream`.
 */
plpsh_status plpsh_error_matvec(double sigma, int32_t n, int32_t s, const void* bins, size_t bins_bytes,
                                const double* x, double* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * plpsh_error_norms -- both norms of E for the hashes (delta[i], u[i]),
 * i < s (host arrays, as plpsh_bins_from_hashes).
 *   maxnorm    : host out, ||E||_max (exact, from the row maxima);
 *   argmax_row : host out or NULL, the first row where it is attained;
 *   spectral   : host out, ||E||_2 = max |eigenvalue| of the symmetric E,
 *                by Lanczos with full reorthogonalisation from a start
 *                vector drawn from `seed`; it stops when the estimate has
 *                changed by at most tol (relative) over three steps, the
 *                Krylov space closes, or after max_steps (1..1000) steps;
 *   steps      : host out or NULL, Lanczos steps taken.
 * workspace: device, 256-byte aligned, >= plpsh_error_workspace_bytes(n, s,
 * max_steps) bytes (holds the bins, max_steps + 1 Lanczos vectors and
 * scratch).  Synchronises `stream` (the iteration reads scalars back every
 * step).
 */
plpsh_status plpsh_error_norms(double sigma, int32_t n, int32_t s, const double* delta, const double* u,
                               int32_t max_steps, double tol, uint64_t seed, void* workspace, size_t workspace_bytes,
                               double* spectral, double* maxnorm, int32_t* argmax_row, int32_t* steps,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PLPSH_H */
