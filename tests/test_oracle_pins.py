"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
closed form, exact rational arithmetic, a brute-force loop, a library
routine in a special case, an invariant, or a statistical law.  Citations
[P, ...] are to the explainer pages of "Positional LSH: Binary Block Matrix
Approximation for Attention with Linear Biases" (gist.science).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.integrate
import scipy.stats
import torch

import oracle
from oracle.sampler import sample_hashes, splitmix64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _draw(rng, sigma, s):
    """Hashes drawn with numpy's generator (independent of the library's
    sampler): delta ~ Gamma(2, sigma), u ~ U[0, delta)."""
    delta = rng.gamma(2.0, sigma, size=s)
    u = rng.uniform(0.0, 1.0, size=s) * delta
    return delta, u


# ---------------------------------------------------------------- P1 -------
# [P, Methodology 1]: L* = E_h[M(h)] exactly, for the Laplace kernel.

@pytest.mark.parametrize("sigma", [0.7, 4.0, 16.0])
def test_p1_gamma_law_integrates_to_laplace(sigma):
    """With u uniform, P[same bin | delta] = max(0, 1 - D/delta); averaging
    over delta ~ Gamma(2, sigma) gives exp(-D / sigma) (closed form)."""
    dens = lambda dl: dl * math.exp(-dl / sigma) / sigma ** 2
    for D in [0.0, 0.5, 1.0, 3.0, 10.0, 40.0]:
        val, _ = scipy.integrate.quad(lambda dl: max(0.0, 1.0 - D / dl) * dens(dl),
                                      D, np.inf, epsabs=1e-13, epsrel=1e-12) if D > 0 else (1.0, 0)
        assert abs(val - math.exp(-D / sigma)) < 1e-9


def test_p1_same_bin_probability_given_width():
    """Fixed delta, u ~ U[0, delta): positions x and x + D share a bin with
    probability max(0, 1 - D / delta) (Monte Carlo through oracle.bin_values)."""
    rng = _rng(1)
    delta, n, trials = 7.3, 24, 20000
    us = rng.uniform(0, delta, size=trials)
    same = np.zeros(n)
    for uu in us:
        b = oracle.bin_values(delta, uu, n)
        same += b == b[0]
    p_hat = same / trials
    D = np.arange(n)
    p = np.maximum(0.0, 1.0 - D / delta)
    se = np.sqrt(np.maximum(p * (1 - p), 1.0 / trials) / trials)
    assert np.all(np.abs(p_hat - p) <= 5 * se + 1e-12)


@pytest.mark.parametrize("sigma", [0.7, 4.0, 16.0])
def test_p1_expected_mask_is_alibi(sigma):
    """Monte Carlo over 40000 hashes: E[M~] -> L* entrywise (5 standard errors)."""
    rng = _rng(int(sigma * 10))
    n, s = 32, 40000
    delta, u = _draw(rng, sigma, s)
    mt = oracle.mtilde(delta, u, n)
    L = oracle.alibi_matrix(sigma, n)
    se = np.sqrt(np.maximum(L * (1 - L), 1.0 / s) / s)
    assert np.all(np.abs(mt - L) <= 5 * se + 1e-12)
    # and the closed form of L* itself
    i = np.arange(n)
    assert np.allclose(L, np.exp(-np.abs(i[:, None] - i[None, :]) / sigma), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- P2 -------
# Sampler: the published generator and the Gamma(2, sigma) / uniform laws.

def test_p2_splitmix64_known_answer():
    with open(os.path.join(GOLDEN, "splitmix64_state0.txt")) as f:
        vals = [int(l, 16) for l in f if l.strip() and not l.startswith("#")]
    assert splitmix64(0, len(vals)) == vals


def test_p2_sampler_laws():
    sigma, s = 3.5, 20000
    delta, u = sample_hashes(12345, [sigma], s)
    delta, u = delta[0], u[0]
    assert scipy.stats.kstest(delta / sigma, scipy.stats.gamma(2.0).cdf).pvalue > 1e-3
    assert scipy.stats.kstest(u / delta, scipy.stats.uniform().cdf).pvalue > 1e-3
    assert abs(delta.mean() - 2 * sigma) < 5 * math.sqrt(2) * sigma / math.sqrt(s)
    assert np.all((u >= 0) & (u <= delta))


def test_p2_sampler_streams_independent_of_shape():
    """Counter mode: hash (h, i) does not depend on how many heads or hashes
    are drawn alongside it."""
    d1, u1 = sample_hashes(7, [2.0, 5.0, 9.0], 6)
    d2, u2 = sample_hashes(7, [2.0, 5.0], 3)
    assert np.array_equal(d1[:2, :3], d2) and np.array_equal(u1[:2, :3], u2)


# ---------------------------------------------------------------- P3 -------
# Bins given (delta, u): brute force with exact rationals, and invariants.

def _exact_bins(delta, u, n):
    D, U = Fraction(delta), Fraction(u)
    out, near = [], []
    for x in range(n):
        qv = (Fraction(x) - U) / D
        fl = math.floor(qv)
        out.append(fl)
        near.append(min(qv - fl, fl + 1 - qv) < Fraction(1, 10 ** 9))
    return np.array(out, dtype=np.float64), np.array(near)


@pytest.mark.parametrize("delta", [0.3, 0.999, 1.0, 1.5, 2.0, 7.3, 100.25, 5e3])
def test_p3_bins_match_exact_arithmetic(delta):
    rng = _rng(int(delta * 1000) % 2 ** 31)
    n = 600
    for uu in list(rng.uniform(0, delta, size=4)) + [0.0]:
        fb = oracle.bin_values(delta, uu, n)
        eb, near = _exact_bins(delta, uu, n)
        assert np.array_equal(fb[~near], eb[~near])


@pytest.mark.parametrize("delta", [0.4, 1.0, 2.5, 7.3, 64.0, 1000.0])
def test_p3_block_invariants(delta):
    rng = _rng(3)
    n = 997  # odd, not a multiple of anything
    for uu in rng.uniform(0, delta, size=5):
        st = oracle.block_starts(delta, uu, n)
        assert st[0] == 0 and np.all(np.diff(st) > 0) and st[-1] < n
        lens = np.diff(np.append(st, n))
        if delta < 1:
            assert st.size == n  # every position is its own block
        else:
            interior = lens[1:-1]
            assert np.all((interior == math.floor(delta)) | (interior == math.ceil(delta)))
            assert lens[0] <= math.ceil(delta) and lens[-1] <= math.ceil(delta)
            # number of blocks = number of bins met, counted exactly
            eb, _ = _exact_bins(delta, uu, n)
            assert st.size == int(eb[-1] - eb[0]) + 1


def test_p3_block_of_matches_brute_force():
    rng = _rng(4)
    n = 300
    for delta in [0.5, 3.0, 17.0]:
        uu = rng.uniform(0, delta)
        b = oracle.bin_values(delta, uu, n)
        a, e = oracle.block_of(delta, uu, n, np.arange(n))
        for x in range(n):
            same = [j for j in range(n) if b[j] == b[x]]
            assert a[x] == min(same) and e[x] == max(same) + 1


# ---------------------------------------------------------------- P4 -------
# Exact laws of the sampled masks (derived from the hash law).

def test_p4_count_is_binomial():
    """s * M~[i, j] ~ Binomial(s, exp(-|i-j| / sigma)): chi-square over seeds."""
    rng = _rng(5)
    sigma, s, n, reps = 6.0, 10, 16, 3000
    counts = np.zeros((reps, 3), dtype=int)
    pairs = [(0, 2), (3, 9), (1, 15)]
    for t in range(reps):
        dl, uu = _draw(rng, sigma, s)
        c = oracle.count_matrix(dl, uu, n)
        counts[t] = [c[i, j] for i, j in pairs]
    for col, (i, j) in enumerate(pairs):
        p = math.exp(-abs(i - j) / sigma)
        expct = scipy.stats.binom(s, p).pmf(np.arange(s + 1)) * reps
        obs = np.bincount(counts[:, col], minlength=s + 1)
        keep = expct >= 5
        o = np.append(obs[keep], obs[~keep].sum())
        e_ = np.append(expct[keep], expct[~keep].sum())
        if e_[-1] == 0:
            o, e_ = o[:-1], e_[:-1]
        assert scipy.stats.chisquare(o, e_ * o.sum() / e_.sum()).pvalue > 1e-4


def test_p4_expected_number_of_blocks():
    rng = _rng(6)
    sigma, n, reps = 5.0, 400, 4000
    nb = np.array([oracle.block_starts(*(_draw(rng, sigma, 1)[k][0] for k in (0, 1)), n).size
                   for _ in range(reps)])
    mean = 1 + (n - 1) * (1 - math.exp(-1 / sigma))
    assert abs(nb.mean() - mean) < 5 * nb.std() / math.sqrt(reps)


def test_p4_distance_to_block_start():
    """P(r - start(r) >= k) = exp(-k / sigma) for k <= r."""
    rng = _rng(7)
    sigma, n, reps, r = 8.0, 200, 20000, 150
    dist = np.empty(reps)
    for t in range(reps):
        dl, uu = _draw(rng, sigma, 1)
        a, _ = oracle.block_of(dl[0], uu[0], n, [r])
        dist[t] = r - a[0]
    for k in [1, 4, 8, 20, 40]:
        p = math.exp(-k / sigma)
        assert abs((dist >= k).mean() - p) < 5 * math.sqrt(p * (1 - p) / reps) + 1e-4


# ---------------------------------------------------------------- P5 -------
# [P, Theorem 2.1] and [P, Key results]: error of M~ decays as O(1/sqrt(s)).

def test_p5_convergence_rate_and_hoeffding():
    rng = _rng(8)
    n, sigma, seeds = 192, 16.0, 6
    L = oracle.alibi_matrix(sigma, n)
    ss = [4, 16, 64, 256, 1024]
    emax, espec = [], []
    eta = 1e-3
    for s in ss:
        m1, m2 = [], []
        for _ in range(seeds):
            dl, uu = _draw(rng, sigma, s)
            E = oracle.mtilde(dl, uu, n) - L
            m1.append(np.abs(E).max())
            m2.append(np.linalg.norm(E, 2))
            # Hoeffding + union bound on n^2 entries, failure prob eta
            assert np.abs(E).max() <= math.sqrt(math.log(2 * n * n / eta) / (2 * s))
        emax.append(np.mean(m1))
        espec.append(np.mean(m2))
    for e in (emax, espec):
        slope = np.polyfit(np.log(ss), np.log(e), 1)[0]
        assert -0.62 < slope < -0.38, slope


# ---------------------------------------------------------------- P6 -------
# [P, Methodology 1]: blocks are contiguous and do not overlap.

@pytest.mark.parametrize("delta", [0.6, 2.2, 9.0, 50.0])
def test_p6_single_mask_is_block_diagonal(delta):
    rng = _rng(9)
    n = 120
    for uu in rng.uniform(0, delta, size=3):
        M = oracle.count_matrix([delta], [uu], n).astype(bool)
        assert np.array_equal(M, M.T) and np.all(np.diag(M))
        idx = np.arange(n)
        for r in range(n):
            ones = idx[M[r]]
            assert ones.size == ones[-1] - ones[0] + 1  # contiguous row support
        # transitivity: r~j and j~k imply r~k
        assert np.array_equal((M.astype(int) @ M.astype(int)) > 0, M)


# ---------------------------------------------------------------- P7 / P8 --
# Special cases that reduce to plain (masked) softmax attention.

def _sdpa(q, k, v, mask=None, causal=False):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else t(mask), is_causal=causal)
    return o.numpy()


def _qkv(seed, B=1, Hq=2, Hkv=1, n=80, d=16, scale=1.0):
    rng = _rng(seed)
    q = rng.standard_normal((B, Hq, n, d)) * scale
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_p7_all_ones_masks_give_plain_attention(causal):
    q, k, v = _qkv(10, B=2, Hq=4, Hkv=2, n=70, d=16, scale=2.0)
    n, s = q.shape[2], 3
    deltas = np.full((4, s), float(n))
    us = np.zeros((4, s))
    t = oracle.plsh_attention(q, k, v, deltas, us, causal)
    kk = np.repeat(k, 2, axis=1)
    vv = np.repeat(v, 2, axis=1)
    ref = _sdpa(q, kk, vv, causal=causal)
    assert np.abs(t - ref).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_p8_tiny_bins_give_identity(causal):
    q, k, v = _qkv(11, n=50)
    deltas = np.array([[0.5, 0.9, 0.2]] * 2)
    us = deltas * 0.3
    t = oracle.plsh_attention(q, k, v, deltas, us, causal)
    assert np.abs(t - np.repeat(v, 2, axis=1)).max() < 1e-14


def test_p8_causal_first_row_is_first_value():
    q, k, v = _qkv(12, n=40)
    rng = _rng(12)
    deltas, us = _draw(rng, 9.0, 5)
    t = oracle.plsh_attention(q, k, v, np.stack([deltas] * 2), np.stack([us] * 2), True)
    assert np.abs(t[0, :, 0] - v[0, 0, 0]).max() < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_p8_fixed_blocks_equal_block_masked_sdpa(causal):
    """s = 1, delta = b, u = 0: the deterministic partition into blocks of b
    positions (the pages' "fixed blocks" baseline); T~ equals softmax
    attention restricted to each block."""
    q, k, v = _qkv(13, n=90)
    b = 16
    t = oracle.plsh_attention(q, k, v, np.full((2, 1), float(b)), np.zeros((2, 1)), causal)
    i = np.arange(90)
    mask = (i[:, None] // b) == (i[None, :] // b)
    if causal:
        mask &= i[None, :] <= i[:, None]
    ref = _sdpa(q, np.repeat(k, 2, 1), np.repeat(v, 2, 1), mask=mask)
    assert np.abs(t - ref).max() < 1e-12


# ---------------------------------------------------------------- P9 -------
# [P, Theorem 2.2] error bound: output error <= mask error / biased row mass.

@pytest.mark.parametrize("causal", [False, True])
def test_p9_output_error_identity_and_bound(causal):
    """T~_r - T*_r = sum_j (M~ - L*)[r,j] A[r,j] (v_j - T*_r) / sum_j M~[r,j] A[r,j]
    with A = C o exp(S): exact identity (from sum_j L* A (v_j - T*_r) = 0),
    hence the absolute-value bound."""
    q, k, v = _qkv(14, Hq=1, n=96)
    rng = _rng(14)
    sigma, s = 12.0, 6
    dl, uu = _draw(rng, sigma, s)
    T = oracle.plsh_attention(q, k, v, dl[None], uu[None], causal)[0, 0]
    Ts = oracle.alibi_attention(q, k, v, [sigma], causal)[0, 0]
    n, d = q.shape[2:]
    S = q[0, 0] @ k[0, 0].T / math.sqrt(d)
    A = np.exp(S - S.max(axis=1, keepdims=True))
    if causal:
        A = np.tril(A)
    M = oracle.mtilde(dl, uu, n)
    L = oracle.alibi_matrix(sigma, n)
    diff = v[0, 0][None, :, :] - Ts[:, None, :]            # [r, j, k]
    num = np.einsum("rj,rjk->rk", (M - L) * A, diff)
    den = (M * A).sum(axis=1)[:, None]
    assert np.abs((T - Ts) - num / den).max() < 1e-10
    bound = np.einsum("rj,rjk->rk", np.abs(M - L) * A, np.abs(diff)) / den
    assert np.all(np.abs(T - Ts) <= bound + 1e-12)


# ---------------------------------------------------------------- P10 ------
# Exact ALiBi by brute force; T~ -> T* as s grows.

@pytest.mark.parametrize("causal", [False, True])
def test_p10_alibi_brute_force(causal):
    q, k, v = _qkv(15, Hq=2, Hkv=1, n=24, d=8)
    sig = [3.0, 11.0]
    T = oracle.alibi_attention(q, k, v, sig, causal)
    n, d = 24, 8
    for h in range(2):
        for r in range(n):
            num = np.zeros(d)
            den = 0.0
            for j in range(n):
                if causal and j > r:
                    continue
                w = math.exp(-abs(r - j) / sig[h]) * math.exp(
                    sum(q[0, h, r, t] * k[0, 0, j, t] for t in range(d)) / math.sqrt(d))
                num += w * v[0, 0, j]
                den += w
            assert np.abs(T[0, h, r] - num / den).max() < 1e-13


def test_p10_plsh_converges_to_alibi():
    q, k, v = _qkv(16, Hq=1, n=128, d=16)
    sigma = 10.0
    Ts = oracle.alibi_attention(q, k, v, [sigma], True)
    rng = _rng(16)
    ss, errs = [4, 16, 64, 256], []
    for s in ss:
        e = []
        for _ in range(5):
            dl, uu = _draw(rng, sigma, s)
            e.append(np.abs(oracle.plsh_attention(q, k, v, dl[None], uu[None], True) - Ts).max())
        errs.append(np.mean(e))
    assert errs[-1] < errs[0] / 4
    slope = np.polyfit(np.log(ss), np.log(errs), 1)[0]
    assert -0.75 < slope < -0.3, slope


def test_p10_numerator_unbiased():
    """E over hashes of (M~ o A) V equals (L* o A) V (the ratio is not
    unbiased, but numerator and denominator are)."""
    q, k, v = _qkv(17, Hq=1, n=40, d=8)
    sigma, reps, s = 5.0, 3000, 1
    n, d = 40, 8
    S = q[0, 0] @ k[0, 0].T / math.sqrt(d)
    A = np.exp(S - S.max())
    rng = _rng(17)
    acc = np.zeros((reps, n, d))
    for t in range(reps):
        dl, uu = _draw(rng, sigma, s)
        acc[t] = (oracle.mtilde(dl, uu, n) * A) @ v[0, 0]
    ref = (oracle.alibi_matrix(sigma, n) * A) @ v[0, 0]
    se = acc.std(axis=0) / math.sqrt(reps) + 1e-12
    assert np.all(np.abs(acc.mean(axis=0) - ref) <= 5.5 * se)


# ---------------------------------------------------------------- P11 ------

def test_p11_convexity():
    q, k, v = _qkv(18, Hq=2, n=100, scale=3.0)
    rng = _rng(18)
    dl = np.stack([_draw(rng, 7.0, 4)[0] for _ in range(2)])
    uu = dl * rng.uniform(size=dl.shape)
    for causal in (False, True):
        T = oracle.plsh_attention(q, k, v, dl, uu, causal)
        for h in range(2):
            lo, hi = oracle.support_interval(dl[h], uu[h], 100, np.arange(100), causal)
            for r in range(100):
                vs = v[0, 0, lo[r]:hi[r]]
                assert np.all(T[0, h, r] >= vs.min(0) - 1e-12) and np.all(T[0, h, r] <= vs.max(0) + 1e-12)


# ---------------------------------------------------------------- P12 ------
# [P, Theorem 2.2]: the reduction to per-block unbiased attentions computes
# the same T~ as the dense M~ formula.

@pytest.mark.parametrize("causal", [False, True])
def test_p12_literal_reduction_equals_dense(causal):
    q, k, v = _qkv(19, B=2, Hq=4, Hkv=2, n=130, d=16, scale=2.0)
    rng = _rng(19)
    dl = np.stack([_draw(rng, sg, 5)[0] for sg in (0.8, 3.0, 9.0, 40.0)])
    uu = dl * rng.uniform(size=dl.shape)
    a = oracle.plsh_attention(q, k, v, dl, uu, causal)
    b = oracle.plsh_attention_literal(q, k, v, dl, uu, causal)
    assert np.abs(a - b).max() / np.abs(a).max() < 1e-12


# ----------------------------------------------------- row / banded forms --
# Consistency of the restricted-key forms with the (pinned) dense form.

@pytest.mark.parametrize("causal", [False, True])
def test_rows_and_bands_equal_dense(causal):
    q, k, v = _qkv(20, B=1, Hq=1, Hkv=1, n=333, d=16)
    rng = _rng(20)
    dl, uu = _draw(rng, 12.0, 7)
    dense = oracle.plsh_attention(q, k, v, dl[None], uu[None], causal)[0, 0]
    rows = np.array([0, 1, 63, 64, 200, 332])
    r = oracle.plsh_attention_rows(q[0, 0], k[0, 0], v[0, 0], dl, uu, rows, causal)
    assert np.abs(r - dense[rows]).max() < 1e-12
    band, _ = oracle.plsh_attention_rowblocks(q[0, 0], k[0, 0], v[0, 0], dl, uu, causal, row_block=64)
    assert np.abs(band - dense).max() < 1e-12
    Ts = oracle.alibi_attention(q, k, v, [12.0], causal)[0, 0]
    assert np.abs(oracle.alibi_attention_rows(q[0, 0], k[0, 0], v[0, 0], 12.0, rows, causal) - Ts[rows]).max() < 1e-12


# ---------------------------------------------------------------- P13 ------
# [P, Theorem 2.1; Key results, experimental validation]: the error
# E = L* - M~ at large n.  The large-n forms (row maxima from the
# definition, E x through the Toeplitz product and per-bin sums, ARPACK
# spectral norm) must agree with the dense matrices, and with closed forms.

@pytest.mark.parametrize("n", [300, 777])
def test_p13_error_matvec_equals_dense(n):
    rng = _rng(21 + n)
    sigma = 9.0
    dl, uu = _draw(rng, sigma, 7)
    dl = np.append(dl, [0.5, 3.0 * n])        # single-position blocks; one block
    uu = np.append(uu, [0.25, 0.0])
    x = rng.standard_normal(n)
    E = oracle.error_dense(sigma, dl, uu, n)
    y = oracle.error_matvec(sigma, dl, uu, n, x)
    assert np.abs(y - E @ x).max() <= 1e-12 * np.abs(E @ x).max()


def test_p13_error_rowmax_equals_dense():
    rng = _rng(23)
    n, sigma = 300, 12.0
    dl, uu = _draw(rng, sigma, 9)
    E = oracle.error_dense(sigma, dl, uu, n)
    rows = np.arange(n)
    assert np.array_equal(oracle.error_rowmax(sigma, dl, uu, n, rows), np.abs(E).max(axis=1))
    assert oracle.error_maxnorm(sigma, dl, uu, n) == np.abs(E).max()


def test_p13_error_spectral_arpack_equals_dense():
    rng = _rng(24)
    n, sigma = 500, 10.0
    dl, uu = _draw(rng, sigma, 5)
    dense = np.linalg.norm(oracle.error_dense(sigma, dl, uu, n), 2)
    arpack = oracle.error_spectral(sigma, dl, uu, n, dense_below=0)
    assert abs(arpack - dense) <= 1e-9 * dense


def test_p13_closed_forms():
    """One block over everything: E = L* - J, whose largest entry is at the
    corners, 1 - exp(-(n-1)/sigma).  Single-position blocks: M~ = I, so the
    largest entry is exp(-1/sigma) and ||E||_2 = ||L* - I||_2 lies below the
    Toeplitz-symbol bound 2 rho / (1 - rho), rho = exp(-1/sigma), and tends
    to it as n grows."""
    n, sigma = 400, 25.0
    assert math.isclose(oracle.error_maxnorm(sigma, [2.0 * n], [0.0], n), 1 - math.exp(-(n - 1) / sigma),
                        rel_tol=1e-14)
    assert math.isclose(oracle.error_maxnorm(sigma, [0.5, 0.9], [0.1, 0.3], n), math.exp(-1 / sigma),
                        rel_tol=1e-14)
    n, sigma = 4096, 4.0
    rho = math.exp(-1 / sigma)
    bound = 2 * rho / (1 - rho)
    spec = oracle.error_spectral(sigma, [0.5], [0.0], n)      # ARPACK path (n >= 2048)
    assert 0.999 * bound < spec < bound


# ---------------------------------------------------------------- P14 ------
# [P, Key results, experimental validation]: training with T~ needs its
# gradients and the row normalisers.  Pinned by central finite differences
# of the forward oracle and by the one-block case.

@pytest.mark.parametrize("causal", [False, True])
def test_p14_gradients_match_finite_differences(causal):
    rng = _rng(31)
    B, Hq, Hkv, n, d = 1, 2, 1, 11, 4
    q = rng.standard_normal((B, Hq, n, d))
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    do = rng.standard_normal((B, Hq, n, d))
    dl = np.stack([_draw(rng, 3.0, 4)[0] for _ in range(Hq)])
    uu = dl * rng.uniform(0, 1, dl.shape)
    dq, dk, dv = oracle.plsh_attention_grad(q, k, v, do, dl, uu, causal)
    f = lambda q_, k_, v_: float((do * oracle.plsh_attention(q_, k_, v_, dl, uu, causal)).sum())
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0, 0), (0, 0, 5, 2), (0, x.shape[1] - 1, n - 1, 3), (0, x.shape[1] - 1, 3, 1)]:
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name] = xp
            args_m[name] = xm
            fd = (f(args_p["q"], args_p["k"], args_p["v"]) - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def test_p14_lse_one_block_is_logsumexp():
    """One block over everything: c = s everywhere, so the normaliser is
    log s + logsumexp of the scaled logits (SciPy)."""
    from scipy.special import logsumexp
    rng = _rng(32)
    B, H, n, d, s = 2, 2, 40, 8, 3
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    dl = np.full((H, s), 10.0 * n)
    uu = np.zeros((H, s))
    got = oracle.plsh_attention_lse(q, k, k, dl, uu, False)
    S = np.einsum("bhrd,bhjd->bhrj", q, k) / math.sqrt(d)
    assert np.allclose(got, math.log(s) + logsumexp(S, axis=-1), rtol=0, atol=1e-12)
    # causal: row r sums over j <= r
    got = oracle.plsh_attention_lse(q, k, k, dl, uu, True)
    Sc = np.where(np.tril(np.ones((n, n), bool)), S, -np.inf)
    assert np.allclose(got, math.log(s) + logsumexp(Sc, axis=-1), rtol=0, atol=1e-12)
