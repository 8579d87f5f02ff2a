"""GPU parity of the error measurements of M~ against L* (Theorem 2.1)
through the C ABI: row maxima, products E x and both norms, against the
fp64 oracle (oracle.convergence).

Hashes are drawn with numpy's generator (delta ~ Gamma(2, sigma), u uniform
in [0, delta)) plus edge widths; any valid hashes define an E.
"""

import math

import numpy as np
import pytest

import oracle
from tests._parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")


def _hashes(seed, sigma, s, n, edges=True):
    rng = np.random.default_rng(seed)
    d = rng.gamma(2.0, sigma, size=s)
    u = rng.uniform(0.0, 1.0, size=s) * d
    if edges and s >= 3:
        d[0], u[0] = 0.5, 0.25          # single-position blocks
        d[1], u[1] = 2.0 * n + 3.0, 0.0  # one block over everything
    return d, u


ROWMAX_CASES = [(1, 3.0, 1), (2, 3.0, 2), (129, 40.0, 5), (1000, 3.0, 20), (1000, 40.0, 20), (4097, 40.0, 7),
                (300, 10.0, 128)]


@pytest.mark.parametrize("case", ROWMAX_CASES, ids=lambda c: f"n{c[0]}sig{c[1]:g}s{c[2]}")
def test_rowmax_every_row(gpu, case):
    n, sigma, s = case
    say(f"error row maxima n={n} sigma={sigma} s={s}")
    d, u = _hashes(n + s, sigma, s, n)
    bins = P.bins_from_hashes(d[None], u[None], n, device=gpu)
    got = P.error_rowmax(sigma, bins).cpu().numpy()
    ref = oracle.error_rowmax(sigma, d, u, n, np.arange(n))
    assert np.abs(got - ref).max() <= 1e-15, np.abs(got - ref).max()


@pytest.mark.parametrize("n", [1, 777, 4097, 131072])
def test_matvec_full_vector(gpu, n):
    sigma, s = 37.0, 20
    say(f"error product n={n}")
    d, u = _hashes(3 * n + 1, sigma, s, n)
    bins = P.bins_from_hashes(d[None], u[None], n, device=gpu)
    x = np.random.default_rng(n).standard_normal(n)
    y = P.error_matvec(sigma, bins, torch.from_numpy(x).to(gpu)).cpu().numpy()
    ref = oracle.error_matvec(sigma, d, u, n, x)
    assert np.abs(y - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1e-300), np.abs(y - ref).max()


@pytest.mark.parametrize("case", [(1, 5.0, 3), (64, 5.0, 3), (1500, 25.0, 16), (2048, 7.0, 1)],
                         ids=lambda c: f"n{c[0]}sig{c[1]:g}s{c[2]}")
def test_norms_against_dense(gpu, case):
    n, sigma, s = case
    say(f"error norms n={n} sigma={sigma} s={s}")
    d, u = _hashes(n + 7, sigma, s, n)
    got = P.error_norms(sigma, d, u, n, max_steps=min(400, n), tol=1e-12, device=gpu)
    E = oracle.error_dense(sigma, d, u, n)
    spec = np.linalg.norm(E, 2)
    mx = np.abs(E).max()
    say(f"  spectral {got['spectral']:.12g} vs {spec:.12g} ({got['steps']} steps); max {got['maxnorm']:.15g}")
    assert abs(got["spectral"] - spec) <= 1e-8 * max(spec, 1e-300)
    assert abs(got["maxnorm"] - mx) <= 1e-15
    assert abs(np.abs(E[got["argmax_row"]]).max() - mx) <= 1e-15


def test_norms_full_size(gpu):
    """n = 131072, sigma = 256, s = 20: the max norm bounds every sampled
    row's maximum and equals the oracle's at the reported row; the spectral
    norm agrees with ARPACK on the oracle's product."""
    n, sigma, s = 131072, 256.0, 20
    say("error norms full size")
    d, u = _hashes(11, sigma, s, n, edges=False)
    got = P.error_norms(sigma, d, u, n, max_steps=300, tol=1e-11, device=gpu)
    rows = np.unique(np.concatenate([[0, 1, n - 1, got["argmax_row"]],
                                     np.random.default_rng(2).integers(0, n, 48)]))
    ref = oracle.error_rowmax(sigma, d, u, n, rows)
    assert ref.max() <= got["maxnorm"] + 1e-15
    at = ref[np.searchsorted(rows, got["argmax_row"])]
    assert abs(at - got["maxnorm"]) <= 1e-15
    spec = oracle.error_spectral(sigma, d, u, n, tol=1e-10)
    say(f"  spectral {got['spectral']:.10g} vs ARPACK {spec:.10g} ({got['steps']} steps), max {got['maxnorm']:.6g}")
    assert abs(got["spectral"] - spec) <= 1e-7 * spec


def test_error_decays_like_inverse_sqrt_s(gpu):
    """[Theorem 2.1; Key results]: both norms fall like 1/sqrt(s)."""
    n, sigma = 16384, 64.0
    ss = [4, 16, 64]
    spec, mx = [], []
    for s in ss:
        a, b = [], []
        for seed in range(3):
            d, u = _hashes(100 * s + seed, sigma, s, n, edges=False)
            r = P.error_norms(sigma, d, u, n, max_steps=200, tol=1e-8, device=gpu)
            a.append(r["spectral"])
            b.append(r["maxnorm"])
        spec.append(np.mean(a))
        mx.append(np.mean(b))
    for e in (spec, mx):
        slope = np.polyfit(np.log(ss), np.log(e), 1)[0]
        say(f"  slope {slope:.3f}")
        assert -0.7 < slope < -0.3, slope
    # Hoeffding + union bound on the n^2 entries, failure probability 1e-3
    assert max(mx[i] - math.sqrt(math.log(2 * n * n / 1e-3) / (2 * s)) for i, s in enumerate(ss)) <= 0
