"""fp64 oracle for the error of the sampled mask mean against the ALiBi bias
matrix at large n: E = L* - M~ with L*[r, j] = exp(-|r - j| / sigma) and
M~ = c / s  [P, Methodology 1; Theorem 2.1].

TEST INFRASTRUCTURE ONLY.  The pages state that the spectral-norm and
max-norm errors of M~ fall like 1/sqrt(s) and that their experiments saw the
matrix-norm error go to zero as s grows [P, Theorem 2.1; Key results,
experimental validation].  These functions give both norms for sequence
lengths where the dense n x n matrices no longer fit:

* ``error_rowmax``  : max_j |E[r, j]| for chosen rows, straight from the
  definition (every j, every hash), O(n s) per row;
* ``error_matvec``  : E x, with L* x through SciPy's Toeplitz product and
  M(h_i) x as the sum of x over the block of each position (one bincount per
  hash, which is the definition of a product with a 0/1 block-diagonal
  matrix);
* ``error_spectral``: ||E||_2, the largest |eigenvalue| of the symmetric E,
  from ARPACK (``scipy.sparse.linalg.eigsh``) on that product, or from the
  dense matrix when n is small.

Small-n versions of all three are pinned against the dense matrices of
``oracle.plsh`` in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import numpy as np

from .plsh import alibi_matrix, bin_values, mtilde

__all__ = ["ErrorOperator", "error_dense", "error_rowmax", "error_matvec", "error_spectral", "error_maxnorm"]


def _hashes(deltas, us):
    d = np.atleast_1d(np.asarray(deltas, dtype=np.float64)).reshape(-1)
    u = np.atleast_1d(np.asarray(us, dtype=np.float64)).reshape(-1)
    if d.shape != u.shape:
        raise ValueError("one offset per bin width")
    return d, u


def error_dense(sigma: float, deltas, us, n: int) -> np.ndarray:
    """E = L* - M~ as a dense n x n matrix (small n only)."""
    d, u = _hashes(deltas, us)
    return alibi_matrix(sigma, n) - mtilde(d, u, n)


def error_rowmax(sigma: float, deltas, us, n: int, rows) -> np.ndarray:
    """max over all j of |exp(-|r - j| / sigma) - c[r, j] / s| for each row r."""
    d, u = _hashes(deltas, us)
    s = d.size
    bins = [bin_values(dl, uu, n) for dl, uu in zip(d, u)]
    j = np.arange(n, dtype=np.float64)
    out = np.empty(len(rows))
    for t, r in enumerate(np.asarray(rows, dtype=np.int64)):
        c = np.zeros(n)
        for b in bins:
            c += b == b[r]
        out[t] = np.abs(np.exp(-np.abs(j - float(r)) / float(sigma)) - c / s).max()
    return out


def error_maxnorm(sigma: float, deltas, us, n: int) -> float:
    """||E||_max over all rows (dense, small n)."""
    return float(np.abs(error_dense(sigma, deltas, us, n)).max())


def _laplace_column(sigma: float, n: int) -> np.ndarray:
    return np.exp(-np.arange(n, dtype=np.float64) / float(sigma))


class ErrorOperator:
    """x -> E x = L* x - (1/s) sum_i M(h_i) x.

    L* is the symmetric Toeplitz matrix whose first column is exp(-k/sigma);
    (M(h_i) x)[r] is the sum of x over the positions sharing r's bin.  The
    bin labels of each hash are computed once.
    """

    def __init__(self, sigma: float, deltas, us, n: int):
        d, u = _hashes(deltas, us)
        self.n, self.s = n, d.size
        self.col = _laplace_column(sigma, n)
        self.labels = [np.unique(bin_values(dl, uu, n), return_inverse=True)[1] for dl, uu in zip(d, u)]

    def matvec(self, x) -> np.ndarray:
        from scipy.linalg import matmul_toeplitz

        x = np.asarray(x, dtype=np.float64).reshape(-1)
        lx = matmul_toeplitz(self.col, x)
        mx = np.zeros(self.n)
        for inv in self.labels:
            mx += np.bincount(inv, weights=x)[inv]
        return lx - mx / self.s


def error_matvec(sigma: float, deltas, us, n: int, x) -> np.ndarray:
    """E x (see ErrorOperator)."""
    return ErrorOperator(sigma, deltas, us, n).matvec(x)


def error_spectral(sigma: float, deltas, us, n: int, dense_below: int = 2048, tol: float = 1e-12) -> float:
    """||E||_2 = max |eigenvalue| of the symmetric E."""
    if n < dense_below:
        return float(np.linalg.norm(error_dense(sigma, deltas, us, n), 2))
    from scipy.sparse.linalg import LinearOperator, eigsh

    E = ErrorOperator(sigma, deltas, us, n)
    op = LinearOperator((n, n), matvec=E.matvec, dtype=np.float64)
    vals = eigsh(op, k=1, which="LM", tol=tol, return_eigenvectors=False,
                 v0=np.random.default_rng(0).standard_normal(n))
    return float(np.abs(vals).max())
