"""fp64 NumPy oracle: what Positional-LSH attention computes, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: dense
n x n masks, no blocking, fusion or reordering beyond what the definitions
state.  Inputs are float64 arrays (bf16/fp32 inputs are upcast exactly by the
caller).  Citations ``[P, ...]`` are to the explainer pages named in the
package docstring.

Notation.  Positions are 0-based integers x = 0..n-1.  One hash of head h is a
pair (delta, u): bin width and offset.  Its bin of position x is
``floor((x - u) / delta)`` evaluated in IEEE-754 binary64 (exact conversion of
x, correctly rounded subtraction and division, then floor).  A hash cuts
[0, n) into maximal runs of equal bin value ("blocks").  M(h)[r, j] = 1 iff r
and j share a bin.  With s hashes, the count c[r, j] = sum_i M(h_i)[r, j] and
M~ = c / s.  Attention logits are S = Q K^T / sqrt(d).  Queries of head h read
key/value head g(h) = h // (Hq // Hkv).  With ``causal`` the weight of (r, j)
is also multiplied by [j <= r].

The approximation computed is

    T~_r = sum_j M~[r,j] C[r,j] exp(S[r,j]) v_j / sum_j M~[r,j] C[r,j] exp(S[r,j])

i.e. the exact ALiBi-attention formula with the Laplace bias matrix L* replaced
by the empirical mean M~ of s random binary block masks [P, Theorem 2.1] and
[P, Theorem 2.2].  The samples are combined as a ratio of sums (numerator and
denominator each summed over the s masks), which is what replacing L* by M~
in the biased attention means.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bin_values",
    "block_starts",
    "block_of",
    "count_matrix",
    "mtilde",
    "alibi_matrix",
    "support_interval",
    "plsh_attention",
    "plsh_attention_literal",
    "plsh_attention_rows",
    "plsh_attention_rowblocks",
    "alibi_attention",
    "alibi_attention_rows",
]


# ---------------------------------------------------------------------------
# Hash -> bins -> masks   [P, Methodology 1]
# ---------------------------------------------------------------------------

def bin_values(delta: float, u: float, n: int) -> np.ndarray:
    """Bin index of every position under one random-binning hash.

    [P, Methodology 1]: the random binning features of Rahimi and Recht,
    applied to the integer positions only, place position x in bin
    floor((x - u) / delta) for a random width delta and offset u.  Values are
    kept as float64 (no integer cast, so delta << 1 cannot overflow).
    Parity: pinned (exact rational arithmetic, monotonicity, block lengths).
    """
    x = np.arange(n, dtype=np.float64)
    return np.floor((x - float(u)) / float(delta))


def block_starts(delta: float, u: float, n: int) -> np.ndarray:
    """Start positions of the blocks of one hash (int64, ascending, first = 0).

    A block is a maximal run of positions with equal bin value; a position
    starts a block when it is 0 or its bin differs from the previous
    position's.  [P, Methodology 1]: the bins of the integer positions are
    contiguous and do not overlap, so these starts describe M(h) completely.
    Empty bins (delta < 1) therefore never produce a block.
    Parity: pinned (brute force against exact rationals; invariants).
    """
    b = bin_values(delta, u, n)
    flags = np.ones(n, dtype=bool)
    flags[1:] = b[1:] != b[:-1]
    return np.flatnonzero(flags).astype(np.int64)


def block_of(delta: float, u: float, n: int, x) -> tuple[np.ndarray, np.ndarray]:
    """[start, end) of the block containing each position in ``x``.

    Since bin values are non-decreasing in x, the positions sharing x's bin
    are exactly those between the first and last occurrence of that value.
    """
    b = bin_values(delta, u, n)
    x = np.asarray(x, dtype=np.int64)
    start = np.searchsorted(b, b[x], side="left")
    end = np.searchsorted(b, b[x], side="right")
    return start.astype(np.int64), end.astype(np.int64)


def count_matrix(deltas, us, n: int) -> np.ndarray:
    """Dense c[r, j] = #{i : bin_i(r) == bin_i(j)}  (int32, n x n).

    The sum over the s sampled masks M(h_i); M~ = c / s is the empirical
    mean of [P, Theorem 2.1].  Parity: pinned (E[M(h)] = L* closed form,
    binomial law, contiguity invariants).
    """
    deltas = np.atleast_1d(np.asarray(deltas, dtype=np.float64))
    us = np.atleast_1d(np.asarray(us, dtype=np.float64))
    c = np.zeros((n, n), dtype=np.int32)
    for dl, uu in zip(deltas, us):
        b = bin_values(dl, uu, n)
        c += (b[:, None] == b[None, :])
    return c


def mtilde(deltas, us, n: int) -> np.ndarray:
    """M~ = (1/s) sum_i M(h_i)  [P, Theorem 2.1]."""
    deltas = np.atleast_1d(np.asarray(deltas, dtype=np.float64))
    return count_matrix(deltas, us, n).astype(np.float64) / deltas.size


def alibi_matrix(sigma: float, n: int) -> np.ndarray:
    """L*[i, j] = exp(-|i - j| / sigma), the Laplace-kernel form of the ALiBi
    bias [P, Methodology 1] (sigma = 1 / ALiBi slope)."""
    i = np.arange(n, dtype=np.float64)
    return np.exp(-np.abs(i[:, None] - i[None, :]) / float(sigma))


def support_interval(deltas, us, n: int, rows, causal: bool):
    """[lo(r), hi(r)) : the smallest interval holding every j with c[r, j] > 0.

    Each hash puts r in one contiguous block; the union of s intervals that
    all contain r is the interval from the smallest block start to the
    largest block end.  With ``causal`` the interval is cut at r + 1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    lo = np.full(rows.shape, n, dtype=np.int64)
    hi = np.zeros(rows.shape, dtype=np.int64)
    for dl, uu in zip(np.atleast_1d(deltas), np.atleast_1d(us)):
        a, e = block_of(dl, uu, n, rows)
        lo = np.minimum(lo, a)
        hi = np.maximum(hi, e)
    if causal:
        hi = np.minimum(hi, rows + 1)
    return lo, hi


# ---------------------------------------------------------------------------
# Attention with a weight matrix   [P, Theorem 2.2]
# ---------------------------------------------------------------------------

def _weighted_attention(S: np.ndarray, Wb: np.ndarray, v: np.ndarray) -> np.ndarray:
    """sum_j Wb[r,j] exp(S[r,j]) v_j / sum_j Wb[r,j] exp(S[r,j]).

    Wb >= 0 is the (bias or mask) weight.  The row maximum of S over the
    support {Wb > 0} is subtracted first; it cancels between numerator and
    denominator and only keeps exp() in range.
    """
    supp = Wb > 0
    m = np.max(np.where(supp, S, -np.inf), axis=1, keepdims=True)
    E = np.exp(np.where(supp, S - m, -np.inf))
    W = Wb * E
    return (W @ v) / W.sum(axis=1, keepdims=True)


def _heads(q, k):
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return B, Hq, Hkv, n, d, Hq // Hkv


def plsh_attention(q, k, v, deltas, us, causal: bool) -> np.ndarray:
    """T~ with the dense M~ materialised (the reference formulation).

    q: [B, Hq, n, d]; k, v: [B, Hkv, n, d]; deltas, us: [Hq, s].
    [P, Theorem 2.1] gives M~; [P, Theorem 2.2] uses it in place of L* in
    the biased attention.  Parity: pinned (all-ones masks reduce to plain
    softmax attention; delta < 1 gives T~ = V; fixed blocks equal a
    block-masked SDPA; agreement with the literal per-sample reduction;
    convergence to exact ALiBi; convexity; the output-error inequality).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Hkv, n, d, grp = _heads(q, k)
    deltas = np.asarray(deltas, np.float64).reshape(Hq, -1)
    us = np.asarray(us, np.float64).reshape(Hq, -1)
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    tri = np.tril(np.ones((n, n), dtype=bool)) if causal else None
    for h in range(Hq):
        mt = mtilde(deltas[h], us[h], n)
        if causal:
            mt = np.where(tri, mt, 0.0)
        g = h // grp
        for b in range(B):
            S = (q[b, h] @ k[b, g].T) * scale
            out[b, h] = _weighted_attention(S, mt, v[b, g])
    return out


def plsh_attention_literal(q, k, v, deltas, us, causal: bool) -> np.ndarray:
    """T~ computed as [P, Theorem 2.2] describes the reduction: a collection
    of short-context attentions with no positional bias, one per block of
    each sampled hash, whose numerators and denominators are summed over
    all blocks containing the query and divided at the end.

    A second, independent formulation of the same quantity (no dense mask).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Hkv, n, d, grp = _heads(q, k)
    deltas = np.asarray(deltas, np.float64).reshape(Hq, -1)
    us = np.asarray(us, np.float64).reshape(Hq, -1)
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    for h in range(Hq):
        g = h // grp
        blocks = []
        for dl, uu in zip(deltas[h], us[h]):
            st = block_starts(dl, uu, n)
            en = np.append(st[1:], n)
            blocks.extend(zip(st.tolist(), en.tolist()))
        for b in range(B):
            # common stabiliser: per-row max over every block the row sits in
            m = np.full(n, -np.inf)
            for a, e in blocks:
                Sb = (q[b, h, a:e] @ k[b, g, a:e].T) * scale
                if causal:
                    Sb = np.where(np.tril(np.ones((e - a, e - a), bool)), Sb, -np.inf)
                m[a:e] = np.maximum(m[a:e], Sb.max(axis=1))
            num = np.zeros((n, d))
            den = np.zeros(n)
            for a, e in blocks:
                Sb = (q[b, h, a:e] @ k[b, g, a:e].T) * scale
                if causal:
                    Sb = np.where(np.tril(np.ones((e - a, e - a), bool)), Sb, -np.inf)
                E = np.exp(Sb - m[a:e, None])
                num[a:e] += E @ v[b, g, a:e]
                den[a:e] += E.sum(axis=1)
            out[b, h] = num / den[:, None]
    return out


def plsh_attention_rows(qh, kh, vh, deltas_h, us_h, rows, causal: bool) -> np.ndarray:
    """T~ for selected query rows of one (batch, head): qh [n, d] (or only
    the needed rows indexed by ``rows``), kh/vh [n, d] of the KV head.

    Row r only needs keys in its support [lo(r), hi(r)); outside it every
    count is zero.  Inside it the count is the plain definition
    c[r, j] = #{i : bin_i(r) == bin_i(j)}.  Used to check full-size
    launches on sampled rows.
    """
    kh = np.asarray(kh, np.float64)
    vh = np.asarray(vh, np.float64)
    n, d = kh.shape
    rows = np.asarray(rows, dtype=np.int64)
    bins = [bin_values(dl, uu, n) for dl, uu in zip(np.atleast_1d(deltas_h), np.atleast_1d(us_h))]
    lo, hi = support_interval(deltas_h, us_h, n, rows, causal)
    scale = 1.0 / math.sqrt(d)
    qh = np.asarray(qh, np.float64)
    out = np.empty((rows.size, d))
    for t, r in enumerate(rows):
        a, e = int(lo[t]), int(hi[t])
        c = np.zeros(e - a)
        for b in bins:
            c += b[a:e] == b[r]
        qr = qh[r] if qh.shape[0] == n else qh[t]
        S = (kh[a:e] @ qr) * scale
        out[t] = _weighted_attention(S[None, :], c[None, :], vh[a:e])[0]
    return out


def plsh_attention_rowblocks(qh, kh, vh, deltas_h, us_h, causal: bool,
                             row_block: int = 64, blocks=None) -> tuple[np.ndarray, list]:
    """Banded T~ for one (batch, head): each block of ``row_block`` rows reads
    only keys in [lo(first row), hi(last row)), the union of its rows'
    supports (lo and hi are non-decreasing in r).  Arithmetically identical
    to the dense form because every excluded count is zero.

    ``blocks``: optional iterable of row-block indices (a bounded sample).
    Returns (rows_out [R, d], list of row ranges).
    """
    qh = np.asarray(qh, np.float64)
    kh = np.asarray(kh, np.float64)
    vh = np.asarray(vh, np.float64)
    n, d = kh.shape
    bins = np.stack([bin_values(dl, uu, n) for dl, uu in
                     zip(np.atleast_1d(deltas_h), np.atleast_1d(us_h))])
    nb = (n + row_block - 1) // row_block
    blocks = range(nb) if blocks is None else blocks
    scale = 1.0 / math.sqrt(d)
    outs, ranges = [], []
    for t in blocks:
        r0, r1 = t * row_block, min(n, (t + 1) * row_block)
        lo, hi = support_interval(deltas_h, us_h, n, [r0, r1 - 1], causal)
        a = int(lo[0])
        e = int(hi[1]) if not causal else r1
        c = (bins[:, r0:r1, None] == bins[:, None, a:e]).sum(axis=0).astype(np.float64)
        if causal:
            c = np.where(np.arange(a, e)[None, :] <= np.arange(r0, r1)[:, None], c, 0.0)
        S = (qh[r0:r1] @ kh[a:e].T) * scale
        outs.append(_weighted_attention(S, c, vh[a:e]))
        ranges.append((r0, r1))
    return (np.concatenate(outs) if outs else np.empty((0, d))), ranges


# ---------------------------------------------------------------------------
# Exact ALiBi attention T*   [P, Methodology 1] (bias) and problem statement
# ---------------------------------------------------------------------------

def alibi_attention(q, k, v, sigmas, causal: bool) -> np.ndarray:
    """T* = (L* o C o exp(S)) V / (L* o C o exp(S)) 1, the exact ALiBi-biased
    attention that T~ approximates; per head h, sigma_h = 1 / slope_h.
    Parity: pinned (brute-force triple loop on tiny n; reduction to plain
    softmax attention as sigma -> infinity)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Hkv, n, d, grp = _heads(q, k)
    sigmas = np.broadcast_to(np.asarray(sigmas, np.float64), (Hq,))
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    for h in range(Hq):
        L = alibi_matrix(sigmas[h], n)
        if causal:
            L = np.tril(L)
        g = h // grp
        for b in range(B):
            S = (q[b, h] @ k[b, g].T) * scale
            out[b, h] = _weighted_attention(S, L, v[b, g])
    return out


def alibi_attention_rows(qh, kh, vh, sigma: float, rows, causal: bool) -> np.ndarray:
    """Rows of T* for one (batch, head), one at a time (full-size checks)."""
    kh = np.asarray(kh, np.float64)
    vh = np.asarray(vh, np.float64)
    qh = np.asarray(qh, np.float64)
    n, d = kh.shape
    rows = np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(d)
    out = np.empty((rows.size, d))
    j = np.arange(n, dtype=np.float64)
    for t, r in enumerate(rows):
        e = r + 1 if causal else n
        L = np.exp(-np.abs(float(r) - j[:e]) / float(sigma))
        qr = qh[r] if qh.shape[0] == n else qh[t]
        S = (kh[:e] @ qr) * scale
        out[t] = _weighted_attention(S[None, :], L[None, :], vh[:e])[0]
    return out
