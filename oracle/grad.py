"""fp64 oracle for training with Positional-LSH attention: the log of each
row's normaliser and the gradients of T~ with respect to Q, K and V.

TEST INFRASTRUCTURE ONLY.  The pages train models with the approximation in
place of exact ALiBi (Qwen3-0.6B from scratch, Mistral-7B fine-tuned) [P, Key
results, experimental validation], which needs the backward pass of
T~ = W V / (W 1) with W = c o C o exp(S), S = Q K^T / sqrt(d), c the integer
counts of the sampled masks and C the causal mask.  The counts do not depend
on Q, K or V, so the gradients are those of softmax attention with the
weights c o C:

    P = W / (W 1)           dV = P^T dO          dP = dO V^T
    D_r = sum_j P_rj dP_rj = <dO_r, O_r>         dS = P o (dP - D)
    dQ = dS K / sqrt(d)     dK = dS^T Q / sqrt(d)

with the gradients of the query heads of one KV group summed into that KV
head.  Written densely; pinned in tests/test_oracle_pins.py by central finite
differences of ``plsh_attention`` and by the one-block case, where the
normaliser is a log-sum-exp.
"""

from __future__ import annotations

import math

import numpy as np

from .plsh import _heads, count_matrix

__all__ = ["plsh_attention_lse", "plsh_attention_grad"]


def _weights(q, k, deltas, us, causal, b, h, g):
    """Count-weighted logits of one (batch, head): (S, c o C)."""
    n, d = q.shape[2], q.shape[3]
    dl = np.asarray(deltas, np.float64).reshape(q.shape[1], -1)
    uu = np.asarray(us, np.float64).reshape(q.shape[1], -1)
    c = count_matrix(dl[h], uu[h], n).astype(np.float64)
    if causal:
        c = np.where(np.tril(np.ones((n, n), dtype=bool)), c, 0.0)
    S = (q[b, h] @ k[b, g].T) / math.sqrt(d)
    return S, c


def plsh_attention_lse(q, k, v, deltas, us, causal: bool) -> np.ndarray:
    """LSE[b, h, r] = log sum_j c[r, j] C[r, j] exp(S[r, j])  (natural log).

    The normaliser of row r of T~ with the counts (not M~ = c / s) as the
    weights.  [B, Hq, n] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, Hq, Hkv, n, d, grp = _heads(q, k)
    out = np.empty((B, Hq, n))
    for h in range(Hq):
        for b in range(B):
            S, c = _weights(q, k, deltas, us, causal, b, h, h // grp)
            supp = c > 0
            m = np.max(np.where(supp, S, -np.inf), axis=1)
            out[b, h] = m + np.log((c * np.exp(np.where(supp, S - m[:, None], -np.inf))).sum(axis=1))
    return out


def plsh_attention_grad(q, k, v, do, deltas, us, causal: bool):
    """(dQ, dK, dV) of sum(dO * T~) for T~ = plsh_attention(q, k, v, ...).

    q, do: [B, Hq, n, d]; k, v: [B, Hkv, n, d]; deltas, us: [Hq, s].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Hq, Hkv, n, d, grp = _heads(q, k)
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // grp
        for b in range(B):
            S, c = _weights(q, k, deltas, us, causal, b, h, g)
            supp = c > 0
            m = np.max(np.where(supp, S, -np.inf), axis=1, keepdims=True)
            W = c * np.exp(np.where(supp, S - m, -np.inf))
            P = W / W.sum(axis=1, keepdims=True)
            O = P @ v[b, g]
            dv[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            D = (do[b, h] * O).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, h] = dS @ k[b, g] * scale
            dk[b, g] += dS.T @ q[b, h] * scale
    return dq, dk, dv
