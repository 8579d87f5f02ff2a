"""Shared helpers of the GPU parity tests: tolerances and oracle plumbing.

Tolerances (stated for the method's outputs):
  * float32 inputs: max |O - O_ref| <= 1e-4 elementwise.
  * bfloat16 inputs (fp32 accumulation, P rounded to bf16 before the value
    product): per (batch, head) slice, max |O - O_ref| / max |O_ref| <= 2e-2.
The oracle receives the exact values the kernel read (bf16 or fp32 upcast to
float64), so only in-kernel arithmetic is measured.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle

TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_slices(out, ref, dtype, where=""):
    """out, ref: float64 [..., n, d] (same shape).  Returns max errors."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"non-finite output {where}"
    err = np.abs(out - ref)
    if dtype == "f32":
        m = err.max() if err.size else 0.0
        assert m <= TOL_F32_ABS, f"{where}: max abs err {m:.3e} > {TOL_F32_ABS}"
        return m
    lead = out.shape[:-2]
    worst = 0.0
    for idx in np.ndindex(*lead):
        e = err[idx].max()
        s = np.abs(ref[idx]).max()
        rel = e / s if s > 0 else e
        worst = max(worst, rel)
        assert rel <= TOL_BF16_REL, f"{where} slice {idx}: rel err {rel:.3e} > {TOL_BF16_REL}"
    return worst


def oracle_full(q, k, v, delta, u, causal):
    """Full T~ with the banded oracle (identical arithmetic to the dense
    form; pinned against it on the CPU).  q [B,Hq,n,d] float64 etc."""
    B, Hq, n, d = q.shape
    grp = Hq // k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            o, _ = oracle.plsh_attention_rowblocks(q[b, h], k[b, h // grp], v[b, h // grp], delta[h], u[h],
                                                   causal, row_block=64)
            out[b, h] = o
    return out


def sample_rows(n, count, rng):
    base = {0, 1, 2, n - 1, n - 2}
    for t in (63, 64, 65, 127, 128, 129, 255, 256):
        if t < n:
            base.add(t)
    extra = rng.choice(n, size=min(count, n), replace=False)
    return np.array(sorted(base.union(int(x) for x in extra)))


def oracle_hashes(seed, sigmas, s, lib_delta=None, lib_u=None):
    """The oracle's own draw of the hashes (its independent SplitMix64); when
    the library's draw is given, it must be bit-identical.  Oracle inputs
    never come from the library."""
    d, u = oracle.sample_hashes(seed, sigmas, s)
    if lib_delta is not None:
        assert np.array_equal(np.asarray(lib_delta).reshape(d.shape), d), "library hash widths differ from the oracle's"
        assert np.array_equal(np.asarray(lib_u).reshape(u.shape), u), "library hash offsets differ from the oracle's"
    return d, u


# ---------------------------------------------------------- bin buffers --

def expected_plan(delta, u, n, tiles=None):
    """Block starts and the plan records of `tiles` (all tiles if None; the
    other rows of the returned array are left zero)."""
    st = oracle.block_starts(delta, u, n)
    ntile = (n + 127) // 128
    rec = np.zeros((ntile, 8), dtype=np.int64)
    starts_set = set(st.tolist()) | {n}
    for q in (range(ntile) if tiles is None else tiles):
        r0 = 128 * q
        rl = min(r0 + 127, n - 1)
        a, e = oracle.block_of(delta, u, n, [r0, rl])
        rec[q, 0], rec[q, 1], rec[q, 2], rec[q, 3] = a[0], e[0], a[1], e[1]
        bits = [0, 0, 0, 0]
        for p in range(1, 128):
            if r0 + p in starts_set:
                bits[p >> 5] |= 1 << (p & 31)
        rec[q, 4:] = bits
    return st, rec


def check_bins(bins, delta, u, n, tiles=None):
    """Block counts and starts of every hash, and the plan records of `tiles`
    (every tile if None), bit-exact against the oracle."""
    nblk = bins.nblk.cpu().numpy()
    starts = bins.starts.cpu().numpy()
    plan = bins.plan.cpu().numpy().view(np.uint32).astype(np.int64)
    H, s = delta.shape
    sel = slice(None) if tiles is None else np.asarray(tiles)
    for h in range(H):
        for i in range(s):
            t = h * s + i
            st, rec = expected_plan(delta[h, i], u[h, i], n, tiles)
            assert nblk[t] == st.size, (h, i, delta[h, i], u[h, i], n)
            assert np.array_equal(starts[t, :st.size + 1], np.append(st, n)), (h, i, delta[h, i], u[h, i], n)
            got = plan[h, :, i, :].copy()
            got[:, :4] = plan[h, :, i, :4].astype(np.uint32).view(np.int32)
            assert np.array_equal(got[sel], rec[sel]), (h, i, delta[h, i], u[h, i], n)
