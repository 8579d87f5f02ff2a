"""Every compiled variant of every kernel, element by element against the
fp64 oracle.

The library compiles its kernels per (head_dim, dtype, causal, hash chunks):
head_dim 64 or 128, fp32 or bf16, causal or not, and s hashes held in 1, 2
or 4 chunks of 32 (s <= 32, s <= 64, s <= 128).  Each test below walks the
full product of the dimensions its kernel is compiled over, so that no
variant the C ABI accepts goes untested:

  * count-weighted attention (plpsh_attention_fwd): 2 x 2 x 2 x 3 = 24,
    plus s at each chunk edge (32, 33, 64, 65);
  * the per-hash kernel (plpsh_attention_fwd_literal): 2 x 2 x 2 = 8;
  * dense exact ALiBi (plpsh_alibi_dense_fwd): 2 x 2 x 2 = 8;
  * the backward pass (plpsh_attention_bwd, bf16 only): 2 x 2 x 3 = 12.

Inputs: 4 query heads over 2 KV heads (GQA), n = 300 (two full 128-row
tiles and a ragged third), widths from about one position to wider than the
sequence, Q scaled by 2 so that the softmax is not flat.  Tolerances are
those of tests/_parity.py.
"""

import itertools

import numpy as np
import pytest

import oracle
import synth
from tests._parity import check_slices, oracle_full, oracle_hashes, say, to64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")

B, HQ, HKV, N = 1, 4, 2, 300
SIGMAS = (1.5, 6.0, 40.0, 300.0)
CHUNK_S = {1: 20, 2: 48, 4: 100}   # one s per hash-chunk count


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _inputs(d, dtype, seed, gpu):
    q, k, v = synth.qkv_numpy(B, HQ, HKV, N, d, dtype, seed, 2.0)
    t = lambda a: torch.from_numpy(a).to(gpu).to(_tdt(dtype)).contiguous()
    return (t(q), t(k), t(v)), (q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))


def _ids(c):
    return "-".join(str(x) for x in c)


FWD = [(d, dt, c, CHUNK_S[ch]) for d, dt, c, ch in itertools.product((64, 128), ("f32", "bf16"), (False, True),
                                                                       (1, 2, 4))]
FWD += [(128, "bf16", True, s) for s in (32, 33, 64, 65)]


@pytest.mark.parametrize("case", FWD, ids=lambda c: f"d{c[0]}-{c[1]}-{'causal' if c[2] else 'full'}-s{c[3]}")
def test_forward_variant(gpu, case):
    d, dtype, causal, s = case
    say(f"forward variant d={d} {dtype} causal={causal} s={s}")
    (q, k, v), (q64, k64, v64) = _inputs(d, dtype, 100 + d + s, gpu)
    delta, u = oracle_hashes(21, SIGMAS, s, *P.draw_hashes(21, SIGMAS, s))
    o = torch.full_like(q, float("nan"))
    P.attention(q, k, v, SIGMAS, s, seed=21, causal=causal, out=o)
    torch.cuda.synchronize()
    ref = oracle_full(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=f"forward {case}")
    say(f"  max err {err:.3e}")


LIT = list(itertools.product((64, 128), ("f32", "bf16"), (False, True)))


@pytest.mark.parametrize("case", LIT, ids=lambda c: f"d{c[0]}-{c[1]}-{'causal' if c[2] else 'full'}")
def test_literal_variant(gpu, case):
    """The per-hash kernel (Theorem 2.2's reduction) against the oracle's
    per-block formulation."""
    d, dtype, causal = case
    s = 20
    say(f"literal variant d={d} {dtype} causal={causal}")
    (q, k, v), (q64, k64, v64) = _inputs(d, dtype, 300 + d, gpu)
    ldelta, lu, bins = P.sample_bins(22, SIGMAS, s, N, device=gpu)
    delta, u = oracle_hashes(22, SIGMAS, s, ldelta, lu)
    o = torch.full_like(q, float("nan"))
    P.attention_literal(q, k, v, bins, causal=causal, delta=ldelta, out=o)
    torch.cuda.synchronize()
    ref = oracle.plsh_attention_literal(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=f"literal {case}")
    say(f"  max err {err:.3e}")


@pytest.mark.parametrize("case", LIT, ids=lambda c: f"d{c[0]}-{c[1]}-{'causal' if c[2] else 'full'}")
def test_dense_alibi_variant(gpu, case):
    d, dtype, causal = case
    say(f"dense ALiBi variant d={d} {dtype} causal={causal}")
    (q, k, v), (q64, k64, v64) = _inputs(d, dtype, 500 + d, gpu)
    o = torch.full_like(q, float("nan"))
    P.alibi_dense(q, k, v, SIGMAS, causal=causal, out=o)
    torch.cuda.synchronize()
    ref = oracle.alibi_attention(q64, k64, v64, SIGMAS, causal)
    err = check_slices(to64(o), ref, dtype, where=f"dense {case}")
    say(f"  max err {err:.3e}")


BWD = list(itertools.product((64, 128), (False, True), (1, 2, 4)))


@pytest.mark.parametrize("case", BWD, ids=lambda c: f"d{c[0]}-{'causal' if c[1] else 'full'}-chunks{c[2]}")
def test_backward_variant(gpu, case):
    """Row normalisers and dQ, dK, dV against the fp64 gradient oracle, per
    (batch, head) slice: max |x - x_ref| / max |x_ref| <= 2e-2."""
    d, causal, ch = case
    s = CHUNK_S[ch]
    say(f"backward variant d={d} causal={causal} s={s}")
    (q, k, v), (q64, k64, v64) = _inputs(d, "bf16", 700 + d + s, gpu)
    do = torch.from_numpy(np.random.default_rng(d + s).standard_normal((B, HQ, N, d)).astype(np.float32))
    do = do.to(gpu).to(torch.bfloat16).contiguous()
    do64 = to64(do)
    ldelta, lu, bins = P.sample_bins(23, SIGMAS, s, N, device=gpu)
    delta, u = oracle_hashes(23, SIGMAS, s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=causal, delta=ldelta)
    dq, dk, dv = P.attention_bwd(q, k, v, o, do, lse, bins, causal=causal, delta=ldelta)
    torch.cuda.synchronize()
    lse_ref = oracle.plsh_attention_lse(q64, k64, v64, delta, u, causal)
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= 1e-4 * max(1.0, np.abs(lse_ref).max())
    gq, gk, gv = oracle.plsh_attention_grad(q64, k64, v64, do64, delta, u, causal)
    worst = []
    for name, got, ref in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
        g = to64(got)
        w = 0.0
        for idx in np.ndindex(*ref.shape[:2]):
            rel = np.abs(g[idx] - ref[idx]).max() / max(np.abs(ref[idx]).max(), 1e-30)
            assert rel <= 2e-2, f"{name} {case} slice {idx}: {rel:.3e}"
            w = max(w, rel)
        worst.append(w)
    say(f"  worst rel err dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")
