"""GPU parity of training support through the C ABI: the forward pass's row
normalisers (plpsh_attention_fwd_lse) and the backward pass
(plpsh_attention_bwd), against the fp64 oracle (oracle.grad).

The oracle sees the bf16-rounded inputs.  Gradients are compared per
(batch, head) slice, max |x - x_ref| / max |x_ref| <= 2e-2 (the products use
P and dS rounded to bf16, as the forward uses P); at the full Mistral size,
dQ on sampled rows from the definition and, for dK and dV, the identities
sum_j dV_j = sum over the group's heads and rows of dO and sum_j dK_j = 0.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from tests._parity import oracle_hashes, say, to64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")

TOL = 2e-2


def _dev(B, Hq, Hkv, n, d, seed, gpu, scale_q=1.0):
    q, k, v = synth.qkv_numpy(B, Hq, Hkv, n, d, "bf16", seed, 2.0)
    q = q * np.float32(scale_q)
    do = np.random.default_rng(seed + 1).standard_normal((B, Hq, n, d)).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu).to(torch.bfloat16).contiguous()
    qt, kt, vt, dot = t(q), t(k), t(v), t(do)
    return (qt, kt, vt, dot), tuple(to64(x) for x in (qt, kt, vt, dot))


def _rel(got, ref, where):
    worst = 0.0
    for idx in np.ndindex(*ref.shape[:2]):
        den = np.abs(ref[idx]).max()
        err = np.abs(got[idx] - ref[idx]).max() / max(den, 1e-30)
        worst = max(worst, err)
        assert err <= TOL, f"{where} slice {idx}: {err:.3e}"
    return worst


CASES = [
    # B, Hq, Hkv, n, d, sigmas, s, causal
    (1, 2, 1, 200, 64, (4.0, 30.0), 8, True),
    (1, 2, 1, 200, 64, (4.0, 30.0), 8, False),
    (2, 4, 2, 333, 128, (1.5, 6.0, 30.0, 200.0), 20, True),
    (1, 4, 2, 333, 128, (1.5, 6.0, 30.0, 200.0), 20, False),
    (1, 2, 2, 300, 128, (3.0, 50.0), 40, False),   # two hash chunks
    (1, 2, 1, 129, 64, (5.0, 80.0), 100, True),    # four hash chunks
    (1, 2, 1, 1, 64, (4.0, 8.0), 5, True),         # n = 1
    (1, 2, 1, 65, 128, (4.0, 8.0), 5, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}s{c[6]}{'c' if c[7] else 'nc'}")
def test_lse_and_gradients_match_oracle(gpu, case):
    B, Hq, Hkv, n, d, sig, s, causal = case
    say(f"backward case {case}")
    (q, k, v, do), (q64, k64, v64, do64) = _dev(B, Hq, Hkv, n, d, 40 + n, gpu)
    ldelta, lu, bins = P.sample_bins(17, sig, s, n, device=gpu)
    delta, u = oracle_hashes(17, sig, s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=causal, delta=ldelta)
    dq, dk, dv = P.attention_bwd(q, k, v, o, do, lse, bins, causal=causal, delta=ldelta)
    torch.cuda.synchronize()
    lse_ref = oracle.plsh_attention_lse(q64, k64, v64, delta, u, causal)
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= 1e-4 * max(1.0, np.abs(lse_ref).max())
    gq, gk, gv = oracle.plsh_attention_grad(q64, k64, v64, do64, delta, u, causal)
    wq = _rel(to64(dq), gq, "dQ")
    wk = _rel(to64(dk), gk, "dK")
    wv = _rel(to64(dv), gv, "dV")
    say(f"  worst rel err dQ {wq:.2e} dK {wk:.2e} dV {wv:.2e}")


LARGE_LOGIT_CASES = [
    # B, Hq, Hkv, n, d, sigmas, s, causal (Q scaled by 16)
    (1, 4, 2, 700, 128, (1.5, 6.0, 40.0, 300.0), 20, True),
    (1, 4, 2, 700, 128, (1.5, 6.0, 40.0, 300.0), 20, False),
    (1, 2, 1, 500, 64, (2.0, 90.0), 40, True),     # two hash chunks
]


def _max_uncounted_exponent(q64, k64, lse, delta, u, causal):
    """Largest (S - LSE) log2(e) over the pairs whose count is 0: above 128
    the backward's exponential of such a pair overflows fp32."""
    B, Hq, n, d = q64.shape
    grp = Hq // k64.shape[1]
    worst = -np.inf
    for b in range(B):
        for h in range(Hq):
            bins = [oracle.bin_values(a, c, n) for a, c in zip(delta[h], u[h])]
            cnt = sum((bb[:, None] == bb[None, :]).astype(np.int32) for bb in bins)
            if causal:
                cnt = np.tril(cnt)
            S = q64[b, h] @ k64[b, h // grp].T / math.sqrt(d)
            x = (S - lse[b, h][:, None]) * math.log2(math.e)
            worst = max(worst, x[cnt == 0].max(initial=-np.inf))
    return worst


@pytest.mark.parametrize("case", LARGE_LOGIT_CASES,
                         ids=lambda c: f"H{c[1]}/{c[2]}n{c[3]}d{c[4]}s{c[6]}{'c' if c[7] else 'nc'}")
def test_large_logits_gradients(gpu, case):
    """Q scaled by 16: the logits spread over hundreds, so pairs whose count
    is 0 have exponents far past fp32's range (checked from the oracle's
    LSE); they must weigh 0, every gradient stays finite and within the
    tolerance of the oracle."""
    B, Hq, Hkv, n, d, sig, s, causal = case
    say(f"backward large logits {case}")
    (q, k, v, do), (q64, k64, v64, do64) = _dev(B, Hq, Hkv, n, d, 90 + n, gpu, scale_q=16.0)
    ldelta, lu, bins = P.sample_bins(23, sig, s, n, device=gpu)
    delta, u = oracle_hashes(23, sig, s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=causal, delta=ldelta)
    dq, dk, dv = P.attention_bwd(q, k, v, o, do, lse, bins, causal=causal, delta=ldelta)
    torch.cuda.synchronize()
    lse_ref = oracle.plsh_attention_lse(q64, k64, v64, delta, u, causal)
    over = _max_uncounted_exponent(q64, k64, lse_ref, delta, u, causal)
    say(f"  largest uncounted exponent {over:.1f}")
    assert over > 128.0, "the case does not reach the overflow it is meant to test"
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    gq, gk, gv = oracle.plsh_attention_grad(q64, k64, v64, do64, delta, u, causal)
    say(f"  worst rel err dQ {_rel(to64(dq), gq, 'dQ'):.2e} dK {_rel(to64(dk), gk, 'dK'):.2e} "
        f"dV {_rel(to64(dv), gv, 'dV'):.2e}")


def _random_cases(count, seed):
    """Seeded random configurations: GQA ratios 1..8, odd n, s across the
    hash-chunk boundaries, log-uniform widths 0.5..600, d 64 and 128,
    causal or not."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        out.append((int(rng.choice([1, 2])), hq, hkv, int(rng.integers(1, 420)), int(rng.choice([64, 128])),
                    tuple(float(x) for x in np.exp(rng.uniform(np.log(0.5), np.log(600.0), size=hq))),
                    int(rng.choice([1, 3, 8, 20, 32, 33, 64, 65, 128])), bool(rng.integers(0, 2)),
                    int(rng.integers(0, 2 ** 32))))
    return out


RANDOM_CASES = _random_cases(16, 4242)


@pytest.mark.parametrize("case", RANDOM_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}s{c[6]}{'c' if c[7] else 'nc'}")
def test_random_configurations_gradients(gpu, case):
    B, Hq, Hkv, n, d, sig, s, causal, seed = case
    say(f"backward random configuration {case}")
    (q, k, v, do), (q64, k64, v64, do64) = _dev(B, Hq, Hkv, n, d, seed % 100000, gpu)
    ldelta, lu, bins = P.sample_bins(seed, sig, s, n, device=gpu)
    delta, u = oracle_hashes(seed, sig, s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=causal, delta=ldelta)
    dq, dk, dv = P.attention_bwd(q, k, v, o, do, lse, bins, causal=causal, delta=ldelta)
    torch.cuda.synchronize()
    gq, gk, gv = oracle.plsh_attention_grad(q64, k64, v64, do64, delta, u, causal)
    say(f"  worst rel err dQ {_rel(to64(dq), gq, 'dQ'):.2e} dK {_rel(to64(dk), gk, 'dK'):.2e} "
        f"dV {_rel(to64(dv), gv, 'dV'):.2e}")


def test_gradients_mid_size_full_compare(gpu):
    B, Hq, Hkv, n, d, s = 1, 4, 2, 1024, 128, 20
    sig = synth.alibi_sigmas(Hq)
    say("backward mid size full compare")
    (q, k, v, do), (q64, k64, v64, do64) = _dev(B, Hq, Hkv, n, d, 77, gpu)
    ldelta, lu, bins = P.sample_bins(5, sig, s, n, device=gpu)
    delta, u = oracle_hashes(5, sig, s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=True, delta=ldelta)
    dq, dk, dv = P.attention_bwd(q, k, v, o, do, lse, bins, causal=True, delta=ldelta)
    torch.cuda.synchronize()
    gq, gk, gv = oracle.plsh_attention_grad(q64, k64, v64, do64, delta, u, True)
    say(f"  worst rel err dQ {_rel(to64(dq), gq, 'dQ'):.2e} dK {_rel(to64(dk), gk, 'dK'):.2e} "
        f"dV {_rel(to64(dv), gv, 'dV'):.2e}")


def _dq_rows(qh, kh, vh, doh, dl, uu, rows, causal):
    """dQ rows from the definition: row r needs only P_r and dP_r."""
    n, d = kh.shape
    bins = [oracle.bin_values(a, b, n) for a, b in zip(dl, uu)]
    out = np.empty((len(rows), d))
    for t, r in enumerate(rows):
        c = np.zeros(n)
        for bb in bins:
            c += bb == bb[r]
        if causal:
            c[r + 1:] = 0
        S = kh @ qh[t] / math.sqrt(d)
        supp = c > 0
        m = S[supp].max()
        W = np.where(supp, c * np.exp(np.where(supp, S - m, 0.0)), 0.0)
        Pr = W / W.sum()
        O = Pr @ vh
        dP = vh @ doh[t]
        dS = Pr * (dP - doh[t] @ O)
        out[t] = dS @ kh / math.sqrt(d)
    return out


def test_gradients_full_size(gpu):
    """Mistral-shaped layer (n = 16384, 32/8 heads, d = 128, s = 20, causal),
    launched as a training step would: dQ on sampled rows from the
    definition; the column identities of dK and dV over every key."""
    W = synth.WORKLOADS["mistral"]
    say("backward full size")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    gen = torch.Generator(device=gpu)
    gen.manual_seed(9)
    do = torch.randn(q.shape, generator=gen, device=gpu, dtype=torch.float32).to(q.dtype)
    ldelta, lu, bins = P.sample_bins(W.hash_seed, W.sigmas, W.s, W.n, device=gpu)
    delta, u = oracle_hashes(W.hash_seed, W.sigmas, W.s, ldelta, lu)
    o, lse = P.attention_lse(q, k, v, bins, causal=W.causal, delta=ldelta)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    P.attention_bwd(q, k, v, o, do, lse, bins, causal=W.causal, delta=ldelta, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any().item(), "gradient not fully written"
    grp = W.heads_q // W.heads_kv
    rng = np.random.default_rng(3)
    for h in range(0, W.heads_q, 4):
        rows = np.unique(np.concatenate([[0, 1, 127, 128, W.n - 1], rng.integers(0, W.n, 10)]))
        ridx = torch.as_tensor(rows, device=gpu)
        ref = _dq_rows(to64(q[0, h, ridx]), to64(k[0, h // grp]), to64(v[0, h // grp]), to64(do[0, h, ridx]),
                       delta[h], u[h], rows, W.causal)
        got = to64(dq[0, h, ridx])
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= TOL, f"dQ head {h}: {err:.3e}"
    # sum over keys of dV = sum over the group's heads and rows of dO; sum of dK = 0
    dv_sum = dv.double().sum(dim=2)[0]                                     # [Hkv, d]
    do_sum = do.double().sum(dim=2)[0].view(W.heads_kv, grp, -1).sum(1)    # [Hkv, d]
    assert (dv_sum - do_sum).abs().max().item() <= 2e-2 * do_sum.abs().max().item()
    dk_sum = dk.double().sum(dim=2)[0]
    dk_scale = dk.double().abs().sum(dim=2)[0]
    assert (dk_sum.abs() <= 2e-2 * dk_scale + 1e-6).all().item()


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4)], ids=["dKdV-on-second-stream", "dQ-on-second-stream"])
def test_gradients_ordered_on_the_callers_stream(gpu, Hq, Hkv):
    """One of the two backward kernels runs on a second stream of the device
    (dK/dV with four or more query heads per KV head, else dQ), forked from
    and joined back to the caller's stream: copies enqueued on the caller's
    (non-default) stream right after the call, with no device-wide
    synchronisation, must see every gradient, bit-identical to a call on the
    default stream.  The outputs are filled with NaN before each call."""
    B, n, d, s = 1, 2048, 128, 20
    sig = synth.alibi_sigmas(Hq)
    say(f"backward ordering on a side stream, Hq={Hq} Hkv={Hkv}")
    (q, k, v, do), _ = _dev(B, Hq, Hkv, n, d, 91, gpu)
    ldelta, lu, bins = P.sample_bins(3, sig, s, n, device=gpu)
    o, lse = P.attention_lse(q, k, v, bins, causal=True, delta=ldelta)
    ref = P.attention_bwd(q, k, v, o, do, lse, bins, causal=True, delta=ldelta)
    torch.cuda.synchronize()
    ref = [t.clone() for t in ref]
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        got = []
        for _ in range(3):
            dq, dk, dv = (torch.full_like(t, float("nan")) for t in ref)
            P.attention_bwd(q, k, v, o, do, lse, bins, causal=True, delta=ldelta, dq=dq, dk=dk, dv=dv, stream=st)
            got.append([t.clone() for t in (dq, dk, dv)])
    st.synchronize()
    for copies in got:
        for g, want in zip(copies, ref):
            assert torch.equal(g, want)
