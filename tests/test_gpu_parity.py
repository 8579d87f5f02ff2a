"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bins are compared bit for bit; attention outputs within the tolerances of
tests/_parity.py.  Small problems are compared element by element over
every output; the full-size workloads are launched exactly as the bench
launches them and compared on sampled rows that the oracle computes one by
one.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from tests._parity import check_bins as _check_bins
from tests._parity import check_slices, oracle_full, oracle_hashes, sample_rows, say, to64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _qkv_dev(B, Hq, Hkv, n, d, dtype, seed, gpu, scale_q=1.0):
    q, k, v = synth.qkv_numpy(B, Hq, Hkv, n, d, dtype, seed, scale_q)
    t = lambda a: torch.from_numpy(a).to(gpu).to(_tdt(dtype)).contiguous()
    return (t(q), t(k), t(v)), (q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))


# ------------------------------------------------------------------ bins --

# Widths within 2^-30 of 1 send the whole launch to the per-hash bin kernel;
# all others take the part kernel, whose start counts have a closed form
# (every position a start below 1 - 2^-30, bins rising by 0 or 1 above
# 1 + 2^-30): the widths next to those bounds are here on both sides.
EDGE_WIDTHS = [0.3, 0.999, 1.0 - 2 ** -29, 1.0 - 2 ** -30, 1.0 + 2 ** -30, 1.0 + 2 ** -29, 1.5, 1.999, 2.0, 2.5,
               7.3, 64.0, 127.5, 1000.0, 1e9]
NEAR_ONE_WIDTHS = [1.0, 1.0 + 2 ** -40, 1.0 - 2 ** -40, 1.0 - 2 ** -31, 1.5, 7.3, 0.3, 1000.0]


@pytest.mark.parametrize("near_one", [False, True], ids=["part_kernel", "per_hash_kernel"])
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4097, 8193, 20000])
def test_bins_bit_exact_edge_widths(gpu, n, near_one):
    widths = (NEAR_ONE_WIDTHS if near_one else EDGE_WIDTHS) + [float(n), 10.0 * n]
    rng = np.random.default_rng(n)
    delta, u = [], []
    for w in widths:
        for uu in (0.0, rng.uniform(0, w), w * (1 - 2 ** -30), w):
            delta.append(w)
            u.append(uu)
    s = 4
    delta = np.array(delta).reshape(-1, s)
    u = np.array(u).reshape(-1, s)
    say(f"bins edge widths n={n} near_one={near_one} hashes={delta.size}")
    bins = P.bins_from_hashes(delta, u, n, device=gpu)
    torch.cuda.synchronize()
    _check_bins(bins, delta, u, n)


@pytest.mark.parametrize("n", [4097, 16384])
def test_bins_bit_exact_wide_hashes(gpu, n):
    """Widths of 32 and more, where the device settles most 32-position words
    from the bins at their two ends and finds a single start by bisection:
    starts on the first and the last position of a word (delta = 32 with
    u = 0 or 1), widths just above 32, offsets at the ends of [0, delta),
    and random wide draws, every block checked against the oracle."""
    rng = np.random.default_rng(77 + n)
    delta, u = [], []
    for w in (32.0, 32.0 + 2 ** -40, 33.3, 64.0, 100.5, 256.0, 1000.0, 4096.0, 5000.25):
        for uu in (0.0, 1.0, 15.5, 31.0, w / 2, w * (1 - 2 ** -30), rng.uniform(0, w), rng.uniform(0, w)):
            delta.append(w)
            u.append(min(uu, w))
    wr = 32.0 + rng.gamma(2.0, 200.0, size=64)
    delta += wr.tolist()
    u += (wr * rng.uniform(size=64)).tolist()
    s = 8
    delta = np.array(delta).reshape(-1, s)
    u = np.array(u).reshape(-1, s)
    say(f"bins wide hashes n={n} hashes={delta.size}")
    bins = P.bins_from_hashes(delta, u, n, device=gpu)
    torch.cuda.synchronize()
    _check_bins(bins, delta, u, n)


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3", "mistral"])
def test_bins_bit_exact_workload_draws(gpu, name):
    W = synth.WORKLOADS[name]
    say(f"bins workload {name}")
    ldelta, lu, bins = P.sample_bins(W.hash_seed, W.sigmas, W.s, W.n, device=gpu)
    torch.cuda.synchronize()
    delta, u = oracle_hashes(W.hash_seed, W.sigmas, W.s, ldelta, lu)
    heads = range(W.heads_q) if W.n <= 4096 else [0, 5, W.heads_q // 2, W.heads_q - 1]
    nblk = bins.nblk.cpu().numpy()
    starts = bins.starts.cpu().numpy()
    for h in heads:
        for i in range(W.s):
            st = oracle.block_starts(delta[h, i], u[h, i], W.n)
            t = h * W.s + i
            assert nblk[t] == st.size
            assert np.array_equal(starts[t, :st.size + 1], np.append(st, W.n))


# ------------------------------------------------------------- attention --

CASES = [
    # B, Hq, Hkv, n, d, dtype, sigmas, s, causal
    (1, 1, 1, 512, 64, "f32", (16.0,), 8, False),          # the tiny workload's shape
    (1, 1, 1, 512, 64, "f32", (16.0,), 8, True),
    (2, 4, 2, 333, 128, "f32", (1.5, 6.0, 30.0, 200.0), 6, True),
    (2, 4, 2, 333, 128, "f32", (1.5, 6.0, 30.0, 200.0), 6, False),
    (1, 4, 4, 1000, 64, "bf16", (1.19, 8.0, 64.0, 512.0), 20, True),
    (1, 4, 4, 1000, 64, "bf16", (1.19, 8.0, 64.0, 512.0), 20, False),
    (2, 6, 2, 777, 128, "bf16", (1.0, 2.0, 4.0, 16.0, 100.0, 300.0), 20, True),
    (1, 2, 1, 777, 128, "bf16", (5.0, 80.0), 32, False),
    (1, 2, 2, 300, 128, "bf16", (3.0, 50.0), 40, True),     # two count chunks
    (1, 2, 2, 300, 64, "bf16", (3.0, 50.0), 100, False),    # four count chunks
    (1, 2, 2, 300, 64, "bf16", (3.0, 50.0), 100, True),
    (1, 2, 1, 257, 128, "bf16", (0.6, 2.0), 128, True),      # s at its maximum; widths under 1
    (1, 2, 1, 200, 64, "f32", (2.5, 40.0), 48, True),        # two count chunks, fp32
    (1, 2, 1, 1, 64, "bf16", (4.0, 8.0), 5, True),           # n = 1
    (1, 2, 1, 65, 128, "bf16", (4.0, 8.0), 5, True),
    (3, 2, 1, 129, 64, "f32", (0.5, 1000.0), 3, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}{c[5]}s{c[7]}{'c' if c[8] else 'nc'}")
def test_attention_matches_oracle_small(gpu, case):
    B, Hq, Hkv, n, d, dtype, sig, s, causal = case
    say(f"attention small case {case}")
    (q, k, v), (q64, k64, v64) = _qkv_dev(B, Hq, Hkv, n, d, dtype, 7 + n, gpu, scale_q=2.0)
    delta, u = oracle_hashes(11, sig, s, *P.draw_hashes(11, sig, s))
    o = P.attention(q, k, v, sig, s, seed=11, causal=causal)
    torch.cuda.synchronize()
    ref = oracle_full(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=str(case))
    say(f"  max err {err:.3e}")


def _random_cases(count, seed):
    """Seeded random configurations: GQA ratios 1..8, odd n, s across the
    hash-chunk boundaries, log-uniform widths 0.5..600, both dtypes and
    head sizes, causal or not, Q scaled by 1, 2 or 4."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        out.append((int(rng.choice([1, 2])), hq, hkv, int(rng.integers(1, 800)), int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f32"])),
                    tuple(float(x) for x in np.exp(rng.uniform(np.log(0.5), np.log(600.0), size=hq))),
                    int(rng.choice([1, 2, 5, 8, 13, 20, 31, 32, 33, 47, 64, 65, 90, 128])),
                    bool(rng.integers(0, 2)), int(rng.integers(0, 2 ** 32)), float(rng.choice([1.0, 2.0, 4.0]))))
    return out


RANDOM_CASES = _random_cases(32, 2026)


@pytest.mark.parametrize("case", RANDOM_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}{c[5]}s{c[7]}{'c' if c[8] else 'nc'}")
def test_random_configurations_match_oracle(gpu, case):
    B, Hq, Hkv, n, d, dtype, sig, s, causal, seed, scale = case
    say(f"random configuration {case}")
    (q, k, v), (q64, k64, v64) = _qkv_dev(B, Hq, Hkv, n, d, dtype, seed % 100000, gpu, scale_q=scale)
    delta, u = oracle_hashes(seed, sig, s, *P.draw_hashes(seed, sig, s))
    o = P.attention(q, k, v, sig, s, seed=seed, causal=causal)
    torch.cuda.synchronize()
    ref = oracle_full(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=str(case))
    say(f"  max err {err:.3e}")


LARGE_LOGIT_CASES = [
    # B, Hq, Hkv, n, d, dtype, sigmas, s, causal (Q scaled by 16)
    (1, 4, 2, 900, 64, "bf16", (1.5, 6.0, 40.0, 300.0), 20, True),
    (1, 4, 2, 900, 64, "bf16", (1.5, 6.0, 40.0, 300.0), 20, False),
    (1, 4, 2, 700, 128, "bf16", (2.0, 12.0, 90.0, 400.0), 20, True),
    (1, 2, 2, 700, 128, "bf16", (2.0, 90.0), 40, False),    # two count chunks
    (1, 2, 1, 500, 128, "f32", (3.0, 60.0), 8, True),
    (1, 2, 1, 500, 64, "f32", (3.0, 60.0), 8, False),
]


@pytest.mark.parametrize("case", LARGE_LOGIT_CASES,
                         ids=lambda c: f"H{c[1]}/{c[2]}n{c[3]}d{c[4]}{c[5]}s{c[7]}{'c' if c[8] else 'nc'}")
def test_large_logits_raise_in_far_tiles(gpu, case):
    """Q scaled by 16, so the logits spread over hundreds and chunks of the
    far tiles raise the running maximum, also on entries whose count is 0
    (a far chunk is masked only when it triggers a raise): every output is
    finite and within the tolerances of the oracle."""
    B, Hq, Hkv, n, d, dtype, sig, s, causal = case
    say(f"large logits {case}")
    (q, k, v), (q64, k64, v64) = _qkv_dev(B, Hq, Hkv, n, d, dtype, 21 + n, gpu, scale_q=16.0)
    delta, u = oracle_hashes(13, sig, s, *P.draw_hashes(13, sig, s))
    o = P.attention(q, k, v, sig, s, seed=13, causal=causal)
    torch.cuda.synchronize()
    ref = oracle_full(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=str(case))
    say(f"  max err {err:.3e}")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_workload_full_compare(gpu, name):
    W = synth.WORKLOADS[name]
    say(f"workload {name} full compare")
    (q, k, v), (q64, k64, v64) = _qkv_dev(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    o = P.attention(q, k, v, W.sigmas, W.s, seed=W.hash_seed, causal=W.causal)
    torch.cuda.synchronize()
    delta, u = oracle.sample_hashes(W.hash_seed, W.sigmas, W.s)
    ref = oracle_full(q64, k64, v64, delta, u, W.causal)
    err = check_slices(to64(o), ref, W.dtype, where=name)
    say(f"  max err {err:.3e}")


@pytest.mark.parametrize("name", ["qwen3", "mistral", "long"])
def test_workload_full_size_sampled_rows(gpu, name):
    W = synth.WORKLOADS[name]
    say(f"workload {name} full size, sampled rows")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    ws = torch.empty(P.workspace_bytes(W.heads_q, W.s, W.n), dtype=torch.uint8, device=gpu)
    o = torch.full_like(q, float("nan"))
    P.attention(q, k, v, W.sigmas, W.s, seed=W.hash_seed, causal=W.causal, out=o, workspace=ws)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item(), "output not fully written"
    delta, u = oracle.sample_hashes(W.hash_seed, W.sigmas, W.s)
    rng = np.random.default_rng(5)
    grp = W.heads_q // W.heads_kv
    heads = range(W.heads_q) if W.n <= 16384 else range(0, W.heads_q, 3)
    nrow = 24 if W.n <= 16384 else 10
    worst = 0.0
    for h in heads:
        rows = sample_rows(W.n, nrow, rng)
        kh = to64(k[0, h // grp])
        vh = to64(v[0, h // grp])
        qh = to64(q[0, h, torch.as_tensor(rows, device=gpu)])
        ref = oracle.plsh_attention_rows(qh, kh, vh, delta[h], u[h], rows, W.causal)
        got = to64(o[0, h, torch.as_tensor(rows, device=gpu)])
        worst = max(worst, check_slices(got[None], ref[None], W.dtype, where=f"{name} head {h}"))
    say(f"  worst rel err {worst:.3e}")


def test_maximum_length(gpu):
    """n at the library's maximum (PLPSH_MAX_N): the bin kernel's word array
    is then at its largest (about 128 KB of LDS per hash), checked bit-exact
    for edge and wide widths, and a causal attention over the whole length is
    checked on sampled rows (first and last rows, tile edges, random rows)."""
    n = P._binding.MAX_N
    say(f"maximum length n={n}: bins")
    delta = np.array([[0.7, 2.5, 37.0, 5000.25]])
    u = np.array([[0.3, 0.0, 36.9, 1234.5]])
    bins = P.bins_from_hashes(delta, u, n, device=gpu)
    torch.cuda.synchronize()
    ntile = (n + 127) // 128
    tiles = sorted({0, 1, 2, ntile - 2, ntile - 1} | set(np.random.default_rng(3).choice(ntile, 40, replace=False).tolist()))
    _check_bins(bins, delta, u, n, tiles)
    say(f"maximum length n={n}: attention")
    B, Hq, Hkv, d, s = 1, 2, 1, 64, 6
    sig = (3.0, 120.0)
    q, k, v = synth.qkv_torch(B, Hq, Hkv, n, d, "bf16", 4242, gpu)
    o = torch.full_like(q, float("nan"))
    P.attention(q, k, v, sig, s, seed=11, causal=True, out=o)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item(), "output not fully written"
    od, ou = oracle.sample_hashes(11, sig, s)
    rng = np.random.default_rng(8)
    kh, vh = to64(k[0, 0]), to64(v[0, 0])
    for h in range(Hq):
        rows = sample_rows(n, 12, rng)
        qh = to64(q[0, h, torch.as_tensor(rows, device=gpu)])
        ref = oracle.plsh_attention_rows(qh, kh, vh, od[h], ou[h], rows, True)
        got = to64(o[0, h, torch.as_tensor(rows, device=gpu)])
        check_slices(got[None], ref[None], "bf16", where=f"n={n} head {h}")


def test_one_block_is_plain_attention(gpu):
    """delta >= n, u = 0: every mask is all ones; T~ = softmax(QK^T/sqrt d) V."""
    (q, k, v), (q64, k64, v64) = _qkv_dev(1, 2, 1, 300, 64, "bf16", 3, gpu, scale_q=3.0)
    for causal in (False, True):
        delta = np.full((2, 3), 300.0)
        u = np.zeros((2, 3))
        o = P.attention_hashes(q, k, v, delta, u, causal=causal)
        torch.cuda.synchronize()
        ref = oracle.plsh_attention(q64, k64, v64, delta, u, causal)
        check_slices(to64(o), ref, "bf16", where=f"one block causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_position_blocks_return_v_exactly(gpu, dtype):
    """delta < 1: each position is its own block, so T~ = V exactly.  In bf16
    the output rounding makes it bit-exact; in fp32 the weight of the only
    key is exp2 of a rounding residue, so the ratio is within 2 ulp."""
    (q, k, v), _ = _qkv_dev(2, 2, 2, 257, 128, dtype, 4, gpu)
    delta = np.array([[0.5, 0.9], [0.25, 0.999]])
    u = delta * 0.5
    for causal in (False, True):
        o = P.attention_hashes(q, k, v, delta, u, causal=causal)
        torch.cuda.synchronize()
        if dtype == "bf16":
            assert torch.equal(o, v), f"causal={causal}"
        else:
            assert torch.all((o - v).abs() <= 2 * 2.0 ** -23 * v.abs()), f"causal={causal}"


def test_fixed_blocks(gpu):
    """s = 1, delta = b, u = 0: deterministic partition into blocks of b."""
    (q, k, v), (q64, k64, v64) = _qkv_dev(1, 2, 2, 500, 128, "bf16", 5, gpu)
    block = np.array([16, 128], dtype=np.int32)
    delta = block.astype(np.float64)[:, None]
    u = np.zeros((2, 1))
    for causal in (False, True):
        o = P.fixed_blocks(q, k, v, block, causal=causal)
        o2 = P.attention_hashes(q, k, v, delta, u, causal=causal)
        torch.cuda.synchronize()
        ref = oracle.plsh_attention(q64, k64, v64, delta, u, causal)
        check_slices(to64(o), ref, "bf16", where=f"fixed blocks causal={causal}")
        assert torch.equal(o, o2), f"fixed blocks vs one deterministic hash, causal={causal}"


LITERAL_CASES = [CASES[i] for i in (0, 3, 4, 5, 6, 8, 9, 10, 11, 13, 14, 15)]


@pytest.mark.parametrize("case", LITERAL_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}{c[5]}s{c[7]}{'c' if c[8] else 'nc'}")
def test_literal_matches_literal_oracle(gpu, case):
    """The per-hash short-attention kernel against the oracle's per-block
    formulation (Theorem 2.2), every output element."""
    B, Hq, Hkv, n, d, dtype, sig, s, causal = case
    say(f"literal small case {case}")
    (q, k, v), (q64, k64, v64) = _qkv_dev(B, Hq, Hkv, n, d, dtype, 7 + n, gpu, scale_q=2.0)
    ldelta, lu, bins = P.sample_bins(11, sig, s, n, device=gpu)
    delta, u = oracle_hashes(11, sig, s, ldelta, lu)
    o = torch.full_like(q, float("nan"))
    P.attention_literal(q, k, v, bins, causal=causal, delta=ldelta, out=o)
    torch.cuda.synchronize()
    ref = oracle.plsh_attention_literal(q64, k64, v64, delta, u, causal)
    err = check_slices(to64(o), ref, dtype, where=f"literal {case}")
    say(f"  max err {err:.3e}")


def test_literal_full_size_sampled_rows(gpu):
    W = synth.WORKLOADS["mistral"]
    say("literal kernel, mistral full size, sampled rows")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    ldelta, lu, bins = P.sample_bins(W.hash_seed, W.sigmas, W.s, W.n, device=gpu)
    delta, u = oracle_hashes(W.hash_seed, W.sigmas, W.s, ldelta, lu)
    o = torch.full_like(q, float("nan"))
    P.attention_literal(q, k, v, bins, causal=W.causal, delta=ldelta, out=o)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item(), "output not fully written"
    rng = np.random.default_rng(9)
    grp = W.heads_q // W.heads_kv
    worst = 0.0
    for h in range(0, W.heads_q, 2):
        rows = sample_rows(W.n, 12, rng)
        kh = to64(k[0, h // grp])
        vh = to64(v[0, h // grp])
        qh = to64(q[0, h, torch.as_tensor(rows, device=gpu)])
        ref = oracle.plsh_attention_rows(qh, kh, vh, delta[h], u[h], rows, W.causal)
        got = to64(o[0, h, torch.as_tensor(rows, device=gpu)])
        worst = max(worst, check_slices(got[None], ref[None], W.dtype, where=f"literal mistral head {h}"))
    say(f"  worst rel err {worst:.3e}")


def test_deterministic_and_canary(gpu):
    W = synth.WORKLOADS["small"]
    (q, k, v), _ = _qkv_dev(1, 8, 8, 1500, 64, "bf16", 6, gpu)
    o1 = torch.full_like(q, float("nan"))
    o2 = torch.full_like(q, float("nan"))
    P.attention(q, k, v, W.sigmas, 10, seed=3, causal=False, out=o1)
    P.attention(q, k, v, W.sigmas, 10, seed=3, causal=False, out=o2)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any().item()
    assert torch.equal(o1, o2)


def test_repeated_launches_across_sizes_and_streams(gpu):
    """Launches of different sizes and kinds in a row, and spread over two
    streams, reproduce the results of launches made one at a time."""
    W = synth.WORKLOADS["small"]
    shapes = [(1, 8, 8, 1500, 64), (2, 4, 2, 200, 64), (1, 8, 8, 1500, 64), (1, 2, 1, 1, 64), (1, 4, 4, 9000, 64)]
    data = [_qkv_dev(*sh, "bf16", 20 + i, gpu)[0] for i, sh in enumerate(shapes)]
    sig = [np.asarray(W.sigmas[:sh[1]]) for sh in shapes]
    ref = []
    for (q, k, v), sg in zip(data, sig):
        ref.append(P.attention(q, k, v, sg, 10, seed=3, causal=True))
        torch.cuda.synchronize()
    ref.append(P.alibi_dense(*data[1], sig[1], causal=False))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        outs = []
        for i, ((q, k, v), sg) in enumerate(zip(data, sig)):
            st = streams[(i + rep) % 2]
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(P.attention(q, k, v, sg, 10, seed=3, causal=True, stream=st))
        with torch.cuda.stream(streams[rep % 2]):
            outs.append(P.alibi_dense(*data[1], sig[1], causal=False, stream=streams[rep % 2]))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"launch {i}, repetition {rep}"


def test_empty_inputs(gpu):
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device=gpu)
    o = P.attention(q, q[:, :1], q[:, :1], [2.0, 3.0], 4, causal=True)
    assert o.shape == q.shape
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=gpu)
    o = P.attention(q, q[:, :1], q[:, :1], [2.0, 3.0], 4, causal=True)
    assert o.shape == q.shape


def test_workspace_too_small_on_device(gpu):
    (q, k, v), _ = _qkv_dev(1, 1, 1, 128, 64, "bf16", 1, gpu)
    ws = torch.empty(64, dtype=torch.uint8, device=gpu)
    with pytest.raises(P.PlpshError):
        P.attention(q, k, v, [4.0], 4, workspace=ws)


# --------------------------------------------------------- dense ALiBi ----

@pytest.mark.parametrize("case", [
    (1, 1, 1, 512, 64, "f32", (16.0,), False),
    (1, 1, 1, 512, 64, "f32", (16.0,), True),
    (2, 4, 2, 333, 128, "f32", (1.5, 6.0, 30.0, 200.0), True),
    (1, 4, 2, 1000, 128, "bf16", (1.19, 8.0, 64.0, 256.0), True),
    (1, 4, 4, 700, 64, "bf16", (2.0, 8.0, 64.0, 1e4), False),
])
def test_alibi_dense_matches_oracle(gpu, case):
    B, Hq, Hkv, n, d, dtype, sig, causal = case
    say(f"alibi dense {case}")
    (q, k, v), (q64, k64, v64) = _qkv_dev(B, Hq, Hkv, n, d, dtype, 9 + n, gpu, scale_q=2.0)
    o = P.alibi_dense(q, k, v, sig, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.alibi_attention(q64, k64, v64, sig, causal)
    check_slices(to64(o), ref, dtype, where=f"alibi {case}")


def test_alibi_dense_full_size_sampled(gpu):
    W = synth.WORKLOADS["mistral"]
    say("alibi dense mistral shape, sampled rows")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    o = P.alibi_dense(q, k, v, W.sigmas, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for h in (0, 13, 31):
        rows = sample_rows(W.n, 8, rng)
        kh = to64(k[0, h // 4])
        vh = to64(v[0, h // 4])
        qh = to64(q[0, h, torch.as_tensor(rows, device=gpu)])
        ref = oracle.alibi_attention_rows(qh, kh, vh, W.sigmas[h], rows, True)
        got = to64(o[0, h, torch.as_tensor(rows, device=gpu)])
        check_slices(got[None], ref[None], "bf16", where=f"alibi mistral head {h}")
