"""The one-launch forward: the attention kernel evaluates the bins of its own
query tiles from (delta, u) and its batch-0 workgroups write the bin buffer.

For every width whose start count has a closed form (none within 2^-30 of
1), plpsh_attention_fwd[_hashes] takes this path.  Checked here:
  * the bin buffer it writes equals the oracle's block counts, block starts
    and plan records bit for bit (the bin kernel's contract);
  * its output equals the two-launch path (the bin kernel, then the
    attention kernel reading that buffer) bit for bit, so every parity
    result of the two-launch path carries over;
  * widths within 2^-30 of 1 still take the two-launch path, correctly.
Edge widths are those of the bin-kernel tests: both sides of 1 +- 2^-30,
widths under 1 (every position a block), wide and one-block widths, and
offsets at both ends of [0, delta].
"""

import numpy as np
import pytest

import synth
from tests._parity import check_bins, check_slices, oracle_full, say, to64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")

CLOSED_FORM_WIDTHS = [0.3, 0.999, 1.0 - 2 ** -29, 1.0 - 2 ** -30, 1.0 + 2 ** -30, 1.0 + 2 ** -29, 1.5, 1.999, 2.0,
                      2.5, 7.3, 31.9, 32.0, 33.3, 64.0, 127.5, 1000.0, 1e9]
NEAR_ONE_WIDTHS = [1.0, 1.0 + 2 ** -40, 1.0 - 2 ** -40, 1.0 - 2 ** -31, 1.5, 7.3, 0.3, 1000.0]


def _edge_hashes(widths, n, s, seed):
    rng = np.random.default_rng(seed)
    delta, u = [], []
    # one-block widths n and 10 n (n = 1 would be a width within 2^-30 of 1)
    for w in widths + [x for x in (float(n), 10.0 * n) if abs(x - 1.0) >= 2 ** -30]:
        for uu in (0.0, rng.uniform(0, w), w * (1 - 2 ** -30), w):
            delta.append(w)
            u.append(uu)
    pad = (-len(delta)) % s
    delta += [3.0] * pad
    u += [1.0] * pad
    return np.array(delta).reshape(-1, s), np.array(u).reshape(-1, s)


def _qkv(B, Hq, Hkv, n, d, dtype, seed, gpu):
    q, k, v = synth.qkv_numpy(B, Hq, Hkv, n, d, dtype, seed, 2.0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda a: torch.from_numpy(a).to(gpu).to(tdt).contiguous()
    return (t(q), t(k), t(v)), (q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))


def _one_launch(q, k, v, delta, u, causal):
    H, s = delta.shape
    ws = torch.empty(P.workspace_bytes(H, s, q.shape[2]), dtype=torch.uint8, device=q.device)
    o = P.attention_hashes(q, k, v, delta, u, causal=causal, workspace=ws)
    return o, P.Bins(ws, H, s, q.shape[2])


def _two_launch(q, k, v, delta, u, causal):
    bins = P.bins_from_hashes(delta, u, q.shape[2], device=q.device)
    return P.attention_from_bins(q, k, v, bins, causal=causal, delta=delta)


@pytest.mark.parametrize("causal", [False, True], ids=["nc", "c"])
@pytest.mark.parametrize("n", [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 1000, 4097, 8193, 20000])
def test_edge_widths_bin_buffer_and_output(gpu, n, causal):
    s = 4
    delta, u = _edge_hashes(CLOSED_FORM_WIDTHS, n, s, n)
    H = delta.shape[0]
    say(f"in-kernel plan, edge widths n={n} causal={causal} heads={H}")
    (q, k, v), _ = _qkv(1, H, 1, n, 64, "bf16", 5 + n, gpu)
    o1, bins = _one_launch(q, k, v, delta, u, causal)
    o2 = _two_launch(q, k, v, delta, u, causal)
    torch.cuda.synchronize()
    check_bins(bins, delta, u, n)
    assert torch.equal(o1, o2), "one-launch output differs from the two-launch path"


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, n, d, dtype, s, causal
    (2, 4, 2, 333, 128, "f32", 6, True),
    (3, 2, 1, 129, 64, "f32", 3, False),
    (2, 6, 2, 777, 128, "bf16", 20, True),
    (1, 2, 2, 300, 128, "bf16", 40, True),      # two count chunks
    (1, 2, 2, 300, 64, "bf16", 100, False),     # four count chunks
    (1, 2, 1, 257, 128, "bf16", 128, True),     # s at its maximum
    (1, 3, 1, 1500, 64, "bf16", 64, False),
], ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}n{c[3]}d{c[4]}{c[5]}s{c[6]}{'c' if c[7] else 'nc'}")
def test_random_draws_match_two_launch_and_oracle(gpu, case):
    B, Hq, Hkv, n, d, dtype, s, causal = case
    rng = np.random.default_rng(n + s)
    sig = rng.choice([0.7, 1.3, 4.0, 30.0, 250.0], size=Hq)
    delta = rng.gamma(2.0, 1.0, size=(Hq, s)) * sig[:, None]
    u = delta * rng.uniform(size=(Hq, s))
    say(f"in-kernel plan, random draws {case}")
    (q, k, v), (q64, k64, v64) = _qkv(B, Hq, Hkv, n, d, dtype, 9 + n, gpu)
    o1, bins = _one_launch(q, k, v, delta, u, causal)
    o2 = _two_launch(q, k, v, delta, u, causal)
    torch.cuda.synchronize()
    check_bins(bins, delta, u, n)
    assert torch.equal(o1, o2), "one-launch output differs from the two-launch path"
    err = check_slices(to64(o1), oracle_full(q64, k64, v64, delta, u, causal), dtype, where=str(case))
    say(f"  max err {err:.3e}")


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3", "mistral"])
def test_workload_draws_match_two_launch(gpu, name):
    """The workloads as the bench runs them: plpsh_attention_fwd (seed) in one
    launch against plpsh_sample_bins + plpsh_attention_fwd_bins; outputs and
    the written parts of the bin buffer identical."""
    W = synth.WORKLOADS[name]
    say(f"in-kernel plan, workload {name}")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, gpu)
    ws = torch.empty(P.workspace_bytes(W.heads_q, W.s, W.n), dtype=torch.uint8, device=gpu)
    o1 = P.attention(q, k, v, W.sigmas, W.s, seed=W.hash_seed, causal=W.causal, workspace=ws)
    delta, u, bins = P.sample_bins(W.hash_seed, W.sigmas, W.s, W.n, device=gpu)
    o2 = P.attention_from_bins(q, k, v, bins, causal=W.causal, delta=delta)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    b1 = P.Bins(ws, W.heads_q, W.s, W.n)
    nb = bins.nblk.cpu().numpy()
    assert np.array_equal(b1.nblk.cpu().numpy(), nb)
    s1, s2 = b1.starts.cpu().numpy(), bins.starts.cpu().numpy()
    for t in range(nb.size):
        assert np.array_equal(s1[t, :nb[t] + 1], s2[t, :nb[t] + 1]), t
    assert torch.equal(b1.plan, bins.plan)


@pytest.mark.parametrize("causal", [False, True], ids=["nc", "c"])
@pytest.mark.parametrize("n", [65, 1000, 4097])
def test_near_one_widths_take_the_bin_kernel(gpu, n, causal):
    s = 4
    delta, u = _edge_hashes(NEAR_ONE_WIDTHS, n, s, 3 * n)
    H = delta.shape[0]
    say(f"near-one widths n={n} causal={causal} heads={H}")
    (q, k, v), (q64, k64, v64) = _qkv(1, H, 1, n, 64, "bf16", 17 + n, gpu)
    o1, bins = _one_launch(q, k, v, delta, u, causal)
    o2 = _two_launch(q, k, v, delta, u, causal)
    torch.cuda.synchronize()
    check_bins(bins, delta, u, n)
    assert torch.equal(o1, o2)
    if n <= 1000:
        err = check_slices(to64(o1), oracle_full(q64, k64, v64, delta, u, causal), "bf16", where=f"n={n}")
        say(f"  max err {err:.3e}")


@pytest.mark.parametrize("s", [1, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["nc", "c"])
def test_plan_task_wave_boundaries(gpu, s, causal):
    """The plan's 4 s flag tasks and 4 s bound tasks fill whole waves (64
    tasks each, a second pass past 256): hash counts on both sides of every
    wave boundary (4 s = 64, 128, 192, 256) and of the second pass give the
    bin buffer bit for bit and the two-launch output."""
    n = 700
    rng = np.random.default_rng(1000 + s)
    H = 2
    sig = np.array([3.0, 90.0])
    delta = rng.gamma(2.0, 1.0, size=(H, s)) * sig[:, None]
    delta = np.where(np.abs(delta - 1.0) < 2 ** -29, 1.5, delta)
    u = delta * rng.uniform(size=(H, s))
    say(f"plan task boundaries s={s} causal={causal}")
    (q, k, v), (q64, k64, v64) = _qkv(1, H, 1, n, 64, "bf16", 31 + s, gpu)
    o1, bins = _one_launch(q, k, v, delta, u, causal)
    o2 = _two_launch(q, k, v, delta, u, causal)
    torch.cuda.synchronize()
    check_bins(bins, delta, u, n)
    assert torch.equal(o1, o2), "one-launch output differs from the two-launch path"
    if s in (17, 65):
        err = check_slices(to64(o1), oracle_full(q64, k64, v64, delta, u, causal), "bf16", where=f"s={s}")
        say(f"  max err {err:.3e}")
