"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, draws hashes bit-identical to the generator's published
definition (re-derived independently in oracle.sampler), and rejects every
invalid argument before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle.sampler import sample_hashes

P = pytest.importorskip("randomized_positional_lsh_amd")
from randomized_positional_lsh_amd import _binding as B  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plpsh.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(plpsh_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(B.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_status_strings_and_version():
    assert B.status_string(0) == "PLPSH_OK"
    assert B.status_string(3) == "PLPSH_ERR_WORKSPACE_TOO_SMALL"
    assert "UNKNOWN" in B.status_string(99)
    assert "gfx950" in B.version()


@pytest.mark.parametrize("seed", [0, 1, 2 ** 63 + 12345, 2 ** 64 - 1])
def test_host_draw_is_bitwise_the_published_generator(seed):
    sig = [1.189, 2.0, 16.0, 256.0, 1e-3, 1e6]
    d, u = P.draw_hashes(seed, sig, 20)
    d2, u2 = sample_hashes(seed, sig, 20)
    assert np.array_equal(d.view(np.uint64), d2.view(np.uint64))
    assert np.array_equal(u.view(np.uint64), u2.view(np.uint64))
    assert np.all((u >= 0) & (u <= d))


def test_sample_bins_host_only_matches_draw():
    lib = B.raw()
    sig = np.array([3.0, 40.0])
    d = np.empty(2 * 5)
    u = np.empty(2 * 5)
    st = lib.plpsh_sample_bins(7, 2, 5, 100, B._ptr(sig), B._ptr(d), B._ptr(u), None, 0, None)
    assert st == 0
    d2, u2 = P.draw_hashes(7, sig, 5)
    assert np.array_equal(d.reshape(2, 5), d2) and np.array_equal(u.reshape(2, 5), u2)


def test_bins_layout_is_consistent():
    for H, s, n in [(1, 1, 1), (32, 20, 16384), (8, 10, 4097), (3, 128, 129)]:
        L = P.bins_layout(H, s, n)
        assert L["nblk"] == 0
        assert L["starts"] >= 4 * H * s and L["starts"] % 256 == 0
        assert L["plan"] >= L["starts"] + 4 * H * s * (n + 1) and L["plan"] % 256 == 0
        ntile = (n + 127) // 128
        assert L["total"] >= L["plan"] + 32 * H * ntile * s
        assert P.workspace_bytes(H, s, n) == L["total"]


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, batch=1, hq=2, hkv=1, n=64, d=64, dtype=1,
             sigma=np.array([2.0, 4.0]), s=4, seed=0, causal=0, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    sig = np.ascontiguousarray(a["sigma"], dtype=np.float64)
    return B.raw().plpsh_attention_fwd(a["q"], a["k"], a["v"], a["o"], a["batch"], a["hq"], a["hkv"], a["n"],
                                       a["d"], a["dtype"], B._ptr(sig) if a["sigma"] is not None else None,
                                       a["s"], a["seed"], a["causal"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.INVALID_ARGUMENT),
    (dict(o=None), B.INVALID_ARGUMENT),
    (dict(ws=None), B.INVALID_ARGUMENT),
    (dict(batch=-1), B.INVALID_ARGUMENT),
    (dict(n=-5), B.INVALID_ARGUMENT),
    (dict(hq=3, sigma=np.array([1.0, 2.0, 3.0])), B.INVALID_ARGUMENT),   # 3 % 1 == 0 but ok: see next
    (dict(hkv=3), B.INVALID_ARGUMENT),                                    # 2 % 3 != 0
    (dict(hq=0), B.INVALID_ARGUMENT),
    (dict(s=0), B.INVALID_ARGUMENT),
    (dict(s=B.MAX_S + 1), B.INVALID_ARGUMENT),
    (dict(sigma=np.array([2.0, -1.0])), B.INVALID_ARGUMENT),
    (dict(sigma=np.array([2.0, np.inf])), B.INVALID_ARGUMENT),
    (dict(sigma=np.array([0.0, 1.0])), B.INVALID_ARGUMENT),
    (dict(sigma=None), B.INVALID_ARGUMENT),
    (dict(causal=2), B.INVALID_ARGUMENT),
    (dict(dtype=7), B.INVALID_ARGUMENT),
    (dict(d=96), B.UNSUPPORTED),
    (dict(d=0), B.INVALID_ARGUMENT),
    (dict(batch=65535, n=B.MAX_N, hq=1024, hkv=1, sigma=np.full(1024, 2.0)), B.UNSUPPORTED),  # > 2^31 work items
    (dict(n=B.MAX_N + 1), B.UNSUPPORTED),
    (dict(wsb=10), B.WORKSPACE_TOO_SMALL),
    (dict(q=ctypes.c_void_p((1 << 20) + 4)), B.INVALID_ARGUMENT),        # misaligned
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), B.INVALID_ARGUMENT),      # workspace not 256-aligned
])
def test_attention_validation_before_any_hip_call(kw, status):
    if "hq" in kw and kw["hq"] == 3:
        # heads_q = 3 with heads_kv = 1 is valid; make it invalid through sigma length mismatch instead
        kw = dict(hq=3, sigma=np.array([1.0, 2.0, -3.0]))
    assert _attn(**kw) == status


def test_hashes_validation():
    lib = B.raw()
    d = np.array([2.0, 3.0])
    for bad_d, bad_u in [([2.0, 0.0], [0.0, 0.0]), ([2.0, np.nan], [0.0, 0.0]), ([2.0, 3.0], [0.0, 3.5]),
                         ([2.0, 3.0], [-0.1, 0.0]), ([2.0, 3.0], [0.0, np.nan])]:
        dd = np.array(bad_d)
        uu = np.array(bad_u)
        st = lib.plpsh_attention_fwd_hashes(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 64, 1, B._ptr(dd), B._ptr(uu), 2, 0,
                                            FAKE, 1 << 30, None)
        assert st == B.INVALID_ARGUMENT
        st = lib.plpsh_bins_from_hashes(1, 2, 64, B._ptr(dd), B._ptr(uu), FAKE, 1 << 30, None)
        assert st == B.INVALID_ARGUMENT
    uu = np.array([0.0, 3.0])  # u == delta allowed
    st = lib.plpsh_bins_from_hashes(1, 2, 64, B._ptr(d), B._ptr(uu), FAKE, 10, None)
    assert st == B.WORKSPACE_TOO_SMALL


def test_fixed_blocks_validation():
    lib = B.raw()
    i32 = ctypes.POINTER(ctypes.c_int32)
    for bad in ([16, 0], [16, -3], [16, B.MAX_N + 1]):
        bl = np.array(bad, dtype=np.int32)
        st = lib.plpsh_fixed_blocks_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 64, 1, bl.ctypes.data_as(i32), 0,
                                        FAKE, 1 << 30, None)
        assert st == B.INVALID_ARGUMENT, bad
    assert lib.plpsh_fixed_blocks_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 64, 1, None, 0, FAKE, 1 << 30,
                                      None) == B.INVALID_ARGUMENT
    bl = np.array([16, 128], dtype=np.int32)
    st = lib.plpsh_fixed_blocks_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 64, 1, bl.ctypes.data_as(i32), 0, FAKE, 10,
                                    None)
    assert st == B.WORKSPACE_TOO_SMALL


def test_error_functions_validation():
    lib = B.raw()
    dl = np.array([4.0, 9.0])
    uu = np.array([1.0, 0.0])
    # workspace sizes: invalid sizes give 0; products need the scan scratch
    assert lib.plpsh_error_workspace_bytes(0, 2, 0) == 0
    assert lib.plpsh_error_workspace_bytes(100, 0, 0) == 0
    assert lib.plpsh_error_workspace_bytes(100, 2, 1001) == 0
    assert lib.plpsh_error_workspace_bytes(100, 2, 0) > 0
    assert lib.plpsh_error_workspace_bytes(100, 2, 10) > lib.plpsh_error_workspace_bytes(100, 2, 0)
    for sigma, n, s in [(0.0, 64, 2), (float("nan"), 64, 2), (-1.0, 64, 2), (4.0, 0, 2), (4.0, 64, 0),
                        (4.0, B.MAX_N + 1, 2), (4.0, 64, B.MAX_S + 1)]:
        assert lib.plpsh_error_rowmax(sigma, n, s, FAKE, 1 << 30, FAKE, None) == B.INVALID_ARGUMENT
        assert lib.plpsh_error_matvec(sigma, n, s, FAKE, 1 << 30, FAKE, ctypes.c_void_p((1 << 21)), FAKE, 1 << 30,
                                      None) == B.INVALID_ARGUMENT
    assert lib.plpsh_error_rowmax(4.0, 64, 2, FAKE, 10, FAKE, None) == B.WORKSPACE_TOO_SMALL
    assert lib.plpsh_error_matvec(4.0, 64, 2, FAKE, 1 << 30, FAKE, FAKE, FAKE, 1 << 30, None) == B.INVALID_ARGUMENT
    assert lib.plpsh_error_matvec(4.0, 64, 2, FAKE, 1 << 30, FAKE, ctypes.c_void_p(1 << 21), FAKE, 10,
                                  None) == B.WORKSPACE_TOO_SMALL
    out = ctypes.c_double()
    i32 = ctypes.c_int32()
    args = lambda **kw: dict(dict(sigma=4.0, n=64, s=2, d=B._ptr(dl), u=B._ptr(uu), steps=20, tol=1e-10,
                                  ws=FAKE, wsb=1 << 30), **kw)
    call = lambda a: lib.plpsh_error_norms(a["sigma"], a["n"], a["s"], a["d"], a["u"], a["steps"], a["tol"], 0,
                                           a["ws"], a["wsb"], ctypes.byref(out), ctypes.byref(out),
                                           ctypes.byref(i32), ctypes.byref(i32), None)
    bad_u = np.array([5.0, 0.0])
    for kw in [dict(steps=0), dict(steps=1001), dict(tol=0.0), dict(d=None), dict(u=B._ptr(bad_u)),
               dict(ws=None), dict(ws=ctypes.c_void_p((1 << 20) + 8)), dict(sigma=0.0)]:
        assert call(args(**kw)) == B.INVALID_ARGUMENT, kw
    assert call(args(wsb=100)) == B.WORKSPACE_TOO_SMALL


def test_backward_validation():
    lib = B.raw()
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, batch=1, hq=2, hkv=1,
                n=64, d=64, dtype=1, s=4, causal=1, bins=FAKE, binsb=1 << 30, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return lib.plpsh_attention_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                       a["batch"], a["hq"], a["hkv"], a["n"], a["d"], a["dtype"], a["s"],
                                       a["causal"], a["bins"], a["binsb"], None, a["ws"], a["wsb"], None)
    for kw in [dict(lse=None), dict(do=None), dict(dk=None), dict(dv=None), dict(o=None), dict(ws=None),
               dict(ws=ctypes.c_void_p((1 << 20) + 16)), dict(do=ctypes.c_void_p((1 << 20) + 4)), dict(hkv=3),
               dict(s=0), dict(causal=2), dict(bins=None), dict(lse=ctypes.c_void_p((1 << 20) + 2))]:
        assert call(**kw) == B.INVALID_ARGUMENT, kw
    assert call(dtype=0) == B.UNSUPPORTED
    assert call(d=80) == B.UNSUPPORTED
    assert call(wsb=16) == B.WORKSPACE_TOO_SMALL
    assert call(binsb=16) == B.WORKSPACE_TOO_SMALL
    assert call(batch=0) == B.OK and call(n=0) == B.OK  # empty: nothing launched
    assert lib.plpsh_attention_bwd_workspace_bytes(2, 4, 100) >= 2 * 4 * 100 * 4
    assert lib.plpsh_attention_bwd_workspace_bytes(1, 0, 100) == 0
    # forward with normalisers: lse is required
    st = lib.plpsh_attention_fwd_lse(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 1, 64, 64, 1, 4, 1, FAKE, 1 << 30, None, None)
    assert st == B.INVALID_ARGUMENT


def test_draw_validation():
    lib = B.raw()
    sig = np.array([1.0])
    out = np.empty(4)
    assert lib.plpsh_draw_hashes(0, 1, 0, B._ptr(sig), B._ptr(out), B._ptr(out)) == B.INVALID_ARGUMENT
    assert lib.plpsh_draw_hashes(0, 0, 1, B._ptr(sig), B._ptr(out), B._ptr(out)) == B.INVALID_ARGUMENT
    assert lib.plpsh_draw_hashes(0, 1, 1, B._ptr(sig), None, B._ptr(out)) == B.INVALID_ARGUMENT
    assert lib.plpsh_draw_hashes(0, 70000, 1, B._ptr(sig), B._ptr(out), B._ptr(out)) == B.INVALID_ARGUMENT


def test_alibi_validation():
    lib = B.raw()
    sig = np.array([1.0, 2.0])
    assert lib.plpsh_alibi_dense_fwd(FAKE, FAKE, FAKE, None, 1, 2, 1, 64, 64, 1, B._ptr(sig), 0, None) == 1
    assert lib.plpsh_alibi_dense_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 80, 1, B._ptr(sig), 0, None) == 2
    bad = np.array([1.0, -2.0])
    assert lib.plpsh_alibi_dense_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 64, 64, 1, B._ptr(bad), 0, None) == 1


def test_empty_calls_are_noops():
    """batch == 0 or n == 0: valid, nothing launched (no HIP call is made)."""
    assert _attn(batch=0) == B.OK
    assert _attn(n=0, wsb=256) == B.OK
    lib = B.raw()
    sig = np.array([1.0, 2.0])
    assert lib.plpsh_alibi_dense_fwd(FAKE, FAKE, FAKE, FAKE, 0, 2, 1, 64, 64, 1, B._ptr(sig), 0, None) == 0


def test_binding_checks_caller_outputs_before_the_c_abi():
    """The Python wrappers reject an output or gradient tensor whose shape,
    dtype or layout differs from what the kernels write (an fp32 input with
    a bf16 output would otherwise be written past its end), before any call
    into the library."""
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.float32)
    k = torch.zeros((1, 1, 64, 64), dtype=torch.float32)
    bad_outs = [torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16),       # dtype
                torch.zeros((1, 2, 63, 64), dtype=torch.float32),        # shape
                torch.zeros((1, 2, 64, 128), dtype=torch.float32)[..., ::2]]  # not contiguous
    for out in bad_outs:
        with pytest.raises(ValueError):
            P.attention(q, k, k, [2.0, 3.0], 4, out=out)
        with pytest.raises(ValueError):
            P.alibi_dense(q, k, k, [2.0, 3.0], out=out)
        with pytest.raises(ValueError):
            P.attention_hashes(q, k, k, np.full((2, 4), 3.0), np.zeros((2, 4)), out=out)
    qb, kb = q.bfloat16(), k.bfloat16()
    lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    bins = type("FakeBins", (), {"heads": 2, "n": 64, "s": 4})()
    # backward: out, dout and lse are read; dq, dk, dv are written
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb[:, :, :32], qb, lse, bins)
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb.float(), lse, bins)
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb, lse.double(), bins)
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb, lse[:, :1], bins)
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb, lse, bins, dq=torch.zeros_like(kb))
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb, lse, bins, dk=torch.zeros_like(qb))
    with pytest.raises(ValueError):
        P.attention_bwd(qb, kb, kb, qb, qb, lse, bins, dv=torch.zeros_like(kb).float())
    with pytest.raises(ValueError):
        P.attention_lse(qb, kb, kb, bins, lse=lse[:, :, :10])


def test_noalloc_validation_and_limits():
    """The no-allocation entry point validates like plpsh_attention_fwd and
    rejects problems beyond its static array before any HIP call."""
    lib = B.raw()
    sig2 = np.array([2.0, 4.0])

    def call(q=FAKE, o=FAKE, batch=1, hq=2, hkv=1, n=64, d=64, dtype=1, sigma=sig2, s=4, causal=0):
        sg = np.ascontiguousarray(sigma, dtype=np.float64)
        return lib.plpsh_attention_fwd_noalloc(q, FAKE, FAKE, o, batch, hq, hkv, n, d, dtype, B._ptr(sg), s, 0,
                                               causal, None)
    assert call(q=None) == B.INVALID_ARGUMENT
    assert call(s=0) == B.INVALID_ARGUMENT
    assert call(sigma=np.array([2.0, -1.0])) == B.INVALID_ARGUMENT
    assert call(dtype=5) == B.INVALID_ARGUMENT
    assert call(d=96) == B.UNSUPPORTED
    assert call(batch=0) == B.OK and call(n=0) == B.OK          # empty: nothing launched
    # more hashes than the array holds (heads_q * s > 4096)
    assert call(hq=64, hkv=1, sigma=np.full(64, 2.0), s=65) == B.UNSUPPORTED
    # a bin buffer larger than the array (32 heads, s = 32, n = 131072: about 537 MB)
    assert call(hq=32, hkv=8, sigma=np.full(32, 2.0), s=32, n=131072) == B.UNSUPPORTED
    # the 32-head, s = 20, n = 16384 layer fits
    assert P.workspace_bytes(32, 20, 16384) <= 64 << 20
