"""plpsh_attention_fwd_noalloc (bin buffer in the library's static device
array) against plpsh_attention_fwd (caller's workspace), through the C ABI:
the same kernels on the same bins, so the outputs must be bit-identical.
Two calls in a row share the array; the second is smaller than the first, so
it runs on what the first left behind."""

import ctypes

import numpy as np
import pytest

import synth
from tests._parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
P = pytest.importorskip("randomized_positional_lsh_amd")
from randomized_positional_lsh_amd import _binding as B  # noqa: E402


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def _reference(lib, q, k, v, sig, s, seed, causal, stream):
    Bt, Hq, n, d = q.shape
    Hkv = k.shape[1]
    o = torch.full_like(q, float("nan"))
    ws = torch.empty(int(lib.plpsh_workspace_bytes(Hq, s, n)), dtype=torch.uint8, device=q.device)
    st = lib.plpsh_attention_fwd(_vp(q), _vp(k), _vp(v), _vp(o), Bt, Hq, Hkv, n, d, B._torch_dtype_code(q),
                                 B._ptr(sig), s, ctypes.c_uint64(seed), int(causal), _vp(ws), ws.numel(), stream)
    assert st == B.OK, B.status_string(st)
    return o


def _noalloc(lib, q, k, v, sig, s, seed, causal, stream):
    Bt, Hq, n, d = q.shape
    Hkv = k.shape[1]
    o = torch.full_like(q, float("nan"))
    st = lib.plpsh_attention_fwd_noalloc(_vp(q), _vp(k), _vp(v), _vp(o), Bt, Hq, Hkv, n, d, B._torch_dtype_code(q),
                                         B._ptr(sig), s, ctypes.c_uint64(seed), int(causal), stream)
    assert st == B.OK, B.status_string(st)
    return o


def test_noalloc_matches_workspace_entry_point(gpu):
    lib = B.raw()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [
        # the 32-head layer at n = 16384 (the array's design size), then a smaller fp32 problem
        (synth.WORKLOADS["mistral"], "bf16"),
        (synth.Workload("small-f32", 2, 4, 2, 1000, 64, "f32", (1.5, 6.0, 40.0, 300.0), 8, False, 5, 77), "f32"),
    ]
    for W, dtype in cases:
        say(f"noalloc vs workspace entry point: {W.name} B={W.batch} Hq={W.heads_q} n={W.n} s={W.s} {dtype}")
        q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, dtype, W.data_seed, gpu)
        sig = np.ascontiguousarray(W.sigmas, dtype=np.float64)
        got = _noalloc(lib, q, k, v, sig, W.s, W.hash_seed, W.causal, stream)
        want = _reference(lib, q, k, v, sig, W.s, W.hash_seed, W.causal, stream)
        torch.cuda.synchronize()
        assert not torch.isnan(got).any().item(), "output not fully written"
        assert torch.equal(got, want), f"{W.name}: outputs differ"
        del q, k, v, got, want
    # beyond the array: rejected on the host, nothing launched
    W = synth.WORKLOADS["long"]
    sig = np.ascontiguousarray(W.sigmas, dtype=np.float64)
    q = torch.empty((1, W.heads_q, 8, W.head_dim), dtype=torch.bfloat16, device=gpu)
    st = lib.plpsh_attention_fwd_noalloc(_vp(q), _vp(q), _vp(q), _vp(q), 1, W.heads_q, W.heads_kv, W.n, W.head_dim,
                                         1, B._ptr(sig), W.s, ctypes.c_uint64(0), 1, stream)
    assert st == B.UNSUPPORTED
