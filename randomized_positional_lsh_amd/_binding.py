"""ctypes binding of libplpsh (C ABI in include/plpsh.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libplpsh.so.  PyTorch supplies device memory and the stream.
If the library has not been built the import fails loudly; there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PLPSH_LIBRARY names another build of the same library (the host-sanitizer
# build of sanitize.py); by default the in-tree libplpsh.so is loaded
LIB_PATH = os.environ.get("PLPSH_LIBRARY") or os.path.join(_HERE, "libplpsh.so")

OK = 0
INVALID_ARGUMENT = 1
UNSUPPORTED = 2
WORKSPACE_TOO_SMALL = 3
HIP_ERROR = 4
DTYPE_F32 = 0
DTYPE_BF16 = 1
MAX_S = 128
MAX_N = 524288
PLAN_TILE = 128

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python randomized_positional_lsh_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")

# torch is loaded first so that libplpsh binds to the HIP runtime torch has
# already mapped (same soname) instead of mapping a second copy: a process
# with two HIP runtimes can find no device in the one initialised second.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_c_int = ctypes.c_int32
_c_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_dp = ctypes.POINTER(ctypes.c_double)
_szp = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "plpsh_status_string": (ctypes.c_char_p, [_c_int]),
    "plpsh_version": (ctypes.c_char_p, []),
    "plpsh_last_hip_error": (ctypes.c_char_p, []),
    "plpsh_draw_hashes": (_c_int, [ctypes.c_uint64, _c_int, _c_int, _dp, _dp, _dp]),
    "plpsh_bins_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "plpsh_bins_layout": (_c_int, [_c_int, _c_int, _c_int, _szp, _szp, _szp]),
    "plpsh_sample_bins": (_c_int, [ctypes.c_uint64, _c_int, _c_int, _c_int, _dp, _dp, _dp, _vp, _c_sz, _vp]),
    "plpsh_bins_from_hashes": (_c_int, [_c_int, _c_int, _c_int, _dp, _dp, _vp, _c_sz, _vp]),
    "plpsh_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "plpsh_attention_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _dp, _c_int, ctypes.c_uint64, _c_int, _vp, _c_sz, _vp]),
    "plpsh_attention_fwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _dp, _c_int, ctypes.c_uint64, _c_int, _vp]),
    "plpsh_attention_fwd_hashes": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _dp, _dp, _c_int, _c_int, _vp, _c_sz, _vp]),
    "plpsh_attention_fwd_bins": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _vp, _c_sz, _dp, _vp]),
    "plpsh_attention_fwd_literal": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _vp, _c_sz, _dp, _vp]),
    "plpsh_attention_fwd_lse": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _vp, _c_sz, _dp, _vp]),
    "plpsh_attention_bwd_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "plpsh_attention_bwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _c_int, _c_int, _c_int, _vp, _c_sz, _dp, _vp, _c_sz, _vp]),
    "plpsh_error_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "plpsh_error_rowmax": (_c_int, [ctypes.c_double, _c_int, _c_int, _vp, _c_sz, _vp, _vp]),
    "plpsh_error_matvec": (_c_int, [ctypes.c_double, _c_int, _c_int, _vp, _c_sz, _vp, _vp, _vp, _c_sz, _vp]),
    "plpsh_error_norms": (_c_int, [ctypes.c_double, _c_int, _c_int, _dp, _dp, _c_int, ctypes.c_double,
                                   ctypes.c_uint64, _vp, _c_sz, _dp, _dp, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32), _vp]),
    "plpsh_fixed_blocks_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        ctypes.POINTER(ctypes.c_int32), _c_int, _vp, _c_sz, _vp]),
    "plpsh_alibi_dense_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _dp, _c_int, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class PlpshError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)}"
        if status == HIP_ERROR:
            msg += f" [{_lib.plpsh_last_hip_error().decode()}]"
        super().__init__(msg)


def status_string(status: int) -> str:
    return _lib.plpsh_status_string(int(status)).decode()


def version() -> str:
    return _lib.plpsh_version().decode()


def raw():
    """The ctypes library handle (for tests of the C ABI itself)."""
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(st: int, where: str):
    if st != OK:
        raise PlpshError(st, where)


def draw_hashes(seed: int, sigma, s: int) -> tuple[np.ndarray, np.ndarray]:
    """Host draw of (delta, u), each float64 [H, s] (plpsh_draw_hashes)."""
    sig = _f64(sigma).reshape(-1)
    H = sig.size
    delta = np.empty((H, s))
    u = np.empty((H, s))
    _check(_lib.plpsh_draw_hashes(ctypes.c_uint64(seed & (2 ** 64 - 1)), H, s, _ptr(sig), _ptr(delta), _ptr(u)),
           "plpsh_draw_hashes")
    return delta, u


def bins_layout(heads: int, s: int, n: int) -> dict:
    a, b, c = (ctypes.c_size_t() for _ in range(3))
    _check(_lib.plpsh_bins_layout(heads, s, n, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "plpsh_bins_layout")
    return {"nblk": a.value, "starts": b.value, "plan": c.value, "total": _lib.plpsh_bins_bytes(heads, s, n)}


def workspace_bytes(heads_q: int, s: int, n: int) -> int:
    return int(_lib.plpsh_workspace_bytes(heads_q, s, n))


def _torch_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _on_stream(stream):
    """Context in which tensors are allocated for work enqueued on `stream`:
    the caching allocator then hands their memory to other work only in that
    stream's order, never while the library's kernels may still use it."""
    import torch
    return torch.cuda.stream(_torch_stream(stream))


def _check_like(t, like, name, dtype=None, shape=None):
    """A caller-supplied output or gradient must match what the kernels write:
    the shape, dtype and device of `like` (or those given), contiguous."""
    want_shape = tuple(like.shape) if shape is None else tuple(shape)
    want_dtype = like.dtype if dtype is None else dtype
    if tuple(t.shape) != want_shape:
        raise ValueError(f"{name} must have shape {want_shape}, not {tuple(t.shape)}")
    if t.dtype != want_dtype:
        raise ValueError(f"{name} must be {want_dtype}, not {t.dtype}")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out_like(out, like, name="out", stream=None):
    import torch
    if out is None:
        with _on_stream(stream):
            return torch.empty_like(like)
    return _check_like(out, like, name)


def _torch_dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


class Bins:
    """Views of a device bin buffer (layout of plpsh.h)."""

    def __init__(self, buf, heads: int, s: int, n: int):
        import torch
        L = bins_layout(heads, s, n)
        self.buffer, self.heads, self.s, self.n = buf, heads, s, n
        hs = heads * s
        b8 = buf.view(torch.uint8)
        self.nblk = b8[L["nblk"]:L["nblk"] + 4 * hs].view(torch.int32)
        self.starts = b8[L["starts"]:L["starts"] + 4 * hs * (n + 1)].view(torch.int32).view(hs, n + 1)
        ntile = (n + PLAN_TILE - 1) // PLAN_TILE
        self.plan = b8[L["plan"]:L["plan"] + 32 * heads * ntile * s].view(torch.int32).view(heads, ntile, s, 8)


def _bins_buffer(heads, s, n, device, stream=None):
    import torch
    nbytes = bins_layout(heads, s, n)["total"]
    with _on_stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sample_bins(seed: int, sigma, s: int, n: int, device="cuda", stream=None, buffer=None, delta=None, u=None):
    """Draw hashes and compute their blocks on the device.  Returns
    (delta, u, Bins) with delta/u float64 numpy [H, s].  ``buffer`` (device
    uint8 tensor) and ``delta``/``u`` (float64 [H, s]) may be supplied to
    reuse storage."""
    sig = _f64(sigma).reshape(-1)
    H = sig.size
    delta = np.empty((H, s)) if delta is None else delta
    u = np.empty((H, s)) if u is None else u
    buf = _bins_buffer(H, s, n, device, stream) if buffer is None else buffer
    _check(_lib.plpsh_sample_bins(ctypes.c_uint64(seed & (2 ** 64 - 1)), H, s, n, _ptr(sig), _ptr(delta), _ptr(u),
                                  ctypes.c_void_p(buf.data_ptr()), buf.numel(), _stream(stream)),
           "plpsh_sample_bins")
    return delta, u, Bins(buf, H, s, n)


def bins_from_hashes(delta, u, n: int, device="cuda", stream=None) -> Bins:
    d = _f64(delta)
    uu = _f64(u)
    H, s = d.shape
    buf = _bins_buffer(H, s, n, device, stream)
    _check(_lib.plpsh_bins_from_hashes(H, s, n, _ptr(d), _ptr(uu), ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                       _stream(stream)), "plpsh_bins_from_hashes")
    return Bins(buf, H, s, n)


def _qkv_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, n, head_dim]")
    B, Hq, n, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != n or k.shape[3] != d:
        raise ValueError("k and v must be [batch, heads_kv, n, head_dim] matching q")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    return B, Hq, k.shape[1], n, d


def _workspace(workspace, heads_q, s, n, device, stream=None):
    import torch
    need = workspace_bytes(heads_q, s, n)
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace


def attention(q, k, v, sigma, s: int, seed: int = 0, causal: bool = False, out=None, workspace=None,
              stream=None):
    """Positional-LSH attention (plpsh_attention_fwd)."""
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    sig = _f64(sigma).reshape(-1)
    if sig.size != Hq:
        raise ValueError("sigma must have one entry per query head")
    out = _out_like(out, q, stream=stream)
    ws = _workspace(workspace, Hq, s, n, q.device, stream)
    st = _lib.plpsh_attention_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, n, d,
                                  _torch_dtype_code(q), _ptr(sig), s, ctypes.c_uint64(seed & (2 ** 64 - 1)),
                                  int(bool(causal)), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "plpsh_attention_fwd")
    return out


def attention_noalloc(q, k, v, sigma, s: int, seed: int = 0, causal: bool = False, out=None, stream=None):
    """plpsh_attention_fwd with the bin buffer in the library's static device
    array (plpsh_attention_fwd_noalloc): no workspace, no allocation inside
    the call (`out` is allocated here only when not supplied)."""
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    sig = _f64(sigma).reshape(-1)
    if sig.size != Hq:
        raise ValueError("sigma must have one entry per query head")
    out = _out_like(out, q, stream=stream)
    st = _lib.plpsh_attention_fwd_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                          ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv,
                                          n, d, _torch_dtype_code(q), _ptr(sig), s,
                                          ctypes.c_uint64(seed & (2 ** 64 - 1)), int(bool(causal)), _stream(stream))
    _check(st, "plpsh_attention_fwd_noalloc")
    return out


def attention_hashes(q, k, v, delta, u, causal: bool = False, out=None, workspace=None, stream=None):
    """Positional-LSH attention with explicit hashes (plpsh_attention_fwd_hashes)."""
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    dl = _f64(delta)
    uu = _f64(u)
    if dl.ndim != 2 or dl.shape[0] != Hq or uu.shape != dl.shape:
        raise ValueError("delta and u must be [heads_q, s]")
    s = dl.shape[1]
    out = _out_like(out, q, stream=stream)
    ws = _workspace(workspace, Hq, s, n, q.device, stream)
    st = _lib.plpsh_attention_fwd_hashes(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                         ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv,
                                         n, d, _torch_dtype_code(q), _ptr(dl), _ptr(uu), s, int(bool(causal)),
                                         ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "plpsh_attention_fwd_hashes")
    return out


def fixed_blocks(q, k, v, block, causal: bool = False, out=None, workspace=None, stream=None):
    """The fixed-blocks baseline: blocks of block[h] positions per query head
    (plpsh_fixed_blocks_fwd)."""
    import numpy as np
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    bl = np.ascontiguousarray(np.broadcast_to(np.asarray(block, dtype=np.int32), (Hq,)))
    out = _out_like(out, q, stream=stream)
    ws = _workspace(workspace, Hq, 1, n, q.device, stream)
    st = _lib.plpsh_fixed_blocks_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                     ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, n, d,
                                     _torch_dtype_code(q), bl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     int(bool(causal)), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "plpsh_fixed_blocks_fwd")
    return out


def _on_bins(fn, name, q, k, v, bins, causal, delta, out, stream):
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    if bins.heads != Hq or bins.n != n:
        raise ValueError("bins were computed for other sizes")
    dl = None if delta is None else _f64(delta)
    out = _out_like(out, q, stream=stream)
    st = fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, n, d, _torch_dtype_code(q), bins.s, int(bool(causal)),
            ctypes.c_void_p(bins.buffer.data_ptr()), bins.buffer.numel(), None if dl is None else _ptr(dl),
            _stream(stream))
    _check(st, name)
    return out


def attention_from_bins(q, k, v, bins: "Bins", causal: bool = False, delta=None, out=None, stream=None):
    """The attention step on a computed bin buffer (plpsh_attention_fwd_bins)."""
    return _on_bins(_lib.plpsh_attention_fwd_bins, "plpsh_attention_fwd_bins", q, k, v, bins, causal, delta, out,
                    stream)


def attention_literal(q, k, v, bins: "Bins", causal: bool = False, delta=None, out=None, stream=None):
    """The same result as one short attention per hash over its blocks
    (plpsh_attention_fwd_literal)."""
    return _on_bins(_lib.plpsh_attention_fwd_literal, "plpsh_attention_fwd_literal", q, k, v, bins, causal, delta,
                    out, stream)


def attention_lse(q, k, v, bins: "Bins", causal: bool = False, delta=None, out=None, lse=None, stream=None):
    """Forward on a bin buffer that also returns each row's log-normaliser
    (plpsh_attention_fwd_lse): (out, lse) with lse float32 [B, Hq, n]."""
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    if bins.heads != Hq or bins.n != n:
        raise ValueError("bins were computed for other sizes")
    dl = None if delta is None else _f64(delta)
    if lse is not None:
        _check_like(lse, q, "lse", dtype=torch.float32, shape=(B, Hq, n))
    out = _out_like(out, q, stream=stream)
    if lse is None:
        with _on_stream(stream):
            lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    else:
        _check_like(lse, q, "lse", dtype=torch.float32, shape=(B, Hq, n))
    st = _lib.plpsh_attention_fwd_lse(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, n, d, _torch_dtype_code(q), bins.s,
                                      int(bool(causal)), ctypes.c_void_p(bins.buffer.data_ptr()), bins.buffer.numel(),
                                      None if dl is None else _ptr(dl), _stream(stream))
    _check(st, "plpsh_attention_fwd_lse")
    return out, lse


def attention_bwd(q, k, v, out, dout, lse, bins: "Bins", causal: bool = False, delta=None, dq=None, dk=None,
                  dv=None, workspace=None, stream=None):
    """(dq, dk, dv) of sum(dout * T~) (plpsh_attention_bwd); bf16 only."""
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    if bins.heads != Hq or bins.n != n:
        raise ValueError("bins were computed for other sizes")
    dl = None if delta is None else _f64(delta)
    _check_like(out, q, "out")
    _check_like(dout, q, "dout")
    _check_like(lse, q, "lse", dtype=torch.float32, shape=(B, Hq, n))
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is not None:
            _check_like(t, like, name)
    dq = _out_like(dq, q, "dq", stream)
    dk = _out_like(dk, k, "dk", stream)
    dv = _out_like(dv, v, "dv", stream)
    need = int(_lib.plpsh_attention_bwd_workspace_bytes(B, Hq, n))
    if workspace is None:
        with _on_stream(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        ws = workspace
        if ws.device != q.device or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = _lib.plpsh_attention_bwd(ptr(q), ptr(k), ptr(v), ptr(out), ptr(dout), ptr(lse), ptr(dq), ptr(dk), ptr(dv),
                                  B, Hq, Hkv, n, d, _torch_dtype_code(q), bins.s, int(bool(causal)),
                                  ptr(bins.buffer), bins.buffer.numel(), None if dl is None else _ptr(dl), ptr(ws),
                                  ws.numel(), _stream(stream))
    _check(st, "plpsh_attention_bwd")
    return dq, dk, dv


def alibi_dense(q, k, v, sigma, causal: bool = False, out=None, stream=None):
    """Exact dense ALiBi attention (plpsh_alibi_dense_fwd)."""
    import torch
    B, Hq, Hkv, n, d = _qkv_shapes(q, k, v)
    sig = _f64(sigma).reshape(-1)
    if sig.size != Hq:
        raise ValueError("sigma must have one entry per query head")
    out = _out_like(out, q, stream=stream)
    st = _lib.plpsh_alibi_dense_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                    ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, n, d,
                                    _torch_dtype_code(q), _ptr(sig), int(bool(causal)), _stream(stream))
    _check(st, "plpsh_alibi_dense_fwd")
    return out


# ------------------------------------------------- error of M~ against L* --

def error_workspace_bytes(n: int, s: int, max_steps: int) -> int:
    return int(_lib.plpsh_error_workspace_bytes(n, s, max_steps))


def error_rowmax(sigma: float, bins: "Bins", out=None, stream=None):
    """max_j |L*[r, j] - c[r, j] / s| for every row r (plpsh_error_rowmax);
    ``bins`` must hold one head."""
    import torch
    if bins.heads != 1:
        raise ValueError("error functions take the bins of one head")
    if out is None:
        with _on_stream(stream):
            out = torch.empty(bins.n, dtype=torch.float64, device=bins.buffer.device)
    else:
        _check_like(out, bins.buffer, "out", dtype=torch.float64, shape=(bins.n,))
    _check(_lib.plpsh_error_rowmax(float(sigma), bins.n, bins.s, ctypes.c_void_p(bins.buffer.data_ptr()),
                                   bins.buffer.numel(), ctypes.c_void_p(out.data_ptr()), _stream(stream)),
           "plpsh_error_rowmax")
    return out


def error_matvec(sigma: float, bins: "Bins", x, out=None, workspace=None, stream=None):
    """(L* - M~) x for a float64 device vector x (plpsh_error_matvec)."""
    import torch
    if bins.heads != 1:
        raise ValueError("error functions take the bins of one head")
    if x.dtype != torch.float64 or x.numel() != bins.n or not x.is_contiguous():
        raise ValueError("x must be a contiguous float64 vector of length n")
    out = _out_like(out, x, stream=stream)
    need = error_workspace_bytes(bins.n, bins.s, 0)
    if workspace is None:
        with _on_stream(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    else:
        ws = workspace
    _check(_lib.plpsh_error_matvec(float(sigma), bins.n, bins.s, ctypes.c_void_p(bins.buffer.data_ptr()),
                                   bins.buffer.numel(), ctypes.c_void_p(x.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                   _stream(stream)), "plpsh_error_matvec")
    return out


def error_norms(sigma: float, delta, u, n: int, max_steps: int = 300, tol: float = 1e-10, seed: int = 0,
                device="cuda", workspace=None, stream=None) -> dict:
    """||L* - M~||_2 and ||L* - M~||_max for one head's hashes
    (plpsh_error_norms).  Returns spectral, maxnorm, argmax_row, steps."""
    import torch
    d = _f64(delta).reshape(-1)
    uu = _f64(u).reshape(-1)
    s = d.size
    need = error_workspace_bytes(n, s, max_steps)
    if need == 0:
        raise ValueError("invalid sizes")
    if workspace is None:
        with _on_stream(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        ws = workspace
    spec = ctypes.c_double()
    mx = ctypes.c_double()
    row = ctypes.c_int32()
    steps = ctypes.c_int32()
    _check(_lib.plpsh_error_norms(float(sigma), n, s, _ptr(d), _ptr(uu), max_steps, float(tol),
                                  ctypes.c_uint64(seed & (2 ** 64 - 1)), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.byref(spec), ctypes.byref(mx), ctypes.byref(row), ctypes.byref(steps),
                                  _stream(stream)), "plpsh_error_norms")
    return {"spectral": spec.value, "maxnorm": mx.value, "argmax_row": row.value, "steps": steps.value}

