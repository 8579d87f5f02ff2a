"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds none of the method's arithmetic: only workload shapes, the per-head
ALiBi scales, and seeded N(0, 1) tensors.  Both the HIP path and the oracle
receive what this module produces.

Workloads (shapes of the pages' experiments: a single attention layer of the
named model families, synthetic activations; the pages' models, weights and
evaluation data are not used):

  tiny      1 x 1/1 heads,  n=512,    d=64,  fp32, sigma=16,               s=8,  non-causal
  small     2 x 8/8 heads,  n=4096,   d=64,  bf16, sigma_h=2^(8(h+1)/8),   s=10, non-causal
  qwen3     1 x 16/8 heads, n=8192,   d=128, bf16, sigma_h=2^(8(h+1)/16),  s=20, causal
  mistral   1 x 32/8 heads, n=16384,  d=128, bf16, sigma_h=2^(8(h+1)/32),  s=20, causal
  long      1 x 32/8 heads, n=131072, d=128, bf16, sigma_h=2^(8(h+1)/32),  s=32, causal

sigma_h = 1 / m_h with the standard ALiBi slopes m_h = 2^(-8(h+1)/H).
Q, K, V are i.i.d. N(0, 1), drawn in the order Q, K, V, C-order [B, H, n, d],
then rounded to the workload's dtype (round to nearest even for bf16).
The hash seed is 0 for every workload.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    n: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    sigmas: tuple
    s: int
    causal: bool
    hash_seed: int = 0
    data_seed: int = 1000
    extra: dict = field(default_factory=dict)


def alibi_sigmas(heads: int) -> tuple:
    """sigma_h = 2^(8(h+1)/H): inverse of the geometric ALiBi slopes."""
    return tuple(float(2.0 ** (8.0 * (h + 1) / heads)) for h in range(heads))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 512, 64, "f32", (16.0,), 8, False, 0, 1000),
    "small": Workload("small", 2, 8, 8, 4096, 64, "bf16", alibi_sigmas(8), 10, False, 0, 1001),
    "qwen3": Workload("qwen3", 1, 16, 8, 8192, 128, "bf16", alibi_sigmas(16), 20, True, 0, 1002),
    "mistral": Workload("mistral", 1, 32, 8, 16384, 128, "bf16", alibi_sigmas(32), 20, True, 0, 1003),
    "long": Workload("long", 1, 32, 8, 131072, 128, "bf16", alibi_sigmas(32), 32, True, 0, 1004),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding exactly representable bf16 values.  NaN/inf untouched."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    finite = np.isfinite(x)
    out = np.where(finite, r.astype(np.uint32), x.view(np.uint32))
    return out.astype(np.uint32).view(np.float32)


def qkv_numpy(batch, heads_q, heads_kv, n, d, dtype="f32", seed=1000, scale_q=1.0):
    """Seeded Q [B,Hq,n,d], K, V [B,Hkv,n,d] as float32 numpy arrays whose
    values are exactly representable in ``dtype``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, heads_q, n, d), dtype=np.float32) * np.float32(scale_q)
    k = rng.standard_normal((batch, heads_kv, n, d), dtype=np.float32)
    v = rng.standard_normal((batch, heads_kv, n, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def qkv_torch(batch, heads_q, heads_kv, n, d, dtype="bf16", seed=1000, device="cuda"):
    """Seeded Q, K, V generated directly on ``device`` with torch's
    generator (for full-size workloads whose host generation would be slow).
    Returns tensors of the workload dtype; callers needing the oracle copy
    the rows they check back to the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = []
    for H in (heads_q, heads_kv, heads_kv):
        t = torch.randn((batch, H, n, d), generator=g, device=device, dtype=torch.float32)
        out.append(t.to(tdt))
    return tuple(out)
