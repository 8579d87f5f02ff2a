"""Positional-LSH approximation of ALiBi attention on AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``libplpsh.so`` (``include/plpsh.h``); this package only marshals
arguments.  See ``_binding`` for the functions.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    Bins,
    PlpshError,
    alibi_dense,
    attention,
    attention_bwd,
    attention_from_bins,
    attention_literal,
    attention_lse,
    attention_hashes,
    attention_noalloc,
    bins_from_hashes,
    bins_layout,
    draw_hashes,
    error_matvec,
    error_norms,
    error_rowmax,
    error_workspace_bytes,
    fixed_blocks,
    raw,
    sample_bins,
    status_string,
    version,
    workspace_bytes,
)
