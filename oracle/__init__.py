"""Plain fp64 CPU oracle for Positional-LSH attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with ``randomized_positional_lsh_amd`` (the HIP path) and never
imports it.

Source pages.  Every citation ``[P, ...]`` refers to the gist.science
explainer of arXiv 2605.09472, "Positional LSH: Binary Block Matrix
Approximation for Attention with Linear Biases" (D. Wolfson, T. Wagner),
available in Dutch ("Technische Samenvatting: Positionele LSH ..."), Chinese
and Japanese with the same section structure:

* [P, Methodology 1]   theoretical framework: positional LSH (Laplace kernel
                       L*_ij = exp(-|i-j|/sigma), random binning of integer
                       positions, contiguous non-overlapping bins, E[M(h)] = L*)
* [P, Theorem 2.1]     structural approximation: empirical mean of s masks,
                       spectral / max-norm bounds, block-size control, Gamma law
* [P, Theorem 2.2]     algorithmic reduction to randomized short-context
                       unbiased attentions; output-error bound
* [P, Key results]     O(1/sqrt(s)) error decay; experiments
* [P, Limitations]     no wall-clock claim against dense kernels

``oracle.grad`` gives the row normalisers and the gradients of T~ for
training with the approximation.  ``oracle.convergence`` gives the error E = L* - M~ of [P, Theorem 2.1] at
sequence lengths where dense matrices no longer fit (row maxima, products
E x, spectral norm).

Parity status of each function is stated in its docstring; all functions
here are pinned by ``tests/test_oracle_pins.py`` (closed forms, exact
rational arithmetic, brute force, special cases reducing to library
routines, invariants and statistical laws).
"""

from .plsh import (  # noqa: F401
    bin_values,
    block_starts,
    block_of,
    count_matrix,
    mtilde,
    alibi_matrix,
    plsh_attention,
    plsh_attention_literal,
    plsh_attention_rows,
    plsh_attention_rowblocks,
    alibi_attention,
    alibi_attention_rows,
    support_interval,
)
from .sampler import splitmix64, sample_hashes  # noqa: F401
from .grad import plsh_attention_grad, plsh_attention_lse  # noqa: F401
from .convergence import (  # noqa: F401
    error_dense,
    error_matvec,
    error_maxnorm,
    error_rowmax,
    error_spectral,
)
