"""fp64 CPU oracle for exact softmax attention (forward and backward).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The HIP library and its Python binding
never import, call or link it, and the two share no code: no kernels, headers,
helpers, tables or pre/post-processing.  The only thing both sides consume is
the seeded input tensors from ``workloads.py``.

Contents
--------
``attention``   the plain definition: S and P materialized, analytic backward;
                also with grouped key/value heads (forward_gqa, backward_gqa)
                and padding-free variable-length batches (forward_varlen,
                backward_varlen); every function takes an optional local
                window (window_visible) and a block-sparse mask
                (block_visible).
``philox``      Philox4x32-10 and the dropout keep mask built from it.
``recurrence``  the online-softmax tile recurrence and the two-tile merge,
                written in the pages' order; used only to pin that the
                recurrence is exact, never as the reference for the GPU path.

Every function in this package is pinned by a ``-m "not gpu"`` test against
values the pages print, closed forms, invariants or brute-force finite
differences (``tests/test_oracle.py``).  No function here is parity-unpinned.
"""
from .attention import (  # noqa: F401
    backward,
    backward_gqa,
    backward_varlen,
    block_visible,
    dropped,
    head_drop,
    backward_head,
    causal_visible,
    forward,
    forward_gqa,
    forward_varlen,
    forward_head,
    probabilities,
    row_softmax,
    scores,
    window_visible,
)
from .recurrence import merge_tile, online_forward_head  # noqa: F401
from . import philox  # noqa: F401
