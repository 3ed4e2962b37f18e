"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The GPU path never
routes through it, and it imports nothing from the GPU package: the two share
no code.  The seeded input generator lives in its own module and holds none of
the method's arithmetic.

Every function is pinned by tests in ``tests/test_oracle.py`` against closed
forms, invariants, brute force and independent library routines; none is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    attention_ref,
    attention_probs_ref,
    attention_bwd_ref,
    attention_varlen_ref,
    online_softmax_blocked,
    merge_partials,
    split_bounds,
    decode_partials_ref,
    score_matrix_bytes,
    paged_to_contiguous,
    to_f64,
)
from .fp8 import decode_fp8, attention_fp8_ref, E4M3, E5M2  # noqa: F401
