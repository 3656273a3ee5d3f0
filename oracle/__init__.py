"""Plain fp64 CPU oracle for the attention KL divergence (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it.
"""
from .streamkl_oracle import (  # noqa: F401
    scores,
    valid_mask,
    head_forward,
    head_backward,
    head_backward_dk_rows,
    head_dk_keys,
    materialised_bytes,
    pair_count,
)
