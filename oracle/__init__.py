"""fp64 CPU oracle for the attention KL divergence (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""
from .reference import (  # noqa: F401
    allowed_mask, forward_head, backward_head, dq_rows, dk_keys, dk_keys_from_state, dlogits_head,
    forward, backward,
)
