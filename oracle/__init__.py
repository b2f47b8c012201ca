"""fp64 CPU oracle for exact softmax attention (forward pass).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg may import it; the product path never does.  It shares no code,
constant or helper with the HIP path.

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself (the Polish notes' worked example, closed forms, invariances, brute
force over the pages' recurrences, and torch's fp64 CPU attention).  No output
of this oracle is "parity unpinned".
"""
from .attention import (attention_head, attention_ref, attention_rows, kv_head,
                        masked_scores, softmax_rows)

__all__ = ["attention_head", "attention_ref", "attention_rows", "kv_head",
           "masked_scores", "softmax_rows"]
