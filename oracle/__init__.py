"""fp64 CPU oracle for exact softmax attention: forward pass and gradients.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg may import it; the product path never does.  It shares no code,
constant or helper with the HIP path.

Every function is pinned to something other than itself:
``tests/test_oracle.py`` pins the forward through the Polish notes' worked
example, closed forms, invariances, brute force over the pages' recurrences
and torch's fp64 CPU attention.  ``tests/test_oracle_backward.py`` pins the
gradients through finite differences of the forward, torch's fp64 autograd,
the blog's blockwise backward, closed forms and invariances.
``tests/test_oracle_dropout.py`` pins the dropout forward and backward
through Philox4x32-10's published known-answer vectors, the statistics of
the keep mask, closed forms, finite differences and torch's fp64 autograd.
No output of this oracle is "parity unpinned".
"""
from .attention import (attention_head, attention_ref, attention_rows, kv_head,
                        masked_scores, softmax_rows)
from .backward import attention_backward_head, attention_backward_ref, backward_blocked
from .dropout import (attention_dropout_backward_head, attention_dropout_backward_ref,
                      attention_dropout_head, attention_dropout_ref, attention_dropout_rows,
                      dropout_keep, philox4x32_10)

__all__ = ["attention_head", "attention_ref", "attention_rows", "kv_head",
           "masked_scores", "softmax_rows", "attention_backward_head",
           "attention_backward_ref", "backward_blocked", "attention_dropout_head",
           "attention_dropout_ref", "attention_dropout_rows", "attention_dropout_backward_head",
           "attention_dropout_backward_ref", "dropout_keep", "philox4x32_10"]
