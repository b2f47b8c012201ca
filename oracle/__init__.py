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
Every output value is pinned, with one exception that concerns an input of
the dropout path rather than its arithmetic: which Philox4x32-10 draw
decides which (row, key) pair.  The pages name no generator and no such
assignment (the reading notes only say that dropout keeps the generator's
state for the backward pass), so the assignment in ``dropout.draw_position``
(key j = 16a + 8b + 4c + w takes half 4b + w of the call at counter
(2a + c, row, head, offset)) is a convention of this library.  Its only pins
restate it (every keep bit against a single generator call at its own
counter), so dropout parity is self-consistent on that convention and the
key-to-draw assignment itself is "parity unpinned".  The generator, the keep
rule and all arithmetic on the kept weights are pinned independently.
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
