"""CPU oracle for causal softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The GPU
library never uses it, and it uses nothing of the GPU library.

Every function is pinned by CPU tests against results fixed independently
of this code.  Attention (``tests/test_oracle_pins.py``): pure-Python brute
force, float64 central differences, closed forms, invariants and torch's own
CPU scaled-dot-product attention.  Dropout
(``tests/test_dropout_oracle_pins.py``): splitmix64's published outputs, and
through them the keep decision of chosen (seed, index) pairs (the golden
multiply of the index, the XOR with the seed and the top-24-bit window),
plus keep-rate and uniformity bounds, brute force and central differences
through the mask.  ``tests/test_oracle_mutants.py`` shows that planted slips
in either module fail these pins.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_backward_head,
    attention_forward,
    attention_forward_head,
    attention_forward_rows,
)
from .dropout import (  # noqa: F401
    attention_dropout_backward_head,
    attention_dropout_forward_head,
    keep_mask,
    splitmix64,
)
