"""CPU float64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__.py and bench.py's CPU-baseline
leg may import this package. The HIP library and its Python binding never do.
"""
from .attention import (allowed_matrix, backward, backward_keys, backward_rows, dropout_keep,  # noqa: F401
                        forward, forward_rows, head_backward, head_forward, head_probabilities, keep_scale)
from .philox import philox4x32  # noqa: F401
