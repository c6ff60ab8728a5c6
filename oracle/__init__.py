"""CPU float64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__.py and bench.py's CPU-baseline
leg may import this package. The HIP library and its Python binding never do.
"""
from .attention import (allowed_matrix, backward, backward_keys, backward_rows, forward,  # noqa: F401
                        forward_rows, head_backward, head_forward, head_probabilities)
