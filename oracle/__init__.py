"""fp64 CPU oracle for exact attention -- test infrastructure only.

Importable only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  The product path never imports it.
"""
from .attention import (backward, backward_keys, backward_rows, forward, forward_rows,  # noqa: F401
                        key_lengths, row_stats, visible, block_count, MASK_BLOCK)
from .philox import dropout_keep, keep_threshold, philox4x32_10  # noqa: F401,E402
