"""fp64 CPU oracle for the fused-attention hot path.  TEST INFRASTRUCTURE ONLY.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product library never imports,
links or runs anything in this package, and this package imports nothing from
the product library.
"""
from .attention import (attention, attention_rows, attention_split, combine,
                        split_partials, visible_mask)
from .brute import brute_attention

__all__ = ["attention", "attention_rows", "attention_split", "combine",
           "split_partials", "visible_mask", "brute_attention"]
