"""fp64 CPU oracle for the fused hot paths (attention; MatMul + MatMul;
RMSNorm + MatMul; SwiGLU).  TEST INFRASTRUCTURE ONLY.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product library never imports,
links or runs anything in this package, and this package imports nothing from
the product library.
"""
from .attention import (attention, attention_rows, attention_split, combine,
                        split_partials, visible_mask)
from .brute import brute_attention, brute_matmul_matmul, brute_rmsnorm_matmul, brute_swiglu
from .matmul_matmul import error_bounds, intermediate, matmul_matmul, matmul_matmul_rows
from .rmsnorm_matmul import (RMS_EPS, rmsnorm, rmsnorm_matmul, rmsnorm_matmul_combine,
                             rmsnorm_matmul_partials, rmsnorm_matmul_split)
from .swiglu import silu, swiglu, swiglu_combine, swiglu_partials, swiglu_split

__all__ = ["attention", "attention_rows", "attention_split", "combine",
           "split_partials", "visible_mask", "brute_attention", "brute_matmul_matmul",
           "error_bounds", "intermediate", "matmul_matmul", "matmul_matmul_rows",
           "brute_rmsnorm_matmul",
           "RMS_EPS", "rmsnorm", "rmsnorm_matmul", "rmsnorm_matmul_combine",
           "rmsnorm_matmul_partials", "rmsnorm_matmul_split", "brute_swiglu", "silu", "swiglu",
           "swiglu_combine", "swiglu_partials", "swiglu_split"]
