"""MI355X (gfx950) fused attention (split-K GQA/MLA decode, causal GQA
prefill, paged and ragged layouts), MatMul+MatMul, RMSNorm followed by a
MatMul, and SwiGLU.

The compute runs in the HIP kernels of ``libattn_mi355x.so`` (C ABI declared
in ``include/attn_mi355x.h``, ``include/rmsnorm_matmul.h`` and
``include/swiglu.h``); this package
is its thin ctypes binding.
"""
from ._lib import (ATTN_BF16, ATTN_ERR_ARG, ATTN_ERR_HIP, ATTN_ERR_UNSUPPORTED,
                   ATTN_ERR_WORKSPACE, ATTN_F32, ATTN_OK, EXPORTED, KERNEL_NAMES, AttnError,
                   AttnPlan, AttnProblem, attn_combine, attn_decode, attn_decode_noalloc,
                   attn_decode_plan,
                   attn_decode_split, attn_matmul_matmul, attn_prefill, decode, load, make_problem, make_rms_problem,
                   matmul_matmul, prefill, rms_workspace, rmsnorm_matmul, rmsnorm_matmul_plan, RmsConfig,
                   RmsProblem, SwigluConfig, SwigluProblem, make_swiglu_problem, swiglu,
                   swiglu_plan, swiglu_workspace, workspace)

__all__ = ["ATTN_BF16", "ATTN_ERR_ARG", "ATTN_ERR_HIP", "ATTN_ERR_UNSUPPORTED",
           "ATTN_ERR_WORKSPACE", "ATTN_F32", "ATTN_OK", "EXPORTED", "KERNEL_NAMES", "AttnError",
           "AttnPlan", "AttnProblem", "attn_combine", "attn_decode", "attn_decode_noalloc",
           "attn_decode_plan",
           "attn_decode_split", "attn_matmul_matmul", "matmul_matmul",
           "attn_prefill", "decode", "load", "make_problem", "make_rms_problem", "prefill",
           "rms_workspace", "rmsnorm_matmul", "rmsnorm_matmul_plan", "RmsConfig", "RmsProblem",
           "SwigluConfig", "SwigluProblem", "make_swiglu_problem", "swiglu", "swiglu_plan",
           "swiglu_workspace", "workspace"]
