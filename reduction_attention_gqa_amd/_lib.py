"""ctypes binding of libattn_mi355x.so: argument marshalling only.

Every step of the attention path runs in the HIP kernels of the library; this
module builds the C structs from torch tensors (device memory and streams are
torch's) and calls the C entry points of the same names.  If the library is
not built, ``load()`` raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_mi355x.so")

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_OK = 0
ATTN_ERR_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_HIP = 4
KERNEL_NAMES = {0: "generic", 1: "gqa_d128", 2: "mla"}

EXPORTED = ("attn_decode_plan", "attn_decode_split", "attn_combine", "attn_decode", "attn_prefill",
            "attn_status_str", "attn_last_error", "attn_version")


class AttnProblem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("kv_len_max", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float), ("reserved0", ctypes.c_int32),
        ("kv_lens", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


class AttnPlan(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32), ("s_max", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("tile_n", ctypes.c_int32), ("rows_per_unit", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32), ("grid", ctypes.c_uint32 * 3), ("block", ctypes.c_uint32),
        ("ws_o_bytes", ctypes.c_uint64), ("ws_lse_bytes", ctypes.c_uint64),
        ("ws_cnt_bytes", ctypes.c_uint64), ("n_items", ctypes.c_int64),
        ("problem_key", ctypes.c_uint64),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


_LIB = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m reduction_attention_gqa_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, PL, V = ctypes.POINTER(AttnProblem), ctypes.POINTER(AttnPlan), ctypes.c_void_p
    lib.attn_decode_plan.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.c_int32, PL]
    lib.attn_decode_split.argtypes = [P, PL, V, V, V, V, ctypes.c_size_t, V, ctypes.c_size_t, V]
    lib.attn_combine.argtypes = [P, PL, V, V, V, V, V]
    lib.attn_decode.argtypes = [P, PL, V, V, V, V, ctypes.c_size_t, V, ctypes.c_size_t, V,
                                ctypes.c_size_t, V, V, V]
    lib.attn_prefill.argtypes = [P, V, V, V, V, V, V]
    for f in ("attn_decode_plan", "attn_decode_split", "attn_combine", "attn_decode",
              "attn_prefill"):
        getattr(lib, f).restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        lib = load()
        raise AttnError(status, f"{lib.attn_status_str(status).decode()}: "
                                f"{lib.attn_last_error().decode()}")


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def make_problem(q, k, v, o, *, kv_lens=None, kv_len_max: Optional[int] = None,
                 causal: bool = False, scale: float = 0.0) -> AttnProblem:
    """Describe tensors q [B, Lq, Hq, Dqk], k [B, Lcap, Hkv, Dqk], v [B, Lcap, Hkv, Dv]
    and o [B, Lq, Hq, Dv] (any strides with a contiguous last dim; v may be a
    view of k).  ``kv_lens`` is a device int32 tensor [B] or None."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    p = AttnProblem()
    p.dtype = _dtype_code(q)
    p.o_dtype = _dtype_code(o)
    p.batch, p.q_len, p.q_heads, p.head_dim_qk = (int(x) for x in q.shape)
    p.kv_heads = int(k.shape[2])
    p.head_dim_v = int(v.shape[3])
    p.kv_len_max = int(k.shape[1]) if kv_len_max is None else int(kv_len_max)
    p.causal = 1 if causal else 0
    p.scale = float(scale)
    p.reserved0 = 0
    p.kv_lens = _ptr(kv_lens) if kv_lens is not None else None
    if kv_lens is not None:
        import torch
        if kv_lens.dtype != torch.int32 or not kv_lens.is_contiguous():
            raise TypeError("kv_lens must be a contiguous int32 tensor")
    for dst, t in ((p.q_stride, q), (p.k_stride, k), (p.v_stride, v), (p.o_stride, o)):
        dst[0], dst[1], dst[2] = t.stride(0), t.stride(1), t.stride(2)
    return p


def attn_decode_plan(problem: AttnProblem, s_request: int = 0,
                     kv_lens_host: Optional[Sequence[int]] = None, num_cus: int = 0) -> AttnPlan:
    lib = load()
    plan = AttnPlan()
    arr = None
    if kv_lens_host is not None:
        arr = (ctypes.c_int32 * len(kv_lens_host))(*[int(x) for x in kv_lens_host])
    _check(lib.attn_decode_plan(ctypes.byref(problem), int(s_request), arr, int(num_cus),
                                ctypes.byref(plan)))
    return plan


def attn_decode_split(problem: AttnProblem, plan: AttnPlan, q, k, v, ws_o, ws_lse,
                      stream=None) -> None:
    lib = load()
    _check(lib.attn_decode_split(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(ws_o), ws_o.numel() * ws_o.element_size(),
                                 _ptr(ws_lse), ws_lse.numel() * ws_lse.element_size(),
                                 _stream(stream)))


def attn_combine(problem: AttnProblem, plan: AttnPlan, ws_o, ws_lse, o, lse_out=None,
                 stream=None) -> None:
    lib = load()
    _check(lib.attn_combine(ctypes.byref(problem), ctypes.byref(plan), _ptr(ws_o), _ptr(ws_lse),
                            _ptr(o), _ptr(lse_out), _stream(stream)))


def attn_decode(problem: AttnProblem, plan: AttnPlan, q, k, v, ws_o, ws_lse, ws_cnt, o,
                lse_out=None, stream=None) -> None:
    lib = load()
    _check(lib.attn_decode(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(ws_o), ws_o.numel() * ws_o.element_size(),
                           _ptr(ws_lse), ws_lse.numel() * ws_lse.element_size(),
                           _ptr(ws_cnt), ws_cnt.numel() * ws_cnt.element_size(),
                           _ptr(o), _ptr(lse_out), _stream(stream)))


def attn_prefill(problem: AttnProblem, q, k, v, o, lse_out=None, stream=None) -> None:
    lib = load()
    _check(lib.attn_prefill(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                            _ptr(lse_out), _stream(stream)))


def workspace(plan: AttnPlan, device):
    """Allocate the workspace a plan asks for (torch owns the memory):
    (ws_o, ws_lse, ws_cnt); the arrival counters start at zero, as attn_decode
    requires, and every attn_decode call leaves them at zero."""
    import torch
    ws_o = torch.empty(max(1, plan.ws_o_bytes // 4), dtype=torch.float32, device=device)
    ws_lse = torch.empty(max(1, plan.ws_lse_bytes // 4), dtype=torch.float32, device=device)
    ws_cnt = torch.zeros(max(1, plan.ws_cnt_bytes // 4), dtype=torch.int32, device=device)
    return ws_o, ws_lse, ws_cnt


def decode(q, k, v, o, *, kv_lens=None, kv_lens_host=None, causal=False, scale=0.0,
           s_request=0, lse_out=None, stream=None, plan=None, ws=None, fused=True):
    """Split decode; returns the plan used.  fused=True calls attn_decode (one
    launch where the kernel family allows), fused=False the split launch
    followed by the combine launch."""
    prob = make_problem(q, k, v, o, kv_lens=kv_lens, causal=causal, scale=scale)
    if plan is None:
        plan = attn_decode_plan(prob, s_request, kv_lens_host)
    if ws is None:
        ws = workspace(plan, q.device)
    if fused:
        attn_decode(prob, plan, q, k, v, ws[0], ws[1], ws[2], o, lse_out, stream)
    else:
        attn_decode_split(prob, plan, q, k, v, ws[0], ws[1], stream)
        attn_combine(prob, plan, ws[0], ws[1], o, lse_out, stream)
    return plan


def prefill(q, k, v, o, *, kv_lens=None, causal=False, scale=0.0, lse_out=None, stream=None):
    prob = make_problem(q, k, v, o, kv_lens=kv_lens, causal=causal, scale=scale)
    attn_prefill(prob, q, k, v, o, lse_out, stream)


def default_scale(dqk: int) -> float:
    return 1.0 / math.sqrt(dqk)
