"""ctypes binding of libattn_mi355x.so: argument marshalling only.

Every step of the attention path runs in the HIP kernels of the library; this
module builds the C structs from torch tensors (device memory and streams are
torch's) and calls the C entry points of the same names.  If the library is
not built, ``load()`` raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
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

EXPORTED = ("attn_decode_plan", "attn_decode_split", "attn_combine", "attn_decode",
            "attn_decode_noalloc", "attn_prefill",
            "attn_matmul_matmul", "attn_status_str", "attn_last_error", "attn_version", "rmsnorm_matmul_plan",
            "rmsnorm_matmul", "swiglu_plan", "swiglu")


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
        ("q_indptr", ctypes.c_void_p), ("kv_indptr", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
        ("pages_per_req", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
    ]


class AttnPlan(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32), ("s_max", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("tile_n", ctypes.c_int32), ("rows_per_unit", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32), ("grid", ctypes.c_uint32 * 3), ("block", ctypes.c_uint32),
        ("ws_o_bytes", ctypes.c_uint64), ("ws_lse_bytes", ctypes.c_uint64),
        ("ws_cnt_bytes", ctypes.c_uint64), ("n_items", ctypes.c_int64),
        ("stream_rounds", ctypes.c_int64), ("stream_grid", ctypes.c_int32),
        ("stream_pieces", ctypes.c_int32), ("problem_key", ctypes.c_uint64),
    ]


class RmsProblem(ctypes.Structure):
    """rmsnorm_matmul_problem (include/rmsnorm_matmul.h)."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("m", ctypes.c_int32),
        ("k", ctypes.c_int32), ("n", ctypes.c_int32), ("eps", ctypes.c_float),
        ("x_stride", ctypes.c_int64), ("w_stride", ctypes.c_int64), ("y_stride", ctypes.c_int64),
    ]


class RmsConfig(ctypes.Structure):
    """rmsnorm_matmul_config (include/rmsnorm_matmul.h)."""
    _fields_ = [
        ("s", ctypes.c_int32), ("k_chunk", ctypes.c_int32), ("grid", ctypes.c_uint32 * 3),
        ("block", ctypes.c_uint32), ("kernel", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("ws_bytes", ctypes.c_uint64), ("problem_key", ctypes.c_uint64),
    ]


class SwigluProblem(ctypes.Structure):
    """swiglu_problem (include/swiglu.h)."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("m", ctypes.c_int32),
        ("k", ctypes.c_int32), ("n", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("x_stride", ctypes.c_int64), ("wg_stride", ctypes.c_int64),
        ("wu_stride", ctypes.c_int64), ("y_stride", ctypes.c_int64),
    ]


class SwigluConfig(ctypes.Structure):
    """swiglu_config (include/swiglu.h)."""
    _fields_ = [
        ("s", ctypes.c_int32), ("k_chunk", ctypes.c_int32), ("grid", ctypes.c_uint32 * 3),
        ("block", ctypes.c_uint32), ("kernel", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("ws_bytes", ctypes.c_uint64), ("problem_key", ctypes.c_uint64),
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
    lib.attn_decode_noalloc.argtypes = [P, PL, V, V, V, V, V, V]
    lib.attn_prefill.argtypes = [P, V, V, V, V, V, V]
    lib.attn_matmul_matmul.argtypes = [P, V, V, V, V, V]
    RP, RC = ctypes.POINTER(RmsProblem), ctypes.POINTER(RmsConfig)
    lib.rmsnorm_matmul_plan.argtypes = [RP, ctypes.c_int32, ctypes.c_int32, RC]
    lib.rmsnorm_matmul.argtypes = [RP, RC, V, V, V, V, V, ctypes.c_size_t, V]
    SP, SC = ctypes.POINTER(SwigluProblem), ctypes.POINTER(SwigluConfig)
    lib.swiglu_plan.argtypes = [SP, ctypes.c_int32, ctypes.c_int32, SC]
    lib.swiglu.argtypes = [SP, SC, V, V, V, V, V, ctypes.c_size_t, V]
    for f in ("attn_decode_plan", "attn_decode_split", "attn_combine", "attn_decode",
              "attn_decode_noalloc", "attn_prefill", "attn_matmul_matmul", "rmsnorm_matmul_plan", "rmsnorm_matmul",
              "swiglu_plan", "swiglu"):
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


def _index_tensor(name, t):
    import torch
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return _ptr(t)


def make_problem(q, k, v, o, *, kv_lens=None, kv_len_max: Optional[int] = None,
                 causal: bool = False, scale: float = 0.0, q_indptr=None,
                 q_len_max: Optional[int] = None, kv_indptr=None,
                 page_table=None) -> AttnProblem:
    """Describe the tensors of one attention call (each with a contiguous last dim).

    Plain layout: q [B, Lq, Hq, Dqk], k [B, Lcap, Hkv, Dqk], v [B, Lcap, Hkv, Dv],
    o [B, Lq, Hq, Dv], any strides; v may be a view of k.  ``kv_lens`` is a
    device int32 tensor [B] or None.

    Packed queries (``q_indptr`` int32 [B + 1], prefill only): q [T, Hq, Dqk] and
    o [T, Hq, Dv]; ``q_len_max`` bounds every request's row count.
    Packed keys (``kv_indptr`` int32 [B + 1]): k [T, Hkv, Dqk], v [T, Hkv, Dv];
    ``kv_len_max`` bounds every request's key count.
    Paged keys (``page_table`` int32 [B, pages_per_req]): k and v are page pools
    [num_pages, page_size, Hkv, D] (any strides, e.g. a permuted head-major
    pool); ``kv_len_max`` defaults to pages_per_req * page_size and key counts
    come from ``kv_lens``.
    """
    if q_indptr is not None:
        qdims, batch = 3, int(q_indptr.numel()) - 1
    else:
        qdims, batch = 4, int(q.shape[0])
    kdims = 3 if kv_indptr is not None else 4
    for name, t, nd in (("q", q, qdims), ("o", o, qdims), ("k", k, kdims), ("v", v, kdims)):
        if t.dim() != nd:
            raise ValueError(f"{name} must be {nd}-D for this layout")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if kv_indptr is not None and (kv_lens is not None or page_table is not None):
        raise ValueError("kv_indptr excludes kv_lens and page_table")
    p = AttnProblem()
    p.dtype = _dtype_code(q)
    p.o_dtype = _dtype_code(o)
    p.batch = batch
    p.q_heads, p.head_dim_qk = int(q.shape[-2]), int(q.shape[-1])
    p.kv_heads = int(k.shape[-2])
    p.head_dim_v = int(v.shape[-1])
    if q_indptr is not None:
        if q_len_max is None:
            raise ValueError("packed queries need q_len_max")
        p.q_len = int(q_len_max)
        p.q_indptr = _index_tensor("q_indptr", q_indptr)
        p.q_stride[0], p.q_stride[1], p.q_stride[2] = 0, q.stride(0), q.stride(1)
        p.o_stride[0], p.o_stride[1], p.o_stride[2] = 0, o.stride(0), o.stride(1)
    else:
        p.q_len = int(q.shape[1])
        p.q_stride[0], p.q_stride[1], p.q_stride[2] = q.stride(0), q.stride(1), q.stride(2)
        p.o_stride[0], p.o_stride[1], p.o_stride[2] = o.stride(0), o.stride(1), o.stride(2)
    if kv_indptr is not None:
        if kv_len_max is None:
            raise ValueError("packed keys need kv_len_max")
        p.kv_len_max = int(kv_len_max)
        p.kv_indptr = _index_tensor("kv_indptr", kv_indptr)
        p.k_stride[0], p.k_stride[1], p.k_stride[2] = 0, k.stride(0), k.stride(1)
        p.v_stride[0], p.v_stride[1], p.v_stride[2] = 0, v.stride(0), v.stride(1)
    else:
        for dst, t in ((p.k_stride, k), (p.v_stride, v)):
            dst[0], dst[1], dst[2] = t.stride(0), t.stride(1), t.stride(2)
        if page_table is not None:
            if page_table.dim() != 2 or int(page_table.shape[0]) != batch:
                raise ValueError("page_table must be [B, pages_per_req]")
            if k.shape[:2] != v.shape[:2]:
                raise ValueError("k and v pools must have the same pages")
            p.page_table = _index_tensor("page_table", page_table)
            p.num_pages, p.page_size = int(k.shape[0]), int(k.shape[1])
            p.pages_per_req = int(page_table.shape[1])
            p.kv_len_max = (p.pages_per_req * p.page_size if kv_len_max is None
                            else int(kv_len_max))
        else:
            p.kv_len_max = int(k.shape[1]) if kv_len_max is None else int(kv_len_max)
    p.causal = 1 if causal else 0
    p.scale = float(scale)
    p.kv_lens = _index_tensor("kv_lens", kv_lens) if kv_lens is not None else None
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


def attn_decode_noalloc(problem: AttnProblem, plan: AttnPlan, q, k, v, o, lse_out=None,
                        stream=None) -> None:
    lib = load()
    _check(lib.attn_decode_noalloc(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(o), _ptr(lse_out), _stream(stream)))


def attn_prefill(problem: AttnProblem, q, k, v, o, lse_out=None, stream=None) -> None:
    lib = load()
    _check(lib.attn_prefill(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                            _ptr(lse_out), _stream(stream)))


def attn_matmul_matmul(problem: AttnProblem, q, k, v, o, stream=None) -> None:
    lib = load()
    _check(lib.attn_matmul_matmul(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _stream(stream)))


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


def matmul_matmul(q, k, v, o, *, kv_lens=None, causal=False, scale=0.0, stream=None):
    """O = (tau Q K^T) V per (request, query head), no softmax between the products."""
    prob = make_problem(q, k, v, o, kv_lens=kv_lens, causal=causal, scale=scale)
    attn_matmul_matmul(prob, q, k, v, o, stream)


# ------------------------------------------------------ RMSNorm + MatMul

def make_rms_problem(x, g, w, y, *, eps: float = 1e-5) -> RmsProblem:
    """Describe X [m, k], g [k], W [n, k] and Y [m, n] (row strides taken from
    the tensors; the last dimension must be contiguous)."""
    if x.dim() != 2 or w.dim() != 2 or y.dim() != 2 or g.dim() != 1:
        raise ValueError("x, w, y must be 2-D and g 1-D")
    for name, t in (("x", x), ("w", w), ("y", y), ("g", g)):
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
    if g.dtype != x.dtype or w.dtype != x.dtype:
        raise TypeError("x, g and w must share one dtype")
    p = RmsProblem()
    p.dtype = _dtype_code(x)
    p.y_dtype = _dtype_code(y)
    p.m, p.k = int(x.shape[0]), int(x.shape[1])
    p.n = int(w.shape[0])
    if int(w.shape[1]) != p.k or int(g.shape[0]) != p.k or tuple(y.shape) != (p.m, p.n):
        raise ValueError("shapes: x [m, k], g [k], w [n, k], y [m, n]")
    p.eps = float(eps)
    p.x_stride, p.w_stride, p.y_stride = x.stride(0), w.stride(0), y.stride(0)
    return p


def rmsnorm_matmul_plan(problem: RmsProblem, s_request: int = 0, num_cus: int = 0) -> RmsConfig:
    lib = load()
    cfg = RmsConfig()
    _check(lib.rmsnorm_matmul_plan(ctypes.byref(problem), int(s_request), int(num_cus),
                                   ctypes.byref(cfg)))
    return cfg


def rms_workspace(plan: RmsConfig, device):
    """The workspace a plan asks for, as float32 elements (torch owns the
    memory), or None."""
    import torch
    if plan.ws_bytes == 0:
        return None
    return torch.empty((plan.ws_bytes + 3) // 4, dtype=torch.float32, device=device)


def rmsnorm_matmul(problem: RmsProblem, plan: RmsConfig, x, g, w, y, ws=None, stream=None) -> None:
    lib = load()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.rmsnorm_matmul(ctypes.byref(problem), ctypes.byref(plan), _ptr(x), _ptr(g), _ptr(w),
                              _ptr(y), _ptr(ws), nbytes, _stream(stream)))


# ----------------------------------------------------------------- SwiGLU

def make_swiglu_problem(x, w_gate, w_up, y) -> SwigluProblem:
    """Describe X [m, k], W_gate and W_up [n, k] and H [m, n] (row strides taken
    from the tensors; the last dimension must be contiguous)."""
    for name, t in (("x", x), ("w_gate", w_gate), ("w_up", w_up), ("y", y)):
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
    if w_gate.dtype != x.dtype or w_up.dtype != x.dtype:
        raise TypeError("x and the weights must share one dtype")
    p = SwigluProblem()
    p.dtype = _dtype_code(x)
    p.y_dtype = _dtype_code(y)
    p.m, p.k = int(x.shape[0]), int(x.shape[1])
    p.n = int(w_gate.shape[0])
    if (tuple(w_gate.shape) != (p.n, p.k) or tuple(w_up.shape) != (p.n, p.k)
            or tuple(y.shape) != (p.m, p.n)):
        raise ValueError("shapes: x [m, k], w_gate and w_up [n, k], y [m, n]")
    p.x_stride, p.wg_stride, p.wu_stride, p.y_stride = (x.stride(0), w_gate.stride(0),
                                                        w_up.stride(0), y.stride(0))
    return p


def swiglu_plan(problem: SwigluProblem, s_request: int = 0, num_cus: int = 0) -> SwigluConfig:
    lib = load()
    cfg = SwigluConfig()
    _check(lib.swiglu_plan(ctypes.byref(problem), int(s_request), int(num_cus), ctypes.byref(cfg)))
    return cfg


def swiglu_workspace(config: SwigluConfig, device):
    """The fp32 workspace a config asks for (torch owns the memory), or None."""
    import torch
    if config.ws_bytes == 0:
        return None
    return torch.empty(config.ws_bytes // 4, dtype=torch.float32, device=device)


def swiglu(problem: SwigluProblem, config: SwigluConfig, x, w_gate, w_up, y, ws=None,
           stream=None) -> None:
    lib = load()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swiglu(ctypes.byref(problem), ctypes.byref(config), _ptr(x), _ptr(w_gate),
                      _ptr(w_up), _ptr(y), _ptr(ws), nbytes, _stream(stream)))
