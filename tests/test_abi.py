"""The C-ABI library on the CPU: it loads, exports what the header declares,
rejects bad arguments before enqueueing anything, and plans splits.

No compute call is made here (there is no GPU in this environment); the
checks below return before the library touches the device.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import reduction_attention_gqa_amd as ra
from reduction_attention_gqa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_mi355x.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from reduction_attention_gqa_amd.build import build
        build()
    return ra.load()


HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


def _declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?((?:attn|rmsnorm|swiglu)\w*)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_matches_header(lib):
    m = re.search(r"#define ATTN_MI355X_VERSION (\d+)", open(HEADER).read())
    assert lib.attn_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(5):
        assert lib.attn_status_str(code)
    assert lib.attn_status_str(99) == b"unknown status"


def _c_layout(tmp_path, struct, fields):
    """sizeof and offsetof of a header struct, from a C program compiled against the header."""
    lines = [f'printf("size %zu\\n", sizeof({struct}));']
    lines += [f'printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"attn_mi355x.h\"\n"
                   "#include \"rmsnorm_matmul.h\"\n#include \"swiglu.h\"\n"
                   "int main(void) {\n" + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    return {k: int(v) for k, v in (line.split() for line in out.splitlines())}


@pytest.mark.parametrize("py,c", [(_lib.AttnProblem, "attn_problem"), (_lib.AttnPlan, "attn_plan"),
                                  (_lib.RmsProblem, "rmsnorm_matmul_problem"),
                                  (_lib.RmsConfig, "rmsnorm_matmul_config"),
                                  (_lib.SwigluProblem, "swiglu_problem"),
                                  (_lib.SwigluConfig, "swiglu_config")])
def test_struct_layout_matches_c(tmp_path, py, c):
    names = [f[0] for f in py._fields_]
    got = _c_layout(tmp_path, c, names)
    assert got["size"] == ctypes.sizeof(py)
    for n in names:
        assert got[n] == getattr(py, n).offset, n


def problem(**kw):
    """A token-major [B, L, H, D] problem with fake (never dereferenced) pointers."""
    f = dict(dtype=ra.ATTN_BF16, o_dtype=ra.ATTN_BF16, batch=32, q_heads=32, kv_heads=8,
             head_dim_qk=128, head_dim_v=128, q_len=1, kv_len_max=4096, causal=0, scale=0.0)
    f.update(kw)
    p = _lib.AttnProblem()
    for k, v in f.items():
        setattr(p, k, v)
    hq, hkv, dqk, dv, lq, lk = (p.q_heads, p.kv_heads, p.head_dim_qk, p.head_dim_v, p.q_len,
                                p.kv_len_max)
    for dst, (l, h, d) in ((p.q_stride, (lq, hq, dqk)), (p.k_stride, (lk, hkv, dqk)),
                           (p.v_stride, (lk, hkv, dv)), (p.o_stride, (lq, hq, dv))):
        dst[0], dst[1], dst[2] = l * h * d, h * d, d
    return p


def plan_status(lib, p, s_request=0, lens=None, num_cus=256):
    plan = _lib.AttnPlan()
    arr = None if lens is None else (ctypes.c_int32 * len(lens))(*lens)
    st = lib.attn_decode_plan(ctypes.byref(p) if p is not None else None, s_request, arr, num_cus,
                              ctypes.byref(plan))
    return st, plan


@pytest.mark.parametrize("field,value,code", [
    ("q_heads", 30, ra.ATTN_ERR_ARG),            # 30 % 8 != 0
    ("batch", -1, ra.ATTN_ERR_ARG),
    ("q_len", 0, ra.ATTN_ERR_ARG),
    ("kv_len_max", -5, ra.ATTN_ERR_ARG),
    ("dtype", 7, ra.ATTN_ERR_ARG),
    ("o_dtype", -1, ra.ATTN_ERR_ARG),
    ("causal", 2, ra.ATTN_ERR_ARG),
    ("kv_heads", 0, ra.ATTN_ERR_ARG),
    ("head_dim_qk", 0, ra.ATTN_ERR_ARG),
    ("reserved0", 1, ra.ATTN_ERR_ARG),
    ("head_dim_qk", 1024, ra.ATTN_ERR_UNSUPPORTED),
    ("head_dim_v", 600, ra.ATTN_ERR_UNSUPPORTED),
])
def test_invalid_problem_is_rejected_everywhere(lib, field, value, code):
    p = problem(**{field: value})
    fake = ctypes.c_void_p(0x1000)
    st, _ = plan_status(lib, p)
    assert st == code
    assert lib.attn_last_error()
    assert lib.attn_prefill(ctypes.byref(p), fake, fake, fake, fake, None, None) == code
    plan = _lib.AttnPlan()
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake,
                                 1 << 30, fake, 1 << 30, None) == code
    assert lib.attn_combine(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None,
                            None) == code
    assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake, 1 << 30,
                           fake, 1 << 30, fake, 1 << 30, fake, None, None) == code
    assert lib.attn_matmul_matmul(ctypes.byref(p), fake, fake, fake, fake, None) == code


@pytest.mark.parametrize("field,value", [("dtype", ra.ATTN_F32), ("head_dim_qk", 64),
                                         ("head_dim_v", 64)])
def test_matmul_matmul_unsupported_shapes_fail_before_launch(lib, field, value):
    # Valid problems the MFMA path does not cover: rejected before any device
    # access (the pointers are never dereferenced).
    kw = {field: value}
    if field == "dtype":
        kw["o_dtype"] = ra.ATTN_F32
    p = problem(q_len=64, kv_len_max=64, **kw)
    fake = ctypes.c_void_p(0x1000)
    assert lib.attn_matmul_matmul(ctypes.byref(p), fake, fake, fake, fake, None) == \
        ra.ATTN_ERR_UNSUPPORTED
    assert b"MatMul+MatMul" in lib.attn_last_error()


def test_matmul_matmul_arguments(lib):
    fake = ctypes.c_void_p(0x1000)
    p = problem(q_len=64, kv_len_max=64)
    assert lib.attn_matmul_matmul(None, fake, fake, fake, fake, None) == ra.ATTN_ERR_ARG
    assert lib.attn_matmul_matmul(ctypes.byref(p), None, fake, fake, fake, None) == ra.ATTN_ERR_ARG
    assert lib.attn_matmul_matmul(ctypes.byref(p), fake, fake, fake, None, None) == ra.ATTN_ERR_ARG
    p0 = problem(batch=0, q_len=64, kv_len_max=64)
    assert lib.attn_matmul_matmul(ctypes.byref(p0), None, None, None, None, None) == ra.ATTN_OK


def test_negative_stride_and_nonfinite_scale(lib):
    p = problem()
    p.k_stride[1] = -1
    assert plan_status(lib, p)[0] == ra.ATTN_ERR_ARG
    p = problem(scale=float("nan"))
    assert plan_status(lib, p)[0] == ra.ATTN_ERR_ARG


def test_null_arguments(lib):
    st, _ = plan_status(lib, None)
    assert st == ra.ATTN_ERR_ARG
    p = problem()
    assert lib.attn_decode_plan(ctypes.byref(p), 0, None, 256, None) == ra.ATTN_ERR_ARG
    fake = ctypes.c_void_p(0x1000)
    assert lib.attn_prefill(ctypes.byref(p), None, fake, fake, fake, None, None) == ra.ATTN_ERR_ARG
    assert lib.attn_prefill(ctypes.byref(p), fake, fake, fake, None, None, None) == ra.ATTN_ERR_ARG
    st, plan = plan_status(lib, p)
    assert st == 0
    assert lib.attn_decode_split(ctypes.byref(p), None, fake, fake, fake, fake, 1 << 30, fake,
                                 1 << 30, None) == ra.ATTN_ERR_ARG
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), fake, None, fake, fake,
                                 1 << 30, fake, 1 << 30, None) == ra.ATTN_ERR_ARG
    assert lib.attn_combine(ctypes.byref(p), ctypes.byref(plan), fake, fake, None, None,
                            None) == ra.ATTN_ERR_ARG


def test_workspace_too_small_and_plan_mismatch(lib):
    p = problem()
    st, plan = plan_status(lib, p)
    assert st == 0
    fake = ctypes.c_void_p(0x1000)
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake,
                                 plan.ws_o_bytes - 4, fake, plan.ws_lse_bytes,
                                 None) == ra.ATTN_ERR_WORKSPACE
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake,
                                 plan.ws_o_bytes, fake, plan.ws_lse_bytes - 4,
                                 None) == ra.ATTN_ERR_WORKSPACE
    other = problem(batch=31)
    assert lib.attn_decode_split(ctypes.byref(other), ctypes.byref(plan), fake, fake, fake, fake,
                                 plan.ws_o_bytes, fake, plan.ws_lse_bytes,
                                 None) == ra.ATTN_ERR_ARG
    assert lib.attn_combine(ctypes.byref(other), ctypes.byref(plan), fake, fake, fake, None,
                            None) == ra.ATTN_ERR_ARG
    zeroed = _lib.AttnPlan()
    assert lib.attn_combine(ctypes.byref(p), ctypes.byref(zeroed), fake, fake, fake, None,
                            None) == ra.ATTN_ERR_ARG
    # attn_decode: each of the three workspace buffers is checked, and o must be given.
    big = 1 << 40
    for sizes in ((plan.ws_o_bytes - 4, big, big), (big, plan.ws_lse_bytes - 4, big),
                  (big, big, plan.ws_cnt_bytes - 4)):
        assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake,
                               fake, sizes[0], fake, sizes[1], fake, sizes[2], fake, None,
                               None) == ra.ATTN_ERR_WORKSPACE
    assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake, big,
                           fake, big, None, big, fake, None, None) == ra.ATTN_ERR_ARG
    assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake, big,
                           fake, big, fake, big, None, None, None) == ra.ATTN_ERR_ARG
    assert lib.attn_decode(ctypes.byref(other), ctypes.byref(plan), fake, fake, fake, fake, big,
                           fake, big, fake, big, fake, None, None) == ra.ATTN_ERR_ARG


def test_empty_batch_is_a_no_op(lib):
    p = problem(batch=0)
    st, plan = plan_status(lib, p)
    assert st == 0 and plan.s_max == 1
    assert lib.attn_prefill(ctypes.byref(p), None, None, None, None, None, None) == 0
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), None, None, None, None, 0,
                                 None, 0, None) == 0
    assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), None, None, None, None, 0,
                           None, 0, None, 0, None, None, None) == 0


# ---------------------------------------------------------------- planner

def _stream_runs(p, lens, cus):
    """The GQA single-launch decomposition, by brute force: every unit's
    rounds of 128 keys laid end to end (an empty unit counts one), equal runs
    [g T / N, (g + 1) T / N) per workgroup, and for every unit the number of
    runs that meet it."""
    cap = p.kv_len_max
    unit_rounds = []
    for n in lens:
        r = max(1, math.ceil(min(max(n, 0), cap) / 128))
        unit_rounds += [r] * p.kv_heads
    total = sum(unit_rounds)

    def pieces_for(grid):
        owner = []  # owner[round] = the workgroup whose run holds it
        for g in range(grid):
            owner += [g] * ((g + 1) * total // grid - g * total // grid)
        assert len(owner) == total
        pieces, u0 = 1, 0
        for r in unit_rounds:
            pieces = max(pieces, len(set(owner[u0:u0 + r])))
            u0 += r
        return pieces

    # One run per compute unit when that cuts no unit, else two.
    grid = max(1, min(cus, total))
    if pieces_for(grid) > 1:
        grid = max(1, min(2 * cus, total))
    return total, grid, pieces_for(grid)


def _check_plan_invariants(p, plan, lens, cus=256):
    lmax = max(lens) if lens else 0
    assert plan.chunk % plan.tile_n == 0 and plan.chunk >= plan.tile_n
    assert plan.s_max == max(1, math.ceil(lmax / plan.chunk))
    assert plan.s_max * plan.chunk >= lmax
    nrows = p.batch * p.q_len * p.q_heads
    ws_o = plan.s_max * nrows * p.head_dim_v * 4
    ws_lse = plan.s_max * nrows * 4
    if ra.KERNEL_NAMES[plan.kernel] == "gqa_d128" and p.batch:
        total, grid, pieces = _stream_runs(p, lens, cus)
        assert (plan.stream_rounds, plan.stream_grid, plan.stream_pieces) == (total, grid, pieces)
        units = p.batch * p.kv_heads
        ws_o = max(ws_o, pieces * units * 16 * 128 * 4)
        ws_lse = max(ws_lse, pieces * units * 16 * 4)
    assert plan.ws_o_bytes == ws_o
    assert plan.ws_lse_bytes == ws_lse
    assert plan.ws_cnt_bytes == p.batch * p.kv_heads * plan.row_tiles * 4
    # Work items (request, KV head, split), counted from the clamped host lengths;
    # an empty request owns one item per KV head.
    cap = p.kv_len_max
    assert plan.n_items == sum(p.kv_heads * max(1, math.ceil(min(max(n, 0), cap) / plan.chunk))
                               for n in lens)
    if ra.KERNEL_NAMES[plan.kernel] == "gqa_d128":
        # One-dimensional grid, a whole number of rounds over the 8 XCDs.
        assert plan.grid[0] == 8 * math.ceil(plan.n_items / 8)
        assert plan.grid[1] == plan.grid[2] == 1
    else:
        assert plan.grid[0] == plan.s_max


def test_plan_tiny_fp32_decode_fixed_s4(lib):
    # 256 keys split 4 ways: Split(A:[m, k], dim=1) -> [s, m, k/s] (Cleave §4), k/s = 64.
    p = problem(dtype=ra.ATTN_F32, o_dtype=ra.ATTN_F32, batch=1, q_heads=8, kv_heads=2,
                head_dim_qk=64, head_dim_v=64, kv_len_max=256)
    st, plan = plan_status(lib, p, s_request=4)
    assert st == 0
    assert plan.kernel == 0 and plan.s_max == 4 and plan.chunk == 64
    _check_plan_invariants(p, plan, [256])


def test_plan_llama_decode_uses_gqa_kernel_and_fills_the_gpu(lib):
    p = problem()
    st, plan = plan_status(lib, p)
    assert st == 0
    assert ra.KERNEL_NAMES[plan.kernel] == "gqa_d128"
    _check_plan_invariants(p, plan, [4096] * 32)
    assert plan.n_items >= 256  # at least one workgroup per compute unit
    # 32 x 8 = 256 (request, KV head) units fill 256 CUs and the lengths are
    # equal: one split per request, the key axis split across the 4 waves of
    # each workgroup instead (no partials, no merge).
    assert plan.s_max == 1 and plan.block == 256 and plan.tile_n == 128
    # With more compute units than units the key axis is split across workgroups.
    st, plan2 = plan_status(lib, p, num_cus=1024)
    assert st == 0 and plan2.s_max > 1 and plan2.block == 256
    _check_plan_invariants(p, plan2, [4096] * 32, cus=1024)
    # The single launch: one run of 32 rounds per compute unit, each exactly
    # one (request, KV head), so no unit is cut.
    assert (plan.stream_rounds, plan.stream_grid, plan.stream_pieces) == (8192, 256, 1)


def test_plan_unbalanced_lengths_split_across_workgroups(lib):
    # One long request among short ones: a single split per request would leave
    # the long one's workgroup running alone, so the key axis is split.
    lens = [32768] + [1024] * 511
    p = problem(batch=512, kv_len_max=32768)
    st, plan = plan_status(lib, p, lens=lens)
    assert st == 0 and plan.s_max > 1 and plan.block == 256
    _check_plan_invariants(p, plan, lens)


@pytest.mark.parametrize("s_req", [1, 2, 3, 7, 8, 16, 10_000])
def test_plan_honours_requested_split(lib, s_req):
    p = problem()
    st, plan = plan_status(lib, p, s_request=s_req)
    assert st == 0
    assert plan.s_max <= s_req
    _check_plan_invariants(p, plan, [4096] * 32)


def test_plan_ragged_uses_host_lengths(lib):
    lens = [128, 32768, 5000, 0] + [300] * 60
    p = problem(batch=64, q_heads=64, kv_heads=8, kv_len_max=32768)
    st, plan = plan_status(lib, p, lens=lens)
    assert st == 0
    _check_plan_invariants(p, plan, lens)
    # lengths above capacity are clamped, not trusted
    st2, plan2 = plan_status(lib, p, lens=lens[:1] + [10 ** 9] + lens[2:])
    assert st2 == 0 and plan2.s_max == plan.s_max


def test_plan_generic_for_other_shapes(lib):
    p = problem(head_dim_qk=64, head_dim_v=64)
    st, plan = plan_status(lib, p)
    assert st == 0 and ra.KERNEL_NAMES[plan.kernel] == "generic"
    _check_plan_invariants(p, plan, [4096] * 32)


# ------------------------------------------------ packed and paged layouts

def paged(ps=16, lmax=4096, **kw):
    """A problem whose K/V are pools of pages [num_pages, ps, Hkv, D] (fake pointers)."""
    p = problem(kv_len_max=lmax, **kw)
    hkv, dqk, dv = p.kv_heads, p.head_dim_qk, p.head_dim_v
    p.page_table = 0x2000
    p.page_size = ps
    p.pages_per_req = -(-lmax // ps)
    p.num_pages = p.batch * p.pages_per_req
    for dst, d in ((p.k_stride, dqk), (p.v_stride, dv)):
        dst[0], dst[1], dst[2] = ps * hkv * d, hkv * d, d
    return p


@pytest.mark.parametrize("edit", [
    dict(reserved1=1),
    dict(page_size=0),
    dict(num_pages=0),
    dict(pages_per_req=1),                       # 16 rows < kv_len_max
    dict(page_table=None),                       # page fields without a table
    dict(kv_indptr=0x3000),                      # kv_indptr with a page table
])
def test_invalid_layout_is_rejected(lib, edit):
    p = paged()
    for k, v in edit.items():
        setattr(p, k, v)
    assert plan_status(lib, p)[0] == ra.ATTN_ERR_ARG
    fake = ctypes.c_void_p(0x1000)
    assert lib.attn_prefill(ctypes.byref(p), fake, fake, fake, fake, None, None) == ra.ATTN_ERR_ARG


def test_kv_indptr_excludes_kv_lens(lib):
    p = problem()
    p.kv_indptr = 0x3000
    p.kv_lens = 0x4000
    assert plan_status(lib, p)[0] == ra.ATTN_ERR_ARG
    p.kv_lens = None
    assert plan_status(lib, p)[0] == 0


def test_packed_queries_are_prefill_only(lib):
    p = problem(q_len=4)
    p.q_indptr = 0x3000
    st, _ = plan_status(lib, p)
    assert st == ra.ATTN_ERR_UNSUPPORTED
    fake = ctypes.c_void_p(0x1000)
    plan = _lib.AttnPlan()
    assert lib.attn_decode_split(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake,
                                 1 << 30, fake, 1 << 30, None) == ra.ATTN_ERR_UNSUPPORTED
    assert lib.attn_combine(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None,
                            None) == ra.ATTN_ERR_UNSUPPORTED
    assert lib.attn_decode(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, fake, 1 << 30,
                           fake, 1 << 30, fake, 1 << 30, fake, None, None) == ra.ATTN_ERR_UNSUPPORTED


def test_paged_plan_is_not_valid_for_the_plain_problem(lib):
    st, plan = plan_status(lib, paged())
    assert st == 0
    fake = ctypes.c_void_p(0x1000)
    assert lib.attn_decode_split(ctypes.byref(problem()), ctypes.byref(plan), fake, fake, fake,
                                 fake, 1 << 30, fake, 1 << 30, None) == ra.ATTN_ERR_ARG


@pytest.mark.parametrize("ps,kernel", [(1, 1), (16, 1), (64, 1), (256, 1), (24, 0), (48, 0)])
def test_paged_gqa_family_and_split_bound(lib, ps, kernel):
    # Power-of-two pages run on the GQA MFMA kernel, whose split must keep its
    # page ids (at most 8448 per split) in LDS; other page sizes run generic.
    lmax = 32768
    p = paged(ps=ps, lmax=lmax, batch=4)
    lens = [lmax, 100, 9000, 0]
    st, plan = plan_status(lib, p, 0, lens)
    assert st == 0
    assert plan.kernel == kernel
    if kernel == 1:
        assert (plan.chunk + ps - 1) // ps + 1 <= 8448
    _check_plan_invariants(p, plan, lens)
    st, plan = plan_status(lib, p, 1, lens)          # one split requested
    assert st == 0
    if kernel == 1:
        assert (plan.chunk + ps - 1) // ps + 1 <= 8448
        assert plan.s_max == math.ceil(lmax / plan.chunk)


@pytest.mark.parametrize("layout,kernel", [("page1", 2), ("page64", 2), ("page48", 0),
                                           ("indptr", 2)])
def test_mla_layout_family_and_split_bound(lib, layout, kernel):
    # Power-of-two pages and packed keys run on the MLA kernel, whose split
    # must keep its page ids (at most 4096) in LDS; other page sizes run generic.
    mla = dict(q_heads=16, kv_heads=1, head_dim_qk=576, head_dim_v=512)
    if layout.startswith("page"):
        ps = int(layout[4:])
        p = paged(ps=ps, lmax=20000, **mla)
    else:
        p = problem(kv_len_max=20000, **mla)
        p.kv_indptr = 0x3000
    for s_request in (0, 1):
        st, plan = plan_status(lib, p, s_request)
        assert st == 0 and plan.kernel == kernel
        if kernel == 2 and layout.startswith("page"):
            assert (plan.chunk + ps - 1) // ps + 1 <= 4096


# ------------------------------------------------------ RMSNorm + MatMul

def rms_problem(**kw):
    f = dict(dtype=ra.ATTN_BF16, y_dtype=ra.ATTN_BF16, m=32, k=4096, n=14336, eps=1e-5)
    f.update(kw)
    p = _lib.RmsProblem()
    for k, v in f.items():
        setattr(p, k, v)
    p.x_stride = kw.get("x_stride", p.k)
    p.w_stride = kw.get("w_stride", p.k)
    p.y_stride = kw.get("y_stride", p.n)
    return p


def rms_plan(lib, p, s_request=0, num_cus=256):
    cfg = _lib.RmsConfig()
    st = lib.rmsnorm_matmul_plan(ctypes.byref(p) if p is not None else None, s_request, num_cus,
                                 ctypes.byref(cfg))
    return st, cfg


@pytest.mark.parametrize("edit,code", [
    (dict(m=-1), ra.ATTN_ERR_ARG),
    (dict(k=0), ra.ATTN_ERR_ARG),
    (dict(eps=float("nan")), ra.ATTN_ERR_ARG),
    (dict(eps=-1.0), ra.ATTN_ERR_ARG),
    (dict(dtype=5), ra.ATTN_ERR_ARG),
    (dict(x_stride=100), ra.ATTN_ERR_ARG),          # shorter than a row
    (dict(dtype=ra.ATTN_F32), ra.ATTN_ERR_UNSUPPORTED),
    (dict(k=4100, x_stride=4100, w_stride=4100), ra.ATTN_ERR_UNSUPPORTED),  # k % 8
    (dict(w_stride=4100), ra.ATTN_ERR_UNSUPPORTED),  # stride % 8
])
def test_rms_invalid_problem(lib, edit, code):
    p = rms_problem(**edit)
    st, _ = rms_plan(lib, p)
    assert st == code and lib.attn_last_error()
    fake = ctypes.c_void_p(0x1000)
    cfg = _lib.RmsConfig()
    assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(cfg), fake, fake, fake, fake, fake,
                              1 << 30, None) == code


@pytest.mark.parametrize("m,k,n,s_req", [(32, 4096, 14336, 0), (32, 4096, 4096, 0), (1, 4096, 6144, 0),
                                         (255, 4096, 4096, 0), (300, 4104, 4096, 0), (300, 288, 300, 0),
                                         (5, 256, 200, 0),
                                         (5, 264, 70, 0), (32, 4096, 14336, 3), (32, 4096, 14336, 1000)])
def test_rms_plan_invariants(lib, m, k, n, s_req):
    st, cfg = rms_plan(lib, rms_problem(m=m, k=k, n=n, x_stride=k, w_stride=k, y_stride=n), s_req)
    assert st == 0
    assert cfg.kernel == 0      # fewer than 256 tokens, or k not a multiple of 64
    steps = -(-k // 32)
    assert cfg.k_chunk % 32 == 0 and cfg.s >= 1
    assert cfg.s * cfg.k_chunk >= k and (cfg.s - 1) * cfg.k_chunk < k   # no empty part
    assert cfg.s <= steps
    if s_req > 0:
        assert cfg.s <= s_req
    # tile_n weight rows (at most 64, a multiple of 4) x 32 tokens per
    # workgroup; the part's columns are split over its four waves.
    assert 16 <= cfg.tile_n <= 64 and cfg.tile_n % 4 == 0
    assert tuple(cfg.grid) == (-(-n // cfg.tile_n), cfg.s, -(-m // 32)) and cfg.block == 256
    assert cfg.ws_bytes == (cfg.s * m * (n + 1) * 4 if cfg.s > 1 else 0)
    if s_req == 0:
        # planner's choice: the most parts that still fit one round, at least
        # four k-steps per wave, and the tile that fills the compute units best
        tiles = cfg.grid[0] * cfg.grid[2]
        assert cfg.s <= max(1, min(256 // tiles, steps // 16))
        wgs = tiles * cfg.s
        fill = wgs / (-(-wgs // 256) * 256)
        for t in range(64, 15, -4):
            tt = -(-n // t) * -(-m // 32)
            s2 = max(1, min(256 // tt, steps // 16))
            s2 = -(-steps // -(-steps // s2))
            w2 = tt * s2
            assert fill >= w2 / (-(-w2 // 256) * 256) - 1e-9


def test_rms_plan_decode_shape_fills_the_gpu(lib):
    # N = 14336 weight rows on 256 CUs: 56-row tiles, 256 workgroups, one part
    # (64-row tiles would leave 32 CUs idle).
    st, cfg = rms_plan(lib, rms_problem(m=32, k=4096, n=14336, x_stride=4096, w_stride=4096,
                                        y_stride=14336))
    assert st == 0 and cfg.kernel == 0 and cfg.tile_n == 56 and cfg.s == 1
    assert tuple(cfg.grid) == (256, 1, 1)
    # 4096 rows: 64-row tiles and four parts fill the GPU as well.
    st, cfg = rms_plan(lib, rms_problem(m=32, k=4096, n=4096, x_stride=4096, w_stride=4096,
                                        y_stride=4096))
    assert st == 0 and cfg.tile_n == 64 and cfg.s == 4 and tuple(cfg.grid) == (64, 4, 1)


@pytest.mark.parametrize("m,k,n,s_req", [(256, 4096, 14336, 0), (300, 4096, 4096, 0),
                                         (4096, 4096, 14336, 5), (300, 320, 300, 0)])
def test_rms_plan_prefill_gemm(lib, m, k, n, s_req):
    # From 256 tokens on with k % 64 == 0: the tiled GEMM, one 256 x 256 output
    # tile per workgroup of 512 threads, s = 1 whatever was requested, and a
    # workspace for X * g as bf16 pairs (256-byte aligned) and the row scales.
    st, cfg = rms_plan(lib, rms_problem(m=m, k=k, n=n, x_stride=k, w_stride=k, y_stride=n), s_req)
    assert st == 0 and cfg.kernel == 1
    assert cfg.s == 1 and cfg.k_chunk == k and cfg.block == 512
    assert tuple(cfg.grid) == ((-(-m // 256)) * (-(-n // 256)), 1, 1)
    assert cfg.ws_bytes == (m * k * 4 + 255) // 256 * 256 + m * 4


def test_rms_workspace_and_plan_checks(lib):
    p = rms_problem()
    st, cfg = rms_plan(lib, p, 4)
    assert st == 0 and cfg.s == 4
    fake = ctypes.c_void_p(0x1000)
    assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(cfg), fake, fake, fake, fake, fake,
                              cfg.ws_bytes - 4, None) == ra.ATTN_ERR_WORKSPACE
    assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(cfg), fake, fake, fake, fake, None,
                              0, None) == ra.ATTN_ERR_WORKSPACE
    other = rms_problem(n=4096, y_stride=4096)
    assert lib.rmsnorm_matmul(ctypes.byref(other), ctypes.byref(cfg), fake, fake, fake, fake, fake,
                              1 << 40, None) == ra.ATTN_ERR_ARG
    bad = _lib.RmsConfig.from_buffer_copy(cfg)
    bad.k_chunk = 100                                     # not a multiple of 32
    assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(bad), fake, fake, fake, fake, fake,
                              1 << 40, None) == ra.ATTN_ERR_ARG
    for tile in (0, 2, 30, 68):                           # not a multiple of 4 in [4, 64]
        bad = _lib.RmsConfig.from_buffer_copy(cfg)
        bad.tile_n = tile
        assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(bad), fake, fake, fake, fake, fake,
                                  1 << 40, None) == ra.ATTN_ERR_ARG
    unaligned = ctypes.c_void_p(0x1008)
    assert lib.rmsnorm_matmul(ctypes.byref(p), ctypes.byref(cfg), unaligned, fake, fake, fake, fake,
                              1 << 40, None) == ra.ATTN_ERR_UNSUPPORTED
    empty = rms_problem(m=0)
    st, cfg0 = rms_plan(lib, empty)
    assert st == 0
    assert lib.rmsnorm_matmul(ctypes.byref(empty), ctypes.byref(cfg0), None, None, None, None, None,
                              0, None) == 0


# ----------------------------------------------------------------- SwiGLU

def sw_problem(**kw):
    f = dict(dtype=ra.ATTN_BF16, y_dtype=ra.ATTN_BF16, m=32, k=4096, n=14336)
    f.update({k: v for k, v in kw.items() if k in f or k == "reserved0"})
    p = _lib.SwigluProblem()
    for k, v in f.items():
        setattr(p, k, v)
    p.x_stride = kw.get("x_stride", p.k)
    p.wg_stride = kw.get("wg_stride", p.k)
    p.wu_stride = kw.get("wu_stride", p.k)
    p.y_stride = kw.get("y_stride", p.n)
    return p


def sw_plan(lib, p, s_request=0, num_cus=256):
    cfg = _lib.SwigluConfig()
    return lib.swiglu_plan(ctypes.byref(p), s_request, num_cus, ctypes.byref(cfg)), cfg


@pytest.mark.parametrize("edit,code", [
    (dict(m=-1), ra.ATTN_ERR_ARG),
    (dict(k=0), ra.ATTN_ERR_ARG),
    (dict(reserved0=3), ra.ATTN_ERR_ARG),
    (dict(wu_stride=10), ra.ATTN_ERR_ARG),
    (dict(dtype=ra.ATTN_F32), ra.ATTN_ERR_UNSUPPORTED),
    (dict(k=4100, x_stride=4104, wg_stride=4104, wu_stride=4104), ra.ATTN_ERR_UNSUPPORTED),
    (dict(wg_stride=4100), ra.ATTN_ERR_UNSUPPORTED),
])
def test_swiglu_invalid_problem(lib, edit, code):
    p = sw_problem(**edit)
    st, _ = sw_plan(lib, p)
    assert st == code and lib.attn_last_error()
    fake = ctypes.c_void_p(0x1000)
    cfg = _lib.SwigluConfig()
    assert lib.swiglu(ctypes.byref(p), ctypes.byref(cfg), fake, fake, fake, fake, fake, 1 << 30,
                      None) == code


@pytest.mark.parametrize("m,k,n,s_req", [(32, 4096, 14336, 0), (1, 4096, 14336, 0),
                                         (5, 256, 200, 0), (33, 264, 70, 3), (32, 4096, 14336, 999),
                                         (255, 4096, 14336, 0), (300, 4104, 200, 0), (300, 288, 200, 0)])
def test_swiglu_plan_invariants(lib, m, k, n, s_req):
    st, cfg = sw_plan(lib, sw_problem(m=m, k=k, n=n), s_req)
    assert st == 0 and cfg.kernel == 0
    assert cfg.k_chunk % 32 == 0 and cfg.s * cfg.k_chunk >= k and (cfg.s - 1) * cfg.k_chunk < k
    # tile_n output columns (at most 64, a multiple of 4) x 32 tokens per
    # workgroup; each part's columns are split over the two waves of a column
    # group.
    assert 16 <= cfg.tile_n <= 64 and cfg.tile_n % 4 == 0
    assert tuple(cfg.grid) == (-(-n // cfg.tile_n), cfg.s, -(-m // 32)) and cfg.block == 256
    assert cfg.ws_bytes == (2 * cfg.s * m * n * 4 if cfg.s > 1 else 0)
    if s_req == 0:
        assert cfg.grid[0] * cfg.grid[1] * cfg.grid[2] <= max(256, cfg.grid[0] * cfg.grid[2])


@pytest.mark.parametrize("m,k,n,s_req", [(256, 4096, 14336, 0), (4096, 4096, 14336, 7),
                                         (300, 320, 200, 0)])
def test_swiglu_plan_prefill_gemm(lib, m, k, n, s_req):
    # From 256 tokens on with k % 64 == 0: one GEMM of both MatMuls, a
    # 256-token x 128-column output tile (gate and up) per workgroup, no
    # workspace.
    st, cfg = sw_plan(lib, sw_problem(m=m, k=k, n=n), s_req)
    assert st == 0 and cfg.kernel == 1
    assert cfg.s == 1 and cfg.k_chunk == k and cfg.block == 512 and cfg.ws_bytes == 0
    assert tuple(cfg.grid) == ((-(-m // 256)) * (-(-n // 128)), 1, 1)


def test_swiglu_workspace_and_config_checks(lib):
    p = sw_problem()
    st, cfg = sw_plan(lib, p, 2)
    assert st == 0 and cfg.s == 2
    fake = ctypes.c_void_p(0x1000)
    assert lib.swiglu(ctypes.byref(p), ctypes.byref(cfg), fake, fake, fake, fake, fake,
                      cfg.ws_bytes - 4, None) == ra.ATTN_ERR_WORKSPACE
    other = sw_problem(n=4096)
    assert lib.swiglu(ctypes.byref(other), ctypes.byref(cfg), fake, fake, fake, fake, fake,
                      1 << 40, None) == ra.ATTN_ERR_ARG
    assert lib.swiglu(ctypes.byref(p), ctypes.byref(cfg), fake, ctypes.c_void_p(0x1004), fake, fake,
                      fake, 1 << 40, None) == ra.ATTN_ERR_UNSUPPORTED
    for tile in (0, 2, 30, 68):                           # not a multiple of 4 in [4, 64]
        bad = _lib.SwigluConfig.from_buffer_copy(cfg)
        bad.tile_n = tile
        assert lib.swiglu(ctypes.byref(p), ctypes.byref(bad), fake, fake, fake, fake, fake,
                          1 << 40, None) == ra.ATTN_ERR_ARG
    # The decode shape: 56-column tiles fill 256 CUs with one part.
    st, cfg1 = sw_plan(lib, p)
    assert st == 0 and cfg1.tile_n == 56 and cfg1.s == 1 and tuple(cfg1.grid) == (256, 1, 1)


def test_plan_generic_small_problem_one_tile_per_split(lib):
    # 256 keys (four 64-key tiles) x 2 KV heads do not fill 256 CUs: one tile
    # per split, so the latency is one tile's.
    p = problem(dtype=ra.ATTN_F32, o_dtype=ra.ATTN_F32, batch=1, q_heads=8, kv_heads=2,
                head_dim_qk=64, head_dim_v=64, kv_len_max=256)
    st, plan = plan_status(lib, p)
    assert st == 0 and plan.kernel == 0 and plan.s_max == 4 and plan.chunk == 64
    _check_plan_invariants(p, plan, [256])


def test_plan_generic_caps_splits_at_the_merge_table(lib):
    # 32768 keys = 512 tiles on one KV head: at most 64 splits (the most the
    # single-launch merge tabulates), whatever the GPU size.
    for cus in (256, 4096):
        p = problem(dtype=ra.ATTN_F32, o_dtype=ra.ATTN_F32, batch=1, q_heads=4, kv_heads=1,
                    head_dim_qk=64, head_dim_v=64, kv_len_max=32768)
        st, plan = plan_status(lib, p, num_cus=cus)
        assert st == 0 and plan.kernel == 0 and plan.s_max <= 64
        _check_plan_invariants(p, plan, [32768])
    # A problem that fills the GPU keeps at least two tiles per split.
    p = problem(dtype=ra.ATTN_F32, o_dtype=ra.ATTN_F32, batch=64, q_heads=8, kv_heads=2,
                head_dim_qk=64, head_dim_v=64, kv_len_max=4096)
    st, plan = plan_status(lib, p)
    assert st == 0 and plan.kernel == 0 and plan.chunk >= 128
