"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before making any HIP call (so every
error path below runs without a GPU)."""
import ctypes
import os
import re

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import split_kv_decode_amd as m
from split_kv_decode_amd import mxfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfa.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MXFA_API\s+[\w\s\*]+?\b(mxfa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = m.lib()
    declared = header_functions()
    assert declared == sorted(mxfa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def header_arity():
    """Number of parameters of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m_ in re.finditer(r"MXFA_API\s+[\w\s\*]+?\b(mxfa_\w+)\s*\(([^)]*)\)", text):
        params = m_.group(2).strip()
        out[m_.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_the_header():
    L = m.lib()
    for name, n in header_arity().items():
        assert len(getattr(L, name).argtypes) == n, name


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mxfa.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines()
                       if " T " in l and l.split()[-1].startswith("mxfa_")})
    assert exported == header_functions()


def test_status_strings_and_version():
    for s in range(5):
        assert m.status_string(s).startswith("MXFA_")
    assert "unknown" in m.status_string(99)
    assert m.version() >= 100


def test_last_plan_before_any_call_is_an_error():
    import threading
    res = {}

    def worker():
        try:
            m.last_plan()
        except m.MxfaError as e:
            res["status"] = e.status
    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert res["status"] == mxfa.MXFA_ERR_INVALID_ARG


# ---------------------------------------------------------------- validation

def _call(**kw):
    """mxfa_fwd_kvcache with fake (never dereferenced) aligned pointers."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, sl=0, out=0x40000, lse=0x50000,
             B=2, Hq=8, Hkv=2, D=128, qLen=1, cap=64, causal=0, dtype=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return m.lib().mxfa_fwd_kvcache(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["sl"]),
                                    vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"], a["Hkv"],
                                    a["D"], a["qLen"], a["cap"], a["causal"], a["dtype"], None)


def _call_ws(num_splits=0, ws=None, ws_bytes=0, **kw):
    a = dict(q=0x10000, k=0x20000, v=0x30000, sl=0, out=0x40000, lse=0x50000,
             B=2, Hq=8, Hkv=2, D=128, qLen=1, cap=64, causal=0, dtype=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return m.lib().mxfa_fwd_kvcache_ws(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["sl"]),
                                       vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"], a["Hkv"],
                                       a["D"], a["qLen"], a["cap"], a["causal"], a["dtype"],
                                       num_splits, vp(ws), ws_bytes, None)


INV, UNS = mxfa.MXFA_ERR_INVALID_ARG, mxfa.MXFA_ERR_UNSUPPORTED


@pytest.mark.fakeptr
@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INV), (dict(k=0), INV), (dict(v=0), INV), (dict(out=0), INV),
    (dict(q=0x10008), INV), (dict(k=0x20004), INV), (dict(v=0x30002), INV),
    (dict(out=0x40001), INV), (dict(lse=0x50002), INV), (dict(sl=0x60001), INV),
    (dict(B=-1), INV), (dict(qLen=-2), INV), (dict(cap=-1), INV), (dict(Hq=0), INV),
    (dict(Hkv=0), INV), (dict(D=0), INV), (dict(Hq=6, Hkv=4), INV),
    (dict(causal=2), INV), (dict(causal=-1), INV), (dict(dtype=2), INV), (dict(dtype=-1), INV),
    (dict(B=2**30, cap=2**30), INV),                       # byte size overflow
    (dict(D=257), UNS), (dict(D=264), UNS), (dict(D=300), UNS), (dict(B=70000), UNS),
    (dict(cap=2**16, Hq=128, Hkv=128), UNS),               # cache past 2^30 bytes per sequence
    (dict(cap=1, Hq=8192, Hkv=8192), UNS),                 # 1024-token slack past 2^30 bytes
])
def test_invalid_arguments_rejected_before_any_hip_call(kw, status):
    assert _call(**kw) == status
    assert _call_ws(**kw) == status


def _call_paged(ws_entry=False, num_splits=0, **kw):
    """mxfa_fwd_kvcache_paged(_ws) with fake (never dereferenced) aligned pointers."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, bt=0x60000, sl=0, out=0x40000, lse=0x50000,
             B=2, Hq=8, Hkv=2, D=128, qLen=1, num_pages=8, page=16, max_pages=4, causal=0,
             dtype=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    args = (vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]), vp(a["sl"]), vp(a["out"]),
            vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["qLen"], a["num_pages"],
            a["page"], a["max_pages"], a["causal"], a["dtype"])
    if ws_entry:
        return m.lib().mxfa_fwd_kvcache_paged_ws(*args, num_splits, None, 0, None)
    return m.lib().mxfa_fwd_kvcache_paged(*args, None)


@pytest.mark.fakeptr
@pytest.mark.parametrize("kw,status", [
    (dict(bt=0), INV), (dict(bt=0x60002), INV), (dict(k=0), INV), (dict(q=0), INV),
    (dict(page=0), INV), (dict(page=-16), INV), (dict(max_pages=-1), INV),
    (dict(num_pages=-1), INV), (dict(num_pages=0), INV),
    (dict(page=8), UNS), (dict(page=24), UNS), (dict(page=1), UNS),
    (dict(page=1 << 17, Hq=64, Hkv=64), UNS),              # one page past 2^30 bytes
    (dict(page=1 << 20, max_pages=1 << 12), UNS),          # logical capacity past INT_MAX
    (dict(num_pages=1 << 40 >> 20, page=1 << 20, Hq=64, Hkv=64, max_pages=1), UNS),
    (dict(D=260), UNS), (dict(Hq=6, Hkv=4), INV), (dict(causal=3), INV), (dict(dtype=5), INV),
])
def test_paged_arguments_rejected_before_any_hip_call(kw, status):
    assert _call_paged(**kw) == status
    assert _call_paged(ws_entry=True, **kw) == status


@pytest.mark.fakeptr
def test_paged_empty_and_pageless_problems():
    assert _call_paged(B=0) == mxfa.MXFA_OK
    assert _call_paged(qLen=0) == mxfa.MXFA_OK
    assert _call_paged(ws_entry=True, num_splits=-1) == INV
    n = ctypes.c_size_t()
    L = m.lib()
    assert L.mxfa_workspace_size_paged(2, 8, 2, 128, 1, 12, 4, 0, 0, 0, ctypes.byref(n)) == UNS
    assert L.mxfa_workspace_size_paged(2, 8, 2, 128, 1, 16, -4, 0, 0, 0, ctypes.byref(n)) == INV
    assert L.mxfa_workspace_size_paged(2, 8, 2, 128, 1, 16, 4, 0, 0, 0, None) == INV


def _call_append(paged=False, **kw):
    """mxfa_fwd_kvcache(_paged)_append with fake (never dereferenced) aligned pointers."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, kn=0x70000, vn=0x80000, sl=0x90000,
             out=0x40000, lse=0x50000, bt=0x60000, B=2, Hq=8, Hkv=2, D=128, qLen=1,
             new_len=1, cap=64, num_pages=8, page=16, max_pages=4, causal=0, dtype=0,
             num_splits=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    if paged:
        return m.lib().mxfa_fwd_kvcache_paged_append(
            vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]), vp(a["kn"]), vp(a["vn"]),
            vp(a["sl"]), vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["D"],
            a["qLen"], a["new_len"], a["num_pages"], a["page"], a["max_pages"], a["causal"],
            a["dtype"], a["num_splits"], None, 0, None)
    return m.lib().mxfa_fwd_kvcache_append(
        vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["kn"]), vp(a["vn"]), vp(a["sl"]),
        vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["qLen"],
        a["new_len"], a["cap"], a["causal"], a["dtype"], a["num_splits"], None, 0, None)


@pytest.mark.fakeptr
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(new_len=-1), INV), (dict(sl=0), INV), (dict(sl=0x90002), INV),
    (dict(kn=0), INV), (dict(vn=0), INV), (dict(kn=0x70008), INV),
    (dict(k=0), INV), (dict(num_splits=-2), INV), (dict(D=272), UNS),
    (dict(qLen=0, k=0), INV),                    # the cache is still written
    (dict(new_len=2 ** 30, B=2 ** 15, Hkv=1024, Hq=1024), INV),   # k_new byte size
])
def test_append_arguments_rejected_before_any_hip_call(paged, kw, status):
    assert _call_append(paged=paged, **kw) == status


@pytest.mark.fakeptr
def test_append_empty_problems():
    assert _call_append(B=0) == mxfa.MXFA_OK
    assert _call_append(paged=True, B=0) == mxfa.MXFA_OK
    assert _call_append(qLen=0, new_len=0) == mxfa.MXFA_OK
    assert _call_append(paged=True, bt=0) == INV


def _call_varlen(**kw):
    """mxfa_fwd_varlen with fake (never dereferenced) aligned pointers."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, cq=0x90000, ck=0xA0000, out=0x40000,
             lse=0x50000, B=2, Hq=8, Hkv=2, D=128, total_q=5, total_k=100, max_q=4,
             max_k=80, causal=1, dtype=1, num_splits=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return m.lib().mxfa_fwd_varlen(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["cq"]),
                                   vp(a["ck"]), vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"],
                                   a["Hkv"], a["D"], a["total_q"], a["total_k"], a["max_q"],
                                   a["max_k"], a["causal"], a["dtype"], a["num_splits"], None, 0,
                                   None)


@pytest.mark.fakeptr
@pytest.mark.parametrize("kw,status", [
    (dict(cq=0), INV), (dict(ck=0), INV), (dict(cq=0x90002), INV), (dict(q=0), INV),
    (dict(k=0), INV), (dict(out=0x40004), INV), (dict(total_q=-1), INV),
    (dict(total_k=-1), INV), (dict(max_q=-1), INV), (dict(max_k=-1), INV),
    (dict(num_splits=-1), INV), (dict(D=258), UNS), (dict(Hq=3), INV),
    (dict(max_k=1 << 22, Hkv=128, Hq=128), UNS),           # one sequence past 2^30 bytes
])
def test_varlen_arguments_rejected_before_any_hip_call(kw, status):
    assert _call_varlen(**kw) == status


@pytest.mark.fakeptr
def test_varlen_empty_problems():
    assert _call_varlen(B=0) == mxfa.MXFA_OK
    assert _call_varlen(total_q=0, q=0, out=0) == mxfa.MXFA_OK
    assert _call_varlen(max_q=0) == mxfa.MXFA_OK


def _call_dkdv(**kw):
    a = dict(q=0x10000, k=0x20000, v=0x30000, sl=0, out=0x40000, lse=0x50000, B=2, Hq=8,
             Hkv=2, Dk=192, Dv=128, qLen=1, cap=64, causal=0, dtype=1, num_splits=0)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return m.lib().mxfa_fwd_kvcache_dkdv(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["sl"]),
                                         vp(a["out"]), vp(a["lse"]), a["B"], a["Hq"], a["Hkv"],
                                         a["Dk"], a["Dv"], a["qLen"], a["cap"], a["causal"],
                                         a["dtype"], a["num_splits"], None, 0, None)


@pytest.mark.fakeptr
@pytest.mark.parametrize("kw,status", [
    (dict(Dk=0), INV), (dict(Dv=-8), INV), (dict(Dk=257), UNS), (dict(Dv=264), UNS),
    (dict(Dv=300), UNS), (dict(q=0), INV), (dict(v=0x30008), INV), (dict(num_splits=-1), INV),
    (dict(cap=1 << 20, Hkv=8, Hq=8, Dk=256), UNS),         # a sequence past 2^30 bytes
])
def test_dkdv_arguments_rejected_before_any_hip_call(kw, status):
    assert _call_dkdv(**kw) == status


def test_plan_routes_head_dims():
    # 64 / 128 keep the VALU path for few rows; every other head shape takes
    # the matrix-core kernel with its padded tiles (fewer rows per block when wide)
    assert m.plan(4, 32, 8, 64, 1, 4096, 0, 1).path == 0       # 4 rows, head dim 64
    assert m.plan(4, 24, 8, 128, 1, 4096, 0, 1).path == 0      # 3 rows, head dim 128
    assert m.plan(4, 32, 8, 128, 1, 4096, 0, 1).path == 1      # 4 rows, head dim 128
    # (4 rows per kv head: the small 16-row variant up to 128 x 128 tiles)
    for D, rb in ((96, 16), (32, 16), (256, 16), (8, 16), (160, 16)):
        p = m.plan(4, 32, 8, D, 1, 4096, 0, 1)
        assert p.path == 1 and p.row_block == rb, D
    for D, rb in ((96, 64), (256, 16), (200, 16)):
        p = m.plan(4, 64, 2, D, 2, 4096, 0, 1, 3)                # 64 rows per kv head
        assert p.path == 1 and p.row_block == rb, D
    for rows, D, rb in ((32, 96, 32), (32, 128, 32), (32, 64, 32), (32, 256, 16),
                        (48, 128, 48), (40, 64, 48), (34, 96, 48), (48, 200, 16)):
        p = m.plan(4, rows // 2 * 2, 2, D, 2, 4096, 0, 1, 3)      # rows per kv head
        assert p.path == 1 and p.row_block == rb and p.rows == rows, (rows, D)
        assert p.head_block == (2 if rb in (32, 48) else 1), (rows, D)
    # head dims that are not multiples of 8: 16-row tiles, one kv head per
    # workgroup, one workgroup per CU in the balanced grid
    for D in (1, 3, 17, 36, 100, 129, 130, 255):
        for G, qLen in ((1, 1), (4, 1), (8, 8)):
            p = m.plan(4, 2 * G, 2, D, qLen, 4096, 0, 1, num_cus=256)
            assert (p.path, p.row_block, p.head_block) == (1, 16, 1), (D, G, qLen)
            assert p.schedule == 0 or p.grid_x == 256, (D, G, qLen)
    assert m.plan(1, 8, 2, 256, 1, 64, 0, 1).row_block == 16
    n = ctypes.c_size_t()
    assert m.lib().mxfa_workspace_size_dkdv(2, 8, 2, 192, 128, 1, 64, 0, 0, -1,
                                            ctypes.byref(n)) == INV


def test_plan_takes_16_row_tiles_when_64_row_tiles_leave_cus_idle():
    # (B, qLen, Hq, Hkv, D, kv_cap) -> row block, with the planner's own
    # partitions; the 64-row plan's busy workgroups decide (at most half the
    # CUs: 16-row tiles)
    cases = [((1, 32, 8, 2, 64, 128), 16),        # the tiny causal batch: 4 workgroups
             ((2, 8, 64, 8, 128, 1024), 16),      # one partition per stream on 64 rows
             ((4, 8, 64, 8, 128, 4096), 16),      # exactly half the CUs busy
             ((4, 8, 64, 8, 128, 8192), 64),      # every CU busy
             ((4, 8, 64, 8, 128, 32768), 64),     # the Llama-70B MTP batch
             ((16, 8, 64, 8, 128, 1100), 64),     # 138 busy
             ((24, 8, 64, 8, 128, 600), 16),      # 113 busy
             ((1, 8, 64, 8, 128, 32768), 64),
             ((1, 8, 64, 8, 128, 8192), 16),
             ((4, 4, 64, 8, 128, 32768), 32),     # 32 rows: two 16-row tiles per wave
             ((2, 4, 64, 8, 128, 1024), 16)]
    for (B, qLen, Hq, Hkv, D, cap), rb in cases:
        p = m.plan(B, Hq, Hkv, D, qLen, cap, 1, 1, 0, 256)
        assert p.path == 1 and p.row_block == rb, (B, qLen, Hq, Hkv, D, cap, p.as_dict())
        if rb == 16:
            assert p.head_block == 1 and p.schedule in (0, 1)
        # a forced partition count keeps the tile the head shape selects
        f = m.plan(B, Hq, Hkv, D, qLen, cap, 1, 1, 3, 256)
        rows = qLen * Hq // Hkv
        assert f.row_block == (32 if rows <= 32 else 48 if rows <= 48 else 64) and \
            f.schedule == 0, \
            (B, qLen, Hq, Hkv, D, cap)
    # the rule counts CUs: the same 4 x 4096 batch fills half of 128 CUs
    assert m.plan(4, 64, 8, 128, 8, 4096, 1, 1, 0, 128).row_block == 64


@pytest.mark.fakeptr
def test_empty_problem_is_a_no_op():
    assert _call(B=0) == mxfa.MXFA_OK
    assert _call(qLen=0) == mxfa.MXFA_OK
    assert _call(B=0, q=0, k=0, v=0, out=0) == mxfa.MXFA_OK
    assert _call_ws(qLen=0) == mxfa.MXFA_OK


@pytest.mark.fakeptr
def test_ws_rejects_negative_splits_and_misaligned_workspace():
    assert _call_ws(num_splits=-1) == INV
    assert _call_ws(ws=0x70010, ws_bytes=1 << 20) == INV


def test_workspace_size_argument_checks():
    n = ctypes.c_size_t()
    L = m.lib()
    assert L.mxfa_workspace_size(1, 8, 2, 128, 1, 64, 0, 0, 0, None) == INV
    assert L.mxfa_workspace_size(1, 8, 3, 128, 1, 64, 0, 0, 0, ctypes.byref(n)) == INV
    assert L.mxfa_workspace_size(1, 8, 2, 300, 1, 64, 0, 0, 0, ctypes.byref(n)) == UNS
    assert L.mxfa_workspace_size(1, 8, 2, 128, 1, 64, 0, 0, -3, ctypes.byref(n)) == INV


# ---------------------------------------------------------------- planner

SHAPES = [
    # B, Hq, Hkv, D, qLen, cap, causal, dtype
    (1, 8, 2, 64, 32, 128, 1, 0),
    (1, 32, 32, 128, 1, 1023, 0, 0),
    (1, 32, 32, 128, 8, 4096, 0, 0),
    (64, 32, 8, 128, 1, 16384, 0, 1),
    (16, 32, 8, 128, 1, 16384, 0, 0),
    (4, 64, 8, 128, 8, 32768, 1, 1),
    (3, 10, 2, 64, 3, 77, 1, 1),
    (2, 4, 4, 128, 1, 0, 0, 0),
    (1, 1, 1, 64, 1, 1, 0, 0),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7, 1000])
def test_plan_covers_the_cache_exactly(shape, num_splits):
    check_plan(*shape, num_splits)


@settings(max_examples=400, deadline=None, derandomize=True)
@given(B=st.integers(1, 70), G=st.sampled_from([1, 2, 3, 4, 5, 8, 16]),
       Hkv=st.integers(1, 12), D=st.sampled_from([64, 128]), qLen=st.integers(1, 40),
       cap=st.integers(0, 40000), causal=st.integers(0, 1), dt=st.integers(0, 1),
       num_splits=st.sampled_from([0, 0, 0, 1, 2, 5, 64, 100000]),
       cus=st.sampled_from([0, 80, 256, 304]))
def test_plan_invariants_over_random_shapes(B, G, Hkv, D, qLen, cap, causal, dt, num_splits,
                                            cus):
    check_plan(B, G * Hkv, Hkv, D, qLen, cap, causal, dt, num_splits, cus)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(B=st.integers(1, 40), G=st.sampled_from([1, 2, 4, 8]), Hkv=st.integers(1, 8),
       D=st.integers(1, 256), qLen=st.integers(1, 20), cap=st.integers(0, 20000),
       causal=st.integers(0, 1), num_splits=st.sampled_from([0, 0, 1, 3, 64]))
def test_plan_invariants_over_any_head_dim(B, G, Hkv, D, qLen, cap, causal, num_splits):
    check_plan(B, G * Hkv, Hkv, D, qLen, cap, causal, 1, num_splits)


def check_plan(B, Hq, Hkv, D, qLen, cap, causal, dt, num_splits, cus=0):
    """The plan routes the shape to the right kernel, covers every cache
    position with a non-empty partition and sizes the scratch for every
    partial result."""
    p = m.plan(B, Hq, Hkv, D, qLen, cap, causal, dt, num_splits, cus)
    assert p.num_cus == (cus if cus > 0 else 256)
    assert p.rows == (Hq // Hkv) * qLen
    cache_bytes = B * cap * Hkv * D * 2 * 2
    valu_stream = D == 128 and p.rows == 4 and cache_bytes >= 256 << 20
    if D % 8:
        # not a multiple of 8: 16-row tiles, one kv head per workgroup
        assert p.path == 1 and p.row_block == 16 and p.head_block == 1
    elif D not in (64, 128) or (p.rows >= (4 if D == 128 else 8) and not valu_stream):
        # matrix-core kernel: 16-row blocks up to 16 rows, 32 up to 32, 48 up
        # to 48, else 64 (other dims pad to tiles of 64, 128 or 256 channels;
        # 16 rows at 256); two kv heads per workgroup when Hkv is even and one
        # block holds every row.  With more than 16 rows the planner may still take
        # 16-row tiles when its first choice would leave most CUs without
        # work (its own partition count only; then one kv head per workgroup)
        tile = 64 if D <= 64 else 128 if D <= 128 else 256
        rb = (16 if (p.rows <= 16 and tile <= 128) or tile == 256
              else 32 if p.rows <= 32 else 48 if p.rows <= 48 else 64)
        pair = Hkv % 2 == 0 and p.rows <= rb
        assert p.path == 1
        if rb in (32, 48, 64) and p.row_block == 16:
            assert num_splits == 0 and p.head_block == 1 and tile <= 128
        else:
            assert p.row_block == rb and p.head_block == (2 if pair else 1)
    else:
        assert p.path == 0 and p.row_block in (1, 2, 4, 8) and p.row_block >= min(p.rows, 8)
        assert p.head_block in (1, 4, 8, 16)
    assert Hkv % p.head_block == 0
    streams = B * (Hkv // p.head_block) * -(-p.rows // p.row_block)
    tile_v = D if p.path == 0 else (64 if D <= 64 else 128 if D <= 128 else 256)
    entry = p.head_block * p.row_block * (tile_v + 1) * 4
    if p.schedule == 1:                      # balanced: planner's own choice only
        assert num_splits == 0 and p.combine == 1 and p.chunk == 0
        assert (p.grid_x, p.grid_y, p.grid_z) == (p.num_splits, 1, 1)
        assert p.grid_x == p.num_cus * (2 if p.path == 1 and p.row_block == 16 and D % 8 == 0
                                        else 1)
        assert p.workspace_bytes >= (p.num_splits + streams) * entry + (B + 2) * 8
        return
    S, C = p.num_splits, p.chunk
    assert S >= 1 and C >= 1
    if cap > 0:
        assert (S - 1) * C < cap <= S * C          # every partition non-empty at kv_cap
        if num_splits:
            assert S <= min(num_splits, cap)
    assert p.grid_x == S and p.grid_z == B
    assert p.grid_y == (Hkv // p.head_block) * -(-p.rows // p.row_block)
    assert p.combine == (1 if S > 1 else 0)
    if S > 1:
        assert p.workspace_bytes >= streams * S * entry
    else:
        assert p.workspace_bytes == 0


def test_balanced_schedule_is_chosen_for_long_ragged_batches():
    p = m.plan(64, 32, 8, 128, 1, 16384, 0, 1, 0, 256)
    assert p.schedule == 1 and p.grid_x == 256
    p = m.plan(64, 32, 8, 128, 1, 16384, 0, 1, 16, 256)
    assert p.schedule == 0 and p.num_splits == 16
    p = m.plan(2000, 32, 8, 128, 1, 4096, 0, 1, 0, 256)     # batch past the LDS table
    assert p.schedule == 0


def test_balanced_grid_is_one_resident_wave_of_workgroups():
    # matrix-core kernel: two workgroups per CU with 16-row tiles, else one;
    # VALU kernel: one per CU
    p = m.plan(2, 32, 8, 128, 1, 8192, 0, 1, 0, 256)
    assert p.path == 1 and p.row_block == 16 and p.grid_x == 512
    p = m.plan(64, 32, 32, 128, 1, 16384, 0, 1, 0, 256)
    assert p.path == 0 and p.schedule == 1 and p.grid_x == 256


def test_four_rows_take_the_valu_kernel_on_large_caches():
    # 4 rows per kv head at head dim 128: the 16-row matrix-core variant below
    # 256 MiB of cache, the VALU kernel from there
    small = m.plan(4, 32, 8, 128, 1, 8192, 0, 1)     # 134 MB
    large = m.plan(8, 32, 8, 128, 1, 8192, 0, 1)     # 268 MB
    assert small.path == 1 and small.row_block == 16
    assert large.path == 0 and large.row_block == 4
    assert m.plan(8, 32, 8, 64, 1, 16384, 0, 1).path == 0       # head dim 64: VALU below 8 rows
    assert m.plan(8, 40, 8, 128, 1, 8192, 0, 1).path == 1       # 5 rows: matrix core
    p = m.plan(4, 64, 8, 128, 8, 32768, 1, 1, 0, 256)
    assert p.path == 1 and p.schedule == 1 and p.grid_x == 256
    assert m.plan(4, 64, 8, 128, 8, 32768, 1, 1, 0, 80).grid_x == 80


def test_valu_head_blocks_follow_the_cache_size():
    # below 256 MiB of K/V: half a token row's heads per workgroup (4 at
    # head dim 128, 8 at 64); from 256 MiB on: the whole row (8, 16)
    for D, small_hb, big_hb in ((128, 4, 8), (64, 8, 16)):
        p = m.plan(1, 32, 32, D, 1, 4096, 0, 0, 0, 256)           # 8-16 MiB
        assert (p.path, p.head_block, p.layout) == (0, small_hb, 1)
        p = m.plan(1, 64, 32, D, 1, 4096, 0, 0, 0, 256)           # two rows
        assert (p.path, p.row_block, p.head_block, p.layout) == (0, 2, small_hb, 1)
        unit = 16 * 16 * 2 * D * 2                                 # bytes per token of capacity
        cap = -(-(256 << 20) // unit)                              # the first at 256 MiB or more
        p = m.plan(16, 16, 16, D, 1, cap, 0, 1, 0, 256)
        assert (p.path, p.head_block, p.layout) == (0, big_hb, 0)
        p = m.plan(16, 16, 16, D, 1, cap - 1, 0, 1, 0, 256)       # just under
        assert (p.path, p.head_block, p.layout) == (0, small_hb, 1)


def test_plan_fills_the_chip_at_low_batch():
    p = m.plan(1, 32, 32, 128, 1, 4096, 0, 0, 0, 256)
    assert p.grid_x * p.grid_y * p.grid_z >= 256       # at least one workgroup per CU
    p = m.plan(4, 64, 8, 128, 8, 32768, 1, 1, 0, 256)
    assert p.grid_x * p.grid_y * p.grid_z >= 256


def test_plan_rejects_bad_arguments():
    with pytest.raises(m.MxfaError):
        m.plan(1, 8, 2, 300, 1, 64)
    with pytest.raises(m.MxfaError):
        m.plan(1, 8, 2, 128, 1, 64, num_splits=-1)
    assert m.lib().mxfa_plan(1, 8, 2, 128, 1, 64, 0, 0, 0, 0, None) == INV


@pytest.mark.fakeptr
@pytest.mark.parametrize("src,nbytes,nt,sink,cus", [
    (0, 1 << 20, 1, 0x50000, 0),              # null source
    (0x10000, 1 << 20, 1, 0, 0),              # null sink
    (0x10008, 1 << 20, 1, 0x50000, 0),        # source not 16-byte aligned
    (0x10000, 1 << 20, 1, 0x50002, 0),        # sink not 4-byte aligned
    (0x10000, 0, 1, 0x50000, 0),              # nothing to read
    (0x10000, 1000, 1, 0x50000, 0),           # not a multiple of 16 bytes
    (0x10000, (1 << 31) + 16, 1, 0x50000, 0), # past 2^31 bytes
    (0x10000, 1 << 20, 2, 0x50000, 0),        # policy flag not 0 / 1
    (0x10000, 1 << 20, 0, 0x50000, 5000),     # absurd CU count
])
def test_read_probe_rejects_bad_arguments(src, nbytes, nt, sink, cus):
    vp = lambda x: ctypes.c_void_p(x) if x else None
    st = m.lib().mxfa_read_probe(vp(src), nbytes, nt, vp(sink), cus, None)
    assert st == mxfa.MXFA_ERR_INVALID_ARG


def test_fake_pointer_tests_with_the_gpu_hidden():
    """Where a GPU is visible the fake-pointer tests are skipped in this
    process; here they run in a child process with every GPU hidden, and the
    child's own collection check skips them again if it still sees one."""
    import subprocess
    import sys

    import conftest
    if not conftest.gpu_visible():
        pytest.skip("no GPU is visible: the fake-pointer tests run directly")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1",
               ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-m", "pytest", __file__, "-q", "-m", "fakeptr",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       timeout=600)
    print(r.stdout[-2000:], r.stderr[-2000:])
    if "skipped" in r.stdout and "passed" not in r.stdout:
        pytest.skip("the child process still saw a GPU")
    assert r.returncode == 0, r.stdout[-2000:]
