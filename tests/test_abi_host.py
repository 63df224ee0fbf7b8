"""The C ABI library on the host: it loads, exports every symbol include/fcp.h
declares, and its host-only calls (validation, workspace sizing, status text) behave.
A compute entry point is called here only with arguments it rejects before any HIP
call."""
import ctypes
import os
import re

import numpy as np
import pytest

import fcp_workloads as W
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs, PAIR_DTYPE

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_wise_varlen_amd import build
        build.build()
    return B.load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "fcp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(fcp_[a-z_]+)\s*\(", text))


def test_exports_every_declared_symbol(lib):
    decl = declared_symbols()
    assert decl == set(B.SYMBOLS)
    for name in decl:
        assert hasattr(lib, name), name
    assert B.fcp_abi_version() == 1


def test_status_strings(lib):
    for code in range(6):
        assert B.fcp_status_string(code)
    assert B.fcp_status_string(99) == "unknown status"


def _dims(**kw):
    base = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, q_rows=4096, kv_rows=4096,
                part_rows=4096 * 4)
    base.update(kw)
    return B.make_dims(**base)


def _pairs(rows):
    return np.array([tuple(r) for r in rows], dtype=PAIR_DTYPE)


GOOD = _pairs([(0, 0, 1024, 0, 1024, 0, 0, 1), (0, 1024, 1024, 0, 1024, 1024, 1024, 1),
               (0, 1024, 1024, 1024, 1024, 0, 2048, 1)])


@pytest.mark.parametrize("op", [B.FCP_OP_FWD, B.FCP_OP_MERGE, B.FCP_OP_BWD, B.FCP_OP_FWD_FUSED])
def test_valid_table(lib, op):
    assert B.fcp_validate(_dims(), GOOD, op) == B.FCP_OK
    assert B.fcp_workspace_bytes(_dims(), GOOD, op) > 0
    assert B.fcp_workspace_bytes(_dims(), GOOD[:0], op) == 0
    assert B.fcp_validate(_dims(), GOOD[:0], op) == B.FCP_OK


@pytest.mark.parametrize("dims_kw,code", [
    (dict(num_q_heads=0), B.FCP_ERR_INVALID_ARG),
    (dict(num_q_heads=12, num_kv_heads=8), B.FCP_ERR_UNSUPPORTED),
    (dict(num_q_heads=48, num_kv_heads=8), B.FCP_ERR_UNSUPPORTED),   # group 6
    (dict(head_dim=96), B.FCP_ERR_UNSUPPORTED),
    (dict(softmax_scale=-1.0), B.FCP_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), B.FCP_ERR_INVALID_ARG),
    (dict(q_rows=-1), B.FCP_ERR_INVALID_ARG),
    (dict(q_rows=1000), B.FCP_ERR_INVALID_ARG),     # pairs reach row 2048
    (dict(kv_rows=1000), B.FCP_ERR_INVALID_ARG),   # checked for fwd, bwd, fused
    (dict(part_rows=100), B.FCP_ERR_INVALID_ARG),
])
def test_bad_dims(lib, dims_kw, code):
    assert B.fcp_validate(_dims(**dims_kw), GOOD, B.FCP_OP_FWD) == code
    assert B.fcp_last_error()
    assert B.fcp_workspace_bytes(_dims(**dims_kw), GOOD, B.FCP_OP_FWD) == 0


@pytest.mark.parametrize("row,ops", [
    ((0, 0, 0, 0, 16, 0, 0, 1), "fmbu"),            # q_len 0
    ((0, 0, 16, 0, 0, 0, 0, 1), "fmbu"),            # kv_len 0
    ((0, -1, 16, 0, 16, 0, 0, 1), "fmbu"),          # negative start
    ((0, 4090, 16, 0, 16, 0, 0, 1), "fmbu"),        # past q_rows
    ((0, 0, 16, 4090, 16, 0, 0, 1), "fbu"),         # past kv_rows (merge reads no KV)
    ((0, 0, 16, 0, 16, 0, 0, 3), "fmbu"),           # unknown flag bit
    ((0, 0, 16, 0, 16, 0, 16380, 1), "fm"),         # partial rows past part_rows
])
def test_bad_pair(lib, row, ops):
    op_of = {"f": B.FCP_OP_FWD, "m": B.FCP_OP_MERGE, "b": B.FCP_OP_BWD, "u": B.FCP_OP_FWD_FUSED}
    bad = _pairs([row])
    for ch, op in op_of.items():
        want = B.FCP_ERR_INVALID_ARG if ch in ops else B.FCP_OK
        assert B.fcp_validate(_dims(), bad, op) == want, (row, ch)


def test_overlaps(lib):
    # overlapping partial-output rows: an error for fwd and merge
    dup = _pairs([(0, 0, 1024, 0, 1024, 0, 0, 1), (0, 1024, 1024, 0, 1024, 1024, 512, 1)])
    assert B.fcp_validate(_dims(), dup, B.FCP_OP_FWD) == B.FCP_ERR_INVALID_ARG
    assert B.fcp_validate(_dims(), dup, B.FCP_OP_MERGE) == B.FCP_ERR_INVALID_ARG
    assert B.fcp_validate(_dims(), dup, B.FCP_OP_BWD) == B.FCP_OK
    # partially overlapping Q ranges: fine for the per-pair forward, an error elsewhere
    part = _pairs([(0, 0, 1024, 0, 1024, 0, 0, 1), (0, 512, 1024, 0, 1024, 512, 1024, 1)])
    assert B.fcp_validate(_dims(), part, B.FCP_OP_FWD) == B.FCP_OK
    for op in (B.FCP_OP_MERGE, B.FCP_OP_BWD, B.FCP_OP_FWD_FUSED):
        assert B.fcp_validate(_dims(), part, op) == B.FCP_ERR_INVALID_ARG
        assert "overlap" in B.fcp_last_error()


def test_null_arguments(lib):
    f = lib.fcp_validate
    assert f(None, GOOD.ctypes.data_as(ctypes.c_void_p), 3, 0) == B.FCP_ERR_INVALID_ARG
    assert f(ctypes.byref(_dims()), None, 3, 0) == B.FCP_ERR_INVALID_ARG
    assert f(ctypes.byref(_dims()), None, 0, 0) == B.FCP_OK
    assert f(ctypes.byref(_dims()), GOOD.ctypes.data_as(ctypes.c_void_p), -1, 0) == \
        B.FCP_ERR_INVALID_ARG
    assert f(ctypes.byref(_dims()), GOOD.ctypes.data_as(ctypes.c_void_p), 3, 9) == \
        B.FCP_ERR_INVALID_ARG


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_workloads_validate(lib, cfg):
    wl = {1: W.config1, 2: W.config2, 3: W.config3, 4: W.config4}[cfg]()
    pairs = build_pairs(wl)
    dims = B.make_dims(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.q_rows, wl.kv_rows,
                       int(pairs["q_len"].sum()))
    for op in (B.FCP_OP_FWD, B.FCP_OP_MERGE, B.FCP_OP_BWD, B.FCP_OP_FWD_FUSED):
        assert B.fcp_validate(dims, pairs, op) == B.FCP_OK, B.fcp_last_error()
        assert B.fcp_workspace_bytes(dims, pairs, op) > 0


def test_noalloc_rejects_tables_beyond_its_static_scratch(lib):
    """fcp_block_attn_fwd_fused_noalloc keeps its work lists in a 4 MiB static device
    array: a table needing more (5e6 query rows -> 156 250 tiles of 32 rows, 5 MB of
    32-byte items) is refused with FCP_ERR_WORKSPACE before any HIP call, so fake
    (never dereferenced) tensor pointers serve here."""
    rows = 5_000_000
    dims = B.make_dims(8, 1, 64, rows, rows)
    pairs = _pairs([(0, 0, rows, 0, 1, 0, 0, 0)])
    assert B.fcp_validate(dims, pairs, B.FCP_OP_FWD_FUSED) == B.FCP_OK
    assert B.fcp_workspace_bytes(dims, pairs, B.FCP_OP_FWD_FUSED) > (4 << 20)
    fake = ctypes.c_void_p(1 << 20)
    arr = np.ascontiguousarray(pairs)
    st = lib.fcp_block_attn_fwd_fused_noalloc(ctypes.byref(dims), fake, fake, fake,
                                              arr.ctypes.data_as(ctypes.c_void_p), 1, fake,
                                              fake, None)
    assert st == B.FCP_ERR_WORKSPACE
    assert "static scratch" in B.fcp_last_error()
    # n_pairs == 0 is a no-op even with NULL tensors
    assert lib.fcp_block_attn_fwd_fused_noalloc(ctypes.byref(dims), None, None, None, None, 0,
                                                None, None, None) == B.FCP_OK


def test_plan_info(lib):
    """The scheduler summary: config 2's heaviest key tiles split into two parts of four
    query heads (the second starting at head 4); a 32K single sequence splits nothing."""
    wl = W.config2(0)
    pairs = build_pairs(wl)
    dims = B.make_dims(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.q_rows, wl.kv_rows)
    info = B.fcp_plan_info(dims, pairs, B.FCP_OP_BWD)
    assert info["split_tiles"] > 0 and info["slots"] == 2 * info["split_tiles"]
    assert info["multihead_parts"] == info["slots"]
    assert info["multihead_offset_parts"] == info["split_tiles"]
    assert info["ws_bytes"] == B.fcp_workspace_bytes(dims, pairs, B.FCP_OP_BWD)
    fwd = B.fcp_plan_info(dims, pairs, B.FCP_OP_FWD_FUSED)
    # one work item per 32-row tile of each distinct Q range (a Q segment here)
    assert fwd["kvitems"] == 0
    assert fwd["qitems"] == sum(-(-s.length // 32) for s in wl.q_segments())
    wl = W.config3(1024, True)
    pairs = build_pairs(wl)
    dims = B.make_dims(64, 8, 128, wl.q_rows, wl.kv_rows)
    info = B.fcp_plan_info(dims, pairs, B.FCP_OP_BWD)
    assert info["split_tiles"] == 0 and info["kvitems"] == 256
    bad = B.make_dims(64, 7, 128, 10, 10)
    with pytest.raises(B.FcpError):
        B.fcp_plan_info(bad, pairs, B.FCP_OP_BWD)


@pytest.mark.parametrize("hq,hkv,per_xcd", [(64, 8, 1), (16, 2, 1), (8, 1, 1), (128, 16, 2)])
def test_xcd_placement(lib, hq, hkv, per_xcd):
    """Workgroup b runs on XCD b % 8: the launch maps give each XCD as few KV heads as an
    even split allows (one when there are at most 8), with padding only where runs differ
    in length, and launch every unit once (checked in tests/sanitize)."""
    wl = W.config3(4096, True, hq=hq, hkv=hkv)
    pairs = build_pairs(wl)
    dims = B.make_dims(hq, hkv, 128, wl.q_rows, wl.kv_rows)
    for op in (B.FCP_OP_FWD_FUSED, B.FCP_OP_BWD):
        info = B.fcp_plan_info(dims, pairs, op)
        assert info["q_kvheads_per_xcd"] == per_xcd, info
        real_q = info["qitems"] * (hq // min(8, hq // hkv))
        assert info["q_workgroups"] >= real_q
        if op == B.FCP_OP_BWD:
            assert info["kv_kvheads_per_xcd"] == per_xcd, info
            assert info["q_workgroups"] + info["kv_workgroups"] == \
                real_q + info["kvitems"] * hkv + info["empty_workgroups"]
        if hkv % 8 == 0:
            assert info["empty_workgroups"] == 0
