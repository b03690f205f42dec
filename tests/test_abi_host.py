"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library loads, exports every entry point include/fa.h declares, rejects malformed
arguments with the documented status before any HIP call, and its block-list generator
agrees element for element with the oracle's own implementation of the pattern.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fa():
    import exact_block_sparse_amd as fa
    return fa


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"FA_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(fa):
    declared = declared_functions()
    assert set(declared) == set(fa.EXPORTS), declared
    so = ctypes.CDLL(fa.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name


def test_library_is_built_for_gfx950(fa):
    with open(fa.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


def test_status_strings(fa):
    for code, name in fa.FA_STATUS.items():
        assert fa.status_str(code) == name
    assert fa.status_str(12345) == "FA_ERR_UNKNOWN"


S = None


def strides(b, h, n):
    from exact_block_sparse_amd import Strides
    return Strides(b, h, n)


def call_fwd(fa, q=16, k=16, v=16, o=16, lse=16, B=1, H=1, N=64, d=128, st=(8192, 8192, 128),
             causal=0, scale=0.1):
    s = strides(*st)
    return fa.lib.fa_fwd(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(o),
                         ctypes.c_void_p(lse), B, H, N, d, s, s, s, s, causal, scale, None)


def test_fwd_argument_errors_before_any_hip_call(fa):
    # pointers are fake: every case must be rejected on the host before a launch
    assert call_fwd(fa, q=0) == 1                    # FA_ERR_NULL
    assert call_fwd(fa, lse=0) == 1
    assert call_fwd(fa, N=-1) == 2                   # FA_ERR_SHAPE
    assert call_fwd(fa, d=96) == 3                   # FA_ERR_HEADDIM
    assert call_fwd(fa, q=24) == 4                   # misaligned pointer -> FA_ERR_LAYOUT
    assert call_fwd(fa, st=(8192, 8192, 100)) == 4   # stride not a multiple of 8
    assert call_fwd(fa, st=(1 << 30, 1 << 30, 1 << 25)) == 4   # token stride past 32-bit tile offsets
    assert "token stride" in fa.lib.fa_last_error().decode()
    assert call_fwd(fa, B=2, H=1 << 10, N=(1 << 19) + 64) == 2   # more than 2^30 query rows
    assert call_fwd(fa, scale=float("inf")) == 8     # FA_ERR_ARG
    assert "scale" in fa.lib.fa_last_error().decode()
    assert call_fwd(fa, q=0, N=0) == 0               # empty problem: OK, nothing launched
    assert call_fwd(fa, q=0, B=0) == 0


def test_sparse_argument_errors(fa):
    s = strides(8192, 8192, 128)
    vp = ctypes.c_void_p
    f = fa.lib.fa_sparse_fwd
    args = lambda **kw: [vp(16)] * 5 + [1, 1, 256, 128, s, s, s, s, kw.get("bs", 128), vp(kw.get("off", 16)),
                                       vp(kw.get("idx", 16)), kw.get("nnz", 4), 1, 0.1, None]
    assert f(*args(bs=64)) == 2
    assert f(*args(off=0)) == 1
    assert f(*args(idx=0)) == 1
    assert f(*args(nnz=-1)) == 5


def test_bwd_workspace_rules(fa):
    assert fa.bwd_workspace_bytes(2, 32, 8192, 128) == 2 * 32 * 8192 * 8
    assert fa.bwd_workspace_bytes(1, 1, 3, 64) == 256
    assert fa.bwd_workspace_bytes(0, 1, 3, 64) == 0
    s = strides(8192, 8192, 128)
    vp = ctypes.c_void_p
    base = [vp(16)] * 9 + [1, 1, 64, 128] + [s] * 8 + [0, 0.1]
    assert fa.lib.fa_bwd(*base, vp(0), 0, None) == 6            # no workspace
    assert fa.lib.fa_bwd(*base, vp(16), 255, None) == 6          # too small
    assert fa.lib.fa_bwd(*base, vp(24), 4096, None) == 4         # misaligned


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful where no GPU is present")
def test_no_device_is_reported_not_faked(fa):
    assert call_fwd(fa) == 7                          # FA_ERR_HIP: no device, nothing ran
    assert "device" in fa.lib.fa_last_error().decode()


@pytest.mark.parametrize("nb,window,stride,causal,rule", [
    (1024, 8, 16, True, "strided"), (1024, 8, 16, True, "fixed"), (1, 8, 16, True, "strided"),
    (50, 3, 7, False, "strided"), (50, 0, 0, True, "strided"), (33, 40, 5, False, "fixed")])
def test_block_lists_equal_oracle(fa, nb, window, stride, causal, rule):
    off, idx = fa.make_block_lists(nb, window, stride, causal=causal, rule=rule)
    off2, idx2 = oracle.block_lists(nb, window, stride, causal=causal, rule=rule)
    assert off.dtype == np.int32 and idx.dtype == np.int32
    assert np.array_equal(off, off2) and np.array_equal(idx, idx2)
    fa.check_block_lists(off, idx, nb, causal=causal)


def test_block_lists_128k_totals(fa):
    off, idx = fa.make_block_lists(1024, 8, 16)
    assert int(off[-1]) == 41436 and int(np.diff(off).max()) == 72


def test_check_block_lists_rejects_malformed(fa):
    off, idx = fa.make_block_lists(20, 2, 4)
    bad = []
    i2 = idx.copy(); i2[5] = 25; bad.append((off, i2))                       # out of range
    i3 = idx.copy(); i3[1], i3[2] = i3[2], i3[1]; bad.append((off, i3))      # not ascending (block 2)
    o4 = off.copy(); o4[0] = 1; bad.append((o4, idx))                        # offsets[0] != 0
    o5 = off.copy(); o5[3] = o5[4] + 1; bad.append((o5, idx))                # decreasing
    for o, i in bad:
        with pytest.raises(fa.FaError) as e:
            fa.check_block_lists(o, i, 20, causal=True)
        assert e.value.name == "FA_ERR_LIST"
    # above the causal diagonal is fine without causal masking, rejected with it
    o6 = np.array([0, 2], dtype=np.int32)
    i6 = np.array([0, 0], dtype=np.int32)
    with pytest.raises(fa.FaError):
        fa.check_block_lists(o6, i6, 1)
    fa.check_block_lists(np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32), 2, causal=False)
    with pytest.raises(fa.FaError):
        fa.check_block_lists(np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32), 2, causal=True)


def test_make_block_lists_capacity(fa):
    off = np.zeros(11, np.int32)
    idx = np.zeros(3, np.int32)
    nnz = ctypes.c_int64(0)
    p = ctypes.POINTER(ctypes.c_int32)
    st = fa.lib.fa_make_block_lists(10, 2, 4, 1, 0, off.ctypes.data_as(p), idx.ctypes.data_as(p), 3,
                                    ctypes.byref(nnz))
    assert st == 9 and nnz.value > 3
    assert fa.lib.fa_make_block_lists(10, -1, 4, 1, 0, off.ctypes.data_as(p), idx.ctypes.data_as(p), 3,
                                      ctypes.byref(nnz)) == 8


# ----------------------------------------------------------------------------- general entry points
def make_desc(fa, **kw):
    x = fa.AttnDesc()
    x.B, x.H, x.H_kv, x.N, x.d, x.causal, x.scale = 1, 4, 2, 64, 128, 1, 0.1
    for k, v in kw.items():
        setattr(x, k, v)
    return x


def call_attn_fwd(fa, desc, q=16, k=16, v=16, o=16, lse=16, st=(8192, 8192, 128)):
    s = strides(*st)
    d = ctypes.byref(desc) if desc is not None else None
    return fa.lib.fa_attn_fwd(d, ctypes.c_void_p(q), s, ctypes.c_void_p(k), s, ctypes.c_void_p(v), s,
                              ctypes.c_void_p(o), s, ctypes.c_void_p(lse), None)


def call_attn_bwd(fa, desc, ws=16, ws_bytes=1 << 30):
    s = strides(8192, 8192, 128)
    p = ctypes.c_void_p(16)
    d = ctypes.byref(desc) if desc is not None else None
    return fa.lib.fa_attn_bwd(d, p, s, p, s, p, s, p, s, p, s, p, p, s, p, s, p, s, ctypes.c_void_p(ws), ws_bytes,
                              None)


def test_attn_desc_layout_matches_header(fa):
    # int64 x5, int + float sharing one 8-byte slot, 8-byte pointers and int64s up to
    # q_indices, then int dtype and three float descales
    assert ctypes.sizeof(fa.AttnDesc) == 128
    assert fa.AttnDesc.cu_seqlens.offset == 48 and fa.AttnDesc.q_indices.offset == 104
    assert fa.AttnDesc.dtype.offset == 112 and fa.AttnDesc.v_descale.offset == 124


def test_fp8_argument_errors(fa):
    ok = dict(dtype=1, q_descale=0.01, k_descale=0.02, v_descale=0.03)
    assert call_attn_fwd(fa, make_desc(fa, dtype=2)) == 8                      # unknown dtype
    assert call_attn_fwd(fa, make_desc(fa, **{**ok, "k_descale": float("inf")})) == 8
    assert call_attn_fwd(fa, make_desc(fa, **ok), st=(8192, 8192, 136)) == 4   # fp8 rows need 16-byte strides
    assert call_attn_bwd(fa, make_desc(fa, **ok)) == 8                         # backward is bf16 only
    assert "bf16" in fa.lib.fa_last_error().decode()
    assert call_attn_fwd(fa, make_desc(fa, B=0, **ok), q=0) == 0


def test_attn_fwd_argument_errors(fa):
    assert call_attn_fwd(fa, None) == 1                                  # NULL desc
    assert call_attn_fwd(fa, make_desc(fa, H_kv=3)) == 2                 # H not a multiple of H_kv
    assert call_attn_fwd(fa, make_desc(fa, H_kv=0)) == 2
    assert call_attn_fwd(fa, make_desc(fa, H_kv=-1)) == 2
    assert call_attn_fwd(fa, make_desc(fa, d=80)) == 3
    assert call_attn_fwd(fa, make_desc(fa, scale=float("nan"))) == 8
    assert call_attn_fwd(fa, make_desc(fa, cu_seqlens=16, total=-5)) == 2
    assert call_attn_fwd(fa, make_desc(fa), q=8) == 4                    # misaligned
    assert call_attn_fwd(fa, make_desc(fa), lse=0) == 1
    assert call_attn_fwd(fa, make_desc(fa, kv_indices=16)) == 1          # lists without offsets
    assert call_attn_fwd(fa, make_desc(fa, kv_offsets=16, block_size=64)) == 2
    assert call_attn_fwd(fa, make_desc(fa, kv_offsets=16, block_size=128, nnz=-1)) == 5
    assert call_attn_fwd(fa, make_desc(fa, kv_offsets=16, block_size=128, nnz=4)) == 1   # no indices
    # empty problems: nothing launched, no device needed
    assert call_attn_fwd(fa, make_desc(fa, B=0), q=0) == 0
    assert call_attn_fwd(fa, make_desc(fa, cu_seqlens=16, total=0), q=0) == 0


def call_attn_fwd_visits(fa, desc, visits=16):
    s = strides(8192, 8192, 128)
    p = ctypes.c_void_p(16)
    d = ctypes.byref(desc) if desc is not None else None
    return fa.lib.fa_attn_fwd_visits(d, p, s, p, s, p, s, p, s, p, ctypes.c_void_p(visits), None)


def test_attn_fwd_visits_argument_errors(fa):
    sparse = dict(kv_offsets=16, kv_indices=16, block_size=128, nnz=4)
    assert call_attn_fwd_visits(fa, make_desc(fa, **sparse), visits=0) == 1    # NULL log
    assert "visits" in fa.lib.fa_last_error().decode()
    assert call_attn_fwd_visits(fa, make_desc(fa)) == 8                        # dense: nothing to log
    assert "kv_offsets" in fa.lib.fa_last_error().decode()
    assert call_attn_fwd_visits(fa, None) == 1
    assert call_attn_fwd_visits(fa, make_desc(fa, B=0, **sparse)) == 0          # empty: nothing launched


def test_attn_bwd_argument_errors(fa):
    assert call_attn_bwd(fa, None) == 1
    assert call_attn_bwd(fa, make_desc(fa, H=6, H_kv=4)) == 2
    sparse = dict(kv_offsets=16, kv_indices=16, block_size=128, nnz=4)
    assert call_attn_bwd(fa, make_desc(fa, **sparse)) == 1               # key-side lists missing
    assert "q_offsets" in fa.lib.fa_last_error().decode()
    assert call_attn_bwd(fa, make_desc(fa, q_offsets=16, **sparse)) == 1
    assert call_attn_bwd(fa, make_desc(fa), ws=0) == 6
    # more than 2^29 query rows in one backward call (the forward takes up to 2^30)
    assert call_attn_bwd(fa, make_desc(fa, B=1, H=1 << 10, H_kv=1 << 10, N=(1 << 19) + 64)) == 2
    assert "query rows" in fa.lib.fa_last_error().decode()
    assert call_attn_bwd(fa, make_desc(fa, H=1 << 10, H_kv=1 << 10, N=1, cu_seqlens=16, total=(1 << 19) + 64)) == 2
    assert call_attn_bwd(fa, make_desc(fa), ws_bytes=100) == 6


def test_attn_workspace_bytes(fa):
    lib = fa.lib
    x = make_desc(fa, B=2, H=8, H_kv=2, N=1000)
    assert lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x)) == (2 * 8 * 1000 * 8 + 255) // 256 * 256
    x = make_desc(fa, B=3, H=8, H_kv=1, N=700, cu_seqlens=16, total=1234)
    assert lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x)) == (8 * 1234 * 8 + 255) // 256 * 256
    assert lib.fa_attn_bwd_workspace_bytes(None) == 0
    assert fa.attn_bwd_workspace_bytes(3, 8, 700, 128, total=1234) == (8 * 1234 * 8 + 255) // 256 * 256
    assert fa.attn_bwd_workspace_bytes(2, 8, 1000, 128) == fa.bwd_workspace_bytes(2, 8, 1000, 128)


def test_stored_ds_workspace_bytes(fa):
    # the stored-dS schedule: base workspace + (sparse) nnz int32 rounded to 256 + one bf16
    # 128 x 128 tile (32 KB) per (sequence, query head, visited pair of blocks)
    base = fa.bwd_workspace_bytes(2, 32, 8192, 128)
    assert fa.bwd_ds_workspace_bytes(2, 32, 8192, 128, causal=True) == base + 2 * 32 * (64 * 65 // 2) * 32768
    assert fa.bwd_ds_workspace_bytes(2, 32, 8192, 128, causal=False) == base + 2 * 32 * 64 * 64 * 32768
    n = -(-1000 // 128)
    assert fa.bwd_ds_workspace_bytes(1, 3, 1000, 128, causal=True) == (
        fa.bwd_workspace_bytes(1, 3, 1000, 128) + 3 * n * (n + 1) // 2 * 32768)
    assert fa.bwd_ds_workspace_bytes(1, 3, 1000, 64, causal=True) == 0      # head dimension 64: recomputation only
    assert fa.bwd_ds_workspace_bytes(0, 3, 1000, 128) == 0
    lib = fa.lib
    x = make_desc(fa, B=3, H=8, H_kv=2, N=700, cu_seqlens=16, total=1234, causal=1)
    n = -(-700 // 128)
    assert lib.fa_attn_bwd_ds_workspace_bytes(ctypes.byref(x)) == (
        lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x)) + 3 * 8 * n * (n + 1) // 2 * 32768)
    nnz = 777
    want = fa.attn_bwd_workspace_bytes(1, 16, 131072, 128) + (nnz * 4 + 255) // 256 * 256 + 16 * nnz * 32768
    assert fa.attn_bwd_ds_workspace_bytes(1, 16, 131072, 128, causal=True, nnz=nnz) == want
    assert fa.attn_bwd_ds_workspace_bytes(1, 16, 131072, 128, causal=True, nnz=0) == 0
    assert lib.fa_attn_bwd_ds_workspace_bytes(None) == 0
    x = make_desc(fa, B=1, H=1, H_kv=1, N=1 << 28, causal=0)                # 2^42 tiles of 32 KB: refused
    assert lib.fa_attn_bwd_ds_workspace_bytes(ctypes.byref(x)) == 0
    x.dtype = 1                                                              # fp8: no backward schedule stores dS
    assert lib.fa_attn_bwd_ds_workspace_bytes(ctypes.byref(x)) == 0


@pytest.mark.parametrize("nb,window,stride,causal,rule", [(1, 0, 0, True, "strided"), (37, 2, 5, True, "strided"),
                                                          (37, 2, 5, False, "fixed"), (64, 8, 16, True, "fixed"),
                                                          (20, 0, 0, False, "strided")])
def test_transposed_lists_equal_oracle(fa, nb, window, stride, causal, rule):
    off, idx = oracle.block_lists(nb, window, stride, causal, rule)
    t_off, t_idx = fa.transpose_block_lists(off, idx, nb)
    o_off, o_idx = oracle.transpose_lists(off, idx, nb)
    assert np.array_equal(t_off, o_off) and np.array_equal(t_idx, o_idx)


def test_transposed_lists_128k(fa):
    off, idx = fa.make_block_lists(1024, 8, 16, True, "strided")
    t_off, t_idx = fa.transpose_block_lists(off, idx, 1024)
    o_off, o_idx = oracle.transpose_lists(off, idx, 1024)
    assert np.array_equal(t_off, o_off) and np.array_equal(t_idx, o_idx) and t_off[-1] == 41436


def test_transpose_rejects_malformed(fa):
    with pytest.raises(fa.FaError) as e:
        fa.transpose_block_lists(np.array([0, 2, 3], np.int32), np.array([1, 0, 0], np.int32), 2)   # unsorted
    assert e.value.status == 5
    with pytest.raises(fa.FaError):
        fa.transpose_block_lists(np.array([0, 1, 2], np.int32), np.array([0, 2], np.int32), 2)      # out of range
    empty = fa.transpose_block_lists(np.zeros(4, np.int32), np.zeros(0, np.int32), 3)
    assert np.array_equal(empty[0], np.zeros(4, np.int32)) and empty[1].size == 0


def test_launch_work_item_limit(fa):
    """Grids stay below 2^31 work-items: many tiny sequences, and a packed batch with one long
    sequence among many, are rejected on the host although their row counts are allowed."""
    no_dev = torch.cuda.device_count() == 0
    accepted = 7 if no_dev else None     # past validation, then no device (FA_ERR_HIP)
    # B*H = 2^30 sequences of one row: 2^30 rows (allowed) but 2^30 workgroups
    assert call_fwd(fa, B=1 << 15, H=1 << 15, N=1) == 2
    assert "work-items" in fa.lib.fa_last_error().decode()
    # 1024 packed sequences, the longest 64K rows, 32 heads: 2.2M rows, 2^33 backward work-items
    skew = dict(B=1024, H=32, H_kv=32, N=1 << 16, cu_seqlens=16, total=(1 << 16) + 1023)
    assert call_attn_fwd(fa, make_desc(fa, **skew)) == 2
    assert call_attn_bwd(fa, make_desc(fa, **skew)) == 2
    assert "work-items" in fa.lib.fa_last_error().decode()
    # exactly at the limit: 2^30 forward rows of 128K tokens (2^31 work-items) and 2^29
    # backward rows (2^31); one more 256-row block of the forward is over
    if no_dev:
        assert call_fwd(fa, B=1, H=1 << 13, N=1 << 17) == accepted
        assert call_attn_bwd(fa, make_desc(fa, B=1, H=1 << 12, H_kv=1 << 12, N=1 << 17), ws_bytes=1 << 32) == accepted
    assert call_fwd(fa, B=1, H=(1 << 13) - 1, N=(1 << 17) + 256) == 2
