"""The C ABI library on the CPU: it loads, exports every entry point the header
declares, and rejects invalid arguments synchronously, before any launch (only
argument checks run here; nothing touches a GPU)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hysparse.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def hs():
    from long_context_split_amd import hysparse
    return hysparse


def test_header_is_plain_c99():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_exports_every_declared_symbol(hs):
    names = _declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", hs.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (hs_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(hs.lib, n)


def test_version_and_strings(hs):
    assert hs.lib.hs_abi_version() == 3
    assert hs.status_string(0) == "HS_OK"
    assert hs.status_string(3) == "HS_ERR_WORKSPACE_TOO_SMALL"


def _cache(hs, dtype=1, head_dim=128, n_kv=1, lens=(100, 200), cap=1000, scales=False, starts=None):
    h_seq = np.asarray(lens, np.int32)
    h_start = np.asarray(starts if starts is not None else np.concatenate([[0], np.cumsum(lens)[:-1]]), np.int64)
    fake = 0x100000
    c = hs.hs_kv_cache(dtype, head_dim, n_kv, len(lens), cap, fake, fake * 2,
                       fake * 3 if scales else None, fake * 4 if scales else None, fake * 5,
                       h_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), fake * 6,
                       h_seq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    c._keep = (h_seq, h_start)
    return c


def _call_full(hs, c, p, q=0x200000, ws=0x300000, nbytes=1 << 40, q_dtype=1):
    return hs.lib.hs_full_attn_select(ctypes.byref(c), ctypes.byref(p), q, q_dtype, 0x400000, None, 0x500000,
                                      0x600000, None, ws, nbytes, None)


@pytest.mark.parametrize("mutate,code", [
    (dict(head_dim=64), 2),
    (dict(n_kv=0), 1),
    (dict(lens=(0, 10)), 1),
    (dict(lens=(600, 600)), 1),                 # rows past capacity
    (dict(starts=(-1, 0)), 1),
    (dict(dtype=2), 1),                         # FP8 without scale pointers
    (dict(dtype=1, scales=True), 1),            # scales on a bf16 cache
    (dict(dtype=7), 1),
])
def test_full_attn_select_rejects_bad_cache(hs, mutate, code):
    c = _cache(hs, **mutate)
    p = hs.params(32, 1)
    assert _call_full(hs, c, p) == code
    assert hs.last_error()


def test_full_attn_select_rejects_bad_params(hs):
    c = _cache(hs)
    assert _call_full(hs, c, hs.params(31, 1)) == 2                # G = 31: unsupported group size
    assert _call_full(hs, _cache(hs, n_kv=2), hs.params(33, 1)) == 1
    assert _call_full(hs, c, hs.params(32, 0)) == 1
    assert _call_full(hs, c, hs.params(32, 1, top_k=-1)) == 1
    assert _call_full(hs, c, hs.params(32, 1, top_k=0, window=0)) == 1
    assert _call_full(hs, c, hs.params(32, 1, softmax_scale=float("nan"))) == 1
    assert _call_full(hs, c, hs.params(32, 1), q=0x200004) == 1   # misaligned q
    assert _call_full(hs, c, hs.params(32, 1), q_dtype=2) == 1    # FP8 queries
    assert _call_full(hs, c, hs.params(32, 1), q=None) == 1
    assert _call_full(hs, c, hs.params(32, 1, select_block=32)) == 2   # block size other than 64


def test_workspace_size_and_too_small(hs):
    c = _cache(hs)
    p = hs.params(32, 1)
    need = hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(c), ctypes.byref(p))
    assert need > 0
    assert _call_full(hs, c, p, nbytes=need - 1) == 3
    assert _call_full(hs, c, p, ws=None, nbytes=0) in (1, 3)
    assert hs.lib.hs_sparse_attn_workspace_size(ctypes.byref(c), ctypes.byref(p)) > 0
    bad = _cache(hs, head_dim=64)
    assert hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(bad), ctypes.byref(p)) == 0


def test_sparse_attn_rejects(hs):
    c = _cache(hs)
    p = hs.params(32, 1)
    f = hs.lib.hs_sparse_attn
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, None, 0x500000, 0x400000, 0x300000, 1 << 40, None) == 1
    # fp32 queries take the split path, which needs a workspace
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 0, 0x700000, 0x500000, 0x400000, 0x300000, 0, None) == 3


def test_select_from_scores_rejects(hs):
    lens = np.array([10, 20], np.int32)
    lp = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = hs.lib.hs_select_from_scores
    assert f(None, 0x100000, lp, 2, 1, 1, 20, 4, 2, 0, 0x200000, 0x300000, None, 0, None) == 1
    assert f(0x100000, 0x100000, lp, 2, 1, 1, 15, 4, 2, 0, 0x200000, 0x300000, None, 0, None) == 1  # L > max_len
    assert f(0x100000, 0x100000, lp, 2, 1, 1, 20, -1, 2, 0, 0x200000, 0x300000, None, 0, None) == 1
    assert f(0x100000, 0x100000, lp, 2, 1, 1, 20, 4, 2, 16, 0x200000, 0x300000, 0x400000, 1 << 20, None) == 2
    big = np.array([3_000_000], np.int32)                     # more candidates than block keys fit in LDS
    bp = big.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert f(0x100000, 0x100000, bp, 1, 1, 1, 3_000_000, 1024, 128, 64, 0x200000, 0x300000, 0x400000, 1 << 40,
             None) == 2


def test_bridge_rejects(hs):
    t = _cache(hs, dtype=2, scales=True, lens=(1,), cap=1000)
    t2 = _cache(hs, dtype=0, lens=(1,), cap=1000)
    tp = (ctypes.POINTER(hs.hs_kv_cache) * 1)(ctypes.pointer(t))
    tp2 = (ctypes.POINTER(hs.hs_kv_cache) * 1)(ctypes.pointer(t2))
    w = (ctypes.c_void_p * 1)(0x800000)
    f = hs.lib.hs_kv_bridge
    assert f(0x900000, 100, 4096, 1, w, w, tp, 950, None) == 1        # offset + T > capacity
    assert f(0x900000, 100, 4000, 1, w, w, tp, 0, None) == 1          # d_model not a multiple of 64
    assert f(0x900000, 100, 4096, 1, w, w, tp2, 0, None) == 1         # fp32 target
    assert f(0x900000, 100, 4096, 1, w, w, tp, -1, None) == 1
    assert f(None, 100, 4096, 1, w, w, tp, 0, None) == 1
    assert f(0x900000, 100, 4096, 9, w, w, tp, 0, None) == 2
    assert f(0x900000, 0, 4096, 1, w, w, tp, 0, None) == 0            # nothing to do: no launch


def test_e4m3_check_rejects(hs):
    f = hs.lib.hs_e4m3_check
    assert f(None, None) == 1
    assert f(0x900004, None) == 1                                      # not 8-byte aligned


def test_append_rejects(hs):
    t = _cache(hs, dtype=2, scales=True, lens=(1,), cap=1000)
    tp = (ctypes.POINTER(hs.hs_kv_cache) * 1)(ctypes.pointer(t))
    w = (ctypes.c_void_p * 1)(0x800000)
    f = hs.lib.hs_kv_append

    def rows(*r):
        a = np.asarray(r, np.int64)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    big = 1 << 20
    a, p = rows(3, 999, 1000)
    assert f(0x900000, 3, 4096, 1, w, w, tp, 0xA00000, p, 0xB00000, big, None) == 1   # row 1000 outside capacity
    a, p = rows(3, -1)
    assert f(0x900000, 2, 4096, 1, w, w, tp, 0xA00000, p, 0xB00000, big, None) == 1   # negative row
    a, p = rows(5, 7, 5)
    assert f(0x900000, 3, 4096, 1, w, w, tp, 0xA00000, p, 0xB00000, big, None) == 1   # row named twice
    a, p = rows(5, 7)
    assert f(0x900000, 2, 4096, 1, w, w, tp, None, p, 0xB00000, big, None) == 1       # no device rows
    assert f(0x900000, 2, 4000, 1, w, w, tp, 0xA00000, p, 0xB00000, big, None) == 1   # d_model not a multiple of 64
    need = hs.lib.hs_kv_append_workspace_size(2, 4096, 1)
    assert need > 0
    assert f(0x900000, 2, 4096, 1, w, w, tp, 0xA00000, p, 0xB00000, need - 16, None) == 3   # workspace too small
    assert f(0x900000, 2, 4096, 1, w, w, tp, 0xA00000, p, None, 0, None) == 1          # no workspace
    assert f(0x900000, 0, 4096, 1, w, w, tp, None, None, None, 0, None) == 0           # nothing to do: no launch


def test_workspace_size_per_query_type(hs):
    """A bf16 plan exists up to 256 heads per KV head, an fp32 one up to 128: the size query answers
    with the largest plan that exists and leaves the caller's last error alone."""
    c = _cache(hs)
    assert _call_full(hs, c, hs.params(31, 1)) == 2                   # sets a last error
    before = hs.last_error()
    assert before
    for H in (32, 128, 256):
        assert hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(c), ctypes.byref(hs.params(H, 1))) > 0, H
    assert hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(c), ctypes.byref(hs.params(160, 1))) == 0
    assert hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(c), ctypes.byref(hs.params(512, 1))) == 0
    assert hs.last_error() == before
    # a G = 256 bf16 call with that workspace passes validation up to the launch (no device here:
    # a too-small workspace is the last check before it)
    need = hs.lib.hs_full_attn_select_workspace_size(ctypes.byref(c), ctypes.byref(hs.params(256, 1)))
    assert _call_full(hs, c, hs.params(256, 1), nbytes=need - 1) == 3
    assert _call_full(hs, c, hs.params(256, 1), q_dtype=0, nbytes=need) == 2   # fp32 queries: G <= 128
    assert _call_full(hs, c, hs.params(96, 1)) == 2                   # not a power of two


def test_output_alignment_and_list_limit(hs):
    c = _cache(hs)
    p = hs.params(32, 1)
    f = hs.lib.hs_full_attn_select

    def call(out=0x400000, lse=None, idx=0x500000, cnt=0x600000, sc=None, cache=c, prm=p):
        return f(ctypes.byref(cache), ctypes.byref(prm), 0x200000, 1, out, lse, idx, cnt, sc, 0x300000, 1 << 40, None)

    assert call(out=0x400008) == 1                                   # out: float4 stores
    assert call(lse=0x400002) == 1
    assert call(idx=0x500002) == 1
    assert call(cnt=0x600001) == 1
    assert call(sc=0x700002) == 1
    many = _cache(hs, lens=[1] * 70000, cap=70000)                   # more lists than a grid dimension holds
    assert call(cache=many) == 2
    assert "lists" in hs.last_error()
    s = hs.lib.hs_sparse_attn
    assert s(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x500000, 0x600000, 0x400008, 0x300000, 1 << 40,
             None) == 1
    assert s(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x500002, 0x600000, 0x400000, 0x300000, 1 << 40,
             None) == 1
    assert s(ctypes.byref(many), ctypes.byref(p), 0x200000, 1, 0x500000, 0x600000, 0x400000, 0x300000, 1 << 40,
             None) == 2


def test_sparse_attn_noalloc_rejects_before_launch(hs):
    """The no-workspace sparse layer validates like hs_sparse_attn, and refuses shapes whose
    partials exceed its static array, all before touching a device."""
    f = hs.lib.hs_sparse_attn_noalloc
    c = _cache(hs)
    p = hs.params(32, 1)
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, None, 0x500000, 0x400000, None) == 1
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x500000, 0x600000, 0x400008, None) == 1
    big = _cache(hs, dtype=0, lens=[1200] * 4096, cap=1200 * 4096)
    pb = hs.params(128, 1)
    assert f(ctypes.byref(big), ctypes.byref(pb), 0x200000, 0, 0x500000, 0x600000, 0x400000, None) == 2
    assert "static" in hs.last_error()


def test_prefill_chunk_rejects_before_launch(hs):
    """The chunk call checks both of its steps (and that they describe the same chunk) first."""
    f = hs.lib.hs_prefill_chunk
    tgt = _cache(hs, dtype=2, scales=True, lens=(1,), cap=1000)
    tp = (ctypes.POINTER(hs.hs_kv_cache) * 1)(ctypes.pointer(tgt))
    w = (ctypes.c_void_p * 1)(0x800000)
    one = _cache(hs, lens=(300,), cap=1000)
    two = _cache(hs, lens=(300, 200), cap=1000)
    p = hs.params(32, 100, 0, 128)
    args = lambda kv, prm, n, off, od=0: (ctypes.byref(kv), ctypes.byref(prm), 0x200000, 1, 0x400000, od, 0x900000,
                                          n, 512, 1, w, w, tp, off, None)
    assert f(*args(one, p, 100, 0, od=2)) == 1                      # output dtype neither F32 nor BF16
    assert f(*args(two, p, 100, 0)) == 1                            # two sequences
    assert f(*args(one, p, 99, 0)) == 1                             # q_tokens != n_tokens
    assert f(*args(one, p, 100, 950)) == 1                          # bridge rows past the target capacity
    assert f(*args(one, hs.params(32, 100, 0, 0), 100, 0)) == 1     # window < 1
    assert f(*args(one, hs.params(32, 400, 0, 128), 400, 0)) == 1   # more queries than cache rows


def test_swa_attn_out_rejects_before_launch(hs):
    """The sliding-window call with a chosen output type validates that type and everything else
    hs_swa_attn validates, before touching a device."""
    f = hs.lib.hs_swa_attn_out
    c = _cache(hs, lens=(300,), cap=1000)
    p = hs.params(32, 100, 0, 128)
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x400000, 2, None) == 1          # E4M3 output
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x400000, 7, None) == 1          # unknown dtype
    assert "output dtype" in hs.last_error()
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, 0x400008, 1, None) == 1          # misaligned out
    assert f(ctypes.byref(c), ctypes.byref(p), 0x200000, 1, None, 1, None) == 1              # NULL out
    assert f(ctypes.byref(c), ctypes.byref(hs.params(32, 100, 0, 0)), 0x200000, 1, 0x400000, 1, None) == 1
