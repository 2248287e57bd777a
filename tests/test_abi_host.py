"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any launch (no GPU is touched: every
call here fails validation first, and validation makes no HIP call)."""

import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_rnn_gated_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    for n in names:
        assert n in exported, n
    L = B.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_contract_id_and_error_strings():
    cid = B.contract_id()
    assert cid.startswith("gdn-cpr/") and "eps=1e-6" in cid
    # the id ends in a digest of the sources and flags this library was built from
    from linear_attention_rnn_gated_amd.build import source_digest
    assert cid.endswith(";src=" + source_digest())
    assert B.contract_check(cid) == B.GDN_OK
    assert B.contract_check(cid[:-1] + ("0" if cid[-1] != "0" else "1")) == B.GDN_ERR_UNSUPPORTED
    assert B.lib().gdn_contract_check(None) == B.GDN_ERR_INVALID_ARG
    L = B.lib()
    for st in [0, -1, -2, -3, -4]:
        assert L.gdn_error_string(st).decode() not in ("", "unknown status")
    assert L.gdn_error_string(7).decode() == "unknown status"


def good_shape(**kw):
    base = dict(H_qk=2, H_v=4, d_k=128, d_v=128, C=64, in_dtype=B.GDN_BF16, qk_l2norm=1,
                scale=1.0)
    base.update(kw)
    return B.Shape(**base)


@pytest.mark.parametrize("kw,want", [
    (dict(d_k=64, d_v=64), B.GDN_ERR_UNSUPPORTED),
    (dict(C=32), B.GDN_ERR_UNSUPPORTED),
    (dict(d_k=16, d_v=16, C=64), B.GDN_ERR_UNSUPPORTED),
    (dict(d_v=16), B.GDN_ERR_UNSUPPORTED),
    (dict(H_v=3), B.GDN_ERR_UNSUPPORTED),
    (dict(H_qk=1, H_v=16), B.GDN_ERR_UNSUPPORTED),
    (dict(H_qk=0), B.GDN_ERR_INVALID_ARG),
    (dict(in_dtype=7), B.GDN_ERR_UNSUPPORTED),
    (dict(qk_l2norm=2), B.GDN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.GDN_ERR_INVALID_ARG),
])
def test_shape_claims(kw, want):
    s = good_shape(**kw)
    L = B.lib()
    assert L.gdn_workspace_bytes(ctypes.byref(s), 4, 1000, B.OP_PREFILL) == 0
    cu = (ctypes.c_int32 * 2)(0, 10)
    dummy = ctypes.c_void_p(16)
    st = L.gdn_prefill(ctypes.byref(s), 1, dummy, cu, dummy, dummy, dummy, dummy, dummy, None,
                       dummy, None, None, dummy, 1 << 40, None)
    assert st == want


def test_good_shape_sizes():
    s = good_shape()
    L = B.lib()
    a = L.gdn_workspace_bytes(ctypes.byref(s), 4, 1000, B.OP_PREFILL)
    b = L.gdn_workspace_bytes(ctypes.byref(s), 4, 2000, B.OP_PREFILL)
    c = L.gdn_workspace_bytes(ctypes.byref(s), 4, 1000, B.OP_FWD_BWD)
    d = L.gdn_workspace_bytes(ctypes.byref(s), 4, 0, B.OP_DECODE)
    assert 0 < a < b and a < c and d > 0
    assert L.gdn_workspace_bytes(ctypes.byref(s), 4, 1000, 9) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(s), -1, 1000, 0) == 0


def _prefill(cu_list, ws_bytes=1 << 40, ws=True, null_q=False):
    s = good_shape()
    L = B.lib()
    n = len(cu_list) - 1
    cu = (ctypes.c_int32 * len(cu_list))(*cu_list)
    dummy = ctypes.c_void_p(16)
    q = None if null_q else dummy
    return L.gdn_prefill(ctypes.byref(s), n, dummy, cu, q, dummy, dummy, dummy, dummy, None,
                         dummy, None, None, dummy if ws else None, ws_bytes, None)


def test_bad_cu_seqlens_rejected():
    assert _prefill([1, 5]) == B.GDN_ERR_INVALID_ARG          # does not start at 0
    assert _prefill([0, 9, 5]) == B.GDN_ERR_INVALID_ARG       # decreasing
    assert _prefill([0, 5], null_q=True) == B.GDN_ERR_INVALID_ARG


def test_workspace_checked():
    assert _prefill([0, 100], ws=False) == B.GDN_ERR_WORKSPACE
    assert _prefill([0, 100], ws_bytes=10) == B.GDN_ERR_WORKSPACE


def test_decode_validation():
    s = good_shape()
    L = B.lib()
    dummy = ctypes.c_void_p(16)
    cache = B.CacheStruct(16, 16, 16, 16, 16, 16, 16)
    ws = 1 << 40
    # NULL cache field
    bad = B.CacheStruct(16, 16, 16, None, 16, 16, 16)
    assert L.gdn_decode_step(ctypes.byref(s), 2, dummy, dummy, dummy, dummy, dummy,
                             ctypes.byref(bad), None, dummy, dummy, ws, None) == B.GDN_ERR_INVALID_ARG
    # pos_host out of range
    pos = (ctypes.c_int32 * 8)(0, 1, 2, 64, 0, 0, 0, 0)
    assert L.gdn_decode_step(ctypes.byref(s), 2, dummy, dummy, dummy, dummy, dummy,
                             ctypes.byref(cache), pos, dummy, dummy, ws,
                             None) == B.GDN_ERR_INVALID_ARG
    # workspace too small
    pos = (ctypes.c_int32 * 8)(*([0] * 8))
    assert L.gdn_decode_step(ctypes.byref(s), 2, dummy, dummy, dummy, dummy, dummy,
                             ctypes.byref(cache), pos, dummy, dummy, 8,
                             None) == B.GDN_ERR_WORKSPACE
    # NULL output
    assert L.gdn_decode_step(ctypes.byref(s), 2, dummy, dummy, dummy, dummy, dummy,
                             ctypes.byref(cache), pos, None, dummy, ws,
                             None) == B.GDN_ERR_INVALID_ARG


def test_cache_init_validation():
    s = good_shape()
    L = B.lib()
    bad = B.CacheStruct(16, None, 16, 16, 16, 16, 16)
    assert L.gdn_cache_init(ctypes.byref(s), 2, None, ctypes.byref(bad), None) == \
        B.GDN_ERR_INVALID_ARG
    assert L.gdn_cache_init(ctypes.byref(s), -1, None, ctypes.byref(bad), None) == \
        B.GDN_ERR_INVALID_ARG


def test_misaligned_pointers_rejected():
    s = good_shape()
    L = B.lib()
    cu = (ctypes.c_int32 * 2)(0, 10)
    a, m = ctypes.c_void_p(16), ctypes.c_void_p(20)
    st = L.gdn_prefill(ctypes.byref(s), 1, a, cu, a, a, m, a, a, None, a, None, None, a,
                       1 << 40, None)
    assert st == B.GDN_ERR_INVALID_ARG
    cache = B.CacheStruct(16, 16, 16, 20, 16, 16, 16)
    assert L.gdn_cache_init(ctypes.byref(s), 2, None, ctypes.byref(cache), None) == \
        B.GDN_ERR_INVALID_ARG


def test_chunked_baseline_claims():
    """The native-mixed baseline prefill runs at d = 128 only."""
    L = B.lib()
    cu = (ctypes.c_int32 * 2)(0, 10)
    a = ctypes.c_void_p(16)
    s16 = good_shape(d_k=16, d_v=16, C=16)
    assert L.gdn_prefill_chunked(ctypes.byref(s16), 1, a, cu, a, a, a, a, a, None, a, None, a,
                                 1 << 40, None) == B.GDN_ERR_UNSUPPORTED
    s = good_shape()
    assert L.gdn_workspace_bytes(ctypes.byref(s), 4, 1000, B.OP_PREFILL_CHUNKED) > 0
    assert L.gdn_prefill_chunked(ctypes.byref(s), 1, a, cu, a, a, a, a, a, None, a, None, None,
                                 1 << 40, None) == B.GDN_ERR_WORKSPACE


def test_prefill_continue_argument_checks():
    """Continuation: pos_host is required and must lie in [0, C); the
    workspace covers the buffered tokens."""
    L = B.lib()
    s = good_shape()
    cu = (ctypes.c_int32 * 3)(0, 10, 20)
    a = ctypes.c_void_p(16)
    cache = B.CacheStruct(*([16] * 7))
    big = 1 << 40
    args = lambda pos: (ctypes.byref(s), 2, a, cu, pos, a, a, a, a, a, ctypes.byref(cache), a,
                        None, a, big, None)
    assert L.gdn_prefill_continue(*args(None)) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_continue(*args((ctypes.c_int32 * 2)(0, 64))) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_continue(*args((ctypes.c_int32 * 2)(-1, 3))) == B.GDN_ERR_INVALID_ARG
    w_pre = L.gdn_workspace_bytes(ctypes.byref(s), 2, 20, B.OP_PREFILL)
    w_con = L.gdn_workspace_bytes(ctypes.byref(s), 2, 20, B.OP_PREFILL_CONTINUE)
    assert w_con > w_pre
    small = (ctypes.byref(s), 2, a, cu, (ctypes.c_int32 * 2)(3, 63), a, a, a, a, a,
             ctypes.byref(cache), a, None, a, w_pre, None)
    assert L.gdn_prefill_continue(*small) == B.GDN_ERR_WORKSPACE


def test_fwd_bwd_ex_grad_dtype_check():
    """gdn_fwd_bwd_ex takes grad_dtype GDN_F32 or GDN_BF16 only."""
    L = B.lib()
    s = good_shape()
    cu = (ctypes.c_int32 * 2)(0, 10)
    a = ctypes.c_void_p(16)
    args = lambda gd: (ctypes.byref(s), 1, a, cu, a, a, a, a, a, None, a, None, a, a, gd, a, a, a,
                       a, a, a, None, 0, None)
    assert L.gdn_fwd_bwd_ex(*args(7)) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_fwd_bwd_ex(*args(B.GDN_BF16)) == B.GDN_ERR_WORKSPACE


def test_host_copy_of_cu_seqlens_checked():
    """The binding takes a caller's host copy of cu_seqlens only as CPU int32
    of the same length."""
    import torch
    cu = torch.tensor([0, 5, 9], dtype=torch.int32)
    dev, host = B._cu_pair(cu, "cpu", None)
    assert host.tolist() == [0, 5, 9] and dev.dtype == torch.int32
    _, host = B._cu_pair(cu, "cpu", cu.clone())
    assert host.tolist() == [0, 5, 9]
    for bad in (cu.to(torch.int64), cu[:2].clone()):
        with pytest.raises(ValueError):
            B._cu_pair(cu, "cpu", bad)


def test_no_alloc_decode_validation():
    """gdn_decode_step_noalloc checks its arguments like gdn_decode_step and
    refuses a shape whose single sequence's resync factors exceed the fixed
    scratch (GDN_NOALLOC_SCRATCH_BYTES = 32 MiB), before any HIP call."""
    L = B.lib()
    a = ctypes.c_void_p(16)
    cache = B.CacheStruct(*([16] * 7))
    s = good_shape()
    pos = (ctypes.c_int32 * 8)(0, 1, 2, 64, 0, 0, 0, 0)
    assert L.gdn_decode_step_noalloc(ctypes.byref(s), 2, a, a, a, a, a, ctypes.byref(cache), pos,
                                     a, None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_decode_step_noalloc(ctypes.byref(s), 2, a, a, a, a, a, ctypes.byref(cache), None,
                                     None, None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_decode_step_noalloc(ctypes.byref(s), 0, a, a, a, a, a, ctypes.byref(cache), None,
                                     a, None) == B.GDN_OK
    # 1024 value heads at d = 128: 1024 * 64 * 257 * 4 bytes per sequence > 32 MiB
    big = good_shape(H_qk=128, H_v=1024)
    assert L.gdn_decode_step_noalloc(ctypes.byref(big), 1, a, a, a, a, a, ctypes.byref(cache),
                                     None, a, None) == B.GDN_ERR_WORKSPACE


def test_native_mixed_entry_points_validation():
    """The baseline's trainer step runs at d = 128 only; its decode step checks
    pointers before any launch."""
    L = B.lib()
    a = ctypes.c_void_p(16)
    cu = (ctypes.c_int32 * 2)(0, 10)
    s16 = good_shape(d_k=16, d_v=16, C=16)
    args = lambda s: (ctypes.byref(s), 1, a, cu, a, a, a, a, a, None, a, None, a, a, a, a, a, a,
                      a, a, a, 1 << 40, None)
    assert L.gdn_fwd_bwd_chunked(*args(s16)) == B.GDN_ERR_UNSUPPORTED
    s = good_shape()
    assert L.gdn_fwd_bwd_chunked(*(args(s)[:-3] + (a, 8, None))) == B.GDN_ERR_WORKSPACE
    assert L.gdn_decode_step_native(ctypes.byref(s), 2, a, a, a, a, a, None, a, None) == \
        B.GDN_ERR_INVALID_ARG
    assert L.gdn_decode_step_native(ctypes.byref(s), 2, a, a, ctypes.c_void_p(20), a, a, a, a,
                                    None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_decode_step_native(ctypes.byref(s), 0, a, a, a, a, a, a, a, None) == B.GDN_OK
