"""The C ABI library loads, exports what include/hysparse.h declares, and
rejects bad arguments on the host before launching anything.

These run without a GPU: every call here fails validation, which happens
before any HIP call (pointers are fake, never dereferenced).
"""
import ctypes
import os
import re

import pytest

from long_context_hybrid_amd import hysparse as hy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hysparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hy.LIB_PATH), reason="libhysparse.so not built")

FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10004)   # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(hysparse_\w+)\s*\(", text)))


def test_exports_match_header():
    L = hy.lib()
    names = declared_functions()
    assert set(names) == set(hy.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = hy.lib()
    assert L.hysparse_status_string(0) == b"ok"
    for s in range(1, 7):
        assert L.hysparse_status_string(s) not in (b"ok", b"unknown status")
    assert L.hysparse_status_string(99) == b"unknown status"
    assert L.hysparse_version() >= 100


def _desc(B=2, Tq=1, Tkv=256, Hq=8, Hkv=2, D=128, dtype=hy.HYS_BF16):
    d = hy.HysAttnDesc()
    d.batch, d.q_len, d.kv_len, d.n_q_heads, d.n_kv_heads, d.head_dim = B, Tq, Tkv, Hq, Hkv, D
    d.dtype, d.scale = dtype, 0.0
    for x, s in enumerate((Tq * Hq * D, Hq * D, D)):
        d.q_stride[x] = s
    for x, s in enumerate((Tkv * Hkv * D, Hkv * D, D)):
        d.kv_stride[x] = s
    return d


def _full(d, sb=1, q=FAKE, out=FAKE, scores=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return hy.lib().hysparse_full_attn_scores(ctypes.byref(d), q, FAKE, FAKE, sb, out, None, scores, ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda d: setattr(d, "q_len", 300), 2),          # q_len > kv_len
    (lambda d: setattr(d, "n_kv_heads", 3), 2),       # Hq % Hkv != 0
    (lambda d: setattr(d, "head_dim", 96), 3),        # unsupported head_dim
    (lambda d: setattr(d, "dtype", 7), 3),            # unknown dtype
    (lambda d: (setattr(d, "n_q_heads", 64), setattr(d, "n_kv_heads", 2)), 3),  # G = 32 > 16
    (lambda d: setattr(d, "batch", 0), 2),
    (lambda d: d.kv_stride.__setitem__(1, 100), 4),   # 200-byte token stride
    (lambda d: d.q_stride.__setitem__(2, -128), 2),
])
def test_desc_validation(mutate, status):
    d = _desc()
    mutate(d)
    assert _full(d) == status
    assert hy.lib().hysparse_last_error() != b""


def test_pointer_and_workspace_checks():
    d = _desc()
    L = hy.lib()
    assert _full(d, q=None) == 1
    assert _full(d, scores=FAKE_ODD) == 4
    assert _full(d, sb=32) == 3
    need = L.hysparse_workspace_bytes(hy.HYS_OP_FULL, ctypes.byref(d), 1, 1, 1)
    assert need > 0
    assert _full(d, ws=None, ws_bytes=0) == 5
    assert _full(d, ws_bytes=need - 1) == 5
    assert b"needed" in L.hysparse_last_error()


def test_topk_validation():
    L = hy.lib()
    assert L.hysparse_topk(FAKE, 4, 100, 100, None, 0, FAKE, FAKE, 1 << 30, None) == 2   # k < 1
    assert L.hysparse_topk(FAKE, 4, 100, 50, None, 8, FAKE, FAKE, 1 << 30, None) == 2    # stride < len
    assert L.hysparse_topk(FAKE, 4, 100, 102, None, 8, FAKE, FAKE, 1 << 30, None) == 4   # stride % 4
    assert L.hysparse_topk(None, 4, 100, 100, None, 8, FAKE, FAKE, 1 << 30, None) == 1
    assert L.hysparse_topk(FAKE, 0, 100, 100, None, 8, FAKE, None, 0, None) == 0        # empty: no-op
    # few long rows: the candidate filter runs in parts and needs a workspace,
    # a slot per part of min(part length, 12288) keys and indices
    assert L.hysparse_topk_workspace_bytes(16, 131072, 2048) >= 16 * 32 * 4096 * 8          # 32 parts of 4096
    assert L.hysparse_topk_workspace_bytes(16, 131072, 2048) < 16 * 32 * 12288 * 8
    assert L.hysparse_topk_workspace_bytes(255, 131072, 2048) >= 255 * 3 * 12288 * 8        # 3 parts of 45056
    assert L.hysparse_topk_workspace_bytes(4096, 32768, 2048) == 0                        # one workgroup per row
    assert L.hysparse_topk_workspace_bytes(16, 12288, 2048) == 0                          # rows fit the LDS
    assert L.hysparse_topk_workspace_bytes(-1, 131072, 2048) == 0
    assert L.hysparse_topk(FAKE, 16, 131072, 131072, None, 2048, FAKE, None, 0, None) == 5   # workspace missing


def test_sparse_and_hybrid_validation():
    L = hy.lib()
    d = _desc()
    args = lambda kt, w: (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, kt, 1, w, FAKE, FAKE, FAKE, 1 << 40, None)
    assert L.hysparse_sparse_attn(*args(0, 128)) == 2
    assert L.hysparse_sparse_attn(*args(64, 0)) == 2
    assert L.hysparse_sparse_attn(ctypes.byref(d), FAKE, FAKE, FAKE, None, 64, 1, 128, FAKE, FAKE, FAKE,
                                  1 << 40, None) == 1
    P = ctypes.c_void_p
    arr = (P * 2)(FAKE.value, None)
    outs = (P * 2)(FAKE.value, FAKE.value)
    st = L.hysparse_hybrid_block(ctypes.byref(d), FAKE, FAKE, FAKE, 2, arr, FAKE, 64, 1, 128, FAKE, outs,
                                 None, None, None, FAKE, 1 << 40, None)
    assert st == 1 and b"q_sparse" in L.hysparse_last_error()
    st = L.hysparse_hybrid_block(ctypes.byref(d), FAKE, FAKE, FAKE, -1, None, None, 64, 1, 128, FAKE, None,
                                 None, None, None, FAKE, 1 << 40, None)
    assert st == 2


def test_hier_validation():
    L = hy.lib()
    d = _desc(Tq=1, Tkv=4096)
    call = lambda dd, blk, keep, kt: L.hysparse_hier_select(ctypes.byref(dd), FAKE, FAKE, FAKE, blk, keep, kt, None,
                                                            None, FAKE, FAKE, 1 << 40, None)
    assert call(d, 0, 8, 64) == 2
    assert call(d, 128, 0, 64) == 2
    assert call(_desc(Tq=4, Tkv=4096), 128, 8, 64) == 3            # decode only
    assert L.hysparse_hier_select(ctypes.byref(d), FAKE, FAKE, None, 128, 8, 64, None, None, FAKE, FAKE,
                                  1 << 40, None) == 1
    assert L.hysparse_hier_workspace_bytes(ctypes.byref(d), 128, 8, 64) > 0


def test_hier_pool_and_pooled_select_validation():
    L = hy.lib()
    d = _desc(Tq=1, Tkv=1000)                                   # 8 blocks of 128
    pool = lambda dd, blk, m0, m1, kb, kbar=FAKE, k=FAKE: L.hysparse_hier_pool(ctypes.byref(dd) if dd else None, k,
                                                                               blk, m0, m1, kbar, kb, None)
    assert pool(None, 128, 0, 8, 8) == 1
    assert pool(d, 0, 0, 8, 8) == 2                             # block < 1
    assert pool(d, 128, -1, 8, 8) == 2                          # m_begin < 0
    assert pool(d, 128, 5, 4, 8) == 2                           # m_end < m_begin
    assert pool(d, 128, 0, 9, 9) == 2                           # past ceil(kv_len / block)
    assert pool(d, 128, 0, 8, 7) == 2                           # kbar_blocks too small
    assert pool(d, 128, 0, 8, 8, kbar=None) == 1
    assert pool(d, 128, 0, 8, 8, kbar=FAKE_ODD) == 4
    sel = lambda dd, kb, kbar=FAKE: L.hysparse_hier_select_pooled(ctypes.byref(dd), FAKE, kbar, kb, FAKE, 128, 4, 64,
                                                                  None, None, FAKE, FAKE, 1 << 40, None)
    assert sel(d, 7) == 2                                       # kbar_blocks too small
    assert sel(d, 8, kbar=None) == 1
    assert sel(_desc(Tq=4, Tkv=1000), 8) == 3                   # decode only


def test_workspace_query_grows_with_problem():
    L = hy.lib()
    small = L.hysparse_workspace_bytes(hy.HYS_OP_HYBRID, ctypes.byref(_desc(Tkv=1024)), 1, 64, 128)
    large = L.hysparse_workspace_bytes(hy.HYS_OP_HYBRID, ctypes.byref(_desc(Tkv=8192)), 1, 64, 128)
    assert 0 < small < large
    bad = _desc()
    bad.head_dim = 80
    assert L.hysparse_workspace_bytes(hy.HYS_OP_FULL, ctypes.byref(bad), 1, 1, 1) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    k = torch.zeros(1, 8, 1, 64)
    with pytest.raises(ValueError):
        hy.hysparse_full_attn_scores(q, k, k, 1)


def test_append_kv_validation():
    L = hy.lib()
    d = _desc(Tkv=100)
    assert L.hysparse_append_kv(None, FAKE, FAKE, 1, 0, FAKE, FAKE, None) == 1
    assert L.hysparse_append_kv(ctypes.byref(d), FAKE, FAKE, 0, 0, FAKE, FAKE, None) == 2      # n_new < 1
    assert L.hysparse_append_kv(ctypes.byref(d), FAKE, FAKE, 1, -1, FAKE, FAKE, None) == 2     # pos < 0
    assert L.hysparse_append_kv(ctypes.byref(d), FAKE, FAKE, 5, 96, FAKE, FAKE, None) == 2     # past capacity
    assert L.hysparse_append_kv(ctypes.byref(d), None, FAKE, 1, 0, FAKE, FAKE, None) == 1
    assert L.hysparse_append_kv(ctypes.byref(d), FAKE, FAKE, 1, 0, FAKE_ODD, FAKE, None) == 4
    bad = _desc(Tkv=100, D=96)
    assert L.hysparse_append_kv(ctypes.byref(bad), FAKE, FAKE, 1, 0, FAKE, FAKE, None) == 3    # head_dim
    # the query fields are not read: a query shape that the attention calls reject is fine here
    q_bad = _desc(Tq=500, Tkv=100, Hq=3)
    assert L.hysparse_append_kv(ctypes.byref(q_bad), FAKE, FAKE, 0, 0, FAKE, FAKE, None) == 2   # still n_new


def test_sparse_ex_validation():
    L = hy.lib()
    d = _desc(Tq=1, Tkv=256)
    w = hy.HysWindowKV()
    w.k, w.v = 0x10000, 0x20000
    for x, s in enumerate((128 * 2 * 128, 2 * 128, 128)):
        w.stride[x] = s
    w.ring = 100                                     # window 128 needs ring >= 128
    args = lambda win, gsb=0: (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, 1, 128, FAKE, gsb, 0, win, FAKE, FAKE,
                               1 << 30, None)
    assert L.hysparse_sparse_attn_ex(*args(ctypes.byref(w))) == 2
    assert L.hysparse_sparse_attn_ex(*args(None, gsb=-1)) == 2
    w.ring = 0
    w.stride[1] = 129                                # not a multiple of 16 bytes
    assert L.hysparse_sparse_attn_ex(*args(ctypes.byref(w))) == 4
    w.stride[1] = 2 * 128
    w.k = 0x10004                                    # misaligned buffer
    assert L.hysparse_sparse_attn_ex(*args(ctypes.byref(w))) == 4
    w.k = None
    assert L.hysparse_sparse_attn_ex(*args(ctypes.byref(w))) == 1


def test_ceiling_helpers_validation():
    L = hy.lib()
    assert L.hysparse_ceiling_workspace_bytes(18 << 20, 0) >= 4 * ((18 << 20) // 16 // 1024)
    assert L.hysparse_ceiling_workspace_bytes(0, 34816) >= 4 * (34816 // 64)
    assert L.hysparse_ceiling_workspace_bytes(-1, 0) == 0
    assert L.hysparse_ceiling_stream_read(FAKE, 100, FAKE, 1 << 20, None) == 2        # not a multiple of 16
    assert L.hysparse_ceiling_stream_read(FAKE_ODD, 4096, FAKE, 1 << 20, None) == 4
    assert L.hysparse_ceiling_stream_read(FAKE, 1 << 20, None, 0, None) == 5          # no sink
    assert L.hysparse_ceiling_stream_read(FAKE, 0, None, 0, None) == 0                # empty: no-op
    assert L.hysparse_ceiling_gather(FAKE, FAKE, 256, 100, FAKE, 10, 512, FAKE, 1 << 20, None) == 3   # row > 256 B
    assert L.hysparse_ceiling_gather(FAKE, FAKE, 128, 100, FAKE, 10, 256, FAKE, 1 << 20, None) == 4   # stride < row
    assert L.hysparse_ceiling_gather(FAKE, None, 256, 100, FAKE, 10, 256, FAKE, 1 << 20, None) == 1
    assert L.hysparse_ceiling_gather(FAKE, FAKE, 256, 100, FAKE, 10, 256, None, 0, None) == 5
    assert L.hysparse_ceiling_gather(FAKE, FAKE, 256, -1, FAKE, 10, 256, FAKE, 1 << 20, None) == 2


def test_noalloc_validation():
    """The no-allocation sparse layer validates like hysparse_sparse_attn and
    refuses, before any HIP call, shapes whose partial states exceed its
    fixed scratch."""
    L = hy.lib()
    assert L.hysparse_noalloc_scratch_bytes() == 16 << 20
    d = _desc()
    call = lambda d, sb=1, kt=64, w=16, q=FAKE, idx=FAKE: L.hysparse_sparse_attn_noalloc(
        ctypes.byref(d), q, FAKE, FAKE, idx, kt, sb, w, FAKE, FAKE, None)
    assert call(d, q=None) == 1
    assert call(d, q=FAKE_ODD) == 4
    assert call(d, kt=0) == 2
    assert call(d, w=0) == 2
    assert call(d, sb=32) == 3
    big = _desc(B=1, Tq=8192, Tkv=8192, Hq=32, Hkv=8)
    need = L.hysparse_workspace_bytes(hy.HYS_OP_SPARSE, ctypes.byref(big), 1, 2048, 128)
    assert need > L.hysparse_noalloc_scratch_bytes()
    assert call(big, kt=2048, w=128) == 5
    assert b"fixed scratch" in L.hysparse_last_error()


def test_check_indices_validation():
    L = hy.lib()
    assert L.hysparse_check_indices(FAKE, -1, 8, 100, None, FAKE, None) == 2
    assert L.hysparse_check_indices(FAKE, 4, 0, 100, None, FAKE, None) == 2
    assert L.hysparse_check_indices(FAKE, 4, 8, 0, None, FAKE, None) == 3
    assert L.hysparse_check_indices(FAKE, 4, 8, (1 << 19) + 1, None, FAKE, None) == 3
    assert L.hysparse_check_indices(None, 4, 8, 100, None, FAKE, None) == 1
    assert L.hysparse_check_indices(FAKE, 4, 8, 100, ctypes.c_void_p(0x10002), FAKE, None) == 4
    assert L.hysparse_check_indices(FAKE, 0, 8, 100, None, None, None) == 0   # empty: no-op
