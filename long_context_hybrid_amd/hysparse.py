"""ctypes binding of libhysparse (the HIP C ABI declared in include/hysparse.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Functions keep the C names:
``hysparse_full_attn_scores``, ``hysparse_topk``, ``hysparse_sparse_attn``,
``hysparse_hybrid_block``, ``hysparse_workspace_bytes``,
``hysparse_topk_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhysparse.so")

HYS_F32, HYS_BF16 = 0, 1
HYS_OP_FULL, HYS_OP_TOPK, HYS_OP_SPARSE, HYS_OP_HYBRID = 0, 1, 2, 3
STATUS = {0: "HYS_OK", 1: "HYS_ERR_NULL_PTR", 2: "HYS_ERR_BAD_SHAPE", 3: "HYS_ERR_UNSUPPORTED",
          4: "HYS_ERR_ALIGN", 5: "HYS_ERR_WORKSPACE", 6: "HYS_ERR_HIP"}

EXPORTS = ("hysparse_full_attn_scores", "hysparse_topk", "hysparse_sparse_attn", "hysparse_hybrid_block",
           "hysparse_workspace_bytes", "hysparse_topk_workspace_bytes", "hysparse_status_string",
           "hysparse_last_error", "hysparse_version", "hysparse_trace_begin", "hysparse_trace_end",
           "hysparse_trace_name", "hysparse_hier_select", "hysparse_hier_workspace_bytes", "hysparse_append_kv",
           "hysparse_sparse_attn_token_gate", "hysparse_sparse_attn_ex", "hysparse_hier_pool",
           "hysparse_hier_select_pooled", "hysparse_ceiling_workspace_bytes", "hysparse_ceiling_stream_read",
           "hysparse_ceiling_gather", "hysparse_sparse_attn_noalloc", "hysparse_noalloc_scratch_bytes",
           "hysparse_check_indices")


class HysWindowKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride", ctypes.c_int64 * 3),
                ("ring", ctypes.c_int32)]


class HysAttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3)]


class HysError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libhysparse.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m long_context_hybrid_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(HysAttnDesc)
    L.hysparse_full_attn_scores.argtypes = [D, _P, _P, _P, i32, _P, _P, _P, _P, sz, _P]
    L.hysparse_topk.argtypes = [_P, i64, i32, i64, _P, i32, _P, _P, sz, _P]
    L.hysparse_sparse_attn.argtypes = [D, _P, _P, _P, _P, i32, i32, i32, _P, _P, _P, sz, _P]
    L.hysparse_hybrid_block.argtypes = [D, _P, _P, _P, i32, ctypes.POINTER(_P), _P, i32, i32, i32, _P,
                                        ctypes.POINTER(_P), _P, _P, _P, _P, sz, _P]
    for f in ("hysparse_full_attn_scores", "hysparse_topk", "hysparse_sparse_attn", "hysparse_hybrid_block"):
        getattr(L, f).restype = i32
    L.hysparse_workspace_bytes.argtypes = [i32, D, i32, i32, i32]
    L.hysparse_workspace_bytes.restype = sz
    L.hysparse_topk_workspace_bytes.argtypes = [i64, i32, i32]
    L.hysparse_topk_workspace_bytes.restype = sz
    L.hysparse_status_string.argtypes = [i32]
    L.hysparse_status_string.restype = ctypes.c_char_p
    L.hysparse_last_error.argtypes = []
    L.hysparse_last_error.restype = ctypes.c_char_p
    L.hysparse_version.restype = i32
    L.hysparse_hier_select.argtypes = [D, _P, _P, _P, i32, i32, i32, _P, _P, _P, _P, sz, _P]
    L.hysparse_hier_select.restype = i32
    L.hysparse_hier_pool.argtypes = [D, _P, i32, i32, i32, _P, i32, _P]
    L.hysparse_hier_pool.restype = i32
    L.hysparse_hier_select_pooled.argtypes = [D, _P, _P, i32, _P, i32, i32, i32, _P, _P, _P, _P, sz, _P]
    L.hysparse_hier_select_pooled.restype = i32
    L.hysparse_hier_workspace_bytes.argtypes = [D, i32, i32, i32]
    L.hysparse_append_kv.argtypes = [D, _P, _P, i32, i32, _P, _P, _P]
    L.hysparse_sparse_attn_token_gate.argtypes = [D, _P, _P, _P, _P, i32, i32, i32, _P, i64, i64, _P, _P, sz, _P]
    L.hysparse_sparse_attn_token_gate.restype = i32
    L.hysparse_sparse_attn_ex.argtypes = [D, _P, _P, _P, _P, i32, i32, i32, _P, i64, i64,
                                          ctypes.POINTER(HysWindowKV), _P, _P, sz, _P]
    L.hysparse_sparse_attn_ex.restype = i32
    L.hysparse_append_kv.restype = i32
    L.hysparse_hier_workspace_bytes.restype = sz
    L.hysparse_sparse_attn_noalloc.argtypes = [D, _P, _P, _P, _P, i32, i32, i32, _P, _P, _P]
    L.hysparse_sparse_attn_noalloc.restype = i32
    L.hysparse_noalloc_scratch_bytes.argtypes = []
    L.hysparse_noalloc_scratch_bytes.restype = sz
    L.hysparse_check_indices.argtypes = [_P, i64, i32, i32, _P, _P, _P]
    L.hysparse_check_indices.restype = i32
    L.hysparse_ceiling_workspace_bytes.argtypes = [i64, i64]
    L.hysparse_ceiling_workspace_bytes.restype = sz
    L.hysparse_ceiling_stream_read.argtypes = [_P, i64, _P, sz, _P]
    L.hysparse_ceiling_stream_read.restype = i32
    L.hysparse_ceiling_gather.argtypes = [_P, _P, i64, i64, _P, i64, i32, _P, sz, _P]
    L.hysparse_ceiling_gather.restype = i32
    L.hysparse_trace_begin.argtypes = [_P, i32]
    L.hysparse_trace_begin.restype = None
    L.hysparse_trace_end.argtypes = []
    L.hysparse_trace_end.restype = i32
    L.hysparse_trace_name.argtypes = [i32]
    L.hysparse_trace_name.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise HysError(status, lib().hysparse_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return HYS_BF16
    if dt == torch.float32:
        return HYS_F32
    raise TypeError(f"unsupported dtype {dt}")


def make_desc(q: torch.Tensor, k: torch.Tensor, scale: float = 0.0) -> HysAttnDesc:
    """Descriptor for q [B, Tq, Hq, D] and k/v [B, Tkv, Hkv, D] (head_dim contiguous)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [B, T, H, D]")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("head_dim must be the contiguous axis")
    B, Tq, Hq, D = q.shape
    d = HysAttnDesc()
    d.batch, d.q_len, d.kv_len = B, Tq, k.shape[1]
    d.n_q_heads, d.n_kv_heads, d.head_dim = Hq, k.shape[2], D
    d.dtype = _dtype_code(q.dtype)
    d.scale = float(scale)
    for x in range(3):
        d.q_stride[x] = q.stride(x)
        d.kv_stride[x] = k.stride(x)
    return d


def hysparse_workspace_bytes(op: int, desc: HysAttnDesc, score_block: int, k_top: int = 1, window: int = 1) -> int:
    return int(lib().hysparse_workspace_bytes(op, ctypes.byref(desc), score_block, k_top, window))


def hysparse_topk_workspace_bytes(n_rows: int, row_len: int, k: int) -> int:
    return int(lib().hysparse_topk_workspace_bytes(n_rows, row_len, k))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if ws is not None:
        return ws
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _same_device(*ts):
    dev = ts[0].device
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on one device")
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return dev


def hysparse_full_attn_scores(q, k, v, score_block: int, out=None, lse=None, scores=None, want_lse: bool = True,
                              workspace=None, scale: float = 0.0):
    """Full-attention layer; returns (out, lse or None, scores)."""
    dev = _same_device(q, k, v)
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    desc = make_desc(q, k, scale)
    B, Tq, Hq, D = q.shape
    Hkv, Tkv = k.shape[2], k.shape[1]
    NB = -(-Tq // score_block)
    out = torch.empty((B, Tq, Hq, D), dtype=q.dtype, device=dev) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hkv, NB, Tkv), dtype=torch.float32, device=dev) if scores is None else scores
    ws = _workspace(hysparse_workspace_bytes(HYS_OP_FULL, desc, score_block), dev, workspace)
    _check(lib().hysparse_full_attn_scores(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), score_block, _ptr(out),
                                           _ptr(lse), _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(dev)))
    return out, lse, scores


def hysparse_topk(scores, k: int, valid_len=None, idx=None, workspace=None):
    """Top-K of each row of a 2-D float32 tensor (last axis contiguous)."""
    dev = _same_device(scores)
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.dtype != torch.float32:
        raise ValueError("scores must be a 2-D float32 tensor with contiguous rows")
    R, L = scores.shape
    idx = torch.empty((R, k), dtype=torch.int32, device=dev) if idx is None else idx
    if valid_len is not None and (valid_len.dtype != torch.int32 or valid_len.numel() != R):
        raise ValueError("valid_len must be int32 [n_rows]")
    ws = _workspace(hysparse_topk_workspace_bytes(R, L, k), dev, workspace)
    _check(lib().hysparse_topk(_ptr(scores), R, L, scores.stride(0) if R > 1 else L, _ptr(valid_len), k, _ptr(idx),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return idx


def hysparse_sparse_attn(q, k, v, idx, k_top: int, score_block: int, window: int, gate_logits, out=None,
                         workspace=None, scale: float = 0.0):
    """One sparse layer over the shared k, v at the given indices; returns out."""
    dev = _same_device(q, k, v, idx, gate_logits)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32 [B, Hkv, NB, k_top]")
    if gate_logits.dtype != torch.float32 or not gate_logits.is_contiguous():
        raise ValueError("gate_logits must be contiguous float32 [Hq]")
    desc = make_desc(q, k, scale)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev) if out is None else out
    ws = _workspace(hysparse_workspace_bytes(HYS_OP_SPARSE, desc, score_block, k_top, window), dev, workspace)
    _check(lib().hysparse_sparse_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), k_top, score_block,
                                      window, _ptr(gate_logits), _ptr(out), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)))
    return out


def hysparse_sparse_attn_noalloc(q, k, v, idx, k_top: int, score_block: int, window: int, gate_logits, out,
                                 scale: float = 0.0):
    """hysparse_sparse_attn with the library's fixed scratch instead of a
    workspace; out must be given (nothing is allocated).  Returns out."""
    dev = _same_device(q, k, v, idx, gate_logits, out)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32 [B, Hkv, NB, k_top]")
    if gate_logits.dtype != torch.float32 or not gate_logits.is_contiguous():
        raise ValueError("gate_logits must be contiguous float32 [Hq]")
    desc = make_desc(q, k, scale)
    _check(lib().hysparse_sparse_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), k_top,
                                              score_block, window, _ptr(gate_logits), _ptr(out), _stream(dev)))
    return out


def hysparse_noalloc_scratch_bytes() -> int:
    return int(lib().hysparse_noalloc_scratch_bytes())


def hysparse_sparse_attn_token_gate(q, k, v, idx, k_top: int, score_block: int, window: int, gate_logits,
                                    out=None, workspace=None, scale: float = 0.0):
    """One sparse layer with one gate logit per token and head: gate_logits
    float32 [B, Tq, Hq] (any strides on the batch and token axes, head axis
    contiguous); returns out."""
    dev = _same_device(q, k, v, idx, gate_logits)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32 [B, Hkv, NB, k_top]")
    B, Tq, Hq, _ = q.shape
    if gate_logits.dtype != torch.float32 or gate_logits.dim() != 3 or tuple(gate_logits.shape) != (B, Tq, Hq) \
            or gate_logits.stride(2) != 1:
        raise ValueError("gate_logits must be float32 [B, Tq, Hq] with the head axis contiguous")
    desc = make_desc(q, k, scale)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev) if out is None else out
    ws = _workspace(hysparse_workspace_bytes(HYS_OP_SPARSE, desc, score_block, k_top, window), dev, workspace)
    _check(lib().hysparse_sparse_attn_token_gate(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), k_top,
                                                 score_block, window, _ptr(gate_logits), gate_logits.stride(0),
                                                 gate_logits.stride(1), _ptr(out), _ptr(ws),
                                                 0 if ws is None else ws.numel(), _stream(dev)))
    return out


def hysparse_hybrid_block(q_full, k, v, q_sparse: Sequence[torch.Tensor], gate_logits, k_top: int,
                          score_block: int, window: int, out_full=None, out_sparse=None, lse=None, scores=None,
                          idx=None, want_scores: bool = True, workspace=None, scale: float = 0.0):
    """Full layer -> top-K -> len(q_sparse) sparse layers.  Returns a dict with
    out_full, out (list), lse, scores, idx (the last three may be None)."""
    dev = _same_device(q_full, k, v, *q_sparse)
    desc = make_desc(q_full, k, scale)
    B, Tq, Hq, D = q_full.shape
    Hkv, Tkv = k.shape[2], k.shape[1]
    NB = -(-Tq // score_block)
    N = len(q_sparse)
    for qs in q_sparse:
        if qs.shape != q_full.shape or qs.stride() != q_full.stride() or qs.dtype != q_full.dtype:
            raise ValueError("every q_sparse must match q_full in shape, strides and dtype")
    if N:
        if gate_logits.dtype != torch.float32 or not gate_logits.is_contiguous() or gate_logits.shape != (N, Hq):
            raise ValueError("gate_logits must be contiguous float32 [n_sparse, Hq]")
        _same_device(q_full, gate_logits)
    out_full = torch.empty(q_full.shape, dtype=q_full.dtype, device=dev) if out_full is None else out_full
    if out_sparse is None:
        out_sparse = [torch.empty(q_full.shape, dtype=q_full.dtype, device=dev) for _ in range(N)]
    if want_scores:
        scores = torch.empty((B, Hkv, NB, Tkv), dtype=torch.float32, device=dev) if scores is None else scores
        idx = torch.empty((B, Hkv, NB, k_top), dtype=torch.int32, device=dev) if idx is None else idx
    ws = _workspace(hysparse_workspace_bytes(HYS_OP_HYBRID, desc, score_block, k_top, window), dev, workspace)
    qs_arr = (_P * max(N, 1))(*[qs.data_ptr() for qs in q_sparse])
    os_arr = (_P * max(N, 1))(*[o.data_ptr() for o in out_sparse])
    _check(lib().hysparse_hybrid_block(ctypes.byref(desc), _ptr(q_full), _ptr(k), _ptr(v), N, qs_arr,
                                       _ptr(gate_logits) if N else None, k_top, score_block, window, _ptr(out_full),
                                       os_arr, _ptr(lse), _ptr(scores), _ptr(idx), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)))
    return {"out_full": out_full, "out": list(out_sparse), "lse": lse, "scores": scores, "idx": idx}


def hysparse_hier_workspace_bytes(desc: HysAttnDesc, block: int, n_keep: int, k_top: int) -> int:
    return int(lib().hysparse_hier_workspace_bytes(ctypes.byref(desc), block, n_keep, k_top))


def hysparse_hier_select(q, k, scores, block: int, n_keep: int, k_top: int, idx=None, block_scores=None,
                         blocks=None, want_blocks: bool = True, workspace=None, scale: float = 0.0):
    """Hierarchical token selection for decode; returns (idx, block_scores, blocks)."""
    dev = _same_device(q, k, scores)
    desc = make_desc(q, k, scale)
    B, Hkv, Tkv = q.shape[0], k.shape[2], k.shape[1]
    M = -(-Tkv // block)
    idx = torch.empty((B, Hkv, 1, k_top), dtype=torch.int32, device=dev) if idx is None else idx
    if want_blocks:
        block_scores = torch.empty((B, Hkv, M), dtype=torch.float32, device=dev) if block_scores is None else block_scores
        blocks = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=dev) if blocks is None else blocks
    ws = _workspace(hysparse_hier_workspace_bytes(desc, block, n_keep, k_top), dev, workspace)
    _check(lib().hysparse_hier_select(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(scores), block, n_keep, k_top,
                                      _ptr(block_scores), _ptr(blocks), _ptr(idx), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)))
    return idx, block_scores, blocks


def hysparse_hier_pool(k, block: int, kbar, m_begin: int = 0, m_end=None):
    """Pooled keys of blocks [m_begin, m_end) of the cache k [B, kv_len, Hkv, D]
    (a view of the tokens it holds now) into kbar [B, kbar_blocks, Hkv, D]
    float32 (contiguous); m_end defaults to ceil(kv_len / block)."""
    _same_device(k, kbar)
    if (kbar.dtype != torch.float32 or not kbar.is_contiguous() or kbar.dim() != 4 or kbar.shape[0] != k.shape[0]
            or kbar.shape[2:] != k.shape[2:]):
        raise ValueError("kbar must be contiguous float32 [B, kbar_blocks, Hkv, D]")
    m_end = -(-k.shape[1] // block) if m_end is None else m_end
    desc = make_desc(k, k)
    _check(lib().hysparse_hier_pool(ctypes.byref(desc), _ptr(k), block, m_begin, m_end, _ptr(kbar), kbar.shape[1],
                                    _stream(k.device)))
    return kbar


def hysparse_hier_select_pooled(q, k, kbar, scores, block: int, n_keep: int, k_top: int, idx=None, block_scores=None,
                                blocks=None, want_blocks: bool = True, workspace=None, scale: float = 0.0):
    """hysparse_hier_select with the pooled keys kbar [B, kbar_blocks, Hkv, D]
    float32 from hysparse_hier_pool; k (the cache view) supplies only the
    shape and strides of the call and is not read."""
    dev = _same_device(q, kbar, scores)
    if kbar.dtype != torch.float32 or not kbar.is_contiguous() or kbar.dim() != 4:
        raise ValueError("kbar must be contiguous float32 [B, kbar_blocks, Hkv, D]")
    desc = make_desc(q, k, scale)
    B, Hkv, Tkv = q.shape[0], k.shape[2], k.shape[1]
    M = -(-Tkv // block)
    idx = torch.empty((B, Hkv, 1, k_top), dtype=torch.int32, device=dev) if idx is None else idx
    if want_blocks:
        block_scores = torch.empty((B, Hkv, M), dtype=torch.float32, device=dev) if block_scores is None else block_scores
        blocks = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=dev) if blocks is None else blocks
    ws = _workspace(hysparse_hier_workspace_bytes(desc, block, n_keep, k_top), dev, workspace)
    _check(lib().hysparse_hier_select_pooled(ctypes.byref(desc), _ptr(q), _ptr(kbar), kbar.shape[1], _ptr(scores),
                                             block, n_keep, k_top, _ptr(block_scores), _ptr(blocks), _ptr(idx),
                                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return idx, block_scores, blocks


class KernelTrace:
    """Per-kernel timing through the library's trace hook.

    While the trace is active the library launches each kernel with a pair of
    these events, which take the dispatch's own begin and end times.  Usage::

        tr = KernelTrace(capacity_kernels=4096)
        tr.begin(); ...library calls...; rows = tr.end()   # [(name, ms), ...]
        tr.span_ms(0, 1)   # begin of kernel 0 to end of kernel 1
    """

    def __init__(self, capacity_kernels: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        self._hip.hipEventSynchronize.argtypes = [_P]
        self._hip.hipEventDestroy.argtypes = [_P]
        self.capacity = 2 * int(capacity_kernels)
        self.events = (_P * self.capacity)()
        for i in range(self.capacity):
            ev = _P()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev

    def begin(self) -> None:
        lib().hysparse_trace_begin(ctypes.cast(self.events, _P), self.capacity)

    def end(self):
        n = lib().hysparse_trace_end()
        names = [lib().hysparse_trace_name(i).decode() for i in range(n)]
        out = []
        if n:
            self._hip.hipEventSynchronize(self.events[2 * n - 1])
        for i in range(n):
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * i], self.events[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((names[i], float(ms.value)))
        self.count = n
        return out

    def span_ms(self, i: int, j: int) -> float:
        """Milliseconds from the begin of traced kernel i to the end of kernel
        j of the last trace (after end())."""
        if not (0 <= i <= j < getattr(self, "count", 0)):
            raise IndexError("kernel index outside the last trace")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * i], self.events[2 * j + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            for i in range(self.capacity):
                self._hip.hipEventDestroy(self.events[i])
        except Exception:
            pass


def hysparse_append_kv(k_new, v_new, k_cache, v_cache, pos: int):
    """Write the rows k_new/v_new [B, n, Hkv, D] (contiguous) into the cache
    tensors [B, capacity, Hkv, D] (head_dim contiguous) at token positions
    [pos, pos + n)."""
    _same_device(k_new, v_new, k_cache, v_cache)
    if k_new.shape != v_new.shape or k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k/v shapes or cache strides differ")
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("new rows must be contiguous [B, n, Hkv, D]")
    if k_new.dtype != k_cache.dtype or k_new.shape[0] != k_cache.shape[0] or k_new.shape[2:] != k_cache.shape[2:]:
        raise ValueError("new rows and cache disagree in dtype, batch, heads or head_dim")
    desc = make_desc(k_cache, k_cache)
    _check(lib().hysparse_append_kv(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), k_new.shape[1], pos,
                                    _ptr(k_cache), _ptr(v_cache), _stream(k_cache.device)))


def hysparse_sparse_attn_ex(q, k, v, idx, k_top: int, score_block: int, window: int, gate_logits,
                            own_k=None, own_v=None, ring: int = 0, out=None, workspace=None, scale: float = 0.0):
    """The general sparse layer: gate_logits float32 [Hq] (one per head) or
    [B, Tq, Hq] (one per token and head, head axis contiguous); own_k / own_v
    [B, rows, Hkv, D] (head_dim contiguous) the layer's own window keys/values
    (position p in row p % ring, or row p when ring == 0), or None for the
    shared cache.  Returns out."""
    dev = _same_device(q, k, v, idx, gate_logits)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32 [B, Hkv, NB, k_top]")
    B, Tq, Hq, _ = q.shape
    if gate_logits.dtype != torch.float32 or gate_logits.stride(-1) != 1:
        raise ValueError("gate_logits must be float32 with the head axis contiguous")
    if gate_logits.dim() == 1 and gate_logits.shape[0] == Hq:
        gsb, gst = 0, 0
    elif gate_logits.dim() == 3 and tuple(gate_logits.shape) == (B, Tq, Hq):
        gsb, gst = gate_logits.stride(0), gate_logits.stride(1)
    else:
        raise ValueError("gate_logits must be [Hq] or [B, Tq, Hq]")
    win = None
    if own_k is not None or own_v is not None:
        _same_device(q, own_k, own_v)
        if own_k.shape != own_v.shape or own_k.stride() != own_v.stride() or own_k.dtype != q.dtype \
                or own_k.dim() != 4 or own_k.stride(3) != 1 or own_k.shape[0] != B or own_k.shape[2:] != k.shape[2:]:
            raise ValueError("own_k / own_v must be matching [B, rows, Hkv, D] tensors of q's dtype")
        win = HysWindowKV()
        win.k, win.v = own_k.data_ptr(), own_v.data_ptr()
        for x in range(3):
            win.stride[x] = own_k.stride(x)
        win.ring = int(ring)
    desc = make_desc(q, k, scale)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev) if out is None else out
    ws = _workspace(hysparse_workspace_bytes(HYS_OP_SPARSE, desc, score_block, k_top, window), dev, workspace)
    _check(lib().hysparse_sparse_attn_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), k_top,
                                         score_block, window, _ptr(gate_logits), gsb, gst,
                                         ctypes.byref(win) if win is not None else None, _ptr(out), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(dev)))
    return out


def hysparse_ceiling_workspace_bytes(n_bytes: int, n_rows: int) -> int:
    return int(lib().hysparse_ceiling_workspace_bytes(n_bytes, n_rows))


def hysparse_ceiling_stream_read(buf, n_bytes: int, workspace=None):
    """Measurement helper: read the first n_bytes of the device tensor buf in
    one launch (nothing computed)."""
    dev = _same_device(buf)
    if n_bytes > buf.numel() * buf.element_size() or not buf.is_contiguous():
        raise ValueError("n_bytes exceeds the contiguous buffer")
    ws = _workspace(hysparse_ceiling_workspace_bytes(n_bytes, 0), dev, workspace)
    _check(lib().hysparse_ceiling_stream_read(_ptr(buf), n_bytes, _ptr(ws), 0 if ws is None else ws.numel(),
                                              _stream(dev)))


def hysparse_ceiling_gather(k, v, rows, workspace=None):
    """Measurement helper: read the K and V rows (last axis) of the contiguous
    caches k, v [..., D] at the flat row indices rows (int32) in one launch."""
    dev = _same_device(k, v, rows)
    if not (k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and rows.dtype == torch.int32
            and rows.is_contiguous()):
        raise ValueError("k, v must be matching contiguous tensors, rows contiguous int32")
    row_bytes = k.shape[-1] * k.element_size()
    n_buf = k.numel() // k.shape[-1]
    ws = _workspace(hysparse_ceiling_workspace_bytes(0, rows.numel()), dev, workspace)
    _check(lib().hysparse_ceiling_gather(_ptr(k), _ptr(v), row_bytes, n_buf, _ptr(rows), rows.numel(), row_bytes,
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))


HYS_IDX_DUPLICATE, HYS_IDX_OUT_OF_RANGE, HYS_IDX_ORDER = 1, 2, 4


def hysparse_check_indices(idx, row_len: int, valid_len=None, status=None):
    """Status bits of each index row (HYS_IDX_*; 0 = a valid top-K row) of a
    contiguous int32 tensor whose last axis holds the rows."""
    dev = _same_device(idx)
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.dim() < 1:
        raise ValueError("idx must be a contiguous int32 tensor")
    k = idx.shape[-1]
    R = idx.numel() // k
    if valid_len is not None and (valid_len.dtype != torch.int32 or valid_len.numel() != R):
        raise ValueError("valid_len must be int32 with one entry per row")
    status = torch.empty(idx.shape[:-1], dtype=torch.int32, device=dev) if status is None else status
    _check(lib().hysparse_check_indices(_ptr(idx), R, k, row_len, _ptr(valid_len), _ptr(status), _stream(dev)))
    return status
