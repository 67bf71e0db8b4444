"""hysparse_sparse_attn_noalloc (the sparse layer with the library's fixed
scratch instead of a caller workspace) gives the same outputs as
hysparse_sparse_attn with a workspace, bit for bit (the same kernels and
split plan), on consecutive calls whose second input is smaller, on the
one-query-row path (decode, per-query scores) and the score-block path; and
the outputs match the oracle.  Calls that would need more scratch than the
library holds are refused before anything is launched."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import assert_attn_close, dev_tensor, say

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


def _case(wl):
    inp = gen.make_inputs(wl)
    _, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    idx = orc.select_indices(S, wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    dt = wl.dtype
    return (inp, idx, dev_tensor(inp.q_sparse[0], dt), dev_tensor(inp.k, dt), dev_tensor(inp.v, dt),
            torch.from_numpy(idx).cuda(), torch.from_numpy(inp.gate_logits[0]).cuda())


def _both(wl, inp, idx, q, k, v, idx_t, gate):
    """The workspace call and the no-allocation call on the same inputs."""
    ref_out = hy.hysparse_sparse_attn(q, k, v, idx_t, wl.k_top, wl.score_block, wl.window, gate)
    out = torch.full_like(q, float("nan"))
    hy.hysparse_sparse_attn_noalloc(q, k, v, idx_t, wl.k_top, wl.score_block, wl.window, gate, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{wl.name}: no-allocation output differs from the workspace call"
    oracle = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, wl.score_block, wl.window, inp.gate_logits[0])
    assert_attn_close(out, oracle, wl.dtype, "no-allocation sparse layer")


@pytest.mark.parametrize("first,second", [
    # decode at 128K's head shape: a larger, then a smaller call (the second reuses the scratch)
    (W["decode128k"].replace(batch=2, kv_len=6000, k_top=512, n_sparse=1, n_planted=8),
     W["decode128k"].replace(batch=1, kv_len=1500, k_top=100, n_sparse=1, n_planted=4)),
    # decode at 8K's head shape, then per-query scores in prefill (score block 1)
    (W["decode8k"].replace(batch=4, kv_len=3000, k_top=300, n_sparse=1),
     W["decode8k"].replace(batch=1, q_len=40, kv_len=200, k_top=24, window=16, n_sparse=1)),
    # the score-block path (no scratch needed), then a fp32 decode
    (W["prefill32k"].replace(q_len=300, kv_len=300, k_top=96, n_sparse=1),
     W["tiny"].replace(batch=2, q_len=1, kv_len=300, k_top=32, n_sparse=1)),
])
def test_noalloc_matches_workspace_call(first, second):
    for wl in (first, second):
        say(f"no-allocation sparse layer B{wl.batch} Tq{wl.q_len} Tkv{wl.kv_len} K{wl.k_top} Sb{wl.score_block}")
        _both(wl, *_case(wl))


def test_noalloc_full_size_decode128k():
    """The 128K decode workload at full size, as bench.py times it."""
    wl = W["decode128k"].replace(n_sparse=1)
    say("no-allocation sparse layer decode128k full size")
    _both(wl, *_case(wl))


def test_noalloc_refuses_oversized_calls():
    wl = W["decode8k"].replace(batch=1, q_len=8192, kv_len=8192, k_top=2048, n_sparse=1)
    q = torch.zeros((1, 8192, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8192, 8, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((1, 8, 8192, 2048), dtype=torch.int32, device="cuda")
    gate = torch.zeros(32, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    desc = hy.make_desc(q, k)
    need = hy.hysparse_workspace_bytes(hy.HYS_OP_SPARSE, desc, 1, wl.k_top, wl.window)
    assert need > hy.hysparse_noalloc_scratch_bytes()
    with pytest.raises(hy.HysError) as e:
        hy.hysparse_sparse_attn_noalloc(q, k, k, idx, wl.k_top, 1, wl.window, gate, out)
    assert e.value.status == 5 and "fixed scratch" in str(e.value)
