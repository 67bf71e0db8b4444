"""GPU parity of the sparse layer whose window branch reads the layer's own
window keys/values (a ring of recent positions in decode, a position-indexed
buffer in prefill), alone and with per-token gates."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import assert_attn_close, dev_tensor, say

pytestmark = pytest.mark.gpu
W = gen.WORKLOADS

CASES = {  # name: (workload, score block, ring length or 0)
    "decode_ring": (W["decode8k"].replace(batch=2, kv_len=3000, k_top=300, n_sparse=1), 1, 160),
    "decode_ring_exact": (W["decode128k"].replace(batch=1, kv_len=2000, k_top=256, n_sparse=1, n_planted=0), 1, 128),
    "decode_linear": (W["decode8k"].replace(batch=2, kv_len=1000, k_top=100, n_sparse=1), 1, 0),
    "prefill_blocks_linear": (W["prefill32k"].replace(q_len=300, kv_len=300, k_top=100, window=50, n_sparse=1), 64, 0),
    "prefill_rows_ring": (W["prefill32k"].replace(q_len=100, kv_len=300, k_top=64, window=50, n_sparse=1), 1, 160),
    "prefill_blocks_ring": (W["prefill32k"].replace(q_len=256, kv_len=700, k_top=96, window=60, n_sparse=1), 64, 320),
}


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


def _setup(wl, sb):
    inp = gen.make_inputs(wl)
    _, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, sb)
    idx = orc.select_indices(S, wl.q_len, wl.kv_len, sb, wl.k_top)
    kw, vw = gen.own_window_kv(wl)
    return inp, idx, kw, vw


def _ring(x: np.ndarray, ring: int, dt: str) -> torch.Tensor:
    """The last `ring` positions of a [B, T, H, D] array in a ring: row p % ring."""
    B, T, H, D = x.shape
    r = np.zeros((B, ring, H, D), np.float32)
    for p in range(max(0, T - ring), T):
        r[:, p % ring] = x[:, p]
    return dev_tensor(r, dt)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("token_gate", [False, True])
def test_own_window_matches_oracle(name, token_gate):
    wl, sb, ring = CASES[name]
    wl = wl.replace(score_block=sb)
    say(f"own window {name} token_gate={token_gate}")
    inp, idx, kw, vw = _setup(wl, sb)
    dt = wl.dtype
    k, v, qs = dev_tensor(inp.k, dt), dev_tensor(inp.v, dt), dev_tensor(inp.q_sparse[0], dt)
    if token_gate:
        gl = np.random.default_rng(11).standard_normal((wl.batch, wl.q_len, wl.n_q_heads)).astype(np.float32)
    else:
        gl = inp.gate_logits[0]
    own_k = _ring(kw, ring, dt) if ring else dev_tensor(kw, dt)
    own_v = _ring(vw, ring, dt) if ring else dev_tensor(vw, dt)
    out = hy.hysparse_sparse_attn_ex(qs, k, v, torch.from_numpy(idx).cuda(), wl.k_top, sb, wl.window,
                                     torch.from_numpy(gl).cuda(), own_k=own_k, own_v=own_v, ring=ring)
    torch.cuda.synchronize()
    ref = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, sb, wl.window, gl, k_win=kw, v_win=vw)
    assert_attn_close(out, ref, dt, f"own window {name}")


@pytest.mark.parametrize("name", ["decode_linear", "prefill_blocks_linear"])
def test_own_window_equal_to_cache_is_the_shared_call(name):
    wl, sb, _ = CASES[name]
    say(f"own window = cache {name}")
    inp, idx, _, _ = _setup(wl, sb)
    dt = wl.dtype
    k, v, qs = dev_tensor(inp.k, dt), dev_tensor(inp.v, dt), dev_tensor(inp.q_sparse[0], dt)
    ti = torch.from_numpy(idx).cuda()
    g = torch.from_numpy(inp.gate_logits[0]).cuda()
    a = hy.hysparse_sparse_attn(qs, k, v, ti, wl.k_top, sb, wl.window, g)
    b = hy.hysparse_sparse_attn_ex(qs, k, v, ti, wl.k_top, sb, wl.window, g, own_k=k.clone(), own_v=v.clone())
    torch.cuda.synchronize()
    assert torch.equal(a, b)
