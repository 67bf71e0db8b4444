"""GPU parity of the hierarchical (block-pooled) selection for decode."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import assert_attn_close, dev_tensor, eps_valid, host, say

pytestmark = pytest.mark.gpu
W = gen.WORKLOADS


def _run(wl, block, n_keep):
    inp = gen.make_inputs(wl)
    qf, k, v = (dev_tensor(x, wl.dtype) for x in (inp.q_full, inp.k, inp.v))
    _, _, S = hy.hysparse_full_attn_scores(qf, k, v, 1)
    idx, bs, blk = hy.hysparse_hier_select(qf, k, S, block, n_keep, wl.k_top)
    torch.cuda.synchronize()
    return inp, (qf, k, v), host(S).astype(np.float32), host(idx), host(bs).astype(np.float32), host(blk)


def _check(wl, inp, S, idx, bs, blk, block, n_keep):
    kb = orc.pooled_keys(inp.k, block)
    bs_ref = orc.block_scores(inp.q_full, kb)
    bad = np.abs(bs - bs_ref) > 1e-4 * np.abs(bs_ref) + 1e-7
    assert not bad.any(), f"block scores: {int(bad.sum())} out of tolerance"
    M = bs.shape[-1]
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            np.testing.assert_array_equal(blk[b, g], orc.topk_row(bs[b, g], M, n_keep))
            assert eps_valid(blk[b, g], bs_ref[b, g], M)
    _, idx_ref, _ = orc.hier_select(inp.q_full, inp.k, S, block, n_keep, wl.k_top, block_scores_f32=bs)
    np.testing.assert_array_equal(idx, idx_ref)


@pytest.mark.parametrize("Tkv,block,n_keep,k_top", [(5000, 128, 8, 256), (3000, 64, 20, 300), (777, 100, 3, 400)])
def test_hier_select_matches_oracle(Tkv, block, n_keep, k_top):
    wl = W["hier128k"].replace(batch=2, kv_len=Tkv, k_top=k_top, n_sparse=1, n_planted=8)
    say(f"hier select Tkv={Tkv} block={block} keep={n_keep} K={k_top}")
    inp, _, S, idx, bs, blk = _run(wl, block, n_keep)
    _check(wl, inp, S, idx, bs, blk, block, n_keep)


def test_hier_select_keeping_all_blocks_is_flat():
    wl = W["hier128k"].replace(batch=1, kv_len=2000, k_top=128, n_sparse=1, n_planted=4)
    say("hier select, all blocks kept")
    inp, _, S, idx, bs, blk = _run(wl, 128, 16)
    flat = orc.select_indices(S, 1, wl.kv_len, 1, wl.k_top)
    np.testing.assert_array_equal(idx, flat)


def test_hier128k_full_size_iou_and_sparse_output():
    """The 128K hierarchical workload: parity of the selection, then the sparse
    layer on the hierarchical indices against the oracle; IoU against the flat
    selection, planted-needle recall and output difference are reported."""
    wl = W["hier128k"].replace(n_sparse=1)
    say("hier128k full size")
    inp, (qf, k, v), S, idx, bs, blk = _run(wl, 128, 64)
    _check(wl, inp, S, idx, bs, blk, 128, 64)
    flat = orc.select_indices(S, 1, wl.kv_len, 1, wl.k_top)
    ious = [orc.selection_iou(idx[b, g], flat[b, g]) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    rec_h = np.mean([np.isin(inp.planted[b], idx[b, g]).mean() for b in range(wl.batch) for g in range(wl.n_kv_heads)])
    rec_f = np.mean([np.isin(inp.planted[b], flat[b, g]).mean() for b in range(wl.batch) for g in range(wl.n_kv_heads)])
    qs = dev_tensor(inp.q_sparse[0], wl.dtype)
    gates = torch.from_numpy(inp.gate_logits[0]).cuda()
    out_h = hy.hysparse_sparse_attn(qs, k, v, torch.from_numpy(idx).cuda(), wl.k_top, 1, wl.window, gates)
    out_f = hy.hysparse_sparse_attn(qs, k, v, torch.from_numpy(flat).cuda(), wl.k_top, 1, wl.window, gates)
    torch.cuda.synchronize()
    ref = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 1, wl.window, inp.gate_logits[0])
    assert_attn_close(out_h, ref, wl.dtype, "sparse layer on hierarchical indices")
    oh, of = host(out_h), host(out_f)
    rel = float(np.linalg.norm(oh - of) / np.linalg.norm(of))
    say(f"  mean IoU vs flat {np.mean(ious):.4f}; planted recall hier {rec_h:.3f} flat {rec_f:.3f}; "
        f"sparse output rel-l2 vs flat {rel:.4f}")
    assert rec_f == 1.0


def test_hier_pooled_select_equals_hier_select():
    """Pooled keys from hysparse_hier_pool (into an array with spare blocks)
    give hysparse_hier_select's outputs bit for bit, and match the oracle's
    block means."""
    wl = W["hier128k"].replace(batch=2, kv_len=3000, k_top=300, n_sparse=1, n_planted=8)
    block, n_keep = 128, 6
    say("hier pooled select vs hier select")
    inp = gen.make_inputs(wl)
    qf, k = dev_tensor(inp.q_full, wl.dtype), dev_tensor(inp.k, wl.dtype)
    _, _, S = hy.hysparse_full_attn_scores(qf, k, dev_tensor(inp.v, wl.dtype), 1)
    M = -(-wl.kv_len // block)
    kbar = torch.full((wl.batch, M + 5, wl.n_kv_heads, wl.head_dim), float("nan"), device="cuda")
    hy.hysparse_hier_pool(k, block, kbar)
    ref = hy.hysparse_hier_select(qf, k, S, block, n_keep, wl.k_top)
    got = hy.hysparse_hier_select_pooled(qf, k, kbar, S, block, n_keep, wl.k_top)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    np.testing.assert_allclose(host(kbar[:, :M]), orc.pooled_keys(inp.k, block), rtol=1e-6, atol=1e-6)
    assert torch.isnan(kbar[:, M:]).all()          # blocks past the cache are not written


def test_hier_pool_refresh_in_decode_loop():
    """Decode loop: append one token per step and refresh only the block that
    holds it; the pooled keys stay equal (bit for bit) to pooling the grown
    cache from scratch, and the selection equals hysparse_hier_select."""
    wl = W["hier128k"].replace(batch=1, kv_len=1400, k_top=128, n_sparse=1, n_planted=4)
    block, n_keep, L0, steps = 100, 4, 1195, 9          # crosses the block boundary at 1200
    say("hier pool refresh over a decode loop")
    inp = gen.make_inputs(wl)
    qf, k_all, v_all = (dev_tensor(x, wl.dtype) for x in (inp.q_full, inp.k, inp.v))
    kc, vc = k_all.clone(), v_all.clone()
    cap_blocks = -(-wl.kv_len // block)
    kbar = torch.zeros((1, cap_blocks, wl.n_kv_heads, wl.head_dim), device="cuda")
    hy.hysparse_hier_pool(kc[:, :L0], block, kbar)
    for s in range(steps):
        L = L0 + s + 1
        hy.hysparse_append_kv(k_all[:, L - 1:L].contiguous(), v_all[:, L - 1:L].contiguous(), kc, vc, L - 1)
        m = (L - 1) // block
        hy.hysparse_hier_pool(kc[:, :L], block, kbar, m, m + 1)
        fresh = torch.zeros_like(kbar)
        hy.hysparse_hier_pool(kc[:, :L], block, fresh)
        M = -(-L // block)
        _, _, S = hy.hysparse_full_attn_scores(qf, kc[:, :L], vc[:, :L], 1)
        ref = hy.hysparse_hier_select(qf, kc[:, :L], S, block, n_keep, wl.k_top)
        got = hy.hysparse_hier_select_pooled(qf, kc[:, :L], kbar, S, block, n_keep, wl.k_top)
        torch.cuda.synchronize()
        assert torch.equal(kbar[:, :M], fresh[:, :M]), f"step {s}"
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"step {s}"
