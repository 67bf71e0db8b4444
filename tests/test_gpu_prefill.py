"""GPU parity of the prefill path (q_len > 1): full layer with per-query or
per-64-query-block scores, and the block-sparse layer."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import (assert_attn_close, assert_scores_close, check_hybrid, dev_tensor, eps_valid, host,
                             say)

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
PREFILL_CASES = {
    "tiny": W["tiny"],
    "prefill32k_small": W["prefill32k"].replace(q_len=700, kv_len=700, k_top=200, n_sparse=2),
    "chunked_q130_kv400": W["prefill32k"].replace(q_len=130, kv_len=400, k_top=96, window=50, n_sparse=1),
    "g16_d128_sb64": W["decode128k"].replace(q_len=300, kv_len=300, score_block=64, k_top=128, n_sparse=1,
                                             n_planted=0, std=1.0),
    "mha_d64_sb1_bf16": W["decode8k"].replace(q_len=200, kv_len=200, n_q_heads=2, n_kv_heads=2, head_dim=64,
                                              score_block=1, k_top=24, window=10, n_sparse=1),
    "f32_sb64_g2": W["tiny"].replace(q_len=200, kv_len=200, n_q_heads=4, n_kv_heads=2, score_block=64,
                                     k_top=40, window=16, n_sparse=1),
    "window_over_ctx": W["prefill32k"].replace(q_len=100, kv_len=100, k_top=500, window=300, n_sparse=1),
    # more selected keys than one LDS index stage holds (the refill path)
    "ktop_over_stage": W["prefill32k"].replace(q_len=2600, kv_len=2600, n_q_heads=4, n_kv_heads=1, k_top=2300,
                                               n_sparse=1),
    # shorter than one 64-key tile: every tile row past the cache is clamped and masked
    "short_ctx_40": W["prefill32k"].replace(q_len=40, kv_len=40, k_top=16, window=8, n_sparse=1),
    # G = 16 with queries after a cached prefix: several score passes, ragged tiles
    "g16_chunk_q70_kv333": W["decode128k"].replace(q_len=70, kv_len=333, score_block=64, k_top=64, n_sparse=1,
                                                   n_planted=0, std=1.0),
    # fp32 with head_dim 128, and bf16 with head_dim 64 and grouped heads
    "f32_d128_g4_sb64": W["tiny"].replace(q_len=150, kv_len=150, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                          std=1.0 / np.sqrt(128.0), score_block=64, k_top=48, window=20,
                                          n_sparse=1),
    "bf16_d64_g8_sb64": W["prefill32k"].replace(q_len=260, kv_len=260, n_q_heads=16, n_kv_heads=2, head_dim=64,
                                                k_top=80, window=32, n_sparse=1),
}


def _dev(inp):
    dt = inp.wl.dtype
    return (dev_tensor(inp.q_full, dt), dev_tensor(inp.k, dt), dev_tensor(inp.v, dt),
            [dev_tensor(q, dt) for q in inp.q_sparse], torch.from_numpy(inp.gate_logits).cuda())


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_full_prefill_matches_oracle(name):
    wl = PREFILL_CASES[name]
    say(f"full prefill {name}")
    inp = gen.make_inputs(wl)
    qf, k, v, _, _ = _dev(inp)
    out, lse, S = hy.hysparse_full_attn_scores(qf, k, v, wl.score_block)
    torch.cuda.synchronize()
    O_ref, LSE_ref, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    assert_attn_close(out, O_ref, wl.dtype, "O_full")
    np.testing.assert_allclose(host(lse), LSE_ref, rtol=0, atol=2e-5 if wl.dtype == "bf16" else 1e-5)
    assert_scores_close(S, S_ref)


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_sparse_prefill_on_oracle_indices(name):
    wl = PREFILL_CASES[name]
    say(f"sparse prefill {name}")
    inp = gen.make_inputs(wl)
    _, k, v, qs, gates = _dev(inp)
    _, _, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    idx = orc.select_indices(S_ref, wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    g = gates[0].clone()
    g[0] = float("inf")
    g[-1] = float("-inf")
    out = hy.hysparse_sparse_attn(qs[0], k, v, torch.from_numpy(idx).cuda(), wl.k_top, wl.score_block,
                                  wl.window, g)
    torch.cuda.synchronize()
    ref = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, wl.score_block, wl.window, host(g))
    assert_attn_close(out, ref, wl.dtype, "sparse out")


def test_sparse_block_unsorted_and_padded_indices():
    """Index rows with -1 entries in the middle and out of order are handled
    per entry (skip negatives, mask entries after the query's position)."""
    wl = PREFILL_CASES["prefill32k_small"]
    say("sparse prefill unsorted indices")
    inp = gen.make_inputs(wl)
    _, k, v, qs, gates = _dev(inp)
    rng = np.random.default_rng(3)
    NB = wl.n_blocks
    idx = np.full((1, wl.n_kv_heads, NB, wl.k_top), -1, np.int32)
    for g in range(wl.n_kv_heads):
        for n in range(NB):
            c = orc.candidate_count(n, wl.q_len, wl.kv_len, wl.score_block)
            m = min(c, wl.k_top - 7)
            row = rng.choice(c, size=m, replace=False).astype(np.int32)
            holes = np.full(wl.k_top - m, -1, np.int32)
            full = np.concatenate([row, holes])
            rng.shuffle(full)
            idx[0, g, n] = full
    out = hy.hysparse_sparse_attn(qs[0], k, v, torch.from_numpy(idx).cuda(), wl.k_top, wl.score_block,
                                  wl.window, gates[0])
    torch.cuda.synchronize()
    ref = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, wl.score_block, wl.window, inp.gate_logits[0])
    assert_attn_close(out, ref, wl.dtype, "sparse out")


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_hybrid_block_prefill(name):
    wl = PREFILL_CASES[name]
    say(f"hybrid prefill {name}")
    inp = gen.make_inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
    torch.cuda.synchronize()
    check_hybrid(wl, inp, res)


def test_hybrid_prefill_deterministic():
    """Twenty runs of the same prefill block give bit-identical results."""
    wl = PREFILL_CASES["prefill32k_small"]
    say("determinism prefill32k_small x20")
    inp = gen.make_inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    first = None
    for _ in range(20):
        res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
        torch.cuda.synchronize()
        cur = [res["out_full"].clone(), res["scores"].clone(), res["idx"].clone()] + [o.clone() for o in res["out"]]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["prefill32k_small", "g16_chunk_q70_kv333"])
def test_hybrid_prefill_head_major_cache_bit_identical(name):
    """A head-major cache ([B, Hkv, T, D] storage passed as a [B, T, Hkv, D]
    view) changes only the row addresses the tile loads use: every output
    must equal the token-major run bit for bit."""
    wl = PREFILL_CASES[name]
    say(f"head-major cache {name}")
    inp = gen.make_inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    khm = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vhm = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert khm.stride(1) == wl.head_dim and torch.equal(khm, k)
    a = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
    b = hy.hysparse_hybrid_block(qf, khm, vhm, qs, gates, wl.k_top, wl.score_block, wl.window)
    torch.cuda.synchronize()
    for key in ("out_full", "scores", "idx"):
        assert torch.equal(a[key], b[key]), key
    for oa, ob in zip(a["out"], b["out"]):
        assert torch.equal(oa, ob)


def test_hybrid_block_prefill32k_full_size_sampled():
    """The 32K prefill workload at full size; the oracle checks a sample of
    (KV group, score block) units including the first and last blocks."""
    wl = W["prefill32k"].replace(n_sparse=1)
    say("hybrid prefill32k full size")
    inp = gen.make_inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
    torch.cuda.synchronize()
    NB = wl.n_blocks
    blocks = [(0, g, n) for g in (0, 5) for n in (0, 1, 31, 32, 200, NB - 2, NB - 1)]
    check_hybrid(wl, inp, res, blocks=blocks)


def test_hybrid_block_prefill128k_sampled():
    """The 128K prefill workload (inputs drawn on the GPU) at full size, in the
    launch configuration bench.py times; the oracle recomputes whole score
    blocks (O, LSE, S row, top-K on the GPU's scores, sparse output on the
    GPU's indices) from host copies of the stored input values."""
    wl = W["prefill128k"].replace(n_sparse=1)
    say("hybrid prefill128k full size")
    qf, k, v, qs, gates = gen.make_device_inputs(wl, torch.device("cuda"))
    lse = torch.empty((1, wl.n_q_heads, wl.q_len), dtype=torch.float32, device="cuda")
    res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window, lse=lse)
    torch.cuda.synchronize()
    f32 = lambda t: t.float().cpu().numpy()  # stored bf16 values, exact in float32
    qh, kh, vh, qsh = f32(qf), f32(k), f32(v), f32(qs[0])
    gh = gates[0].cpu().numpy()
    G, NB, Sb, K = wl.group, wl.n_blocks, wl.score_block, wl.k_top
    for (g, n) in [(0, 0), (1, 777), (3, NB - 1)]:
        say(f"  block (g={g}, n={n})")
        i0, i1 = n * Sb, min((n + 1) * Sb, wl.q_len)
        O, LSE, S = orc.full_layer_block(qh, kh, vh, 0, g, n, Sb)
        assert_attn_close(res["out_full"][0, i0:i1, g * G:(g + 1) * G], O, wl.dtype, f"O_full block {n}")
        np.testing.assert_allclose(host(res["lse"][0, g * G:(g + 1) * G, i0:i1]), LSE, rtol=0, atol=2e-5)
        S_gpu = res["scores"][0, g, n]
        assert_scores_close(S_gpu, S.astype(np.float32))
        c = orc.candidate_count(n, wl.q_len, wl.kv_len, Sb)
        idx_row = host(res["idx"][0, g, n])
        np.testing.assert_array_equal(idx_row, orc.topk_row(host(S_gpu).astype(np.float32), c, K))
        assert eps_valid(idx_row, S.astype(np.float32), c)
        out, _, _ = orc.sparse_layer_block(qsh, kh, vh, idx_row, 0, g, n, Sb, wl.window, gh)
        assert_attn_close(res["out"][0][0, i0:i1, g * G:(g + 1) * G], out, wl.dtype, f"sparse block {n}")
