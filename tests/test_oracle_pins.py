"""Pins of the CPU oracle to facts outside itself (runs without a GPU).

Each test ties one oracle function to a closed form, a brute-force
enumeration, an independent library routine (torch's
scaled_dot_product_attention in float64) or a figure printed on the pages.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import hysparse_oracle as orc
from long_context_hybrid_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in float64; q [Tq,D], k/v [L,D], mask [Tq,L] bool."""
    tq = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    tk = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    tv = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    tm = torch.from_numpy(np.ascontiguousarray(mask))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)[0, 0].numpy()


# ----------------------------------------------------------------- full layer

@pytest.mark.parametrize("Tq,Tkv", [(37, 37), (1, 50), (9, 30)])
def test_full_layer_matches_sdpa(Tq, Tkv):
    B, Hq, Hkv, D = 2, 6, 2, 16
    q, k, v = _rand(1, B, Tq, Hq, D), _rand(2, B, Tkv, Hkv, D), _rand(3, B, Tkv, Hkv, D)
    O, LSE, _ = orc.full_layer(q, k, v, score_block=1)
    G = Hq // Hkv
    pos = Tkv - Tq + np.arange(Tq)
    mask = np.arange(Tkv)[None, :] <= pos[:, None]
    sc = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(Hq):
            ref = _sdpa(q[b, :, h], k[b, :, h // G], v[b, :, h // G], mask, sc)
            np.testing.assert_allclose(O[b, :, h], ref, rtol=0, atol=1e-12)
            lg = torch.from_numpy(sc * q[b, :, h] @ k[b, :, h // G].T)
            lg = lg.masked_fill(~torch.from_numpy(mask), -math.inf)
            np.testing.assert_allclose(LSE[b, h], torch.logsumexp(lg, -1).numpy(), rtol=0, atol=1e-12)


def test_full_layer_closed_forms():
    D, T = 8, 11
    v = _rand(4, 1, T, 1, D)
    # identical keys -> uniform weights over the causal prefix
    k = np.repeat(_rand(5, 1, 1, 1, D), T, axis=1)
    q = _rand(6, 1, T, 1, D)
    O, LSE, _ = orc.full_layer(q, k, v, score_block=1)
    for i in range(T):
        np.testing.assert_allclose(O[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-13)
    # q = 0 -> uniform weights too, LSE = log(i+1)
    O0, LSE0, _ = orc.full_layer(np.zeros_like(q), _rand(7, 1, T, 1, D), v, score_block=1)
    for i in range(T):
        np.testing.assert_allclose(O0[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-13)
        assert abs(LSE0[0, 0, i] - math.log(i + 1)) < 1e-13
    # first query sees a single key -> O = v_0
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=0)


@pytest.mark.parametrize("Tq,Tkv,Sb", [(130, 130, 64), (1, 77, 1), (1, 77, 64), (20, 20, 1)])
def test_scores_sum_to_group_times_block(Tq, Tkv, Sb):
    """Each query head's probabilities sum to 1, so a score row sums to
    G * (queries in the block); scores are >= 0 and zero past the block."""
    B, Hq, Hkv, D = 2, 8, 2, 16
    G = Hq // Hkv
    q, k, v = _rand(8, B, Tq, Hq, D), _rand(9, B, Tkv, Hkv, D), _rand(10, B, Tkv, Hkv, D)
    _, _, S = orc.full_layer(q, k, v, score_block=Sb)
    NB = -(-Tq // Sb)
    assert S.shape == (B, Hkv, NB, Tkv) and S.dtype == np.float32
    for n in range(NB):
        nq = min((n + 1) * Sb, Tq) - n * Sb
        last = orc.candidate_count(n, Tq, Tkv, Sb)
        np.testing.assert_allclose(S[:, :, n].astype(np.float64).sum(-1), G * nq, rtol=1e-6)
        assert np.all(S[:, :, n, :] >= 0)
        assert np.all(S[:, :, n, last:] == 0)


def test_scores_single_head_equal_probability_row():
    """With one head per group and one query per block, S is exactly the
    softmax row of that query (computed here with torch)."""
    T, D = 25, 8
    q, k, v = _rand(11, 1, T, 1, D), _rand(12, 1, T, 1, D), _rand(13, 1, T, 1, D)
    _, _, S = orc.full_layer(q, k, v, score_block=1)
    sc = 1.0 / math.sqrt(D)
    lg = torch.from_numpy(sc * q[0, :, 0] @ k[0, :, 0].T)
    lg = lg.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), -math.inf)
    p = torch.softmax(lg, -1).numpy().astype(np.float32)
    np.testing.assert_array_equal(S[0, 0], p)


def test_scores_group_mapping():
    """Query heads 0..G-1 belong to KV head 0, heads G..2G-1 to KV head 1:
    a key made to match only the second group's queries must top only that
    group's score row."""
    Hq, Hkv, D, T = 4, 2, 8, 12
    G = Hq // Hkv
    q = np.zeros((1, 1, Hq, D))
    q[0, 0, :G, 0] = 4.0       # group 0 queries point along e0
    q[0, 0, G:, 1] = 4.0       # group 1 queries point along e1
    k = np.zeros((1, T, Hkv, D))
    k[0, 3, 0, 0] = 4.0        # key 3 of KV head 0 along e0
    k[0, 7, 1, 1] = 4.0        # key 7 of KV head 1 along e1
    v = _rand(14, 1, T, Hkv, D)
    _, _, S = orc.full_layer(q, k, v, score_block=1)
    assert int(np.argmax(S[0, 0, 0])) == 3
    assert int(np.argmax(S[0, 1, 0])) == 7


# ---------------------------------------------------------------------- top-K

def test_order_key_is_numeric_order():
    x = gen.random_scores(3, 1, 4000, "signed")[0]
    x = np.concatenate([x, np.array([np.inf, -np.inf, 1e-45, -1e-45], np.float32)])
    keys = orc.order_key(x)
    by_key = np.argsort(keys, kind="stable")
    xs = x[by_key]
    assert np.all(np.diff(xs.astype(np.float64)) >= 0)
    # -0 sorts below +0
    zeros = x[by_key][(xs == 0)]
    signs = np.signbit(zeros)
    assert np.all(signs[:signs.sum()]) and not np.any(signs[signs.sum():])


def _brute_topk(s, k):
    """Enumerate every k-subset; keep the one whose descending key vector is
    lexicographically largest, ties to the lexicographically smallest index tuple."""
    keys = [int(x) for x in orc.order_key(s)]
    n = len(s)
    best = None
    for comb in itertools.combinations(range(n), min(k, n)):
        desc = sorted((keys[j] for j in comb), reverse=True)
        cand = (tuple(desc), tuple(-j for j in comb))
        if best is None or cand > best[0]:
            best = (cand, comb)
    out = np.full(k, -1, np.int32)
    out[:len(best[1])] = best[1]
    return out


@pytest.mark.parametrize("kind", ["probs", "ties", "signed"])
def test_topk_brute_force(kind):
    S = gen.random_scores(7, 40, 12, kind)
    rng = np.random.default_rng(0)
    for r in range(S.shape[0]):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(1, 14))
        np.testing.assert_array_equal(orc.topk_row(S[r], n, k), _brute_topk(S[r, :n], k))


def test_topk_special_cases():
    s = np.full(100, 0.25, np.float32)
    np.testing.assert_array_equal(orc.topk_row(s, 100, 10), np.arange(10))
    r = gen.random_scores(8, 1, 50)[0]
    np.testing.assert_array_equal(orc.topk_row(r, 30, 64)[:30], np.arange(30))
    assert np.all(orc.topk_row(r, 30, 64)[30:] == -1)
    # cross-check with a stable torch sort on keys (descending by key, ascending index)
    r = gen.random_scores(9, 1, 5000, "ties")[0]
    keys = torch.from_numpy(orc.order_key(r).astype(np.int64))
    order = torch.sort(-keys, stable=True).indices[:700]
    np.testing.assert_array_equal(orc.topk_row(r, 5000, 700), np.sort(order.numpy()))


# --------------------------------------------------------------- sparse layer

def _tiny_case(seed, B=1, Tq=40, Tkv=40, Hq=4, Hkv=2, D=16, Sb=1, K=6, W=5):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, Tq, Hq, D)), rng.standard_normal((B, Tkv, Hkv, D)),
               rng.standard_normal((B, Tkv, Hkv, D)))
    NB = -(-Tq // Sb)
    idx = np.full((B, Hkv, NB, K), -1, np.int32)
    for b in range(B):
        for g in range(Hkv):
            for n in range(NB):
                c = orc.candidate_count(n, Tq, Tkv, Sb)
                m = min(K, c)
                idx[b, g, n, :m] = np.sort(rng.choice(c, size=m, replace=False))
    return q, k, v, idx


@pytest.mark.parametrize("Sb,Tq,Tkv", [(1, 40, 40), (8, 40, 40), (1, 1, 40), (8, 13, 40)])
def test_sparse_branches_match_masked_dense(Sb, Tq, Tkv):
    """Gather-then-attend equals dense attention under the equivalent boolean mask."""
    B, Hq, Hkv, D, K, W = 1, 4, 2, 16, 9, 5
    q, k, v, idx = _tiny_case(20 + Sb, B, Tq, Tkv, Hq, Hkv, D, Sb, K, W)
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D)
    pos = Tkv - Tq + np.arange(Tq)
    gl = np.linspace(-1.5, 2.0, Hq)
    for g in range(Hkv):
        for n in range(-(-Tq // Sb)):
            out, og, ol = orc.sparse_layer_block(q, k, v, idx[0, g, n], 0, g, n, Sb, W, gl)
            i0, i1 = n * Sb, min((n + 1) * Sb, Tq)
            sel = idx[0, g, n][idx[0, g, n] >= 0]
            jj = np.arange(Tkv)
            for t, i in enumerate(range(i0, i1)):
                mg = np.isin(jj, sel) & (jj <= pos[i])
                ml = (jj <= pos[i]) & (jj > pos[i] - W)
                for hh in range(G):
                    h = g * G + hh
                    if mg.any():
                        rg = _sdpa(q[0, i:i + 1, h], k[0, :, g], v[0, :, g], mg[None], sc)[0]
                        np.testing.assert_allclose(og[t, hh], rg, atol=1e-12)
                    else:
                        assert np.all(og[t, hh] == 0)
                    rl = _sdpa(q[0, i:i + 1, h], k[0, :, g], v[0, :, g], ml[None], sc)[0]
                    np.testing.assert_allclose(ol[t, hh], rl, atol=1e-12)
                    gt = 1.0 / (1.0 + math.exp(-gl[h]))
                    np.testing.assert_allclose(out[t, hh], gt * og[t, hh] + (1 - gt) * ol[t, hh], atol=1e-13)


def test_sparse_empty_global_set_gives_zero():
    """A block whose selection lies after an early query's position leaves that
    query with no global keys: its global branch is 0 and out = (1-g) * local."""
    Tq = Tkv = 16
    q, k, v, _ = _tiny_case(30, 1, Tq, Tkv, 2, 1, 8, 8, 2, 3)
    idx = np.full((1, 1, 2, 2), -1, np.int32)
    idx[0, 0, 0] = [6, 7]
    idx[0, 0, 1] = [3, 12]
    out, og, ol = orc.sparse_layer_block(q, k, v, idx[0, 0, 0], 0, 0, 0, 8, 3, np.zeros(2))
    assert np.all(og[:6] == 0) and np.all(np.abs(og[6:]).sum(-1) > 0)
    np.testing.assert_allclose(out[:6], 0.5 * ol[:6], atol=0)


@pytest.mark.parametrize("Tq,Tkv,Sb", [(32, 32, 1), (32, 32, 8), (1, 50, 1)])
def test_sparse_full_selection_gate_one_is_dense(Tq, Tkv, Sb):
    """K >= context with gate 1 reproduces dense causal attention; with Q' = Q
    it equals the full layer's output."""
    B, Hq, Hkv, D = 2, 4, 2, 16
    q, k, v = _rand(40, B, Tq, Hq, D), _rand(41, B, Tkv, Hkv, D), _rand(42, B, Tkv, Hkv, D)
    O, _, S = orc.full_layer(q, k, v, Sb)
    idx = orc.select_indices(S, Tq, Tkv, Sb, k_top=Tkv + 3)
    out = orc.sparse_layer(q, k, v, idx, Sb, window=4, gate_logits=np.full(Hq, np.inf))
    np.testing.assert_allclose(out, O, atol=1e-12)


@pytest.mark.parametrize("W", [1, 5, 16])
def test_sparse_gate_zero_is_sliding_window(W):
    B, T, Hq, Hkv, D = 1, 30, 4, 1, 8
    q, k, v, idx = _tiny_case(50, B, T, T, Hq, Hkv, D, 1, 4, W)
    out = orc.sparse_layer(q, k, v, idx, 1, W, np.full(Hq, -np.inf))
    sc = 1.0 / math.sqrt(D)
    jj = np.arange(T)
    mask = (jj[None, :] <= jj[:, None]) & (jj[None, :] > jj[:, None] - W)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, :, h], _sdpa(q[0, :, h], k[0, :, 0], v[0, :, 0], mask, sc), atol=1e-12)


def test_sparse_wide_window_gate_zero_is_dense():
    B, T, Hq, Hkv, D = 1, 24, 2, 1, 8
    q, k, v, idx = _tiny_case(60, B, T, T, Hq, Hkv, D, 1, 3, T)
    out = orc.sparse_layer(q, k, v, idx, 1, T + 5, np.full(Hq, -np.inf))
    O, _, _ = orc.full_layer(q, k, v, 1)
    np.testing.assert_allclose(out, O, atol=1e-12)


def test_gate_is_affine_with_global_weight():
    """out(w) = g(w) * global + (1 - g(w)) * local; the page's initial global
    weight 0.7 corresponds to the logit ln(7/3)."""
    gold = json.load(open(os.path.join(GOLDEN, "gate_init.json")))
    w07 = math.log(gold["global_weight"] / (1 - gold["global_weight"]))
    assert abs(float(orc.sigmoid(w07)) - gold["global_weight"]) < 1e-15
    assert float(orc.sigmoid(np.inf)) == 1.0 and float(orc.sigmoid(-np.inf)) == 0.0
    q, k, v, idx = _tiny_case(70, 1, 20, 20, 2, 1, 8, 4, 5, 6)
    og = orc.sparse_layer(q, k, v, idx, 4, 6, np.full(2, np.inf))
    ol = orc.sparse_layer(q, k, v, idx, 4, 6, np.full(2, -np.inf))
    o7 = orc.sparse_layer(q, k, v, idx, 4, 6, np.full(2, w07))
    np.testing.assert_allclose(o7, 0.7 * og + 0.3 * ol, atol=1e-13)


# ---------------------------------------------------------------- composition

def test_hybrid_block_composition_and_planted_recall():
    """The block's indices are the top-K of its own scores, and planted
    needles (keys aligned with the group's summed query) are all selected."""
    wl = gen.WORKLOADS["decode128k"].replace(kv_len=4096, batch=2, n_sparse=2, k_top=128)
    inp = gen.make_inputs(wl)
    res = orc.hybrid_block(inp.q_full, inp.k, inp.v, inp.q_sparse, inp.gate_logits,
                           wl.score_block, wl.k_top, wl.window)
    S, idx = res["S"], res["idx"]
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            np.testing.assert_array_equal(idx[b, g, 0], orc.topk_row(S[b, g, 0], wl.kv_len, wl.k_top))
            assert set(inp.planted[b].tolist()) <= set(idx[b, g, 0].tolist())
    assert len(res["out"]) == 2 and np.all(np.isfinite(res["out"][1]))


def test_tiny_workload_runs_and_is_normalised():
    wl = gen.WORKLOADS["tiny"]
    inp = gen.make_inputs(wl)
    res = orc.hybrid_block(inp.q_full, inp.k, inp.v, inp.q_sparse, inp.gate_logits,
                           wl.score_block, wl.k_top, wl.window)
    S = res["S"].astype(np.float64)
    np.testing.assert_allclose(S.sum(-1), wl.group, rtol=1e-6)
    assert res["idx"].shape == (1, 1, 256, 32)
    # query i has min(32, i+1) candidates
    nvalid = (res["idx"] >= 0).sum(-1)[0, 0]
    np.testing.assert_array_equal(nvalid, np.minimum(32, np.arange(256) + 1))


# ---------------------------------------------------------- pages' figures

def test_block_mask_sparsity_matches_page():
    """The glossary's create_block_mask example prints sparsity 85.47% for a
    1024-token causal window plus 4 sink tokens on 8192^2 with 128^2 blocks."""
    gold = json.load(open(os.path.join(GOLDEN, "flex_block_mask.json")))
    w, s = gold["window"], gold["sinks"]

    def mask(qi, ki):
        return (qi >= ki) & (((qi - ki) <= w) | (ki < s))

    ne, tot = orc.block_mask_nonempty(mask, gold["seq_len"], gold["seq_len"], gold["tile"])
    assert tot == 4096
    assert round(100.0 * (1 - ne / tot), 2) == gold["printed_sparsity_percent"]


def test_selection_helpers():
    assert orc.selection_iou([1, 2, 3, -1], [2, 3, 4, -1]) == 0.5
    p = np.array([0.5, 0.25, 0.125, 0.125])
    assert orc.attention_mass_covered(p, [0, 2, -1]) == 0.625


# ------------------------------------------------------ hierarchical select

def test_pooled_keys_and_block_scores_closed_forms():
    rng = np.random.default_rng(80)
    B, T, Hkv, D, blk = 1, 300, 2, 8, 64
    k = rng.standard_normal((B, T, Hkv, D))
    kb = orc.pooled_keys(k, blk)
    assert kb.shape == (1, 5, 2, 8)
    np.testing.assert_allclose(kb[0, 1, 0], k[0, 64:128, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(kb[0, 4, 1], k[0, 256:300, 1].mean(axis=0), atol=1e-14)   # partial last block
    q = rng.standard_normal((B, 1, 6, D))
    bs = orc.block_scores(q, kb)
    np.testing.assert_allclose(bs.sum(-1), 3.0, rtol=1e-12)                           # G heads x softmax
    # constant keys inside a block: the pooled key is that key
    kc = np.repeat(k[:, ::blk][:, :, None], blk, axis=2).reshape(B, -1, Hkv, D)[:, :T]
    np.testing.assert_allclose(orc.pooled_keys(kc, blk)[0, 2, 1], kc[0, 128, 1], atol=1e-14)


def test_hier_select_keeping_every_block_equals_flat():
    """With as many kept blocks as there are blocks, the hierarchical selection
    is the flat top-K (IoU 1)."""
    wl = gen.WORKLOADS["decode128k"].replace(kv_len=2048, batch=1, n_sparse=1, k_top=100, n_planted=8)
    inp = gen.make_inputs(wl)
    _, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, 1)
    flat = orc.select_indices(S, 1, wl.kv_len, 1, wl.k_top)
    blk, idx, _ = orc.hier_select(inp.q_full, inp.k, S, 128, 16, wl.k_top)
    np.testing.assert_array_equal(idx, flat)
    np.testing.assert_array_equal(blk[0, 0], np.arange(16))
    blk, idx, _ = orc.hier_select(inp.q_full, inp.k, S, 128, 4, wl.k_top)
    for g in range(wl.n_kv_heads):
        sel = idx[0, g, 0][idx[0, g, 0] >= 0]
        assert sel.size == wl.k_top and np.all(np.isin(sel // 128, blk[0, g]))
        assert np.all(np.diff(sel) > 0)
        # the kept tokens are the best of the kept blocks by the flat scores
        cand = np.concatenate([np.arange(m * 128, (m + 1) * 128) for m in blk[0, g]])
        rest = np.setdiff1d(cand, sel)
        assert S[0, g, 0, sel].min() >= S[0, g, 0, rest].max()
    assert 0.0 <= orc.selection_iou(idx[0, 0], flat[0, 0]) < 1.0


def test_block_scores_with_unit_blocks_are_the_full_layer_scores():
    """Blocks of one key: the pooled keys are the keys and the block scores
    are the full layer's decode scores S (softmax per head summed over the
    group), computed independently by full_layer."""
    wl = gen.WORKLOADS["decode128k"].replace(kv_len=700, batch=2, n_sparse=1, k_top=64, n_planted=4)
    inp = gen.make_inputs(wl)
    _, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, 1)
    kb = orc.pooled_keys(inp.k, 1)
    np.testing.assert_array_equal(kb, inp.k.astype(np.float64))
    bs = orc.block_scores(inp.q_full, kb)
    np.testing.assert_allclose(bs, S[:, :, 0], rtol=1.2e-7, atol=0)   # S is stored rounded to float32
    blk, idx, _ = orc.hier_select(inp.q_full, inp.k, S, 1, wl.kv_len, wl.k_top)
    np.testing.assert_array_equal(idx, orc.select_indices(S, 1, wl.kv_len, 1, wl.k_top))


def test_planted_block_outranks_the_rest():
    """A block whose keys all point along a group's summed query direction
    gets that group's largest block score and is kept; other groups are not
    affected."""
    rng = np.random.default_rng(81)
    B, T, Hq, Hkv, D, blk = 1, 1024, 8, 2, 16, 64
    q = rng.standard_normal((B, 1, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D)) * 0.5
    u = q[0, 0, 0:4].sum(axis=0)
    k[0, 5 * blk:6 * blk, 0] = 6.0 * u / np.linalg.norm(u)
    bs = orc.block_scores(q, orc.pooled_keys(k, blk))
    assert int(np.argmax(bs[0, 0])) == 5
    assert int(np.argmax(bs[0, 1])) != 5 or bs[0, 1, 5] < 0.5
    S = np.zeros((B, Hkv, 1, T))
    kept, _, _ = orc.hier_select(q, k, S, blk, 3, 8)
    assert 5 in kept[0, 0]


# ------------------------------------------------- per-token (input-dependent) gate

def _tok_gate_case():
    wl = gen.WORKLOADS["prefill32k"].replace(q_len=150, kv_len=150, k_top=40, window=20, n_sparse=1)
    inp = gen.make_inputs(wl)
    _, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, 64)
    idx = orc.select_indices(S, wl.q_len, wl.kv_len, 64, wl.k_top)
    return wl, inp, idx


def test_token_gate_equal_per_token_is_the_head_gate():
    wl, inp, idx = _tok_gate_case()
    gh = inp.gate_logits[0]
    gt = np.broadcast_to(gh, (wl.batch, wl.q_len, wl.n_q_heads)).copy()
    a = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 64, wl.window, gh)
    b = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 64, wl.window, gt)
    np.testing.assert_array_equal(a, b)


def test_token_gate_is_local_and_selects_branches_per_token():
    wl, inp, idx = _tok_gate_case()
    G = wl.group
    rng = np.random.default_rng(90)
    gt = rng.standard_normal((wl.batch, wl.q_len, wl.n_q_heads))
    base = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 64, wl.window, gt)
    gt2 = gt.copy()
    gt2[0, 70, 5] += 1.5                      # one (token, head) logit
    moved = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 64, wl.window, gt2)
    diff = np.abs(moved - base).max(axis=-1)[0]
    assert diff[70, 5] > 0 and np.count_nonzero(diff) == 1
    # +inf / -inf per token: that token's global / window output, exactly
    gsel = np.where((np.arange(wl.q_len) % 2 == 0)[None, :, None], np.inf, -np.inf) * np.ones_like(gt)
    out = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, 64, wl.window, gsel)
    for n in range(wl.n_blocks):
        i0, i1 = n * 64, min((n + 1) * 64, wl.q_len)
        _, o_g, o_l = orc.sparse_layer_block(inp.q_sparse[0], inp.k, inp.v, idx[0, 1, n], 0, 1, n, 64, wl.window,
                                             gsel)
        rows = np.arange(i0, i1)
        np.testing.assert_array_equal(out[0, rows[rows % 2 == 0], G:2 * G], o_g[(rows % 2 == 0)])
        np.testing.assert_array_equal(out[0, rows[rows % 2 == 1], G:2 * G], o_l[(rows % 2 == 1)])


# ------------------------------------------------- own window KV per sparse layer

def test_own_window_kv_gate_zero_is_sliding_window_on_it():
    """Gate 0: the output is W-key sliding-window attention over the layer's
    own keys/values (torch SDPA with the band mask), the shared cache unused."""
    B, T, Hq, Hkv, D, W = 1, 40, 4, 2, 16, 7
    q, k, v = _rand(31, B, T, Hq, D), _rand(32, B, T, Hkv, D), _rand(33, B, T, Hkv, D)
    kw, vw = _rand(34, B, T, Hkv, D), _rand(35, B, T, Hkv, D)
    idx = np.tile(np.arange(8, dtype=np.int32), (B, Hkv, T, 1))
    out = orc.sparse_layer(q, k, v, idx, 1, W, np.full(Hq, -np.inf), k_win=kw, v_win=vw)
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    for h in range(Hq):
        ref = _sdpa(q[0, :, h], kw[0, :, h // 2], vw[0, :, h // 2], band, 1.0 / math.sqrt(D))
        np.testing.assert_allclose(out[0, :, h], ref, atol=1e-12)


def test_own_window_kv_equal_to_cache_and_gate_one():
    """Own window K/V equal to the shared cache give the shared-window result
    exactly; with gate 1 the window K/V do not matter."""
    B, T, Hq, Hkv, D, W = 2, 30, 4, 1, 16, 5
    q, k, v = _rand(41, B, T, Hq, D), _rand(42, B, T, Hkv, D), _rand(43, B, T, Hkv, D)
    idx = np.tile(np.arange(0, 24, 3, dtype=np.int32), (B, Hkv, T, 1))
    gl = _rand(44, Hq)
    a = orc.sparse_layer(q, k, v, idx, 1, W, gl)
    b = orc.sparse_layer(q, k, v, idx, 1, W, gl, k_win=k.copy(), v_win=v.copy())
    np.testing.assert_array_equal(a, b)
    c = orc.sparse_layer(q, k, v, idx, 1, W, np.full(Hq, np.inf))
    d = orc.sparse_layer(q, k, v, idx, 1, W, np.full(Hq, np.inf), k_win=_rand(45, B, T, Hkv, D),
                         v_win=_rand(46, B, T, Hkv, D))
    np.testing.assert_array_equal(c, d)
    e = orc.sparse_layer(q, k, v, idx, 1, W, gl, k_win=_rand(45, B, T, Hkv, D), v_win=_rand(46, B, T, Hkv, D))
    assert np.abs(e - a).max() > 1e-3
