"""GPU parity of the decode path (one query row per sequence) and of top-K.

Every case compares the HIP library, called through its C ABI, with the CPU
oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import assert_attn_close, assert_scores_close, check_hybrid, dev_tensor, host, say

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
DECODE_CASES = {
    # name: workload (reduced sizes span several splits and ragged tails)
    "decode8k_small": W["decode8k"].replace(batch=2, kv_len=1000, k_top=100, n_sparse=2),
    "decode128k_small": W["decode128k"].replace(batch=1, kv_len=5000, k_top=256, n_sparse=2, n_planted=16),
    "tiny_decode_f32": W["tiny"].replace(batch=2, q_len=1, kv_len=300, k_top=32, n_sparse=2),
    "mha_d64_bf16": W["decode8k"].replace(batch=1, kv_len=777, n_q_heads=3, n_kv_heads=3, head_dim=64,
                                          k_top=64, window=40, n_sparse=1),
    "g16_window300": W["decode128k"].replace(batch=1, kv_len=2000, k_top=300, window=300, n_sparse=1,
                                             n_planted=8),
    "short_ctx": W["decode8k"].replace(batch=1, kv_len=20, k_top=64, window=128, n_sparse=1),
    # one key in the cache: every attention is over key 0 (O = v0, S = G)
    "single_key": W["decode8k"].replace(batch=2, kv_len=1, k_top=16, window=8, n_sparse=1),
    # logits with std 8 (Q, K std 2.83, V std 1): base-2 logits spread over
    # about +-45, so most per-head probabilities fall far below their step's
    # maximum; the decode full layer's three-byte probability scratch keeps
    # fp32's exponent range, so they keep their 2^-16 relative precision
    "wide_logits": W["decode128k"].replace(batch=1, kv_len=5000, k_top=256, n_sparse=1, n_planted=8,
                                           std=float(np.sqrt(8.0)), v_std=1.0),
    # kv_len on and one past the 1024-key score chunks and 32-key steps of
    # the decode full layer's probability scratch
    "chunk_exact": W["decode128k"].replace(batch=1, kv_len=2048, k_top=256, n_sparse=1, n_planted=4),
    "chunk_plus1": W["decode128k"].replace(batch=1, kv_len=1025, k_top=128, n_sparse=1, n_planted=4),
    "step_plus1_g8": W["decode8k"].replace(batch=2, kv_len=33, k_top=16, window=8, n_sparse=1),
    # 128 units (batch 32 x 4 KV heads): the split plan caps the global
    # splits so that the split workgroups fit one resident round (3 splits of
    # 384 entries here), with a K that is not a multiple of the split
    "capped_splits_128_units": W["decode128k"].replace(batch=32, kv_len=3000, k_top=777, n_sparse=1, n_planted=4),
    # one query with score block 64: a block of one query (NB 1, last(0) = the
    # query's own position), the same rows as score block 1
    "one_query_block64": W["decode8k"].replace(batch=2, kv_len=900, k_top=100, n_sparse=1, score_block=64),
    # fp32 with head_dim 128 (no other case covers this instantiation)
    "f32_d128_g4": W["tiny"].replace(batch=2, q_len=1, kv_len=1300, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                     std=1.0 / np.sqrt(128.0), k_top=200, window=64, n_sparse=2),
}


def _inputs(wl):
    return gen.make_inputs(wl)


def _dev(inp):
    dt = inp.wl.dtype
    return (dev_tensor(inp.q_full, dt), dev_tensor(inp.k, dt), dev_tensor(inp.v, dt),
            [dev_tensor(q, dt) for q in inp.q_sparse], torch.from_numpy(inp.gate_logits).cuda())


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


# ---------------------------------------------------------------------- top-K

@pytest.mark.parametrize("kind", ["probs", "ties", "signed"])
@pytest.mark.parametrize("k", [1, 7, 1024, 2048])
def test_topk_bit_exact(kind, k):
    say(f"topk kind={kind} k={k}")
    R, L = 24, 9000
    S = gen.random_scores(11 + k, R, L, kind)
    vl = np.random.default_rng(k).integers(0, L + 1, size=R).astype(np.int32)
    vl[0], vl[1], vl[2] = 0, L, min(k, L)
    ref = orc.topk_rows(S, vl, k)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), k, valid_len=torch.from_numpy(vl).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


def test_topk_long_rows_decode128k_shape():
    """16 rows of 131072 scores, K = 2048: the decode-time selection shape."""
    say("topk 16x131072 k=2048")
    S = gen.random_scores(5, 16, 131072, "probs")
    ref = orc.topk_rows(S, 131072, 2048)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), 2048)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


@pytest.mark.parametrize("kind", ["probs", "ties", "signed"])
@pytest.mark.parametrize("k", [1, 100, 2048])
def test_topk_few_long_rows_in_parts(kind, k):
    """Few rows longer than the LDS capacity: the filter runs over parts of
    each row in separate workgroups; ragged row length, valid lengths from 0 to
    the full row (including <= k and <= the capacity), ties and signed keys."""
    say(f"topk parts kind={kind} k={k}")
    R, L = 20, 50001  # rows of 50001 scores in a buffer 50004 wide (row stride % 4 == 0)
    S = gen.random_scores(31 + k, R, L + 3, kind)
    vl = np.random.default_rng(100 + k).integers(0, L + 1, size=R).astype(np.int32)
    vl[0], vl[1], vl[2], vl[3], vl[4] = 0, L, min(k, L), 12288, 12289
    ref = orc.topk_rows(S[:, :L], vl, k)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda()[:, :L], k, valid_len=torch.from_numpy(vl).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


@pytest.mark.parametrize("R,L,k", [(3, 40000, 15000), (16, 131072, 13000), (2, 20000, 19999), (2, 13000, 13000)])
def test_topk_k_above_the_candidate_capacity(R, L, k):
    """K above the 12,288 candidates a row workgroup holds: the filtered
    candidates cannot hold the top K, so every path (one workgroup per row,
    and the part filter with its select) selects over the whole row; K one
    below and equal to the row length."""
    say(f"topk R{R} L{L} k{k}")
    S = gen.random_scores(61 + k, R, L, "probs")
    ref = orc.topk_rows(S, L, k)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


@pytest.mark.parametrize("kind", ["cluster", "cluster_wide"])
@pytest.mark.parametrize("R,L", [(8, 20000), (300, 10000), (300, 30000), (400, 3000), (400, 20000)])
def test_topk_clustered_rows_multi_digit(kind, R, L):
    """A dense cluster of near-tied keys, with outliers stretching the key
    range, holds the K-th key, so the radix select's selected bin still has
    more keys than the rank list takes after the first digit: later digit
    passes run (their histogram cleared under their own barrier), ending in
    the last digit ("cluster", 64 values) or in the rank list
    ("cluster_wide").  Rows cover the part-and-select path (8 x 20000), the
    large row workgroups with the whole row as candidates (300 x 10000) and
    with the sampled filter (300 x 30000), and the small row workgroups
    without (400 x 3000) and with (400 x 20000) the filter."""
    c = min(3000, L // 3)
    k = 5 + c // 2
    say(f"topk {kind} R{R} L{L} k{k}")
    S = gen.random_scores(77 + R + L, R, L, kind)
    ref = orc.topk_rows(S, L, k)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


def test_topk_parts_strided_rows_and_fallback():
    """Parts with a row stride wider than the row, and a K above the sample's
    reach (the filter keeps too many candidates and the whole-row select
    runs)."""
    say("topk parts strided / fallback")
    S = gen.random_scores(41, 6, 40004, "signed")
    t = torch.from_numpy(S).cuda()[:, :40000]
    got = host(hy.hysparse_topk(t, 777))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, orc.topk_rows(S[:, :40000], 40000, 777))
    S2 = gen.random_scores(42, 3, 131072, "probs")
    got2 = host(hy.hysparse_topk(torch.from_numpy(S2).cuda(), 5000))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got2, orc.topk_rows(S2, 131072, 5000))


@pytest.mark.parametrize("kind", ["probs", "ties", "signed"])
@pytest.mark.parametrize("k", [1, 100, 2048])
def test_topk_many_rows_small_workgroups(kind, k):
    """Many rows (the prefill shape: one row per KV group and 64-query block)
    run in the small row workgroups: valid lengths across the short-row path
    (<= 4096 candidates), the sampled filter and, for tied rows (more
    survivors than the capacity), the whole-row fallback."""
    say(f"topk many rows kind={kind} k={k}")
    R, L = 512, 9000
    S = gen.random_scores(61 + k, R, L, kind)
    vl = np.random.default_rng(200 + k).integers(0, L + 1, size=R).astype(np.int32)
    vl[:8] = [0, L, min(k, L), 4096, 4097, min(2 * k, L), 8191, 8192]
    ref = orc.topk_rows(S, vl, k)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), k, valid_len=torch.from_numpy(vl).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


def test_topk_many_long_rows_small_workgroups():
    """400 rows of up to 131072 scores with K = 2048 (the 128K prefill's row
    lengths) in the small row workgroups: the 8192-key sample keeps the
    survivors between K and the 4096-entry capacity."""
    say("topk 400 rows x 131072")
    R, L = 400, 131072
    S = gen.random_scores(71, R, L, "probs")
    vl = np.linspace(4097, L, R).astype(np.int32)
    ref = orc.topk_rows(S, vl, 2048)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), 2048, valid_len=torch.from_numpy(vl).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


def test_topk_many_rows_k_above_small_capacity():
    """Many rows with K above half the small workgroups' capacity run in the
    large ones."""
    say("topk many rows k=2500")
    R, L = 400, 7000
    S = gen.random_scores(81, R, L, "signed")
    vl = np.random.default_rng(300).integers(0, L + 1, size=R).astype(np.int32)
    ref = orc.topk_rows(S, vl, 2500)
    got = hy.hysparse_topk(torch.from_numpy(S).cuda(), 2500, valid_len=torch.from_numpy(vl).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), ref)


def test_topk_row_stride_and_all_equal():
    say("topk strided rows, all-equal rows")
    base = np.full((5, 4100), 0.5, np.float32)
    base[3, 17] = 0.75
    t = torch.from_numpy(base).cuda()[:, :4096]
    got = host(hy.hysparse_topk(t, 10))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0], np.arange(10))
    np.testing.assert_array_equal(got[3], np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 17]))


# --------------------------------------------------------------- full decode

@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_full_decode_matches_oracle(name):
    wl = DECODE_CASES[name]
    say(f"full decode {name}")
    inp = _inputs(wl)
    qf, k, v, _, _ = _dev(inp)
    out, lse, S = hy.hysparse_full_attn_scores(qf, k, v, wl.score_block)
    torch.cuda.synchronize()
    O_ref, LSE_ref, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    assert_attn_close(out, O_ref, wl.dtype, "O_full")
    np.testing.assert_allclose(host(lse), LSE_ref, rtol=0, atol=2e-5 if wl.dtype == "bf16" else 1e-5)
    assert_scores_close(S, S_ref)


# -------------------------------------------------------------- sparse decode

@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_sparse_decode_on_oracle_indices(name):
    wl = DECODE_CASES[name]
    say(f"sparse decode {name}")
    inp = _inputs(wl)
    _, k, v, qs, gates = _dev(inp)
    _, _, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    idx = orc.select_indices(S_ref, wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    g = gates[0].clone()
    g[0] = float("inf")      # pure global branch
    g[-1] = float("-inf")    # pure window branch
    out = hy.hysparse_sparse_attn(qs[0], k, v, torch.from_numpy(idx).cuda(), wl.k_top, wl.score_block,
                                  wl.window, g)
    torch.cuda.synchronize()
    ref = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, wl.score_block, wl.window, host(g))
    assert_attn_close(out, ref, wl.dtype, "sparse out")


# ----------------------------------------------------------- hybrid block e2e

@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_hybrid_block_decode(name):
    wl = DECODE_CASES[name]
    say(f"hybrid decode {name}")
    inp = _inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
    torch.cuda.synchronize()
    _, idx_gpu = check_hybrid(wl, inp, res)
    if inp.planted is not None:
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                assert set(inp.planted[b].tolist()) <= set(idx_gpu[b, g, 0].tolist())


@pytest.mark.parametrize("name", ["decode8k_small", "g16_window300"])
def test_hybrid_block_deterministic(name):
    """Twenty runs of the same block give bit-identical outputs, scores and
    indices (no atomics-order or scheduling effects)."""
    wl = DECODE_CASES[name]
    say(f"determinism {name} x20")
    inp = _inputs(wl)
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


# ------------------------------------------------------------- full sizes

# agreement of the GPU's index rows (the top-K of its own scores) with the
# oracle's selection on the oracle's scores, at full size: every row is
# eps-valid; rows can differ only where candidates' scores lie within the
# score tolerance of each other at the K-th place
MIN_MEAN_IOU = {"decode8k": 0.99, "decode128k": 0.99}


@pytest.mark.parametrize("name", ["decode8k", "decode128k"])
def test_hybrid_block_full_size(name):
    """The real decode workloads (two of their sparse layers checked)."""
    wl = W[name].replace(n_sparse=2)
    say(f"hybrid decode full size {name}")
    inp = _inputs(wl)
    qf, k, v, qs, gates = _dev(inp)
    res = hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window)
    torch.cuda.synchronize()
    _, idx_gpu = check_hybrid(wl, inp, res)
    agree = check_hybrid.last_agreement
    say(f"  RECORD index agreement {name}: {agree}")
    assert agree["mean_iou"] >= MIN_MEAN_IOU[name]
    if inp.planted is not None:
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                assert set(inp.planted[b].tolist()) <= set(idx_gpu[b, g, 0].tolist())


@pytest.mark.parametrize("name", ["tiny", "decode8k"])
def test_topk_on_oracle_scores_bit_exact(name):
    """The GPU top-K fed the oracle's own fp32 scores of a workload selects
    exactly the oracle's index rows (the tiny workload: 256 per-query rows;
    the 8K decode workload at full size, whose near-uniform scores put many
    exactly equal fp32 values at the K-th place)."""
    wl = W[name]
    say(f"topk on oracle scores {name}")
    inp = _inputs(wl)
    _, _, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    S32 = S_ref.astype(np.float32)
    B, Hkv, NB, Tkv = S32.shape
    ref = orc.select_indices(S32, wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    rows = np.array([orc.candidate_count(n, wl.q_len, wl.kv_len, wl.score_block)
                     for b in range(B) for g in range(Hkv) for n in range(NB)], np.int32)
    kth = [np.sort(S32.reshape(-1, Tkv)[r, :rows[r]])[::-1][min(wl.k_top, rows[r]) - 1] for r in range(len(rows))]
    ties = [int((S32.reshape(-1, Tkv)[r, :rows[r]] == kth[r]).sum()) for r in range(len(rows))]
    say(f"  candidates equal to the K-th score per row: mean {np.mean(ties):.1f}, max {max(ties)}")
    got = hy.hysparse_topk(torch.from_numpy(S32.reshape(-1, Tkv)).cuda(), wl.k_top,
                           valid_len=torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got).reshape(ref.shape), ref)
