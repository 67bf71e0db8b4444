"""CPU oracle for HySparse hybrid-block attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run this module.  The HIP library never calls it and
shares no code with it; the only common dependency is the seeded input
generator, which holds none of the arithmetic below.

Everything is computed in float64 from the exact stored input values (fp32, or
bf16 held in fp32), with numpy's matmul as the one library primitive.  Each
function follows the plain definition it cites:

* Pages cited: "HySparse: A Hybrid Sparse Attention Architecture with Oracle
  Token Selection and KV Cache Sharing" (abstract); the intelliparadigm HySparse
  article, sections 2.1 (hybrid block), 2.2 (dual-branch sparse attention and
  its gate formula) and 3.1 (cross-layer sharing of indices and KV cache); the
  Baidu article "Sparse Evolution of Hybrid Attention Architectures", section
  "Fine-Grained Sparse Attention: Indexer + Top-K" (gather-then-attend
  pseudocode); the Ultralytics "Sparse Attention" glossary, section
  "Transformer un motif en gains de calcul" (block-mask example); the HISA
  abstract (block-pooled coarse filter, IoU of selections).

Readings where the pages are silent (each is also listed in the design notes):

* importance score of key j for KV group g and score block n:
  ``S[b,g,n,j] = sum over heads h of g and queries i of block n of P[b,h,i,j]``,
  accumulated in float64 and rounded once to float32;
* query i sits at position ``pos(i) = Tkv - Tq + i``; attention is causal;
* softmax scale ``1/sqrt(D)`` in all three attentions; KV head of query head h
  is ``h // (Hq/Hkv)``;
* top-K orders candidates ``j <= last(n)`` by (order key of the float32 bits,
  descending; index ascending), keeps ``min(K, candidates)``, returns them
  sorted ascending and pads with -1;
* sparse layer: global branch over ``{j in idx : j <= pos(i)}`` (empty -> 0),
  window branch over the W keys ``[pos(i)-W+1, pos(i)]``, both on the full
  layer's K/V, separately normalised, no de-duplication; gate ``sigmoid(w_h)``
  with one logit per (layer, query head).

Parity is pinned by the ``-m "not gpu"`` tests (closed forms, brute force,
torch's scaled_dot_product_attention in float64, the page's block-mask figure).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(D) (reading: the pages do not state it)."""
    return 1.0 / np.sqrt(float(head_dim))


def query_positions(q_len: int, kv_len: int) -> np.ndarray:
    """Absolute position of each query: the last Tq rows of a Tkv-row cache."""
    return kv_len - q_len + np.arange(q_len)


def n_score_blocks(q_len: int, score_block: int) -> int:
    return -(-q_len // score_block)


def block_query_range(n: int, q_len: int, score_block: int):
    return n * score_block, min((n + 1) * score_block, q_len)


def candidate_count(n: int, q_len: int, kv_len: int, score_block: int) -> int:
    """Keys a score block may select: every key up to its last query's position."""
    _, i1 = block_query_range(n, q_len, score_block)
    return kv_len - q_len + i1


def _softmax_masked(logits: np.ndarray, mask: np.ndarray):
    """Softmax over the last axis where ``mask`` is True.

    Returns (p, lse, any_valid).  Rows with no valid entry get p = 0 and
    lse = -inf.
    """
    x = np.where(mask, logits, -np.inf)
    any_valid = mask.any(axis=-1)
    m = np.max(np.where(mask, logits, -np.inf), axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(x - m)
    z = e.sum(axis=-1, keepdims=True)
    p = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
    with np.errstate(divide="ignore"):
        lse = np.where(any_valid, m[..., 0] + np.log(np.where(z[..., 0] > 0, z[..., 0], 1.0)), -np.inf)
    return p, lse, any_valid


# ---------------------------------------------------------------------------
# Full-attention layer with score emission
# (HySparse abstract: the full layer is the oracle that picks important tokens;
#  intelliparadigm article section 3.1: its importance scores are used directly
#  by the next N layers)
# ---------------------------------------------------------------------------

def full_layer_block(q, k, v, b: int, g: int, n: int, score_block: int, scale=None):
    """Causal softmax attention for the queries of score block n and the heads
    of KV group g, plus that block's importance-score row.

    q: [B, Tq, Hq, D]; k, v: [B, Tkv, Hkv, D].
    Returns (O [nq, G, D], LSE [G, nq], S [Tkv] float64).
    """
    B, Tq, Hq, D = q.shape
    Tkv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = default_scale(D) if scale is None else scale
    i0, i1 = block_query_range(n, Tq, score_block)
    pos = query_positions(Tq, Tkv)[i0:i1]
    L = int(pos[-1]) + 1
    Kg = k[b, :L, g].astype(F64)
    Vg = v[b, :L, g].astype(F64)
    Qb = q[b, i0:i1, g * G:(g + 1) * G].astype(F64)          # [nq, G, D]
    logits = scale * (Qb @ Kg.T)                               # [nq, G, L]
    mask = np.arange(L)[None, None, :] <= pos[:, None, None]
    p, lse, _ = _softmax_masked(logits, mask)
    O = p @ Vg                                                 # [nq, G, D]
    S = np.zeros(Tkv, dtype=F64)
    S[:L] = p.sum(axis=(0, 1))
    return O, lse.T, S


def full_layer(q, k, v, score_block: int, scale=None, blocks=None):
    """Full-attention layer over all (or the listed) (b, g, n) units.

    Returns O [B,Tq,Hq,D] f64, LSE [B,Hq,Tq] f64 and S [B,Hkv,NB,Tkv] float32
    (S rounded once from float64).  Units not listed in ``blocks`` are NaN.
    """
    B, Tq, Hq, D = q.shape
    Tkv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    NB = n_score_blocks(Tq, score_block)
    O = np.full((B, Tq, Hq, D), np.nan)
    LSE = np.full((B, Hq, Tq), np.nan)
    S = np.full((B, Hkv, NB, Tkv), np.nan)
    units = blocks if blocks is not None else [(b, g, n) for b in range(B)
                                               for g in range(Hkv) for n in range(NB)]
    for (b, g, n) in units:
        i0, i1 = block_query_range(n, Tq, score_block)
        o, lse, s = full_layer_block(q, k, v, b, g, n, score_block, scale)
        O[b, i0:i1, g * G:(g + 1) * G] = o
        LSE[b, g * G:(g + 1) * G, i0:i1] = lse
        S[b, g, n] = s
    return O, LSE, S.astype(np.float32)


# ---------------------------------------------------------------------------
# Top-K selection (Baidu article, "Fine-Grained Sparse Attention: Indexer +
# Top-K": pick the K highest-scoring historical positions per query)
# ---------------------------------------------------------------------------

def order_key(x) -> np.ndarray:
    """Monotone map of float32 bit patterns to uint32 (larger float -> larger key).

    Negative numbers have every bit flipped, others only the sign bit, so the
    unsigned order of keys is the numeric order of the floats with -0 < +0.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return np.where(u >> 31, u ^ np.uint32(0xFFFFFFFF), u ^ np.uint32(0x80000000)).astype(np.uint32)


def topk_row(s_row, valid_len: int, k_top: int) -> np.ndarray:
    """K largest of ``s_row[:valid_len]`` by (key desc, index asc), sorted
    ascending, padded with -1 to length K."""
    s = np.asarray(s_row, dtype=np.float32)[:valid_len]
    keys = order_key(s).astype(np.int64)
    j = np.arange(valid_len)
    order = np.lexsort((j, -keys))
    sel = np.sort(order[:min(k_top, valid_len)])
    out = np.full(k_top, -1, dtype=np.int32)
    out[:sel.size] = sel
    return out


def topk_rows(scores, valid_len, k_top: int) -> np.ndarray:
    """Row-wise ``topk_row``; ``valid_len`` is an int or a per-row sequence."""
    scores = np.asarray(scores, dtype=np.float32)
    R = scores.shape[0]
    vl = np.broadcast_to(np.asarray(valid_len), (R,))
    return np.stack([topk_row(scores[r], int(vl[r]), k_top) for r in range(R)]) if R else \
        np.zeros((0, k_top), dtype=np.int32)


def select_indices(S, q_len: int, kv_len: int, score_block: int, k_top: int, blocks=None):
    """Top-K index sets for every (b, g, n) row of the score tensor."""
    B, Hkv, NB, _ = S.shape
    idx = np.full((B, Hkv, NB, k_top), -1, dtype=np.int32)
    units = blocks if blocks is not None else [(b, g, n) for b in range(B)
                                               for g in range(Hkv) for n in range(NB)]
    for (b, g, n) in units:
        idx[b, g, n] = topk_row(S[b, g, n], candidate_count(n, q_len, kv_len, score_block), k_top)
    return idx


# ---------------------------------------------------------------------------
# Sparse layer (intelliparadigm article section 2.2: a global branch on the
# shared KV cache at the full layer's top-K indices, a 128-token local window
# branch, merged as out = gate * global + (1 - gate) * local with a learnable
# sigmoid gate; Baidu article pseudocode: gather the selected K/V rows, then
# ordinary softmax attention over them)
# ---------------------------------------------------------------------------

def sigmoid(w):
    w = np.asarray(w, dtype=F64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-w))


def sparse_layer_block(qs, k, v, idx_row, b: int, g: int, n: int, score_block: int,
                       window: int, gate_logits, scale=None, k_win=None, v_win=None):
    """Sparse-layer output for the queries of block n and heads of group g.

    gate_logits: [Hq] (one learnable logit per head) or [B, Tq, Hq] (one per
    token and head: the input-dependent reading g = sigmoid(x . w_h) of the
    intelliparadigm article's learnable sigmoid gate, section 2.2).
    k_win, v_win: [B, Tkv, Hkv, D] keys and values of the layer's own window
    branch, by position (the reading in which each sparse layer maintains its
    own 128-token window, section 2.2); None reads the shared k, v.

    Returns (out [nq, G, D], o_global, o_local) in float64.
    """
    B, Tq, Hq, D = qs.shape
    Tkv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = default_scale(D) if scale is None else scale
    i0, i1 = block_query_range(n, Tq, score_block)
    pos = query_positions(Tq, Tkv)[i0:i1]
    Qb = qs[b, i0:i1, g * G:(g + 1) * G].astype(F64)          # [nq, G, D]
    nq = i1 - i0

    # global branch: gather k_cache[idx], v_cache[idx], attend causally
    sel = np.asarray(idx_row)
    sel = sel[sel >= 0].astype(np.int64)
    if sel.size:
        Ks = k[b, sel, g].astype(F64)
        Vs = v[b, sel, g].astype(F64)
        lg = scale * (Qb @ Ks.T)                               # [nq, G, m]
        mask = np.broadcast_to(sel[None, None, :] <= pos[:, None, None], lg.shape)
        p, _, _ = _softmax_masked(lg, mask)
        o_g = p @ Vs
    else:
        o_g = np.zeros((nq, G, D))

    # local branch: the W keys ending at each query's own position
    lo = max(0, int(pos[0]) - window + 1)
    hi = int(pos[-1]) + 1
    wk = np.arange(lo, hi)
    kwin = k if k_win is None else k_win
    vwin = v if v_win is None else v_win
    Kw = kwin[b, lo:hi, g].astype(F64)
    Vw = vwin[b, lo:hi, g].astype(F64)
    lw = scale * (Qb @ Kw.T)
    mw = (wk[None, None, :] <= pos[:, None, None]) & (wk[None, None, :] > pos[:, None, None] - window)
    mw = np.broadcast_to(mw, lw.shape)
    pw, _, _ = _softmax_masked(lw, mw)
    o_l = pw @ Vw

    gl = np.asarray(gate_logits)
    if gl.ndim == 3:   # one logit per (batch, query, head): [B, Tq, Hq]
        gate = sigmoid(gl[b, i0:i1, g * G:(g + 1) * G])[:, :, None]
    else:              # one logit per head: [Hq]
        gate = sigmoid(gl[g * G:(g + 1) * G])[None, :, None]
    out = gate * o_g + (1.0 - gate) * o_l
    return out, o_g, o_l


def sparse_layer(qs, k, v, idx, score_block: int, window: int, gate_logits,
                 scale=None, blocks=None, k_win=None, v_win=None):
    """One sparse layer over all (or the listed) (b, g, n) units -> [B,Tq,Hq,D] f64
    (k_win, v_win: the layer's own window keys/values by position, or None)."""
    B, Tq, Hq, D = qs.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    NB = n_score_blocks(Tq, score_block)
    out = np.full((B, Tq, Hq, D), np.nan)
    units = blocks if blocks is not None else [(b, g, n) for b in range(B)
                                               for g in range(Hkv) for n in range(NB)]
    for (b, g, n) in units:
        i0, i1 = block_query_range(n, Tq, score_block)
        o, _, _ = sparse_layer_block(qs, k, v, idx[b, g, n], b, g, n, score_block,
                                     window, gate_logits, scale, k_win, v_win)
        out[b, i0:i1, g * G:(g + 1) * G] = o
    return out


# ---------------------------------------------------------------------------
# Hybrid block (intelliparadigm article section 2.1: one full layer as the
# information hub followed by N sparse layers; section 3.1: the sparse layers
# only read the full layer's cache and reuse its indices)
# ---------------------------------------------------------------------------

def hybrid_block(q_full, k, v, q_sparse, gate_logits, score_block: int, k_top: int,
                 window: int, scale=None, blocks=None):
    """Full layer -> top-K -> N sparse layers sharing K, V and the indices.

    Returns dict with O_full, LSE, S (float32), idx (int32) and out (list of N).
    """
    Tq, Tkv = q_full.shape[1], k.shape[1]
    O, LSE, S = full_layer(q_full, k, v, score_block, scale, blocks)
    idx = select_indices(S, Tq, Tkv, score_block, k_top, blocks)
    outs = [sparse_layer(qs, k, v, idx, score_block, window, gate_logits[l], scale, blocks)
            for l, qs in enumerate(q_sparse)]
    return {"O_full": O, "LSE": LSE, "S": S, "idx": idx, "out": outs}


# ---------------------------------------------------------------------------
# Helpers used by pins and reports
# ---------------------------------------------------------------------------

def block_mask_nonempty(mask_fn, q_len: int, kv_len: int, tile: int):
    """Count the tile x tile blocks of a boolean mask that hold any allowed pair
    (Ultralytics glossary, "Transformer un motif en gains de calcul": kernels
    skip the empty blocks of the score matrix).  Returns (non_empty, total)."""
    nq, nk = -(-q_len // tile), -(-kv_len // tile)
    nonempty = 0
    qi = np.arange(q_len)
    ki = np.arange(kv_len)
    for a in range(nq):
        qq = qi[a * tile:(a + 1) * tile][:, None]
        for c in range(nk):
            kk = ki[c * tile:(c + 1) * tile][None, :]
            if np.any(mask_fn(qq, kk)):
                nonempty += 1
    return nonempty, nq * nk


def selection_iou(a, b) -> float:
    """Intersection over union of two index sets (-1 entries ignored)
    (HISA abstract: mean IoU of token-selection sets)."""
    sa = set(int(x) for x in np.asarray(a).ravel() if x >= 0)
    sb = set(int(x) for x in np.asarray(b).ravel() if x >= 0)
    if not sa and not sb:
        return 1.0
    return len(sa & sb) / len(sa | sb)


def attention_mass_covered(p_row, idx_row) -> float:
    """Share of a full-attention probability row that the selected keys hold
    (Baidu article, "Key Engineering Considerations": how much of the true
    attention the Top-K selection covers)."""
    sel = np.asarray(idx_row)
    sel = sel[sel >= 0]
    p = np.asarray(p_row, dtype=F64)
    return float(p[sel].sum() / p.sum())


# ---------------------------------------------------------------------------
# Hierarchical selection (HISA abstract: a block-level coarse filter scores
# pooled block representatives and prunes regions, then the token-level
# selection runs only inside the surviving blocks; the Baidu article's
# "Configuration Considerations" mention pooled representations for scoring).
# Decode only (one query row): the token-level refinement uses the full
# layer's own scores S restricted to the kept blocks.
# ---------------------------------------------------------------------------

def pooled_keys(k, block: int):
    """Mean of each run of `block` consecutive keys (the last run may be
    shorter): [B, T, Hkv, D] -> [B, M, Hkv, D] float64."""
    B, T, Hkv, D = k.shape
    M = -(-T // block)
    out = np.empty((B, M, Hkv, D))
    for m in range(M):
        out[:, m] = k[:, m * block:min((m + 1) * block, T)].astype(F64).mean(axis=1)
    return out


def block_scores(q, kbar, scale=None):
    """Block score of a KV group for one query row: the group's query heads'
    softmax over the pooled keys, summed over the heads.  q: [B, 1, Hq, D];
    kbar: [B, M, Hkv, D] -> [B, Hkv, M] float64."""
    B, _, Hq, D = q.shape
    M, Hkv = kbar.shape[1], kbar.shape[2]
    G = Hq // Hkv
    scale = default_scale(D) if scale is None else scale
    out = np.empty((B, Hkv, M))
    for b in range(B):
        for g in range(Hkv):
            lg = scale * (q[b, 0, g * G:(g + 1) * G].astype(F64) @ kbar[b, :, g].T)   # [G, M]
            p, _, _ = _softmax_masked(lg, np.ones_like(lg, dtype=bool))
            out[b, g] = p.sum(axis=0)
    return out


def hier_select(q, k, S, block: int, n_keep: int, k_top: int, scale=None, block_scores_f32=None):
    """Kept blocks (ascending, -1 padded) and token indices (ascending, -1
    padded) of the hierarchical selection for decode.

    Blocks: the n_keep largest block scores (rounded once to float32) by the
    same order rule as the token top-K.  Tokens: the k_top largest entries of
    the flat scores S among the tokens of the kept blocks.  ``block_scores_f32``
    lets a caller supply the block scores (to check a selection made on
    another implementation's block scores)."""
    B, T, Hkv, _ = k.shape
    M = -(-T // block)
    bs = (block_scores(q, pooled_keys(k, block), scale).astype(np.float32)
          if block_scores_f32 is None else np.asarray(block_scores_f32, dtype=np.float32))
    blk = np.full((B, Hkv, n_keep), -1, dtype=np.int32)
    idx = np.full((B, Hkv, 1, k_top), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            kept = topk_row(bs[b, g], M, n_keep)
            blk[b, g] = kept
            kept = kept[kept >= 0]
            cand = np.concatenate([np.arange(m * block, min((m + 1) * block, T)) for m in kept]) if kept.size \
                else np.zeros(0, dtype=np.int64)
            pos_in = topk_row(np.asarray(S[b, g, 0], dtype=np.float32)[cand], cand.size, k_top)
            sel = pos_in[pos_in >= 0]
            idx[b, g, 0, :sel.size] = cand[sel]
    return blk, idx, bs
