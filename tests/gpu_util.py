"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import hysparse_oracle as orc

# Tolerances on attention outputs: the stated max-abs bounds plus a relative
# l2 bound (outputs here are often ~1e-2, where max-abs alone would accept 0).
TOL = {"bf16": dict(max_abs=2e-2, rel_l2=1e-2), "f32": dict(max_abs=1e-4, rel_l2=1e-5)}
# Score elements: |dS| <= 1e-4 |S| + 1e-7 on every path (the scores are formed
# from fp32 logits of the stored inputs; the decode full layer's per-head
# probabilities pass between its two kernels with a relative error of at most
# 2^-16).
S_RTOL, S_ATOL = 1e-4, 1e-7


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def assert_attn_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "", mask=None):
    g = host(gpu)
    r = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    tol = TOL[dtype]
    assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3e} > {tol['max_abs']}"
    assert rel <= tol["rel_l2"], f"{what}: rel-l2 {rel:.3e} > {tol['rel_l2']}"
    return mx, rel


def assert_scores_close(gpu: torch.Tensor, ref: np.ndarray, what: str = "scores", rtol: float = S_RTOL):
    g = host(gpu)
    r = np.asarray(ref, dtype=np.float64)
    bad = np.abs(g - r) > rtol * np.abs(r) + S_ATOL
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, worst " \
                          f"{float(np.max(np.abs(g - r) / (np.abs(r) + 1e-30))):.3e}"


def eps_valid(idx_row: np.ndarray, s_ref_row: np.ndarray, valid: int, eps_rel=S_RTOL, eps_abs=S_ATOL) -> bool:
    """Every selected score >= every unselected candidate's score - eps."""
    sel = idx_row[idx_row >= 0]
    if sel.size >= valid:
        return True
    s = np.asarray(s_ref_row[:valid], dtype=np.float64)
    m = np.ones(valid, bool)
    m[sel] = False
    lo = s[sel].min()
    hi = s[m].max()
    return lo >= hi - (eps_rel * abs(hi) + eps_abs)


def _unit_mask(shape_btHd, units, Tq, Sb, G):
    """Boolean mask over [B, Tq, Hq, D] selecting the rows of the listed (b, g, n) units."""
    m = np.zeros(shape_btHd[:3], dtype=bool)
    for (b, g, n) in units:
        m[b, n * Sb:min((n + 1) * Sb, Tq), g * G:(g + 1) * G] = True
    return m


def check_hybrid(wl, inp, res, n_check_layers=None, blocks=None):
    """End-to-end criteria: GPU scores within tolerance of the oracle's; GPU
    indices equal the oracle's top-K of the GPU scores (bit-exact) and are
    eps-valid against the oracle's scores; sparse outputs match the oracle
    evaluated on the GPU's indices.  ``blocks`` restricts every check to the
    listed (b, g, n) units (the oracle then computes only those)."""
    Tq, Tkv, Sb, K = wl.q_len, wl.kv_len, wl.score_block, wl.k_top
    O_ref, LSE_ref, S_ref = orc.full_layer(inp.q_full, inp.k, inp.v, Sb, blocks=blocks)
    B, Hkv, NB, _ = S_ref.shape
    units = blocks if blocks is not None else [(b, g, n) for b in range(B) for g in range(Hkv) for n in range(NB)]
    rows = _unit_mask(O_ref.shape, units, Tq, Sb, wl.group) if blocks is not None else None
    assert_attn_close(res["out_full"], O_ref, wl.dtype, "O_full", mask=rows)
    S_gpu = host(res["scores"]).astype(np.float32)
    sel = tuple(np.array(units).T)
    assert_scores_close(torch.from_numpy(S_gpu[sel]), S_ref[sel])
    idx_gpu = host(res["idx"])
    idx_from_gpu_S = orc.select_indices(S_gpu, Tq, Tkv, Sb, K, blocks=units)
    np.testing.assert_array_equal(idx_gpu[sel], idx_from_gpu_S[sel])
    agree = index_agreement(wl, idx_gpu, S_ref, units)
    say(f"  index rows differing from the oracle's own selection: {agree['rows_differing']}/{agree['rows']}, "
        f"mean IoU {agree['mean_iou']:.6f}")
    layers = range(len(inp.q_sparse)) if n_check_layers is None else range(n_check_layers)
    for l in layers:
        ref = orc.sparse_layer(inp.q_sparse[l], inp.k, inp.v, idx_gpu, Sb, wl.window, inp.gate_logits[l],
                               blocks=blocks)
        assert_attn_close(res["out"][l], ref, wl.dtype, f"sparse layer {l}", mask=rows)
    check_hybrid.last_agreement = agree
    return S_ref, idx_gpu


def iou(a: np.ndarray, b: np.ndarray) -> float:
    """|A & B| / |A | B| of two index rows, padding (-1) ignored."""
    sa, sb = np.unique(a[a >= 0]), np.unique(b[b >= 0])
    union = np.union1d(sa, sb).size
    return np.intersect1d(sa, sb).size / union if union else 1.0


def index_agreement(wl, idx_gpu, S_ref, units):
    """Compare the GPU's index rows (the top-K of its own scores) with the
    oracle's selection on the oracle's scores: every GPU row must be eps-valid
    against the oracle's scores (no unselected candidate beats a selected one
    by more than the score tolerance); returns how many rows differ from the
    oracle's selection and the mean IoU over all rows."""
    Tq, Tkv, Sb, K = wl.q_len, wl.kv_len, wl.score_block, wl.k_top
    idx_ref = orc.select_indices(S_ref, Tq, Tkv, Sb, K, blocks=units)
    differ, ious = 0, []
    for (b, g, n) in units:
        c = orc.candidate_count(n, Tq, Tkv, Sb)
        assert eps_valid(idx_gpu[b, g, n], S_ref[b, g, n], c), f"index row {(b, g, n)} is not eps-valid"
        differ += int(not np.array_equal(idx_gpu[b, g, n], idx_ref[b, g, n]))
        ious.append(iou(idx_gpu[b, g, n], idx_ref[b, g, n]))
    return {"rows": len(units), "rows_differing": differ, "mean_iou": float(np.mean(ious)),
            "min_iou": float(np.min(ious))}
