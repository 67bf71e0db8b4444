"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances on attention outputs: the stated max-abs bounds plus a relative
# l2 bound (outputs here are often ~1e-2, where max-abs alone would accept 0).
TOL = {"bf16": dict(max_abs=2e-2, rel_l2=1e-2), "f32": dict(max_abs=1e-4, rel_l2=1e-5)}
# Score elements: |dS| <= 1e-4 |S| + 1e-7 (fp32 logits from the stored inputs).
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


def assert_scores_close(gpu: torch.Tensor, ref: np.ndarray, what: str = "scores"):
    g = host(gpu)
    r = np.asarray(ref, dtype=np.float64)
    bad = np.abs(g - r) > S_RTOL * np.abs(r) + S_ATOL
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
