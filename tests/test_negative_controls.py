"""Negative controls of the parity checks (run without a GPU).

The GPU parity tests accept an output when the checks in tests/gpu_util.py
pass.  These tests show that the same checks reject wrong results that a
faulty kernel could plausibly produce: an all-zero or a slightly perturbed
attention output, scores off by more than the tolerance, an index row with
one entry changed, and an index set that drops a clearly better candidate.
The reference values come from the oracle; the "GPU" values are CPU tensors
built from them, so no GPU is involved.
"""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import (assert_attn_close, assert_scores_close, eps_valid, index_agreement, iou)

W = gen.WORKLOADS


@pytest.fixture(scope="module")
def tiny_ref():
    wl = W["tiny"]
    inp = gen.make_inputs(wl)
    O, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    idx = orc.select_indices(S.astype(np.float32), wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    out = orc.sparse_layer(inp.q_sparse[0], inp.k, inp.v, idx, wl.score_block, wl.window, inp.gate_logits[0])
    return wl, O, S, idx, out


@pytest.fixture(scope="module")
def decode_ref():
    """A bf16 decode case whose outputs are ~1e-2, where max-abs 2e-2 alone
    would accept an all-zero output."""
    wl = W["decode8k"].replace(batch=2, kv_len=1000, k_top=100, n_sparse=1)
    inp = gen.make_inputs(wl)
    O, _, S = orc.full_layer(inp.q_full, inp.k, inp.v, wl.score_block)
    return wl, O, S


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32))


def test_reference_itself_passes(tiny_ref, decode_ref):
    wl, O, S, idx, out = tiny_ref
    assert_attn_close(_t(O), O, "f32")
    assert_attn_close(_t(out), out, "f32")
    assert_scores_close(_t(S), S)
    wl8, O8, S8 = decode_ref
    assert_attn_close(_t(O8).to(torch.bfloat16), O8, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_zero_output_fails(tiny_ref, decode_ref, dtype):
    O = tiny_ref[1] if dtype == "f32" else decode_ref[1]
    assert np.abs(O).max() < 2e-2 or dtype == "f32"  # the case max-abs alone would not catch
    with pytest.raises(AssertionError):
        assert_attn_close(torch.zeros(O.shape), O, dtype, "zero output")


def test_output_off_by_more_than_tolerance_fails(tiny_ref):
    _, O, _, _, out = tiny_ref
    bad = out.copy()
    bad[0, 100, 2, 5] += 5e-4  # one element, above the fp32 max-abs bound 1e-4
    with pytest.raises(AssertionError):
        assert_attn_close(_t(bad), out, "f32")
    scaled = O * (1 + 3e-5)  # every element, small but above the relative l2 bound 1e-5
    with pytest.raises(AssertionError):
        assert_attn_close(_t(scaled), O, "f32")


def test_wrong_head_or_query_order_fails(tiny_ref):
    _, O, _, _, _ = tiny_ref
    with pytest.raises(AssertionError):
        assert_attn_close(_t(O[:, :, ::-1]), O, "f32", "heads swapped")
    with pytest.raises(AssertionError):
        assert_attn_close(_t(np.roll(O, 1, axis=1)), O, "f32", "queries shifted")


def test_scores_off_by_more_than_tolerance_fail(tiny_ref):
    _, _, S, _, _ = tiny_ref
    bad = S.astype(np.float32).copy()
    r = np.unravel_index(np.argmax(S), S.shape)
    bad[r] *= 1 + 3e-4
    with pytest.raises(AssertionError):
        assert_scores_close(_t(bad), S)
    with pytest.raises(AssertionError):  # a score past the block's last key that should be 0
        z = S.astype(np.float32).copy()
        z[0, 0, 10, 200] = 1e-6
        assert_scores_close(_t(z), S)


def test_perturbed_index_row_fails_bit_exact(tiny_ref):
    wl, _, S, idx, _ = tiny_ref
    S32 = S.astype(np.float32)
    got = orc.select_indices(S32, wl.q_len, wl.kv_len, wl.score_block, wl.k_top)
    np.testing.assert_array_equal(got, idx)  # the unperturbed row passes
    bad = idx.copy()
    n = 200  # a row with more candidates (201) than K (32)
    row = bad[0, 0, n]
    unselected = np.setdiff1d(np.arange(n + 1), row)
    row[np.argmin(S32[0, 0, n, row])] = unselected[0]
    bad[0, 0, n] = np.sort(row)
    with pytest.raises(AssertionError):
        np.testing.assert_array_equal(bad, idx)
    assert iou(bad[0, 0, n], idx[0, 0, n]) < 1.0


def test_index_set_missing_a_better_candidate_is_not_eps_valid(tiny_ref):
    wl, _, S, idx, _ = tiny_ref
    S32 = S.astype(np.float32)
    n = 255
    c = orc.candidate_count(n, wl.q_len, wl.kv_len, wl.score_block)
    row = idx[0, 0, n].copy()
    assert eps_valid(row, S32[0, 0, n], c)
    # replace the best selected key by the worst candidate
    worst = int(np.argmin(S32[0, 0, n, :c]))
    row[np.argmax(S32[0, 0, n, row])] = worst
    assert not eps_valid(np.sort(row), S32[0, 0, n], c)
    bad = idx.copy()
    bad[0, 0, n] = np.sort(row)
    units = [(0, 0, m) for m in range(wl.n_blocks)]
    with pytest.raises(AssertionError):
        index_agreement(wl, bad, S32, units)
    ok = index_agreement(wl, idx, S32, units)
    assert ok["rows_differing"] == 0 and ok["mean_iou"] == 1.0
