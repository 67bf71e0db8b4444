"""hysparse_check_indices: status bits of index rows, compared with the rule
stated in include/hysparse.h written out below in numpy; rows that top-K
writes (from generated scores and from the oracle's selection) are valid."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from long_context_hybrid_amd import inputs as gen
from oracle import hysparse_oracle as orc
from tests.gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


def expected_status(row: np.ndarray, n: int, row_len: int) -> int:
    """The header's rule for one row, entry by entry."""
    flags, seen = 0, set()
    for e, x in enumerate(row.tolist()):
        if x >= 0:
            if x >= n:
                flags |= hy.HYS_IDX_OUT_OF_RANGE
            if x < row_len:
                if x in seen:
                    flags |= hy.HYS_IDX_DUPLICATE
                seen.add(x)
            if e > 0 and (row[e - 1] < 0 or row[e - 1] >= x):
                flags |= hy.HYS_IDX_ORDER
        elif x < -1:
            flags |= hy.HYS_IDX_OUT_OF_RANGE
    return flags


def test_check_indices_on_topk_rows_and_faults():
    say("check indices")
    R, L, K = 40, 3000, 300
    S = gen.random_scores(77, R, L, "ties")
    vl = np.random.default_rng(5).integers(0, L + 1, size=R).astype(np.int32)
    idx = orc.topk_rows(S, vl, K).astype(np.int32)
    rng = np.random.default_rng(6)
    bad = idx.copy()
    bad[1, 3] = bad[1, 4]                      # duplicate (and not ascending)
    bad[2, 0], bad[2, 1] = bad[2, 1], bad[2, 0]  # swapped: order only
    bad[3, 10] = -1                            # padding in the middle
    bad[4, -1] = L + 5                         # beyond the row
    bad[5, 7] = -3                             # below -1
    bad[6] = rng.permutation(bad[6])           # shuffled, still distinct
    bad[7, :] = 0                              # all the same key
    for name, rows in (("top-K rows", idx), ("faulty rows", bad)):
        got = host(hy.hysparse_check_indices(torch.from_numpy(rows).cuda(), L,
                                             valid_len=torch.from_numpy(vl).cuda()))
        torch.cuda.synchronize()
        want = np.array([expected_status(rows[r], int(vl[r]), L) for r in range(R)])
        np.testing.assert_array_equal(got, want, err_msg=name)
    assert (want[[1, 7]] & hy.HYS_IDX_DUPLICATE).all() and not (want[[2, 3, 6]] & hy.HYS_IDX_DUPLICATE).any()


def test_check_indices_on_hybrid_block_indices():
    """The hybrid block's own indices at the 8K decode shape are valid."""
    wl = gen.WORKLOADS["decode8k"].replace(batch=2, kv_len=3000, k_top=512, n_sparse=1)
    inp = gen.make_inputs(wl)
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    res = hy.hysparse_hybrid_block(to(inp.q_full), to(inp.k), to(inp.v), [to(q) for q in inp.q_sparse],
                                   torch.from_numpy(inp.gate_logits).cuda(), wl.k_top, 1, wl.window)
    st = host(hy.hysparse_check_indices(res["idx"], wl.kv_len))
    torch.cuda.synchronize()
    assert (st == 0).all()


def test_check_indices_at_the_maximum_row_length():
    """Rows of the largest supported length (a 64 KiB LDS bitmap), with entries
    at both ends of the row and a duplicate of the last position."""
    L, K = 524288, 64
    rng = np.random.default_rng(9)
    rows = np.stack([np.sort(rng.choice(L, size=K, replace=False)) for _ in range(3)]).astype(np.int32)
    rows[0, 0], rows[0, -1] = 0, L - 1
    rows[1, -2], rows[1, -1] = L - 1, L - 1   # duplicate of the last position
    got = host(hy.hysparse_check_indices(torch.from_numpy(rows).cuda(), L))
    torch.cuda.synchronize()
    want = np.array([expected_status(rows[r], L, L) for r in range(3)])
    np.testing.assert_array_equal(got, want)
    assert want[0] == 0 and want[1] & hy.HYS_IDX_DUPLICATE
