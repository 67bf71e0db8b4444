"""The bandwidth-ceiling helpers read exactly the bytes they are given: each
workgroup's word equals the XOR of the 32-bit words it was meant to read
(a streaming read of 16 KB per workgroup; a gather of 64 K and V rows per
workgroup, row indices outside the buffer skipped)."""
import numpy as np
import pytest
import torch

from long_context_hybrid_amd import hysparse as hy
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib():
    hy.lib()


def _xor_words(a: np.ndarray) -> np.uint32:
    return np.bitwise_xor.reduce(a.view(np.uint32).ravel()) if a.size else np.uint32(0)


def test_stream_read_covers_its_bytes():
    say("ceiling stream read")
    rng = np.random.default_rng(7)
    n = 5 * 16384 + 16 * 37  # a ragged last workgroup
    buf = rng.integers(0, 2**31, size=n // 4 + 8, dtype=np.int64).astype(np.uint32)
    dev = torch.from_numpy(buf.view(np.int32)).cuda()
    ws = torch.zeros(hy.hysparse_ceiling_workspace_bytes(n, 0), dtype=torch.uint8, device="cuda")
    hy.hysparse_ceiling_stream_read(dev, n, workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy().view(np.uint32)
    raw = buf.view(np.uint8)[:n]
    nb = -(-n // 16384)
    for b in range(nb):
        assert got[b] == _xor_words(raw[b * 16384:(b + 1) * 16384].copy()), b


def test_gather_covers_its_rows():
    say("ceiling gather")
    rng = np.random.default_rng(8)
    n_buf, D = 3000, 128
    k = rng.integers(0, 2**15, size=(n_buf, D), dtype=np.int64).astype(np.int16)
    v = rng.integers(0, 2**15, size=(n_buf, D), dtype=np.int64).astype(np.int16)
    rows = rng.integers(0, n_buf, size=200).astype(np.int32)
    rows[5], rows[77] = -1, n_buf  # skipped
    kt = torch.from_numpy(k).cuda().view(torch.bfloat16)
    vt = torch.from_numpy(v).cuda().view(torch.bfloat16)
    ws = torch.zeros(hy.hysparse_ceiling_workspace_bytes(0, rows.size), dtype=torch.uint8, device="cuda")
    hy.hysparse_ceiling_gather(kt, vt, torch.from_numpy(rows).cuda(), workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy().view(np.uint32)
    for b in range(-(-rows.size // 64)):
        acc = np.uint32(0)
        for r in rows[b * 64:(b + 1) * 64]:
            if 0 <= r < n_buf:
                acc ^= _xor_words(k[r].copy()) ^ _xor_words(v[r].copy())
        assert got[b] == acc, b
