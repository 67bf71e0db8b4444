"""Seeded synthetic inputs for the hybrid-block attention path.

This module only draws numbers: it holds none of the attention, scoring,
selection or gating arithmetic.  Both the CPU oracle (``oracle/``) and the
HIP path consume what it produces, so it is the one thing they share.

Recipe (one generator per tensor, so every tensor is reproducible alone):

* ``numpy.random.Generator(PCG64(SeedSequence([config_id, tensor_id, layer])))``
  with tensor ids 0 = full-layer query, 1 = keys, 2 = values, 3 = sparse-layer
  query (``layer`` = 0..N-1), 4 = gate logits, 5 = planted positions, 6 / 7 =
  a sparse layer's own window keys / values (``own_window_kv``).
* Values are drawn in float64, cast to float32 (round to nearest even), and for
  bf16 workloads rounded once more to bf16 (round to nearest even).  The arrays
  returned are float32 whose values are exactly the stored ones, so every
  consumer reads identical numbers.
* Layouts are logical: queries ``[B, Tq, Hq, D]``, keys/values ``[B, Tkv, Hkv, D]``.

Workloads (shapes from the HySparse pages: 8K-128K contexts on the Baidu
article's background section, K = 2048 as the DeepSeek sparse-attention
figure on the Ultralytics glossary page, a 128-token window and a sigmoid gate
from the intelliparadigm article section 2.2, about one full layer in ten from
the HySparse abstract):

* ``tiny``       B1, T 256 prefill, Hq 4 / Hkv 1, D 64, fp32, N(0,1)/8; gates U(-2,2);
                 score block 1, K 32, window 16, one sparse layer.
* ``decode8k``   B16, context 8192, Hq 32 / Hkv 8, D 128, bf16, N(0,1)/sqrt(128);
                 gates N(0,1); K 1024, window 128, 3 sparse layers.
* ``prefill32k`` B1, T 32768 prefill, Hq 32 / Hkv 8, D 128, bf16, N(0,1)/sqrt(128);
                 score block 64, K 2048, window 128, 3 sparse layers.
* ``decode128k`` B4, context 131072, Hq 64 / Hkv 4, D 128, bf16, N(0,1); 64 planted
                 key rows per sequence; K 2048, window 128, 9 sparse layers.
* ``hier128k``   as ``decode128k`` (block-pooled selection variant).
* ``prefill128k`` B1, T 131072 prefill with the 128K model's attention shape
                 (Hq 64 / Hkv 4, D 128), bf16, N(0,1) (unit-std logits, as the 128K
                 decode); score block 64,
                 K 2048, window 128, 9 sparse layers.  Too large to draw on the
                 host in float64: ``make_device_inputs`` draws it on the GPU.

Planting (``decode128k``): per sequence, 64 positions drawn without replacement
from ``[0, ctx - 128)``; at each, the key row of every KV group g is set to
``32 * u`` where ``u`` is the unit vector along the sum of group g's full-layer
query heads.  This gives needles that a correct selection must find.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

T_QFULL, T_K, T_V, T_QSPARSE, T_GATE, T_PLANT, T_KWIN, T_VWIN = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    q_len: int
    kv_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    std: float            # standard deviation of Q, K (and V unless v_std is set)
    gate_dist: str        # "uniform2" (U(-2,2)) or "normal" (N(0,1))
    score_block: int
    k_top: int
    window: int
    n_sparse: int
    n_planted: int = 0
    v_std: Optional[float] = None  # standard deviation of V (None: std)

    @property
    def value_std(self) -> float:
        return self.std if self.v_std is None else self.v_std

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks(self) -> int:
        return -(-self.q_len // self.score_block)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 256, 256, 4, 1, 64, "f32", 1.0 / 8.0,
                     "uniform2", 1, 32, 16, 1),
    "decode8k": Workload("decode8k", 1, 16, 1, 8192, 32, 8, 128, "bf16",
                         1.0 / np.sqrt(128.0), "normal", 1, 1024, 128, 3),
    "prefill32k": Workload("prefill32k", 2, 1, 32768, 32768, 32, 8, 128, "bf16",
                           1.0 / np.sqrt(128.0), "normal", 64, 2048, 128, 3),
    "decode128k": Workload("decode128k", 3, 4, 1, 131072, 64, 4, 128, "bf16",
                           1.0, "normal", 1, 2048, 128, 9, n_planted=64),
    "hier128k": Workload("hier128k", 4, 4, 1, 131072, 64, 4, 128, "bf16",
                         1.0, "normal", 1, 2048, 128, 9, n_planted=64),
    "prefill128k": Workload("prefill128k", 5, 1, 131072, 131072, 64, 4, 128, "bf16",
                            1.0, "normal", 64, 2048, 128, 9),
}


def _rng(config_id: int, tensor_id: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(config_id), int(tensor_id), int(layer)])))


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), kept as float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(x32.shape)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return round_bf16(x32) if dtype == "bf16" else x32


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    rng.standard_normal(out=out, dtype=np.float64)
    if std != 1.0:
        out *= std
    return out


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q_full: np.ndarray             # [B, Tq, Hq, D] float32 (stored values)
    k: np.ndarray                  # [B, Tkv, Hkv, D]
    v: np.ndarray                  # [B, Tkv, Hkv, D]
    q_sparse: list                 # N x [B, Tq, Hq, D]
    gate_logits: np.ndarray        # [N, Hq] float32
    planted: Optional[np.ndarray]  # [B, n_planted] int64 positions, or None

    def sha256(self) -> dict:
        h = {}
        for name in ("q_full", "k", "v", "gate_logits"):
            h[name] = hashlib.sha256(np.ascontiguousarray(getattr(self, name)).tobytes()).hexdigest()[:16]
        h["q_sparse"] = [hashlib.sha256(np.ascontiguousarray(q).tobytes()).hexdigest()[:16]
                         for q in self.q_sparse]
        return h


def make_inputs(wl: Workload, n_sparse: Optional[int] = None) -> Inputs:
    """Draw every input of one hybrid block for workload ``wl``."""
    B, Tq, Tkv = wl.batch, wl.q_len, wl.kv_len
    Hq, Hkv, D = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    N = wl.n_sparse if n_sparse is None else n_sparse
    cid = wl.config_id

    q_full64 = _normal(_rng(cid, T_QFULL), (B, Tq, Hq, D), wl.std)
    q_full = _store(q_full64, wl.dtype)
    del q_full64
    k64 = _normal(_rng(cid, T_K), (B, Tkv, Hkv, D), wl.std)
    planted = None
    if wl.n_planted:
        G = wl.group
        prng = _rng(cid, T_PLANT)
        planted = np.stack([np.sort(prng.choice(Tkv - 128, size=wl.n_planted, replace=False))
                            for _ in range(B)]).astype(np.int64)
        # direction of each group's summed full-layer queries (last query row)
        qs = q_full[:, -1].astype(np.float64).reshape(B, Hkv, G, D).sum(axis=2)
        u = qs / np.linalg.norm(qs, axis=-1, keepdims=True)
        for b in range(B):
            k64[b, planted[b]] = 32.0 * u[b][None, :, :]
    k = _store(k64, wl.dtype)
    del k64
    v = _store(_normal(_rng(cid, T_V), (B, Tkv, Hkv, D), wl.value_std), wl.dtype)
    q_sparse = [_store(_normal(_rng(cid, T_QSPARSE, l), (B, Tq, Hq, D), wl.std), wl.dtype)
                for l in range(N)]
    grng = _rng(cid, T_GATE)
    if wl.gate_dist == "uniform2":
        gates = grng.uniform(-2.0, 2.0, size=(N, Hq))
    else:
        gates = grng.standard_normal(size=(N, Hq))
    return Inputs(wl, q_full, k, v, q_sparse, gates.astype(np.float32), planted)


def random_scores(seed: int, n_rows: int, row_len: int, kind: str = "probs") -> np.ndarray:
    """Score rows for standalone top-K checks (float32).

    ``kind``: "probs" - positive, softmax-like magnitudes with many near-ties;
    "ties"  - values from a set of 7 levels, so equal keys cross the K boundary;
    "signed" - normal values of both signs, including -0.0 and +0.0;
    "cluster" - a small background, a few large outliers at the start of the
    row (indices 0..4) and a dense cluster of ``min(3000, row_len // 3)``
    keys at random positions taking 64 adjacent float32 values just above
    0.5 (many ties, and a key range so stretched by the outliers that the
    cluster shares one bin of any coarse radix digit);
    "cluster_wide" - the same with 16384 adjacent values (few ties).
    """
    rng = _rng(1000 + seed, 0)
    if kind == "probs":
        x = np.exp(rng.standard_normal((n_rows, row_len)) * 2.0) / row_len
    elif kind == "ties":
        x = rng.integers(0, 7, size=(n_rows, row_len)).astype(np.float64) * 0.125
    elif kind == "signed":
        x = rng.standard_normal((n_rows, row_len))
        z = rng.random((n_rows, row_len))
        x[z < 0.02] = 0.0
        x[(z >= 0.02) & (z < 0.04)] = -0.0
    elif kind in ("cluster", "cluster_wide"):
        x = rng.random((n_rows, row_len)) * 1e-3
        c = min(3000, row_len // 3)
        levels = 64 if kind == "cluster" else 16384
        for r in range(n_rows):
            pos = 5 + rng.choice(row_len - 5, size=c, replace=False)
            x[r, pos] = 0.5 + rng.integers(0, levels, size=c) * 2.0 ** -24
        x[:, :5] = np.array([1e4, 1e3, 1e2, 10.0, 2.0])[: min(5, row_len)]
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def make_device_inputs(wl: Workload, device, n_sparse: Optional[int] = None):
    """Inputs of the same shapes and distributions as ``make_inputs``, drawn on
    the GPU with torch's generator (one seed per tensor, from the same
    (config, tensor, layer) triple), for workloads too large to draw on the
    host.  Values differ from ``make_inputs``; planting is not supported.
    Returns (q_full, k, v, [q_sparse], gate_logits) as device tensors."""
    import torch
    if wl.n_planted:
        raise ValueError("device inputs do not plant needles")
    B, Tq, Tkv = wl.batch, wl.q_len, wl.kv_len
    Hq, Hkv, D = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    N = wl.n_sparse if n_sparse is None else n_sparse
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def draw(shape, tensor_id, layer=0, std=wl.std):
        seed = int(np.random.SeedSequence([wl.config_id, tensor_id, layer]).generate_state(1, np.uint64)[0] >> 1)
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(0.0, std, generator=g)
        return x.to(dt)

    q_full = draw((B, Tq, Hq, D), T_QFULL)
    k = draw((B, Tkv, Hkv, D), T_K)
    v = draw((B, Tkv, Hkv, D), T_V, std=wl.value_std)
    q_sparse = [draw((B, Tq, Hq, D), T_QSPARSE, l) for l in range(N)]
    grng = _rng(wl.config_id, T_GATE)
    gates = grng.uniform(-2.0, 2.0, size=(N, Hq)) if wl.gate_dist == "uniform2" else grng.standard_normal(size=(N, Hq))
    return q_full, k, v, q_sparse, torch.from_numpy(gates.astype(np.float32)).to(device)


def own_window_kv(wl: Workload, layer: int = 0):
    """Keys and values of sparse layer ``layer``'s own window branch, by
    position: [B, Tkv, Hkv, D] each, same distribution and rounding as k, v."""
    shape = (wl.batch, wl.kv_len, wl.n_kv_heads, wl.head_dim)
    kw = _store(_normal(_rng(wl.config_id, T_KWIN, layer), shape, wl.std), wl.dtype)
    vw = _store(_normal(_rng(wl.config_id, T_VWIN, layer), shape, wl.value_std), wl.dtype)
    return kw, vw
