#!/usr/bin/env python3
"""Benchmark of the HySparse hybrid-block hot path on one MI355X.

Default workload: decode at 128K context (B 4, Hq 64 / Hkv 4, D 128, bf16,
K 2048, window 128, 9 sparse layers).  ``value`` is the sparse layer's decode
tokens per second (batch / time of one sparse layer), measured cold: a 1 GiB
write evicts the caches before each timed layer, and the layer's time is the
sum of its split and merge kernels' durations, each bracketed by HIP events
that the library records on its launch stream.  The line also carries the
same layer warm (layers back to back, rows partly served from the last-level
cache), its per-kernel cold durations, the bandwidth a launch of the same
size reaches with nothing else to do (a streaming read of the layer's bytes,
a gather of its rows), the roofline of the step's dominant kernel (the full
layer's split kernel) with a streaming read of the same K and V bytes beside
it, the whole hybrid block (full layer + top-K + all sparse layers: the K
timed steps), and the 128K prefill full layer (both sweeps) against the bf16
MFMA peak.

Inputs are resident in HBM before any timed region.  Per-kernel durations
come from HIP events that the library records around each kernel on its
launch stream (separate passes, so the timed steps carry no extra events).
The ``cpu_baseline`` leg times the CPU oracle on a bounded sample of the same
workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "sparse-layer decode tokens/s + HBM GB/s (% roofline) at 128K ctx, K=2048"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3


# workloads whose inputs are drawn on the GPU (too large to draw on the host)
DEVICE_INPUTS = ("prefill128k",)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode128k",
                    choices=["decode128k", "decode8k", "prefill32k", "prefill128k", "tiny", "hier128k",
                             "decode128k_loop"])
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference for HBM counters")
    ap.add_argument("--layer-reps", type=int, default=50, help="cold / warm sparse-layer repetitions")
    ap.add_argument("--prefill128k", type=int, default=1,
                    help="decode128k: also time the 128K prefill full layer (0 skips it)")
    return ap.parse_args()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs (profiles/
    hbm_traffic.json), or None once the kernel's source has changed."""
    from long_context_hybrid_amd.profiling import recorded_traffic
    return recorded_traffic(workload, kernel)


def copy_calibration(mib: int):
    import torch
    x = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": mib << 20, "bytes_written_per_launch": mib << 20,
                      "launches": 5}), flush=True)


def sparse_layer_bytes(wl, idx_np):
    """Algorithmic bytes of one sparse layer: the gathered K and V rows of both
    branches (valid entries only), the layer's queries and outputs, the indices."""
    e = 2 if wl.dtype == "bf16" else 4
    row = wl.head_dim * e
    B, Hkv, NB, K = idx_np.shape
    Tq, Tkv, Sb, W = wl.q_len, wl.kv_len, wl.score_block, wl.window
    rows = 0
    for n in range(NB):
        i0, i1 = n * Sb, min((n + 1) * Sb, Tq)
        last = Tkv - Tq + i1 - 1
        first = Tkv - Tq + i0
        nsel = int((idx_np[:, :, n] >= 0).sum())
        nwin = B * Hkv * (last + 1 - max(0, first - W + 1))
        rows += nsel + nwin
    q_out = 2 * wl.batch * Tq * wl.n_q_heads * wl.head_dim * e
    return 2 * rows * row + q_out + idx_np.size * 4


def full_layer_flops(wl):
    """Algorithmic FLOPs of the causal full layer: QK^T and PV over every
    (query, head, key <= position) triple, 2 FLOPs per multiply-add."""
    Tq, Tkv = wl.q_len, wl.kv_len
    pairs = Tq * (Tkv - Tq) + Tq * (Tq + 1) // 2
    return 4 * wl.head_dim * wl.batch * wl.n_q_heads * pairs


def sparse_layer_flops(wl, idx_np):
    """Algorithmic FLOPs of one sparse layer: QK^T and PV over each query
    head's global keys (selected, <= position) and window keys."""
    B, Hkv, NB, K = idx_np.shape
    Tq, Tkv, Sb, W = wl.q_len, wl.kv_len, wl.score_block, wl.window
    pos = Tkv - Tq + np.arange(Tq)
    total = 0
    for n in range(NB):
        i0, i1 = n * Sb, min((n + 1) * Sb, Tq)
        p = pos[i0:i1]
        rows = np.sort(np.where(idx_np[:, :, n] >= 0, idx_np[:, :, n], np.iinfo(np.int32).max), axis=-1)
        rows = rows.reshape(-1, K)
        glob = sum(int(np.searchsorted(r, p, side="right").sum()) for r in rows)
        win = int(np.minimum(W, p + 1).sum()) * B * Hkv
        total += glob + win
    return 4 * wl.head_dim * wl.group * total


def full_split_bytes(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return 2 * wl.batch * wl.kv_len * wl.n_kv_heads * wl.head_dim * e + wl.batch * wl.q_len * wl.n_q_heads * wl.head_dim * e


def cpu_baseline(wl, inp, budget_s: float):
    """Time the oracle on the same inputs, within a bounded budget.

    Decode workloads: the oracle's sparse layer (the metric's subject) over
    every (batch, KV-group) unit of the workload, repeated over the layers'
    queries until half the budget is spent, with indices from the oracle's
    own full layer and top-K (computed before the timed part); then the whole
    block (full layer, top-K, every sparse layer) on (batch, KV-group) units
    for the other half, scaled to the block.  Prefill workloads: the block on
    (batch, KV-group) units, scaled."""
    from threadpoolctl import threadpool_info
    from oracle import hysparse_oracle as orc
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    units = [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    NB = wl.n_blocks
    res = {"unit": "tokens/s", "cores": int(threads), "kind": "oracle"}
    block_budget = budget_s
    if wl.q_len == 1:
        idx = {}
        for (b, g) in units:
            _, _, s = orc.full_layer_block(inp.q_full, inp.k, inp.v, b, g, 0, 1)
            idx[b, g] = orc.topk_row(s.astype(np.float32), wl.kv_len, wl.k_top)
        layers = 0
        t0 = time.perf_counter()
        while True:
            l = layers % wl.n_sparse
            for (b, g) in units:
                orc.sparse_layer_block(inp.q_sparse[l], inp.k, inp.v, idx[b, g], b, g, 0, 1, wl.window,
                                       inp.gate_logits[l])
            layers += 1
            if time.perf_counter() - t0 > budget_s / 2:
                break
        el = time.perf_counter() - t0
        res["value"] = wl.batch * layers / el
        res["sample"] = (f"{layers} whole sparse layers (all {len(units)} (batch, KV-group) units, K {wl.k_top}, "
                         f"window {wl.window}) in {el:.1f} s, on the oracle's own indices")
        block_budget = budget_s / 2
    done = 0
    t0 = time.perf_counter()
    for (b, g) in units:
        for n in range(NB):
            _, _, s = orc.full_layer_block(inp.q_full, inp.k, inp.v, b, g, n, wl.score_block)
            c = orc.candidate_count(n, wl.q_len, wl.kv_len, wl.score_block)
            ix = orc.topk_row(s.astype(np.float32), c, wl.k_top)
            for l in range(wl.n_sparse):
                orc.sparse_layer_block(inp.q_sparse[l], inp.k, inp.v, ix, b, g, n, wl.score_block, wl.window,
                                       inp.gate_logits[l])
        done += 1
        if time.perf_counter() - t0 > block_budget:
            break
    el = time.perf_counter() - t0
    block_tps = wl.batch * wl.q_len / (el * len(units) / done)
    res["block_tokens_per_s"] = block_tps
    res["block_sample"] = (f"{done} of {len(units)} (batch, KV-group) units of one block (full layer, top-K, "
                           f"{wl.n_sparse} sparse layers) in {el:.1f} s, scaled to the whole block")
    if wl.q_len != 1:
        res["value"] = block_tps
        res["sample"] = res["block_sample"]
    return res


def events_ms(pairs):
    return np.array([a.elapsed_time(b) for a, b in pairs])


def timed_reps(torch, fn, reps, before=None):
    """Run fn reps times, each bracketed by HIP events on the current stream
    (the stream the library launches on); before() runs ahead of each
    bracket.  Returns the per-rep durations in ms."""
    pairs = []
    for r in range(reps):
        if before is not None:
            before(r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(r)
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return events_ms(pairs)


def traced(hy, torch, fn, reps, before=None):
    """Per-kernel durations (us) of fn over reps runs from the library's
    trace (each kernel's dispatch begin/end times): {name: [durations]}, and
    the span of each run (begin of its first kernel to end of its last, us)."""
    trace = hy.KernelTrace(capacity_kernels=64)
    per, spans = {}, []
    for r in range(reps):
        if before is not None:
            before(r)
        trace.begin()
        fn(r)
        rows = trace.end()
        for name, t in rows:
            per.setdefault(name, []).append(1e3 * t)
        if rows:
            spans.append(1e3 * trace.span_ms(0, len(rows) - 1))
    torch.cuda.synchronize()
    return per, np.array(spans)


def decode_layer_measurements(args, wl, hy, torch, k, v, qs, gates, idx, sb_bytes, dev):
    """The sparse decode layer cold and warm, per-kernel cold durations, and
    the size-matched bandwidth ceilings (module docstring)."""
    B, Tkv, Hkv, D = k.shape
    N = len(qs)
    outs = [torch.empty_like(q) for q in qs]
    desc = hy.make_desc(qs[0], k)
    ws = torch.empty(hy.hysparse_workspace_bytes(hy.HYS_OP_SPARSE, desc, 1, wl.k_top, wl.window), dtype=torch.uint8,
                     device=dev)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def flush(r):
        flush_buf.fill_(r & 0xFF)  # 1 GiB written: evicts the L2s and the last-level cache

    def layer(r):
        l = r % N
        hy.hysparse_sparse_attn(qs[l], k, v, idx, wl.k_top, 1, wl.window, gates[l], out=outs[l], workspace=ws)

    reps = args.layer_reps
    for r in range(5):
        layer(r)
    spin = lambda r: torch.cuda._sleep(2_000_000)
    # cold: each layer after the flush.  The layer's time is the sum of its
    # kernels' durations (dispatch begin/end timestamps, as a kernel trace
    # gives them); the same layers between two ordinary HIP events (launch
    # gaps and the events' own overhead included) are reported beside it
    per, _ = traced(hy, torch, layer, reps, before=flush)
    cold = np.sum([np.array(t) for t in per.values()], axis=0) / 1e3
    cold_ev = timed_reps(torch, layer, reps, before=flush)
    kern_cold = {n: float(np.median(t)) for n, t in per.items()}
    # warm: the N layers of a block back to back between two HIP events, per
    # layer; a spin kernel ahead of each run keeps the GPU busy while the host
    # enqueues the run, so that host-side call overhead is not timed
    warm = timed_reps(torch, lambda r: [layer(l) for l in range(N)], max(reps // N, 5), before=spin) / N

    # ceilings of one launch of the same size
    row_bytes = D * k.element_size()
    idx_np = idx.cpu().numpy()
    rows = []
    for b in range(B):
        for g in range(Hkv):
            sel = idx_np[b, g, 0]
            sel = sel[sel >= 0].astype(np.int64)
            win = np.arange(max(0, Tkv - wl.window), Tkv, dtype=np.int64)
            rows.append((b * Tkv + np.concatenate([sel, win])) * Hkv + g)
    rows_t = torch.from_numpy(np.concatenate(rows).astype(np.int32)).to(dev)
    gather_bytes = 2 * rows_t.numel() * row_bytes + 4 * rows_t.numel()
    stream_bytes = (sb_bytes + 15) // 16 * 16
    kflat, vflat = k.view(-1), v.view(-1)
    cws = torch.empty(hy.hysparse_ceiling_workspace_bytes(stream_bytes, rows_t.numel()), dtype=torch.uint8, device=dev)
    for _ in range(3):
        hy.hysparse_ceiling_stream_read(kflat, stream_bytes, workspace=cws)
        hy.hysparse_ceiling_gather(k, v, rows_t, workspace=cws)
    _, c_stream = traced(hy, torch, lambda r: hy.hysparse_ceiling_stream_read(kflat, stream_bytes, workspace=cws),
                         reps, before=flush)
    _, c_gather = traced(hy, torch, lambda r: hy.hysparse_ceiling_gather(k, v, rows_t, workspace=cws), reps,
                         before=flush)
    c_stream, c_gather = c_stream / 1e3, c_gather / 1e3
    torch.cuda.synchronize()
    del flush_buf

    def rate(nbytes, ms):
        us = float(np.median(ms)) * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us_median": us, "us_mean": float(np.mean(ms)) * 1e3, "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}

    cold_r, warm_r = rate(sb_bytes, cold), rate(sb_bytes, warm)
    st_r, ga_r = rate(stream_bytes, c_stream), rate(gather_bytes, c_gather)
    cold_r.update({"tokens_per_s": B / (cold_r["us_median"] * 1e-6),
                   "us_median_event_bracket": float(np.median(cold_ev)) * 1e3,
                   "method": f"median over {reps} layers, each after a 1 GiB write (caches evicted), of the sum of "
                             "the layer's kernel durations (dispatch begin/end timestamps, as a kernel trace gives "
                             "them); us_median_event_bracket: the same layers between two ordinary HIP events "
                             "(launch gaps and event overhead included)"})
    warm_r.update({"tokens_per_s": B / (warm_r["us_median"] * 1e-6),
                   "method": f"the {N} layers of a block back to back (gathered rows partly in the last-level "
                             f"cache) between two HIP events, enqueued behind a spin kernel, per layer (launch "
                             "gaps included)"})
    st_r.update({"bytes": stream_bytes, "what": "one launch reading the layer's byte count as one contiguous "
                                                "stream (non-temporal 16-byte loads), cold, kernel duration"})
    ga_r.update({"bytes": gather_bytes, "rows": int(rows_t.numel()),
                 "what": "one launch reading the layer's own K and V rows (selected + window, 256 B each) at "
                         "their row indices, indices loaded first, cold, kernel duration"})
    return {"alg_bytes": sb_bytes, "cold": cold_r, "warm": warm_r, "kernels_cold_us": kern_cold,
            "ceiling": {"stream_read": st_r, "gather_rows": ga_r,
                        "cold_frac_of_stream_ceiling": st_r["us_median"] / cold_r["us_median"],
                        "cold_frac_of_gather_ceiling": ga_r["us_median"] / cold_r["us_median"]}}


def full_split_ceiling(hy, torch, k, v, dev, reps=5):
    """What one launch that only streams the full decode layer's K and V
    reaches on this GPU (the streaming-read ceiling kernel, non-temporal
    16-byte loads, nothing computed; one launch for K, one for V): the
    attainable rate beside the 8 TB/s peak for the full layer's split
    kernel, which reads the same bytes."""
    kflat, vflat = k.reshape(-1), v.reshape(-1)
    nbytes = kflat.numel() * kflat.element_size()
    cws = torch.empty(hy.hysparse_ceiling_workspace_bytes(nbytes, 0), dtype=torch.uint8, device=dev)

    def run(r):
        hy.hysparse_ceiling_stream_read(kflat, nbytes, workspace=cws)
        hy.hysparse_ceiling_stream_read(vflat, nbytes, workspace=cws)

    run(0)
    per, _ = traced(hy, torch, run, reps)
    pair_us = np.array(per["ceiling_stream"]).reshape(reps, 2).sum(axis=1)
    us = float(np.median(pair_us))
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    return {"GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "us_median": us, "bytes": 2 * nbytes,
            "what": "K and V of the cache read once as two contiguous streams (one launch each, non-temporal "
                    "16-byte loads, nothing computed), kernel durations"}


def prefill128k_full_layer(hy, torch, gen, dev, reps=2):
    """The 128K prefill full layer (both sweeps), inputs drawn on the GPU,
    against the bf16 MFMA peak."""
    wl = gen.WORKLOADS["prefill128k"]
    qf, k, v, _, _ = gen.make_device_inputs(wl, dev, n_sparse=0)
    B, Tq, Hq, D = qf.shape
    Hkv, Tkv = k.shape[2], k.shape[1]
    out = torch.empty_like(qf)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hkv, wl.n_blocks, Tkv), dtype=torch.float32, device=dev)
    desc = hy.make_desc(qf, k)
    ws = torch.empty(hy.hysparse_workspace_bytes(hy.HYS_OP_FULL, desc, wl.score_block), dtype=torch.uint8, device=dev)

    def run(r):
        hy.hysparse_full_attn_scores(qf, k, v, wl.score_block, out=out, lse=lse, scores=scores, workspace=ws)

    run(0)
    torch.cuda.synchronize()
    ms = timed_reps(torch, run, reps)
    per, _ = traced(hy, torch, run, reps)
    ff = full_layer_flops(wl)
    t_us = float(np.median(ms)) * 1e3
    fwd = float(np.median(per["full_prefill_fwd"]))
    sco = float(np.median(per["full_prefill_scores"]))
    res = {"workload": "prefill128k full layer (B 1, 131072 queries and keys, Hq 64 / Hkv 4, D 128, bf16, "
                       "scores per 64-query block)",
           "alg_flops": ff, "us": t_us, "tflops_algorithmic": ff / (t_us * 1e-6) / 1e12,
           "frac_bf16_peak": ff / (t_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
           "fwd_sweep_us": fwd, "fwd_sweep_frac_bf16_peak": ff / (fwd * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
           "score_sweep_us": sco,
           "score_sweep_qk_frac_bf16_peak": (ff // 2) / (sco * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
           "note": "algorithmic FLOPs = QK^T + PV over every causal (query, head, key) triple; the score sweep "
                   "recomputes QK^T once the final LSE is known", "inputs": "drawn on the GPU"}
    del qf, k, v, out, lse, scores, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library and this benchmark run on one GPU; --gpus above 1 is not supported (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_hybrid_amd import hysparse as hy
    from long_context_hybrid_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hy.lib()
    # decode128k_loop: the decode loop on the 128K workload; every step appends
    # one token's K/V to the cache and runs the block on the grown cache
    loop = args.workload.endswith("_loop")
    wl = gen.WORKLOADS[args.workload[:-len("_loop")] if loop else args.workload]
    t_gen = time.perf_counter()
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    if wl.name in DEVICE_INPUTS:
        inp = None
        qf, k, v, qs, gates = gen.make_device_inputs(wl, dev)
    else:
        inp = gen.make_inputs(wl)
        to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(tdt).to(dev)
        qf, k, v = to(inp.q_full), to(inp.k), to(inp.v)
        qs = [to(q) for q in inp.q_sparse]
        gates = torch.from_numpy(inp.gate_logits).to(dev)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    B, Tq, Hq, D = qf.shape
    Hkv, Tkv = k.shape[2], k.shape[1]
    NB = wl.n_blocks
    out_full = torch.empty_like(qf)
    outs = [torch.empty_like(qf) for _ in qs]
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hkv, NB, Tkv), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, NB, wl.k_top), dtype=torch.int32, device=dev)
    desc = hy.make_desc(qf, k)
    ws = torch.empty(hy.hysparse_workspace_bytes(hy.HYS_OP_HYBRID, desc, wl.score_block, wl.k_top, wl.window),
                     dtype=torch.uint8, device=dev)

    def step():
        hy.hysparse_hybrid_block(qf, k, v, qs, gates, wl.k_top, wl.score_block, wl.window, out_full=out_full,
                                 out_sparse=outs, lse=lse, scores=scores, idx=idx, workspace=ws)

    if loop:
        # cache = the workload's keys/values; steps append rows L0, L0 + 1, ...
        n_loop = args.warmup + 2 * args.steps
        L0 = Tkv - n_loop
        # token-major copies, so each step's rows [B, 1, Hkv, D] are contiguous
        k_rows = k[:, L0:].transpose(0, 1).contiguous().unsqueeze(2)
        v_rows = v[:, L0:].transpose(0, 1).contiguous().unsqueeze(2)
        kc, vc = k.clone(), v.clone()
        t_loop = [0]

        def step():
            t = t_loop[0] % n_loop
            L = L0 + t + 1
            hy.hysparse_append_kv(k_rows[t], v_rows[t], kc, vc, L - 1)
            hy.hysparse_hybrid_block(qf, kc[:, :L], vc[:, :L], qs, gates, wl.k_top, wl.score_block, wl.window,
                                     out_full=out_full, out_sparse=outs, lse=lse,
                                     scores=scores.view(-1)[:B * Hkv * L].view(B, Hkv, 1, L), idx=idx, workspace=ws)
            t_loop[0] += 1

    hier = wl.name == "hier128k"
    if hier:
        # full layer -> hierarchical selection (128-key pooled blocks, keep 64) -> sparse layers
        HB, HKEEP = 128, 64
        ws_full = torch.empty(hy.hysparse_workspace_bytes(hy.HYS_OP_FULL, desc, 1), dtype=torch.uint8, device=dev)
        ws_sp = torch.empty(hy.hysparse_workspace_bytes(hy.HYS_OP_SPARSE, desc, 1, wl.k_top, wl.window),
                            dtype=torch.uint8, device=dev)
        ws_h = torch.empty(hy.hysparse_hier_workspace_bytes(desc, HB, HKEEP, wl.k_top), dtype=torch.uint8, device=dev)
        bsc = torch.empty((B, Hkv, -(-Tkv // HB)), dtype=torch.float32, device=dev)
        blk = torch.empty((B, Hkv, HKEEP), dtype=torch.int32, device=dev)
        # pooled keys kept beside the cache: pooled once here; a decode step
        # refreshes only the block that holds the newest token
        kbar = torch.empty((B, -(-Tkv // HB), Hkv, D), dtype=torch.float32, device=dev)
        hy.hysparse_hier_pool(k, HB, kbar)
        m_last = (Tkv - 1) // HB

        def step():
            hy.hysparse_full_attn_scores(qf, k, v, 1, out=out_full, lse=lse, scores=scores, workspace=ws_full)
            hy.hysparse_hier_pool(k, HB, kbar, m_last, m_last + 1)
            hy.hysparse_hier_select_pooled(qf, k, kbar, scores, HB, HKEEP, wl.k_top, idx=idx, block_scores=bsc,
                                           blocks=blk, workspace=ws_h)
            for l in range(len(qs)):
                hy.hysparse_sparse_attn(qs[l], k, v, idx, wl.k_top, 1, wl.window, gates[l], out=outs[l],
                                        workspace=ws_sp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    tokens_per_step = B * Tq
    block_tps = tokens_per_step / (ms * 1e-3)
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step (wall {1e3 * wall / args.steps:.4f})", file=sys.stderr,
          flush=True)

    # per-kernel durations: second pass with the library's event trace
    per, _ = traced(hy, torch, lambda r: step(), args.steps)
    kernels = {n: {"launches_per_step": len(t) / args.steps, "avg_us": float(np.mean(t)),
                   "us_per_step": float(np.sum(t)) / args.steps} for n, t in per.items()}
    traced_ms = sum(v["us_per_step"] for v in kernels.values()) / 1e3

    idx_np = idx.cpu().numpy()
    decode = Tq == 1 and not loop and not hier and len(qs) > 0
    result = {"metric": METRIC, "value": block_tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
              "config": {"workload": wl.name, "batch": B, "q_len": Tq, "context": Tkv, "q_heads": Hq,
                         "kv_heads": Hkv, "head_dim": D, "k_top": wl.k_top, "window": wl.window,
                         "n_sparse": len(qs), "score_block": wl.score_block,
                         "step": "hybrid block: full layer + top-K + all sparse layers"}}

    def roof(name, alg_bytes, us=None):
        if name not in kernels and us is None:
            return None
        us = kernels[name]["avg_us"] if us is None else us
        gbs = alg_bytes / (us * 1e-6) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, name),
                "alg_bytes_per_launch": alg_bytes, "avg_us": us}

    mfma_peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS

    def roof_flops(name, flops):
        if name not in kernels:
            return None
        us = kernels[name]["avg_us"]
        tf = flops / (us * 1e-6) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": tf, "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": tf / mfma_peak, "traffic": measured_traffic(wl.name, name), "alg_flops_per_launch": flops,
                "avg_us": us}

    dom = max(kernels, key=lambda n: kernels[n]["us_per_step"])
    result["dominant_kernel"] = dom
    if Tq == 1:
        sb = sparse_layer_bytes(wl, idx_np)
        rf = roof("full_decode_split", full_split_bytes(wl))
        if rf:
            c = full_split_ceiling(hy, torch, k, v, dev)
            rf["ceiling"] = c
            rf["frac_of_ceiling"] = rf["achieved"] / c["GB_per_s"]
        result["roofline"] = rf
        result["hybrid_block"] = {"tokens_per_s": block_tps, "ms_per_step": ms,
                                  "what": "full layer + top-K + all sparse layers, the timed steps"}
        if decode:
            print("[bench] sparse layer cold / warm, ceilings", file=sys.stderr, flush=True)
            sl = decode_layer_measurements(args, wl, hy, torch, k, v, qs, gates, idx, sb, dev)
            result["value"] = sl["cold"]["tokens_per_s"]
            result["value_is"] = ("sparse-layer decode tokens/s, cold (batch / median time of one sparse layer "
                                  "after a 1 GiB cache-evicting write, kernel durations); sparse_layer.cold.frac_hbm "
                                  "is its fraction of the 8 TB/s HBM peak")
            result["sparse_layer"] = sl
            result["roofline_sparse"] = roof("sparse_decode", sb, us=sl["kernels_cold_us"].get("sparse_decode"))
            if result["roofline_sparse"]:
                result["roofline_sparse"]["note"] = ("cold split kernel alone (gather, both branches' softmax); "
                                                     "the merge kernel is the rest of the layer")
    else:
        ff = full_layer_flops(wl)
        rf = roof_flops("full_prefill_fwd", ff)
        rsc = roof_flops("full_prefill_scores", ff // 2)
        sf = sparse_layer_flops(wl, idx_np)
        rsp = roof_flops("sparse_prefill", sf)
        by = {"full_prefill_fwd": rf, "full_prefill_scores": rsc, "sparse_prefill": rsp}
        result["roofline"] = by.get(dom) or rf
        result["roofline_full_fwd"] = rf
        result["roofline_full_scores"] = rsc
        result["roofline_sparse"] = rsp
        if rf and rsc:
            t_full = (rf["avg_us"] + rsc["avg_us"]) * 1e-6
            result["full_layer"] = {"tflops_algorithmic": ff / t_full / 1e12, "frac_peak": ff / t_full / 1e12 / mfma_peak,
                                    "us": t_full * 1e6, "alg_flops": ff,
                                    "note": "two sweeps: the score sweep recomputes QK^T after the final LSE"}
    if hier:
        flat = hy.hysparse_topk(scores.view(B * Hkv, Tkv), wl.k_top).view(B, Hkv, 1, wl.k_top)
        o_flat = hy.hysparse_sparse_attn(qs[0], k, v, flat, wl.k_top, 1, wl.window, gates[0])
        torch.cuda.synchronize()
        fl, hi = flat.cpu().numpy(), idx_np
        def iou(a, b):  # set overlap of two index lists, padding (-1) ignored
            sa, sb = np.unique(a[a >= 0]), np.unique(b[b >= 0])
            union = np.union1d(sa, sb).size
            return np.intersect1d(sa, sb).size / union if union else 1.0

        ious = [iou(hi[b, g], fl[b, g]) for b in range(B) for g in range(Hkv)]
        rec = lambda sel: float(np.mean([np.isin(inp.planted[b], sel[b, g]).mean() for b in range(B)
                                          for g in range(Hkv)]))
        oh, of = outs[0].float().cpu().numpy(), o_flat.float().cpu().numpy()
        result["hierarchical"] = {"block": 128, "blocks_kept": 64, "mean_iou_vs_flat": float(np.mean(ious)),
                                  "planted_recall": rec(hi), "planted_recall_flat": rec(fl),
                                  "sparse_out_rel_l2_vs_flat": float(np.linalg.norm(oh - of) / np.linalg.norm(of))}
    result["kernels"] = kernels
    result["traced_ms_per_step"] = traced_ms
    if loop:
        result["config"]["workload"] = args.workload
        result["config"]["context"] = f"{L0 + 1}..{L0 + n_loop} (grows by one token per step)"
        result["config"]["step"] = ("decode step: append one token's K/V to the cache, full layer on the grown cache, "
                                    "top-K, all sparse layers")
    if inp is not None:
        result["input_sha256"] = inp.sha256()
    else:
        result["inputs"] = "drawn on the GPU: torch generator seeded per (config, tensor, layer)"
    if decode and wl.name == "decode128k" and args.prefill128k:
        print("[bench] 128K prefill full layer", file=sys.stderr, flush=True)
        del ws
        torch.cuda.empty_cache()
        result["full_layer_prefill128k"] = prefill128k_full_layer(hy, torch, gen, dev)
    if args.cpu_baseline and not hier and inp is not None:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
