#!/usr/bin/env python3
"""Benchmark of the HySparse hybrid-block hot path on one MI355X.

One step = one hybrid block over one batch of synthetic input: the full
attention layer with score emission, the top-K select, then every sparse
layer (all of them reading the full layer's K/V and indices).  Default
workload: decode at 128K context (B 4, Hq 64 / Hkv 4, D 128, bf16, K 2048,
window 128, 9 sparse layers); ``value`` is decoded tokens per second of the
whole block, inputs resident in HBM.

Prints one JSON line.  Per-kernel durations come from HIP events that the
library records around each kernel on its launch stream (a second pass over
the same steps, so the timed pass carries no extra events).  The
``cpu_baseline`` leg times the CPU oracle on a bounded sample of the same
workload.
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
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.json")


def kernel_source_hash(kernel: str) -> str:
    """Hash of the HIP source that defines a kernel (traffic figures are only
    reported while the kernel is unchanged since its counters were taken)."""
    import hashlib
    src = {"full_decode_split": "decode.hip", "sparse_decode": "decode.hip", "full_prefill_fwd": "prefill.hip",
           "full_prefill_scores": "prefill.hip", "sparse_prefill": "prefill.hip", "topk": "topk.hip"}.get(kernel)
    if src is None:
        return ""
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_hybrid_amd", "csrc")
    h = hashlib.sha256()
    for f in (src, "hys_common.h", "attn_tile.h"):
        h.update(open(os.path.join(root, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, or None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


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
    """Time the oracle on (b, g) units of the block until the budget is spent,
    then scale to the whole block."""
    from threadpoolctl import threadpool_info
    from oracle import hysparse_oracle as orc
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    units = [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    NB = wl.n_blocks
    done = 0
    t0 = time.perf_counter()
    for (b, g) in units:
        for n in range(NB):
            _, _, s = orc.full_layer_block(inp.q_full, inp.k, inp.v, b, g, n, wl.score_block)
            c = orc.candidate_count(n, wl.q_len, wl.kv_len, wl.score_block)
            idx = orc.topk_row(s.astype(np.float32), c, wl.k_top)
            for l in range(wl.n_sparse):
                orc.sparse_layer_block(inp.q_sparse[l], inp.k, inp.v, idx, b, g, n, wl.score_block, wl.window,
                                       inp.gate_logits[l])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    step_s = el * len(units) / done
    return {"value": wl.batch * wl.q_len / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(units)} (batch, KV-group) units of one block (full layer, top-K, "
                      f"{wl.n_sparse} sparse layers) in {el:.1f} s, scaled to the whole block"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU; multi-GPU runs are not part of it (use --gpus 1)",
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
    value = tokens_per_step / (ms * 1e-3)
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step (wall {1e3 * wall / args.steps:.4f})", file=sys.stderr,
          flush=True)

    # decode: the sparse layers' share of the untraced step, from the same block
    # without sparse layers (full layer + top-K), timed the same way
    sparse_b2b_us = None
    if Tq == 1 and not loop and not hier and qs:
        def step0():
            hy.hysparse_hybrid_block(qf, k, v, [], gates, wl.k_top, wl.score_block, wl.window, out_full=out_full,
                                     lse=lse, scores=scores, idx=idx, workspace=ws)

        for _ in range(args.warmup):
            step0()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step0()
        e1.record()
        torch.cuda.synchronize()
        ms0 = e0.elapsed_time(e1) / args.steps
        sparse_b2b_us = 1e3 * (ms - ms0) / len(qs)

    # per-kernel durations: second pass with the library's event trace
    trace = hy.KernelTrace(capacity_kernels=64 * (args.steps + 1))
    trace.begin()
    for _ in range(args.steps):
        step()
    rows = trace.end()
    torch.cuda.synchronize()
    per = {}
    for name, t in rows:
        per.setdefault(name, []).append(t)
    kernels = {n: {"launches_per_step": len(t) / args.steps, "avg_us": 1e3 * float(np.mean(t)),
                   "us_per_step": 1e3 * float(np.sum(t)) / args.steps} for n, t in per.items()}
    traced_ms = float(sum(np.sum(t) for t in per.values())) / args.steps

    idx_np = idx.cpu().numpy()
    result = {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
              "config": {"workload": wl.name, "batch": B, "q_len": Tq, "context": Tkv, "q_heads": Hq,
                         "kv_heads": Hkv, "head_dim": D, "k_top": wl.k_top, "window": wl.window,
                         "n_sparse": len(qs), "score_block": wl.score_block,
                         "step": "hybrid block: full layer + top-K + all sparse layers"}}

    def roof(name, alg_bytes):
        if name not in kernels:
            return None
        us = kernels[name]["avg_us"]
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
        rs = roof("sparse_decode", sb)
        result["roofline"] = rf if dom == "full_decode_split" else (rs if dom == "sparse_decode" else rf)
        result["roofline_full"] = rf
        result["roofline_sparse"] = rs
        if rs:
            traced_us = rs["avg_us"] + kernels.get("sparse_merge", {"avg_us": 0.0})["avg_us"]
            # per layer: the untraced share of the step when it was measured
            # (back to back, launch gaps included), else the two traced kernels
            layer_us = sparse_b2b_us if sparse_b2b_us else traced_us
            result["sparse_layer"] = {"tokens_per_s": tokens_per_step / (layer_us * 1e-6), "us_per_layer": layer_us,
                                      "method": "step minus the block without sparse layers, per layer"
                                      if sparse_b2b_us else "traced split + merge kernels",
                                      "us_per_layer_traced": traced_us,
                                      "GB_per_s": sb / (layer_us * 1e-6) / 1e9,
                                      "frac_hbm": sb / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "alg_bytes": sb,
                                      "split_kernel_us": rs["avg_us"]}
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
    if args.cpu_baseline and not hier and inp is not None:
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
