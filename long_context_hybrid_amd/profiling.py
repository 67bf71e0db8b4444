"""Summaries of rocprofv3 CSV output for the kernels of libhysparse.

``python -m long_context_hybrid_amd.profiling stats DIR`` prints a markdown
table of per-kernel durations from ``--kernel-trace --stats -f csv`` output.

``python -m long_context_hybrid_amd.profiling counters DIR...`` prints SQ
counter ratios (MFMA busy, co-issue, wave-time split, LDS bank conflicts) per
kernel from ``--pmc`` runs of the counters named in the table's header.

``python -m long_context_hybrid_amd.profiling traffic --workload W --fetch DIR
--write DIR --copy-fetch DIR --copy-write DIR`` turns two ``--pmc FETCH_SIZE``
/ ``--pmc WRITE_SIZE`` runs of ``bench.py`` into HBM bytes per launch for each
library kernel, scaled by what the same counters report for a plain device
copy of known size (``bench.py --copy-calibration``), and merges the result
into ``profiles/hbm_traffic.json`` (read by ``bench.py``).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics

KERNELS = {  # symbol fragment -> name used by the library's trace hook
    "decode_split_kernel<hys::BF16, 128, true>": "full_decode_split",
    "decode_full_finish_kernel": "full_decode_finish",
    "decode_split_kernel<hys::BF16, 128, false>": "sparse_decode",
    "sparse_merge_kernel": "sparse_merge",
    "topk_row_kernel": "topk",
    "topk_part_kernel": "topk_part",
    "topk_select_kernel": "topk_select",
    "prefill_fwd_kernel": "full_prefill_fwd",
    "prefill_scores_kernel": "full_prefill_scores",
    "prefill_block_scores_kernel": "full_prefill_scores",
    "sparse_block_kernel": "sparse_prefill",
    "pool_keys_kernel": "hier_pool_keys",
    "block_logits_kernel": "hier_block_logits",
    "block_softmax_kernel": "hier_block_softmax",
    "gather_candidates_kernel": "hier_gather",
    "map_positions_kernel": "hier_map",
    "ceiling_stream_kernel": "ceiling_stream",
    "ceiling_gather_kernel": "ceiling_gather",
}

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {"full_decode_split": "decode.hip", "full_decode_finish": "decode.hip", "sparse_decode": "decode.hip",
                  "sparse_merge": "decode.hip", "full_prefill_fwd": "prefill.hip",
                  "full_prefill_scores": "prefill.hip", "sparse_prefill": "prefill.hip", "topk": "topk.hip",
                  "topk_part": "topk.hip", "topk_select": "topk.hip"}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the HIP sources that define a kernel: traffic figures are only
    reported while the kernel is unchanged since its counters were taken."""
    import hashlib
    src = KERNEL_SOURCES.get(kernel)
    if src is None:
        return ""
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in (src, "hys_common.h", "attn_tile.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of a kernel from the committed counter runs, or
    None (no record, or the kernel's source changed since)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def short_name(symbol: str) -> str:
    for frag, name in KERNELS.items():
        if frag in symbol:
            return name
    return symbol.split("(")[0][-60:]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def stats_table(d: str) -> str:
    path = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def counter_per_kernel(d: str, counter: str) -> dict:
    """Median counter value (KiB) per kernel name over its dispatches."""
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def counters_table(dirs, xcds: int = 8, simds: int = 1024) -> str:
    """Markdown table of SQ counter ratios per library kernel (medians over
    dispatches) from one or more ``--pmc`` runs.  GRBM_GUI_ACTIVE is the sum
    over the XCDs (``xcds``); ``simds`` is the chip's SIMD count.  Wave-cycle
    counters are in units of four cycles, as the hardware reports them."""
    vals = {}
    for d in dirs:
        path = _one(os.path.join(d, "**", "*counter_collection.csv"))
        for r in csv.DictReader(open(path)):
            name = short_name(r["Kernel_Name"])
            if name not in KERNELS.values():
                continue
            per = vals.setdefault(name, {})
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            per.setdefault("_ns", []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    med = {k: {c: statistics.median(v) for c, v in per.items()} for k, per in vals.items()}
    out = ["| kernel | clock GHz | MFMA busy % | VALU issued beside MFMA % | wave time issuing / waiting to "
           "issue / waiting on counters % | LDS bank-conflict % | VALU per MFMA | LDS per MFMA |",
           "|---|---|---|---|---|---|---|---|"]
    for k in sorted(med):
        m = med[k]
        need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAVE_CYCLES",
                "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_LDS_BANK_CONFLICT",
                "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS")
        if any(c not in m for c in need):
            continue
        cyc = m["GRBM_GUI_ACTIVE"] / xcds
        wave = m["SQ_WAVE_CYCLES"]
        out.append(
            f"| {k} | {cyc / m['_ns']:.2f} | {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * simds):.1f} | "
            f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / (cyc * simds):.1f} | "
            f"{100 * m['SQ_ACTIVE_INST_ANY'] / wave:.0f} / {100 * m['SQ_WAIT_INST_ANY'] / wave:.0f} / "
            f"{100 * m['SQ_WAIT_ANY'] / wave:.0f} | "
            f"{100 * m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'], 1.0):.1f} | "
            + (f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} | {m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f} |"
               if m["SQ_INSTS_MFMA"] > 0 else "— | — |"))
    return "\n".join(out)


def copy_factor(d: str, counter: str, nbytes: int) -> float:
    v = counter_per_kernel(d, counter)
    copy = [x for k, x in v.items() if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise RuntimeError(f"no copy kernel in {d}")
    return nbytes / (max(copy) * 1024.0)


def traffic(args) -> dict:
    nbytes = args.copy_mib << 20
    ff = copy_factor(args.copy_fetch, "FETCH_SIZE", nbytes)
    wf = copy_factor(args.copy_write, "WRITE_SIZE", nbytes)
    fe = counter_per_kernel(args.fetch, "FETCH_SIZE")
    wr = counter_per_kernel(args.write, "WRITE_SIZE")
    out = {}
    for name in sorted(set(fe) & set(wr)):
        if name not in KERNELS.values():
            continue
        rb, wb = fe[name] * 1024.0 * ff, wr[name] * 1024.0 * wf
        out[name] = {"bytes_per_launch": rb + wb, "read_bytes": rb, "write_bytes": wb,
                     "fetch_kib_raw": fe[name], "write_kib_raw": wr[name], "fetch_scale": ff, "write_scale": wf,
                     "source_hash": kernel_source_hash(name)}
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--out", default=TRAFFIC_FILE)
    args = ap.parse_args()
    if args.cmd == "stats":
        print(stats_table(args.dir))
        return
    if args.cmd == "counters":
        print(counters_table(args.dirs))
        return
    res = traffic(args)
    try:
        allr = json.load(open(args.out))
    except (OSError, ValueError):
        allr = {}
    allr[args.workload] = res
    json.dump(allr, open(args.out, "w"), indent=1, sort_keys=True)
    for k, v in res.items():
        print(f"{args.workload} {k}: {v['bytes_per_launch'] / 1e6:.2f} MB per launch "
              f"(read {v['read_bytes'] / 1e6:.2f}, write {v['write_bytes'] / 1e6:.2f})")


if __name__ == "__main__":
    main()
