"""HBM traffic per kernel from rocprofv3 counter passes.

Two counter passes over the same benchmark command, one with FETCH_SIZE and
one with WRITE_SIZE (KiB per dispatch), each also running a plain device copy
of a known size (bench.py --copy-bytes).  The copy calibrates the counters:
factor = bytes the copy must move / bytes the counter reports for it.  Each
MoE kernel's traffic is its counter value times that factor, averaged over its
dispatches.

    python -m fine_grained_mixture_top_amd.hbm_traffic FETCH.csv WRITE.csv COPY_BYTES OUT.json

(FETCH_SIZE and WRITE_SIZE count the L2's read and write traffic to the
memory side of the chip -- the memory-attached last-level cache (MALL) and
HBM alike; a MALL hit counts as traffic too.)  A second mode summarises any
other counter passes per kernel (see counters_main).

The result records a hash of the kernel sources; bench.py reports the traffic
only while the sources still hash the same.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def classify(name: str, wgt_seen: dict) -> str:
    """Bench kernel name of one dispatch (None for kernels that are not tracked)."""
    if "grouped_gemm4_kernel" in name:
        m = re.search(r"grouped_gemm4_kernel<(true|false), (true|false), (true|false), moe::(?:g\d::)?(\w+)", name)
        if not m:
            return None
        wgt, bmn, epi = m.group(1) == "true", m.group(2) == "true", m.group(4)
        if epi in ("EpiSwiGLU", "G4SwiGLU"):
            return "up"
        if epi in ("EpiDH", "G4DH"):
            return "dh"
        if wgt:  # dw1 and dw2 share an instantiation: first per step is dw1
            k = wgt_seen["n"] % 2
            wgt_seen["n"] += 1
            return "dw1" if k == 0 else "dw2"
        return "down" if bmn else "dxt"
    if "grouped_gemm5_kernel" in name:
        m = re.search(r"grouped_gemm5_kernel<(true|false), (true|false), moe::(?:\w+::)?(\w+)", name)
        if not m:
            return None
        bmn, epi = m.group(1) == "true", m.group(3)
        if epi in ("EpiSwiGLU", "G4SwiGLU", "SplitSwiGLU"):
            return "up"
        if epi in ("EpiDH", "G4DH", "G5DH"):
            return "dh"
        return "down" if bmn else "dxt"
    if "grouped_gemm_kernel" in name:
        m = re.search(r"grouped_gemm_kernel<([^,]+), (\d+), (\d+), (true|false), (\d), (true|false), moe::(\w+)<([^>]*)>", name)
        if not m:
            return None
        wgt, bl, epi, args = m.group(4) == "true", m.group(5), m.group(7), m.group(8)
        if epi == "EpiSwiGLU":
            return "up"
        if epi == "EpiDH":
            return "dh"
        to_float = args.split(",")[1].strip() == "float"
        if to_float:
            return "dwr" if wgt else "router_logits"
        if wgt:  # dw1 and dw2 share an instantiation: first per step is dw1
            k = wgt_seen["n"] % 2
            wgt_seen["n"] += 1
            return "dw1" if k == 0 else "dw2"
        return "down" if bl == "1" else "dxt"
    if "k_aggregate_o" in name:  # O (forward) and dX (backward) share the kernel: O comes first
        k = wgt_seen.get("agg", 0)
        wgt_seen["agg"] = k + 1
        return "agg_o" if k % 2 == 0 else "agg_dx"
    if "k_router_dz" in name:
        return "router_grad"
    if "copyBuffer" in name or "elementwise_kernel" in name and "copy" in name.lower():
        return "copy"
    return None


def per_kernel(path: str, counter: str):
    """{kernel: [KiB per dispatch]} from one counter-collection CSV."""
    rows = list(csv.DictReader(open(path)))
    by = collections.defaultdict(float)
    names = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        by[did] += float(r["Counter_Value"])  # summed over the reporting instances
        names[did] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    seen = {"n": 0}
    for did in sorted(by):
        k = classify(names[did], seen)
        if k:
            out[k].append(by[did])
    return out


def main(fetch_csv, write_csv, copy_bytes, out_json):
    copy_bytes = float(copy_bytes)
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    if not f.get("copy") or not w.get("copy"):
        raise SystemExit("no calibration copy dispatch found")
    # the calibration copy is the largest copy dispatch of the run
    f_copy = max(f["copy"]) * 1024.0
    w_copy = max(w["copy"]) * 1024.0
    kf, kw = copy_bytes / f_copy, copy_bytes / w_copy
    res = {"source_hash": source_hash(), "copy_bytes": copy_bytes, "fetch_factor": kf, "write_factor": kw,
           "kernels": {}}
    for k in sorted(set(f) | set(w)):
        if k == "copy":
            continue
        fb = sum(f.get(k, [0])) / max(1, len(f.get(k, []))) * 1024.0 * kf
        wb = sum(w.get(k, [0])) / max(1, len(w.get(k, []))) * 1024.0 * kw
        res["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb,
                             "dispatches": len(f.get(k, []))}
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


# ----------------------------------------------------------------------------
# other counters: per-kernel means and the ratios the GEMM analysis uses
#
#     python -m fine_grained_mixture_top_amd.hbm_traffic counters OUT.json A.csv [B.csv ...]
# ----------------------------------------------------------------------------

CUS, SIMDS, XCDS = 256, 1024, 8  # MI355X: compute units, SIMDs, accelerator complex dies


def counter_means(paths):
    """{kernel: {counter: mean over the kernel's dispatches}} from any number
    of counter-collection CSVs.  rocprofv3 reports one value per dispatch,
    summed over the counter's instances: GRBM_GUI_ACTIVE is the sum of the 8
    XCDs' busy clocks (it reads about 8 x the dispatch's duration times the
    clock), so it is divided by 8 to give one XCD's cycles.  A counter still
    reported by several instances is summed over them."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        vals = collections.defaultdict(list)
        names = {}
        for r in rows:
            did = int(r["Dispatch_Id"])
            vals[(did, r["Counter_Name"])].append(float(r["Counter_Value"]))
            names[did] = r["Kernel_Name"]
        seen = {"n": 0}
        kernel_of = {did: classify(names[did], seen) for did in sorted(names)}
        for (did, cname), v in vals.items():
            k = kernel_of[did]
            if k:
                acc[k][cname].append(sum(v) / XCDS if cname == "GRBM_GUI_ACTIVE" else sum(v))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def derived(m: dict) -> dict:
    """Ratios of one kernel's counter means (those whose counters are present)."""
    out = {}
    gui = m.get("GRBM_GUI_ACTIVE")
    if gui:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            out["mfma_busy_pct"] = 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS)
        if "TCP_PENDING_STALL_CYCLES_sum" in m:
            out["tcp_pending_stall_pct"] = 100.0 * m["TCP_PENDING_STALL_CYCLES_sum"] / (gui * CUS)
        if "SQ_LDS_BANK_CONFLICT" in m:
            out["lds_bank_conflict_pct"] = 100.0 * m["SQ_LDS_BANK_CONFLICT"] / (gui * CUS)
        out["gui_active_cycles"] = gui
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
        out["mfma_bf16_flop"] = 512.0 * m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    h, x = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
    if h is not None and x is not None and h + x > 0:
        out["l2_hit_pct"] = 100.0 * h / (h + x)
    rq = m.get("TCC_EA0_RDREQ_sum")
    if rq:
        for c, key in (("TCC_EA0_RDREQ_128B_sum", "rdreq_128b_pct"), ("TCC_EA0_RDREQ_64B_sum", "rdreq_64b_pct"),
                       ("TCC_EA0_RDREQ_32B_sum", "rdreq_32b_pct"), ("TCC_BUBBLE_sum", "bubble_pct"),
                       ("TCC_EA0_RDREQ_DRAM_sum", "rdreq_dram_pct")):
            if c in m:
                out[key] = 100.0 * m[c] / rq
    return out


def counters_main(out_json, *paths):
    means = counter_means(paths)
    res = {"source_hash": source_hash(), "kernels": {k: {"counters": v, "derived": derived(v)}
                                                     for k, v in sorted(means.items())}}
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps({k: v["derived"] for k, v in res["kernels"].items()}, indent=1))


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        counters_main(*sys.argv[2:])
    else:
        main(*sys.argv[1:5])
