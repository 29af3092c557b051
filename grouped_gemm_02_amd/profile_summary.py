"""Summaries of rocprofv3 output for the layer's kernels.

    python -m grouped_gemm_02_amd.profile_summary stats <kernel_stats.csv> <out.txt> --cmd "<command>"
    python -m grouped_gemm_02_amd.profile_summary traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <out.json> --cmd "<command>"
    python -m grouped_gemm_02_amd.profile_summary mfma <counter_collection.csv> <out.txt> --cmd "<command>" \
        --title "<workload>"
    python -m grouped_gemm_02_amd.profile_summary lds <counter_collection.csv> <out.txt> --cmd "<command>" \
        --title "<workload>" [--config qwen3_30b]

`stats` turns the --kernel-trace --stats table into a short text table.
`traffic` turns two --pmc runs (FETCH_SIZE, then WRITE_SIZE, both in KiB per
dispatch) into HBM bytes per launch of each layer kernel. Both counters are
calibrated against the largest device-to-device copy in the same run, whose
size is known (it reads and writes `--copy-bytes` bytes): factor =
known bytes / counter reading. The JSON records the sha256 of the GEMM
sources it was measured with, so a reader can tell when it has gone stale.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/gemm.hip", "csrc/device_common.h", "csrc/combine.hip", "csrc/permute.hip",
                  "csrc/quant.hip")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = name.split("(")[0]
    if n.startswith("void "):
        n = n[5:]
    return n.replace("moe::", "")


def stats(csv_path: str, out_path: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"# command: {cmd}", "#",
             f"{'kernel':34s} {'calls':>6s} {'avg_us':>10s} {'total_us':>12s} {'pct':>6s}"]
    for r in rows:
        name = r.get("Name") or r.get("KERNEL_NAME") or ""
        if "moe::" not in name:
            continue
        calls = int(float(r.get("Calls", r.get("TotalCalls", 0))))
        tot = float(r.get("TotalDurationNs", 0)) / 1e3
        avg = float(r.get("AverageNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        lines.append(f"{short_name(name):34s} {calls:6d} {avg:10.1f} {tot:12.1f} {pct:6.2f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(csv_path: str, counter: str):
    vals = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        vals[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return vals, names


def traffic(fetch_csv: str, write_csv: str, out_path: str, cmd: str, copy_bytes: int, workload: str) -> None:
    res = {"command": cmd, "workload": workload, "source_sha256": source_hash(), "copy_bytes": copy_bytes,
           "kernels": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals, names = _per_dispatch(path, counter)
        copies = [d for d, n in names.items() if "copy" in n.lower() and "moe::" not in n]
        if not copies:
            raise SystemExit(f"no copy kernel found in {path}")
        cal = max(copies, key=lambda d: vals[d])
        factor = copy_bytes / (vals[cal] * 1024.0)
        res[f"{counter.lower()}_calibration"] = {"copy_kib": vals[cal], "factor": factor}
        agg = collections.defaultdict(list)
        for d, v in vals.items():
            if "moe::" in names[d]:
                agg[short_name(names[d])].append(v * 1024.0 * factor)
        for k, vs in agg.items():
            ent = res["kernels"].setdefault(k, {})
            ent[f"{counter.lower()}_bytes"] = sum(vs) / len(vs)
            ent["dispatches"] = len(vs)
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)


def mfma(csv_path: str, out_path: str, cmd: str, title: str, simds: int = 1024, xcds: int = 8) -> None:
    """MFMA utilisation per layer kernel from one --pmc pass of
    SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) and GRBM_GUI_ACTIVE
    (summed over the XCDs): busy = mfma / (gui_active / xcds * simds)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(csv_path)):
        d = r["Dispatch_Id"]
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    agg = collections.defaultdict(list)
    for d, v in vals.items():
        if "moe::" in names[d] and v.get("GRBM_GUI_ACTIVE", 0) > 0:
            agg[short_name(names[d])].append((v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v["GRBM_GUI_ACTIVE"]))
    lines = [f"# rocprofv3 MFMA-busy counters, {title} (one pass)", f"# command: {cmd}",
             "# values: average per dispatch. GRBM_GUI_ACTIVE is summed over the "
             f"{xcds} XCDs (the kernel's cycles are gui_active / {xcds});",
             f"# SQ_VALU_MFMA_BUSY_CYCLES is summed over all {simds} SIMDs; busy = mfma_busy / "
             f"(gui_active / {xcds} * {simds}).", "#",
             f"{'kernel':36s} {'mfma_busy_cycles':>17s} {'gui_active':>11s} {'busy':>6s}"]
    for k in sorted(agg):
        mb = sum(a for a, _ in agg[k]) / len(agg[k])
        ga = sum(b for _, b in agg[k]) / len(agg[k])
        if mb <= 0:
            continue
        lines.append(f"{k:36s} {mb:17.0f} {ga:11.0f} {mb / (ga / xcds * simds):6.3f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _tiles_per_launch(config: str) -> dict:
    """Output tiles of each GEMM launch for the seeded routing of `config`
    (256 x 256 tiles; the row-tile GEMMs have sum_e ceil(rows_e / 256) m-tiles)."""
    import torch
    from grouped_gemm_02_amd import inputs
    cfg = inputs.CONFIGS[config]
    d = inputs.make_layer_inputs(cfg, "cpu", with_dy=False)
    counts = torch.bincount(d["topk_idx"].flatten(), minlength=cfg.E)
    mt = int(((counts + 255) // 256).sum())
    n_i = (cfg.I + 255) // 256
    return {"gemm1_swiglu": mt * (2 * cfg.I // 256), "gemm2": mt * (cfg.H // 256), "gemm_dh": mt * n_i,
            "gemm_dx": mt * (cfg.H // 256), "gemm_dw13": cfg.E * (2 * cfg.I // 256) * (cfg.H // 256),
            "gemm_dw2": cfg.E * (cfg.H // 256) * n_i}


def lds(csv_path: str, out_path: str, cmd: str, title: str, config: str) -> None:
    """SQ_LDS_BANK_CONFLICT and SQ_ACTIVE_INST_LDS per dispatch of each GEMM,
    and the conflict cycles per output tile."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(csv_path)):
        d = r["Dispatch_Id"]
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    agg = collections.defaultdict(list)
    for d, v in vals.items():
        if "moe::gemm" in names[d]:
            agg[short_name(names[d])].append((v.get("SQ_LDS_BANK_CONFLICT", 0.0), v.get("SQ_ACTIVE_INST_LDS", 0.0)))
    tiles = _tiles_per_launch(config)
    lines = [f"# rocprofv3 LDS counters, {title} (one pass, two SQ counters)", f"# command: {cmd}",
             "# values: average per dispatch, summed over the chip; tiles per launch from the seeded routing",
             "#", f"{'kernel':36s} {'bank_conflict_cycles':>21s} {'active_lds_inst_cycles':>23s} {'tiles':>6s} "
             f"{'conflict_cycles_per_tile':>25s}"]
    for k in sorted(agg):
        bc = sum(a for a, _ in agg[k]) / len(agg[k])
        ai = sum(b for _, b in agg[k]) / len(agg[k])
        n = next((v for key, v in tiles.items() if k.startswith(key)), 0)
        per = f"{bc / n:25.0f}" if n else f"{'-':>25s}"
        lines.append(f"{k:36s} {bc:21.0f} {ai:23.0f} {n:6d} {per}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--workload", default="qwen3_30b/bf16", help="<config>/<precision> the counters were taken on")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("out")
    m.add_argument("--cmd", required=True)
    m.add_argument("--title", required=True)
    ls = sub.add_parser("lds")
    ls.add_argument("csv")
    ls.add_argument("out")
    ls.add_argument("--cmd", required=True)
    ls.add_argument("--title", required=True)
    ls.add_argument("--config", default="qwen3_30b")
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.csv, a.out, a.cmd)
    elif a.what == "lds":
        lds(a.csv, a.out, a.cmd, a.title, a.config)
    elif a.what == "mfma":
        mfma(a.csv, a.out, a.cmd, a.title)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out, a.cmd, a.copy_bytes, a.workload)


if __name__ == "__main__":
    main()
