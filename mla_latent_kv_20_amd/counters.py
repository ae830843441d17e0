"""Summaries of rocprofv3 counter runs: one markdown row per kernel, from the CSV files that
`rocprofv3 --pmc ... --output-format csv` writes.

    python -m mla_latent_kv_20_amd.counters DIR [DIR ...] [--kernels REGEX]
    python -m mla_latent_kv_20_amd.counters --stats KERNEL_STATS_CSV [--kernels REGEX]

Each DIR holds one pass (*_counter_collection.csv and *_agent_info.csv).  Counters of the same
kernel are averaged over its dispatches (the first dispatch of each kernel is dropped as a
warm-up when there are more), then merged across passes.  Derived columns, where their
counters were collected:
  - cycles: SQ_BUSY_CYCLES per shader engine (the engines run the same kernel in parallel);
  - clock: those cycles over the dispatch's duration;
  - MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES over (SIMDs x cycles);
  - MFMA FLOP: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;
  - LDS active: SQ_LDS_IDX_ACTIVE over (CUs x cycles); LDS bank-conflict cycles per CU;
  - HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB) as read, before any calibration factor.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import re


def _load(dirpath):
    cc = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    ai = glob.glob(os.path.join(dirpath, "**", "*agent_info.csv"), recursive=True)
    if not cc:
        raise FileNotFoundError(f"no counter_collection.csv under {dirpath}")
    agent = {}
    if ai:
        for row in csv.DictReader(open(ai[0])):
            if row.get("Agent_Type") == "GPU" or row.get("Name", "").startswith("gfx"):
                agent = row
                break
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    meta = {}
    for row in csv.DictReader(open(cc[0])):
        d = int(row["Dispatch_Id"])
        per[d][row["Counter_Name"]] += float(row["Counter_Value"])
        meta[d] = (row["Kernel_Name"], int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    return per, meta, agent


def short_name(name: str) -> str:
    """A kernel's readable name from a mangled or demangled symbol (template argument kept)."""
    m = re.search(r"([a-z][a-z_0-9]*_kernel)", name)
    if not m:
        return name[:60]
    base = m.group(1)
    tail = name[m.end():]
    if tail.startswith("IDF16_") or "<_Float16>" in tail:
        base += "<f16>"
    elif tail.startswith("IfE") or "<float>" in tail:
        base += "<f32>"
    return base


def summarize(dirs, kernels: str = ".*"):
    pat = re.compile(kernels)
    agg = collections.defaultdict(dict)          # kernel -> counter -> mean
    dur = collections.defaultdict(list)
    agent = {}
    for dpath in dirs:
        per, meta, ag = _load(dpath)
        agent = agent or ag
        by_kernel = collections.defaultdict(list)
        for d in sorted(per):
            name = meta[d][0]
            if pat.search(name):
                by_kernel[name].append(d)
        for name, ds in by_kernel.items():
            use = ds[1:] if len(ds) > 1 else ds
            for c in {k for d in use for k in per[d]}:
                agg[name][c] = sum(per[d].get(c, 0.0) for d in use) / len(use)
            dur[name].extend(meta[d][1] for d in use)
    n_se = float(agent.get("Num_Shader_Banks") or 32)
    n_simd = float(agent.get("Simd_Count") or 1024)
    n_cu = float(agent.get("Cu_Count") or 256)
    rows = []
    for name, c in agg.items():
        ns = sorted(dur[name])[len(dur[name]) // 2] if dur[name] else 0
        r = {"kernel": short_name(name), "duration_us": ns / 1e3}
        if "SQ_BUSY_CYCLES" in c:
            cyc = c["SQ_BUSY_CYCLES"] / n_se
            r["cycles"] = cyc
            if ns:
                r["clock_GHz"] = cyc / ns
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                r["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * cyc)
            if "SQ_LDS_IDX_ACTIVE" in c:
                r["lds_active"] = c["SQ_LDS_IDX_ACTIVE"] / (n_cu * cyc)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            r["mfma_flop"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        if "SQ_LDS_BANK_CONFLICT" in c:
            r["lds_bank_conflict_cycles_per_cu"] = c["SQ_LDS_BANK_CONFLICT"] / n_cu
        for k in ("FETCH_SIZE", "WRITE_SIZE"):
            if k in c:
                r[k + "_KiB"] = c[k]
        r["counters"] = c
        rows.append(r)
    return rows


def markdown(rows):
    cols = [("kernel", "{}"), ("duration_us", "{:.2f}"), ("cycles", "{:.0f}"), ("clock_GHz", "{:.2f}"),
            ("mfma_busy", "{:.3f}"), ("mfma_flop", "{:.4g}"), ("lds_active", "{:.3f}"),
            ("lds_bank_conflict_cycles_per_cu", "{:.0f}"), ("FETCH_SIZE_KiB", "{:.0f}"), ("WRITE_SIZE_KiB", "{:.0f}")]
    used = [(k, f) for k, f in cols if any(k in r for r in rows)]
    out = ["| " + " | ".join(k for k, _ in used) + " |", "|" + "---|" * len(used)]
    for r in sorted(rows, key=lambda r: -r.get("duration_us", 0)):
        out.append("| " + " | ".join(f.format(r[k]) if k in r else "" for k, f in used) + " |")
    return "\n".join(out)


def stats_table(path: str, kernels: str = ".*") -> str:
    """The kernel-trace statistics (`rocprofv3 --kernel-trace --stats`) as a markdown table."""
    pat = re.compile(kernels)
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for row in csv.DictReader(open(path)):
        if not pat.search(row["Name"]):
            continue
        out.append(f"| {short_name(row['Name'])} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | "
                   f"{float(row['MinNs']) / 1e3:.2f} | {float(row['MaxNs']) / 1e3:.2f} | {float(row['Percentage']):.1f}% |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dirs", nargs="*")
    ap.add_argument("--stats", help="a *_kernel_stats.csv of a kernel-trace run")
    ap.add_argument("--kernels", default=".*")
    ap.add_argument("--raw", action="store_true", help="also print every averaged counter")
    a = ap.parse_args()
    if a.stats:
        print(stats_table(a.stats, a.kernels))
        return
    rows = summarize(a.dirs, a.kernels)
    print(markdown(rows))
    if a.raw:
        for r in rows:
            print(f"\n{r['kernel']}:")
            for k, v in sorted(r["counters"].items()):
                print(f"  {k} = {v:.6g}")


if __name__ == "__main__":
    main()
