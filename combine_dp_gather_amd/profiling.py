"""Text summaries of rocprofv3 runs, and the HBM-traffic figure bench.py reports.

    # per-kernel durations of a --kernel-trace --stats run
    python -m combine_dp_gather_amd.profiling stats DIR/stats_kernel_stats.csv --cmd "..."

    # matrix-core busy fraction, engine clock and counted flops per kernel of a --pmc run
    python -m combine_dp_gather_amd.profiling mfma --counters DIR/run_counter_collection.csv \
        --agent DIR/run_agent_info.csv

    # HBM bytes per launch of one kernel from a FETCH_SIZE run and a WRITE_SIZE run, each
    # scaled by what the same counter reads for a plain device copy of known size made in the
    # same process (bench.py --copy-calibration MIB)
    python -m combine_dp_gather_amd.profiling traffic --fetch F.csv --write W.csv \
        --copy-mib 1024 --kernel grouped_gemm_pp_kernel<true, false> --sources a.hip b.h --cmd "..."

The traffic summary records a SHA-256 over the kernel's source files; bench.py reports the
figure only while the sources still hash to it (counters taken on an older kernel say
nothing about the current one).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
from typing import Dict, List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# the device copy torch launches for a uint8 tensor copy_
COPY_KERNEL_PATTERN = r"direct_copy_kernel|copyBuffer"


def short_name(name: str) -> str:
    n = name.replace("void ", "").replace("moe::(anonymous namespace)::", "")
    n = n.replace("at::native::", "").replace("HIP_vector_type<unsigned int, 4u>", "uint4")
    depth, out = 0, []
    for ch in n:  # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)[:90]


def sources_sha256(paths: Sequence[str]) -> str:
    h = hashlib.sha256()
    for p in paths:
        full = p if os.path.isabs(p) else os.path.join(ROOT, p)
        h.update(os.path.relpath(full, ROOT).encode())
        with open(full, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_stats(path: str) -> List[dict]:
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                     "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                     "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_per_dispatch(path: str, counter: str) -> Dict[str, List[float]]:
    """Counter value of every dispatch, grouped by short kernel name."""
    by = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            by[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return by


def _copy_reading(by: Dict[str, List[float]]) -> float:
    vals = [v for name, vs in by.items() if re.search(COPY_KERNEL_PATTERN, name) for v in vs]
    if not vals:
        raise SystemExit("no copy kernel in the counter run: pass --copy-calibration to bench.py")
    return max(vals)


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, kernel: str) -> dict:
    copy_kib = copy_mib * 1024.0
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        by = counter_per_dispatch(path, counter)
        factor = copy_kib / _copy_reading(by)
        hits = [v for name, vs in by.items() if name.startswith(kernel) for v in vs]
        if not hits:
            raise SystemExit(f"kernel {kernel!r} not in {path}")
        mean_kib = sum(hits) / len(hits)
        res[counter] = {"factor": factor, "raw_kib": mean_kib, "dispatches": len(hits),
                        "bytes": mean_kib * 1024.0 * factor}
    res["bytes_per_launch"] = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    return res


def agent_geometry(agent_csv: str) -> dict:
    """SIMD count, XCD count and the maximum engine clock (MHz) of the GPU agent."""
    for r in csv.DictReader(open(agent_csv)):
        if r.get("Agent_Type") == "GPU":
            return {"simds": int(r["Simd_Count"]), "xcds": int(r["Num_Xcc"]),
                    "max_mhz": float(r["Max_Engine_Clk_Fcompute"])}
    raise SystemExit(f"no GPU agent in {agent_csv}")


def mfma_util(counter_csv: str, agent_csv: str) -> List[dict]:
    """Per kernel, averaged over its dispatches: duration, the engine clock it ran at
    (GRBM_GUI_ACTIVE is summed over the XCDs, so cycles per XCD over the duration), the
    fraction of SIMD cycles with a busy matrix core (SQ_VALU_MFMA_BUSY_CYCLES over SIMDs x
    cycles per XCD) and the matrix-core flops the hardware counted (MOPS x 512)."""
    geo = agent_geometry(agent_csv)
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    spans = collections.defaultdict(dict)
    for r in csv.DictReader(open(counter_csv)):
        name = short_name(r["Kernel_Name"])
        vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        spans[name][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = []
    for name, c in vals.items():
        if not c.get("SQ_VALU_MFMA_BUSY_CYCLES") or not c.get("GRBM_GUI_ACTIVE"):
            continue
        mean = {k: sum(v) / len(v) for k, v in c.items()}
        if mean["SQ_VALU_MFMA_BUSY_CYCLES"] <= 0:
            continue
        dur_ns = sum(spans[name].values()) / len(spans[name])
        cycles = mean["GRBM_GUI_ACTIVE"] / geo["xcds"]
        flops = 512.0 * sum(mean.get(k, 0.0) for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                                                       "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_F64",
                                                       "SQ_INSTS_VALU_MFMA_MOPS_FP8"))
        out.append({"name": name, "dispatches": len(spans[name]), "avg_us": dur_ns / 1e3,
                    "clock_mhz": cycles / dur_ns * 1e3,
                    "mfma_busy": mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * geo["simds"]),
                    "counted_flops": flops})
    return sorted(out, key=lambda r: -r["avg_us"])


def read_traffic_summary(path: str, source_paths: Sequence[str]) -> Optional[float]:
    """bytes per launch from a committed summary, or None if absent or the sources changed."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^([a-z_0-9]+):\s*(\S+)", line.strip())
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("source_sha256") != sources_sha256(source_paths):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--sources", nargs="+", required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    t.add_argument("--cmd", nargs="*", default=[])
    u = sub.add_parser("mfma")
    u.add_argument("--counters", required=True, help="counter_collection.csv of a --pmc run")
    u.add_argument("--agent", required=True, help="agent_info.csv of the same run")
    a = ap.parse_args()
    if a.what == "mfma":
        geo = agent_geometry(a.agent)
        print(f"GPU: {geo['simds']} SIMDs, {geo['xcds']} XCDs, max engine clock {geo['max_mhz']:.0f} MHz")
        print(f"{'kernel':50s} {'calls':>5s} {'avg_us':>9s} {'clock_MHz':>9s} {'mfma_busy':>9s} {'counted_flop':>13s}")
        for r in mfma_util(a.counters, a.agent):
            print(f"{r['name'][:50]:50s} {r['dispatches']:5d} {r['avg_us']:9.1f} {r['clock_mhz']:9.0f} "
                  f"{r['mfma_busy']:9.3f} {r['counted_flops']:13.4e}")
        return
    if a.what == "stats":
        if a.cmd:
            print(f"command: {a.cmd}\n")
        print(f"{'kernel':90s} {'calls':>5s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
        for r in kernel_stats(a.csv):
            print(f"{r['name']:90s} {r['calls']:5d} {r['avg_us']:10.1f} {r['min_us']:10.1f} "
                  f"{r['max_us']:10.1f} {r['pct']:6.2f}")
        return
    res = traffic(a.fetch, a.write, a.copy_mib, a.kernel)
    for c in a.cmd:
        print(f"command: {c}")
    print(f"kernel: {a.kernel}")
    print(f"sources: {' '.join(a.sources)}")
    print(f"source_sha256: {sources_sha256(a.sources)}")
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[counter]
        print(f"{counter.lower()}_kib_per_dispatch_raw: {r['raw_kib']:.1f}  (dispatches {r['dispatches']})")
        print(f"{counter.lower()}_scale_factor: {r['factor']:.4f}  (copy of {a.copy_mib} MiB)")
        print(f"{counter.lower()}_bytes_per_launch: {r['bytes']:.0f}")
    print(f"traffic_bytes_per_launch: {res['bytes_per_launch']:.0f}")
    if a.algorithmic_bytes:
        print(f"algorithmic_bytes_per_launch: {a.algorithmic_bytes:.0f}")
        print(f"traffic_over_algorithmic: {res['bytes_per_launch'] / a.algorithmic_bytes:.3f}")


if __name__ == "__main__":
    main()
