"""Markdown summaries of rocprofv3 runs over bench.py.

Two readers:

* ``trace``: a ``--kernel-trace`` CSV of one bench.py run.  bench.py runs W
  warm-up steps, then K cold steps (each after a 512 MB read, the "flush",
  outside its events), then K warm steps back to back.  The dispatches are
  split into those phases by where the flush kernels fall, so the cold
  average printed here is the one bench.py's HIP events time.
* ``counters``: a ``--pmc`` CSV (MFMA busy cycles, GPU active cycles, MFMA
  op counts) of one run, with the agent CSV for the SIMD count.  MFMA
  utilisation is rocprofv3's own derived MfmaUtil: the MFMA busy cycles summed
  over the SIMDs over (the GPU active cycles of the busiest XCD times the
  number of SIMDs).  The clock is that XCD's active cycles over the
  dispatch's duration; the counter window is a little longer than the
  dispatch, which matters for short kernels, so the table also gives the busy
  cycles per SIMD over the duration at the 2.4 GHz peak clock (a lower bound).

    python -m paged_mla_decode_04_amd.rocprof_summary trace T_kernel_trace.csv
    python -m paged_mla_decode_04_amd.rocprof_summary counters C_counter_collection.csv C_agent_info.csv
"""

from __future__ import annotations

import argparse
import csv
from collections import defaultdict

FLUSH = "reduce_kernel"  # the flush is a torch sum over a 512 MB buffer
DECODE = ("decode", "combine", "plan_kernel")
PEAK_CLOCK_GHZ = 2.4     # MI355X peak engine clock


def short_name(name: str) -> str:
    for cut in ("void ", "(anonymous namespace)::", "mla::"):
        name = name.replace(cut, "")
    return name.split("(", 1)[0]


def trace_phases(path: str) -> dict:
    """kernel -> {"all": [us], "warmup": [us], "cold": [us], "warm": [us]}."""
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    out: dict = defaultdict(lambda: defaultdict(list))
    seen_flush = False
    flushed = False       # a flush since the last step started
    phase = "warmup"
    prev = ""             # the previous kernel of a step
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if FLUSH in name:
            seen_flush = True
            flushed = True
            continue
        if not any(k in name for k in DECODE):
            continue
        # a step starts with its plan kernel, or with its decode kernel when
        # the decode plans for itself (no plan kernel right before it)
        starts = "plan_kernel" in name or ("combine" not in name and "plan_kernel" not in prev)
        if starts:
            if flushed:
                phase = "cold"
            elif seen_flush:
                phase = "warm"
            flushed = False
        prev = name
        k = short_name(name)
        out[k]["all"].append(dur)
        out[k][phase].append(dur)
    return out


def _avg(v):
    return sum(v) / len(v) if v else float("nan")


def trace_table(path: str) -> str:
    ph = trace_phases(path)
    lines = ["| kernel | calls | cold avg (us) | cold min | cold max | warm avg (us) | all calls avg (us) |",
             "|---|---|---|---|---|---|---|"]
    order = sorted(ph, key=lambda k: -_avg(ph[k]["all"]))
    for k in order:
        d = ph[k]
        c = d["cold"]
        lines.append(f"| `{k}` | {len(d['all'])} | {_avg(c):.1f} | {min(c) if c else float('nan'):.1f} | "
                     f"{max(c) if c else float('nan'):.1f} | {_avg(d['warm']):.1f} | {_avg(d['all']):.1f} |")
    cold_call = sum(_avg(ph[k]["cold"]) for k in ph)
    warm_call = sum(_avg(ph[k]["warm"]) for k in ph)
    lines.append("")
    lines.append(f"One step (the kernels above, summed averages): cold {cold_call:.1f} us, "
                 f"warm {warm_call:.1f} us.")
    return "\n".join(lines)


def counter_means(path: str) -> dict:
    """kernel -> {counter: mean per dispatch, "dur_us": mean duration}."""
    vals: dict = defaultdict(lambda: defaultdict(list))
    durs: dict = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        durs[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for k, cs in vals.items():
        out[k] = {c: _avg(v) for c, v in cs.items()}
        out[k]["dur_us"] = _avg(list(durs[k].values()))
        out[k]["dispatches"] = len(durs[k])
    return out


def agent_simds(path: str) -> tuple[int, int]:
    for r in csv.DictReader(open(path)):
        if r["Agent_Type"] == "GPU":
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    raise ValueError("no GPU agent")


def counters_table(path: str, agent_path: str) -> str:
    simds, xcc = agent_simds(agent_path)
    cm = counter_means(path)
    lines = [f"SIMDs: {simds}, XCDs: {xcc}.  GRBM_GUI_ACTIVE is read per XCD and summed; the table "
             f"divides by {xcc} for one XCD (they run the same time to within a few percent).", "",
             "| kernel | dispatches | duration (us) | MFMA busy (sum over SIMDs) | GUI active per XCD | clock (GHz) | "
             "MfmaUtil | busy / (duration x 2.4 GHz) | MFMA flops (MOPS_BF16 x 512) |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(cm, key=lambda k: -cm[k].get("SQ_VALU_MFMA_BUSY_CYCLES", 0)):
        d = cm[k]
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        if busy <= 0:
            continue
        gui = d.get("GRBM_GUI_ACTIVE", float("nan")) / xcc
        util = busy / (gui * simds)
        clock = gui / (d["dur_us"] * 1e3)
        flops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        at_peak = busy / simds / (d["dur_us"] * 1e3 * PEAK_CLOCK_GHZ)
        lines.append(f"| `{k}` | {d['dispatches']} | {d['dur_us']:.1f} | {busy:.4g} | {gui:.4g} | {clock:.2f} | "
                     f"{100 * util:.1f}% | {100 * at_peak:.1f}% | {flops:.4g} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("agent_csv")
    a = ap.parse_args()
    if a.cmd == "trace":
        print(trace_table(a.csv))
    else:
        print(counters_table(a.csv, a.agent_csv))


if __name__ == "__main__":
    main()
