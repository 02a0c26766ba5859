"""Benchmark of paged MLA decode on one MI355X.

One step = one pass of the whole hot path over one batch: the split-KV plan,
the decode and its lse merge, on synthetic inputs already resident in HBM.
The step is one mla_decode_with_kvcache call without metadata, which plans
for itself (inside the decode kernel at the 128-row, bf16-cache shapes; with
the plan kernel first otherwise); --separate-plan times an mla_get_metadata
call followed by the decode given its metadata instead.  The default workload is the
wide-head shape of the PAI FlashMLA tutorial's bandwidth plot (segmentfault,
"云上玩转DeepSeek系列之五", section 二.4): b=128, s_q=1, h_q=128, h_kv=1,
seqlens ~ N(4096, 1024) clipped to [1, 8192], 64-token pages, identity block
table, bf16 N(0,1) data.

Throughput uses the tutorial's formulas: bytes = (sum(seqlens) * 576 +
b * s_q * h_q * (576 + 512)) * 2 and FLOPs = s_q * sum(seqlens) * h_q *
(576 + 512) * 2, over milliseconds, in decimal GB/s and TFLOPS.

Prints one JSON line.  Runs on one GPU only.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_mla_decode_04_amd import traffic
from paged_mla_decode_04_amd import (_lib, default_num_parts, get_mla_metadata,  # noqa: E402
                                     mla_decode_with_kvcache, workspace_size)
from paged_mla_decode_04_amd import metrics  # noqa: E402
from paged_mla_decode_04_amd.workloads import D_V, FP8_KV_SCALE, WORKLOADS, draw  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, 2.5 PFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wide", choices=sorted(WORKLOADS))
    ap.add_argument("--num-parts", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle sample budget (whole sequences until this much work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    # layout and shape overrides of the chosen workload (ablations and sweeps)
    ap.add_argument("--pitch", type=int, choices=(576, 640), default=None,
                    help="cache entry pitch in elements (the pad is never read)")
    ap.add_argument("--table", choices=("arange", "randperm"), default=None,
                    help="identity or seeded-permutation block table")
    ap.add_argument("--seqlen-mean", type=int, default=None,
                    help="seqlens ~ N(mean, mean/4) clipped to [1, 2 mean] instead of the recipe")
    ap.add_argument("--s-q", type=int, default=None, help="query tokens per sequence")
    ap.add_argument("--h-q", type=int, default=None, help="query heads")
    ap.add_argument("--causal", choices=("yes", "no"), default=None)
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="cache element type: bf16, or E4M3 bytes times a per-cache scale "
                         "(the byte count then takes one byte per cached element)")
    ap.add_argument("--separate-plan", action="store_true",
                    help="plan with an mla_get_metadata call before each decode (the plan a "
                         "decode step computes once for all layers) instead of inside the call")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (plan + decode) in a HIP graph and time its replays "
                         "(removes the host's launch overhead, which small workloads feel)")
    ap.add_argument("--warm", action="store_true",
                    help="time the steps back to back with warm caches only (by default every "
                         "timed step is preceded by a 512 MB read of another buffer, outside the "
                         "step's events, so that no input stays in L2 or the 256 MB Infinity "
                         "Cache; warm steps are then timed as well and reported beside the cold "
                         "ones)")
    return ap.parse_args()


def chosen_workload(args):
    """The named workload with any layout or shape overrides applied (renamed if changed)."""
    w = WORKLOADS[args.workload]
    changes, tags = {}, []
    if args.pitch is not None and args.pitch != w.pitch:
        changes["pitch"] = args.pitch
        tags.append(f"pitch {args.pitch}")
    if args.table is not None and args.table != w.table:
        changes["table"] = args.table
        tags.append(f"{'identity' if args.table == 'arange' else 'permuted'} table")
    if args.seqlen_mean is not None:
        m = int(args.seqlen_mean)
        changes["seqlens"] = f"normal_{m}_{max(1, m // 4)}"
        tags.append(f"seqlens ~ N({m},{max(1, m // 4)}) clipped to [1,{2 * m}]")
    if args.s_q is not None and args.s_q != w.s_q:
        changes["s_q"] = args.s_q
        tags.append(f"s_q={args.s_q}")
    if args.h_q is not None and args.h_q != w.h_q:
        changes["h_q"] = args.h_q
        tags.append(f"h_q={args.h_q}")
    if args.causal is not None and (args.causal == "yes") != w.causal:
        changes["causal"] = args.causal == "yes"
        tags.append("causal" if args.causal == "yes" else "non-causal")
    if args.kv == "fp8":
        changes["kv_format"] = "fp8_e4m3"
        changes["kv_scale"] = FP8_KV_SCALE
        tags.append("fp8 cache (E4M3 bytes, scale 1/64)")
    if not changes:
        return w
    return dataclasses.replace(w, name=w.name + "+" + "+".join(t.split()[0] for t in tags),
                               description=w.description + "; with " + ", ".join(tags), **changes)


def copy_probe():
    """A plain copy of known size, to scale profiler byte counters against."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))


def copy_bandwidth(dev, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """Measured HBM bandwidth of a plain device copy (bytes read + written per second).

    A reference beside the 8 TB/s peak: what streaming reads and writes reach
    on this GPU with torch's copy kernel, timed with HIP events.
    """
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"value": round(metrics.gbps(2 * nbytes, ms), 1), "unit": "GB/s",
            "what": f"device copy of {nbytes >> 20} MiB (read + write bytes), mean of {reps}"}


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle on whole sequences of the same inputs, until budget_s of work."""
    from oracle import mla_ref

    def raw(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    fp8 = inp.kv_format == "fp8_e4m3"
    qb = raw(inp.q)
    kb = inp.k_storage.contiguous().numpy() if fp8 else raw(inp.k_storage)
    bt, sl = inp.block_table.numpy(), inp.cache_seqlens.numpy()
    w = inp.workload
    done, elapsed = [], 0.0
    for b in range(w.batch):
        t0 = time.perf_counter()
        mla_ref.mla_decode_ref(qb, kb, bt, sl, w.softmax_scale, w.causal, batch_indices=[b],
                               kv_format=inp.kv_format, kv_scale=inp.kv_scale)
        elapsed += time.perf_counter() - t0
        done.append(b)
        if elapsed >= budget_s:
            break
    tokens = int(sl[done].sum())
    nbytes = metrics.workload_cost(sl[done].tolist(), len(done), w.s_q, w.h_q, w.h_kv,
                                   1 if fp8 else 2)["bytes"]
    flops = metrics.decode_flops(w.s_q, tokens, w.h_q)
    threads = None
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:
        threads = os.cpu_count()
    ms = elapsed * 1e3
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": round(metrics.gbps(nbytes, ms), 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "tflops": round(metrics.tflops(flops, ms), 6),
            "seconds": round(elapsed, 3),
            "sample": f"{len(done)} of {w.batch} sequences ({tokens} cached tokens), fp64 NumPy "
                      f"oracle, {os.cpu_count()} host cores visible ({cpu})"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the decode path has no "
                                   "multi-GPU mode (it would shard by sequence, one plan per GPU)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    _lib.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    inp_host = draw(chosen_workload(args))
    inp = inp_host.to(dev)
    w = inp.workload
    rows = w.s_q * w.h_q
    parts = args.num_parts or default_num_parts(rows, w.h_kv)
    b = w.batch
    out = torch.empty((b, w.s_q, w.h_q, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((workspace_size(b, w.s_q, w.h_q, w.h_kv, D_V, parts),), dtype=torch.uint8,
                     device=dev)
    kv_scale = w.kv_scale if w.kv_format == "fp8_e4m3" else None

    def plan():
        if args.separate_plan:
            return get_mla_metadata(inp.cache_seqlens, rows, w.h_kv, num_parts=parts)
        return None

    def decode(meta):
        mla_decode_with_kvcache(inp.q, inp.blocked_k, inp.block_table, inp.cache_seqlens, D_V,
                                w.softmax_scale, w.causal, metadata=meta, num_parts=parts, out=out,
                                lse=lse, workspace=ws, kv_scale=kv_scale)

    def step():
        decode(plan())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()

    def timed(n_steps: int, flush):
        """n_steps steps with events around the plan call (if any) and the decode call of each."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i, (e0, e1, e2) in enumerate(ev):
            if flush is not None:
                flush.sum()  # reads 512 MB: L2 and MALL then hold clean lines of another buffer
            e0.record()
            if graph is not None:  # plan and decode in one replay
                ev[i] = (e0, e0, e2)
                graph.replay()
                e2.record()
                continue
            if args.separate_plan:
                meta = plan()
                e1.record()
            else:  # the step is the decode call (events recorded twice in a row read ~5 us apart)
                meta = None
                ev[i] = (e0, e0, e2)
            decode(meta)
            e2.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        step_ms = np.array([a.elapsed_time(c) for a, _, c in ev])
        plan_ms = np.array([a.elapsed_time(b_) for a, b_, _ in ev])
        decode_ms = np.array([b_.elapsed_time(c) for _, b_, c in ev])
        # with a flush between steps the step time comes from the events (the
        # flush is not part of a step); back to back, from the wall clock
        per_step = float(step_ms.mean()) if flush is not None else wall_ms / n_steps
        return {"ms_per_step": per_step, "plan_ms": float(plan_ms.mean()),
                "decode_ms": float(decode_ms.mean()), "decode_median": float(np.median(decode_ms)),
                "decode_p10": float(np.percentile(decode_ms, 10)),
                "decode_p90": float(np.percentile(decode_ms, 90))}

    # timed region: exactly `steps` steps (cold: a 512 MB write before each,
    # outside its events), then, unless --warm made the warm steps the official
    # ones, the same number of warm steps back to back for reference
    cold = not args.warm
    # a read, not a write: written lines would stay dirty in the caches and be
    # written back to HBM while the next step runs
    flush = torch.ones((128 << 20,), dtype=torch.float32, device=dev) if cold else None
    main_t = timed(args.steps, flush)
    warm_t = timed(args.steps, None) if cold else None
    if flush is not None:
        del flush
    ms_per_step = main_t["ms_per_step"]
    plan_ms = main_t["plan_ms"]
    dec_avg = main_t["decode_ms"]

    seqlens = inp_host.cache_seqlens
    cost = metrics.workload_cost(seqlens.tolist(), b, w.s_q, w.h_q, w.h_kv,
                                 1 if w.kv_format == "fp8_e4m3" else 2)
    gbs = metrics.gbps(cost["bytes"], ms_per_step)
    tfl = metrics.tflops(cost["flops"], ms_per_step)
    achieved = metrics.gbps(cost["bytes"], dec_avg)

    line = {
        "metric": "paged MLA decode GB/s + TFLOPS (% roofline), b=128 h_q=128 seqlen~4096",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "batch": b, "s_q": w.s_q, "h_q": w.h_q, "h_kv": w.h_kv, "d": 576, "dv": 512,
            "block_size": 64, "entry_pitch": w.pitch, "block_table": w.table, "causal": w.causal,
            "cache_dtype": "fp8_e4m3" if w.kv_format == "fp8_e4m3" else "bf16",
            "caches": "flushed before each step" if cold else "warm",
            "launch": "HIP graph replay" if args.graph else "eager",
            "plan": ("mla_get_metadata call before the decode" if args.separate_plan
                     else "inside the decode call (no metadata passed)"),
            "total_seqlens": cost["total_seqlens"], "num_parts": parts,
            "parallelism": "single GPU",
        },
        "tflops": round(tfl, 2),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "frac_bf16_peak": round(tfl / BF16_PEAK_TFLOPS, 4),
        "algorithmic_bytes": cost["bytes"],
        "algorithmic_flops": cost["flops"],
        "stage_ms": {"plan_call": round(plan_ms, 5) if args.separate_plan else None,
                     "decode_call": round(dec_avg, 5),
                     "decode_median": round(main_t["decode_median"], 5),
                     "decode_p10": round(main_t["decode_p10"], 5),
                     "decode_p90": round(main_t["decode_p90"], 5)},
        "roofline": {
            "bound": "hbm",
            "kernel": ("plan + split-KV decode + lse merge (one graph replay)" if args.graph
                       else "mla_decode_with_kvcache (split-KV decode + lse merge"
                       + (")" if args.separate_plan else ", planning for itself)")),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
    if warm_t is not None:
        line["warm"] = {"value": round(metrics.gbps(cost["bytes"], warm_t["ms_per_step"]), 2),
                        "unit": "GB/s", "ms_per_step": round(warm_t["ms_per_step"], 5),
                        "decode_call_ms": round(warm_t["decode_ms"], 5),
                        "steps": args.steps}
    line["copy_bandwidth"] = copy_bandwidth(dev)
    line["roofline"]["frac_of_copy"] = round(achieved / line["copy_bandwidth"]["value"], 4)
    # measured HBM bytes per decode call (FETCH_SIZE + WRITE_SIZE, copy-calibrated),
    # only when the counters were taken on the current kernel sources
    tr = traffic.load(w.name)
    if tr is not None:
        line["roofline"]["traffic"] = round(tr["bytes_per_call"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp_host, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
