"""Benchmark of paged MLA decode on one MI355X.

One step = one pass of the whole hot path over one batch: the split-KV plan
(mla_get_metadata) and the decode with its lse merge (mla_decode_with_kvcache),
on synthetic inputs already resident in HBM.  The default workload is the
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
from paged_mla_decode_04_amd.workloads import D_V, WORKLOADS, draw  # noqa: E402

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
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (plan + decode) in a HIP graph and time its replays "
                         "(removes the host's launch overhead, which small workloads feel)")
    ap.add_argument("--flush", action="store_true",
                    help="write 512 MB before every timed step so that no input stays in L2 or the "
                         "256 MB Infinity Cache; the step time is then taken from HIP events")
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


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle on whole sequences of the same inputs, until budget_s of work."""
    from oracle import mla_ref

    def raw(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    qb, kb = raw(inp.q), raw(inp.k_storage)
    bt, sl = inp.block_table.numpy(), inp.cache_seqlens.numpy()
    w = inp.workload
    done, elapsed = [], 0.0
    for b in range(w.batch):
        t0 = time.perf_counter()
        mla_ref.mla_decode_ref(qb, kb, bt, sl, w.softmax_scale, w.causal, batch_indices=[b])
        elapsed += time.perf_counter() - t0
        done.append(b)
        if elapsed >= budget_s:
            break
    tokens = int(sl[done].sum())
    nbytes = metrics.decode_bytes(tokens, len(done), w.s_q, w.h_q, w.h_kv)
    flops = metrics.decode_flops(w.s_q, tokens, w.h_q)
    threads = None
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:
        threads = os.cpu_count()
    ms = elapsed * 1e3
    return {"value": round(metrics.gbps(nbytes, ms), 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "tflops": round(metrics.tflops(flops, ms), 6),
            "seconds": round(elapsed, 3),
            "sample": f"{len(done)} of {w.batch} sequences ({tokens} cached tokens), fp64 NumPy "
                      f"oracle, {os.cpu_count()} host cores visible"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not "
                                   "part of this build", "n_gpus": args.gpus}))
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

    def step():
        meta = get_mla_metadata(inp.cache_seqlens, rows, w.h_kv, num_parts=parts)
        mla_decode_with_kvcache(inp.q, inp.blocked_k, inp.block_table, inp.cache_seqlens, D_V,
                                w.softmax_scale, w.causal, metadata=meta, out=out, lse=lse,
                                workspace=ws)
        return meta

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

    # timed region: exactly `steps` steps; events bracket the decode call of each
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev) if args.flush else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (e0, e1, e2) in enumerate(ev):
        if flush is not None:
            flush.fill_(i & 255)
        e0.record()
        if graph is not None:  # plan and decode in one replay (e1 marks nothing)
            e1.record()
            graph.replay()
            e2.record()
            continue
        meta = get_mla_metadata(inp.cache_seqlens, rows, w.h_kv, num_parts=parts)
        e1.record()
        mla_decode_with_kvcache(inp.q, inp.blocked_k, inp.block_table, inp.cache_seqlens, D_V,
                                w.softmax_scale, w.causal, metadata=meta, out=out, lse=lse,
                                workspace=ws)
        e2.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    if flush is not None:  # the flush is not part of a step
        ms_per_step = float(np.mean([a.elapsed_time(c) for a, _, c in ev]))
    plan_ms = float(np.mean([a.elapsed_time(b_) for a, b_, _ in ev]))
    decode_ms = np.array([b_.elapsed_time(c) for _, b_, c in ev])

    seqlens = inp_host.cache_seqlens
    cost = metrics.workload_cost(seqlens.tolist(), b, w.s_q, w.h_q, w.h_kv)
    gbs = metrics.gbps(cost["bytes"], ms_per_step)
    tfl = metrics.tflops(cost["flops"], ms_per_step)
    dec_avg = float(decode_ms.mean())
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
            "caches": "flushed before each step" if args.flush else "warm",
            "launch": "HIP graph replay" if args.graph else "eager",
            "total_seqlens": cost["total_seqlens"], "num_parts": parts,
            "parallelism": "single GPU",
        },
        "tflops": round(tfl, 2),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "frac_bf16_peak": round(tfl / BF16_PEAK_TFLOPS, 4),
        "algorithmic_bytes": cost["bytes"],
        "algorithmic_flops": cost["flops"],
        "stage_ms": {"plan": round(plan_ms, 5), "decode_and_merge": round(dec_avg, 5),
                     "decode_p10": round(float(np.percentile(decode_ms, 10)), 5),
                     "decode_p90": round(float(np.percentile(decode_ms, 90)), 5)},
        "roofline": {
            "bound": "hbm",
            "kernel": ("plan + split-KV decode + lse merge (one graph replay)" if args.graph
                       else "mla_decode_with_kvcache (split-KV decode + lse merge)"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
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
