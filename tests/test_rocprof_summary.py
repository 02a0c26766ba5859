"""The kernel-trace reader splits a bench.py run into warm-up, cold and warm
steps, whether a step starts with the plan kernel or with a decode kernel
that plans for itself."""

import csv

from paged_mla_decode_04_amd import rocprof_summary


def write_trace(path, kernels):
    t = 0
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, us in kernels:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
            t += us * 1000 + 500


FLUSH = "void at::native::reduce_kernel<512, 1>(float)"


def run(tmp_path, step, warmup=2, steps=3):
    kernels = []
    for _ in range(warmup):
        kernels += step("w")
    for _ in range(steps):
        kernels += [(FLUSH, 50)] + step("c")
    for _ in range(steps):
        kernels += step("h")
    path = tmp_path / "trace.csv"
    write_trace(path, kernels)
    return rocprof_summary.trace_phases(str(path))


def durations(phase):  # "w", "c", "h" -> distinct durations per phase
    return {"w": 10, "c": 20, "h": 30}[phase]


def test_steps_that_start_with_the_plan_kernel(tmp_path):
    ph = run(tmp_path, lambda p: [("mla::plan_kernel(int const*)", 1),
                                  ("void mla::decode_kernel<1>(mla::DecodeArgs)", durations(p)),
                                  ("mla::combine_kernel(mla::DecodeArgs)", 2)])
    d = ph["decode_kernel<1>"]
    assert d["warmup"] == [10, 10] and d["cold"] == [20] * 3 and d["warm"] == [30] * 3
    assert len(ph["plan_kernel"]["cold"]) == 3 and len(ph["combine_kernel"]["warm"]) == 3


def test_steps_whose_decode_plans_for_itself(tmp_path):
    name = "void mla::(anonymous namespace)::decode_wide_kernel<false, true>(mla::DecodeArgs)"
    ph = run(tmp_path, lambda p: [(name, durations(p)), ("mla::combine_tiles_kernel(mla::DecodeArgs)", 2)])
    d = ph["decode_wide_kernel<false, true>"]
    assert d["warmup"] == [10, 10] and d["cold"] == [20] * 3 and d["warm"] == [30] * 3
    assert len(ph["combine_tiles_kernel"]["cold"]) == 3
