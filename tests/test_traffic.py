"""The counter summary behind bench.py's roofline.traffic: copy calibration and
per-call totals from rocprofv3 counter CSVs (synthetic files here)."""

import csv
import json

from paged_mla_decode_04_amd import traffic

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, vals in rows.items():
            for v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_summary_scales_by_the_copy_calibration(tmp_path):
    gib_kib = (1 << 30) / 1024
    write_csv(tmp_path / "cf.csv", "FETCH_SIZE", {"__amd_rocclr_copyBuffer": [gib_kib / 2]})
    write_csv(tmp_path / "cw.csv", "WRITE_SIZE", {"__amd_rocclr_copyBuffer": [gib_kib]})
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", {"void mla::decode_kernel<4>(mla::DecodeArgs)": [100.0, 300.0],
                                                 "mla::combine_kernel(mla::DecodeArgs)": [10.0],
                                                 "mla::(anonymous namespace)::decode_wide_kernel(mla::DecodeArgs)": [8.0],
                                                 "mla::plan_kernel(int const*)": [1.0]})
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", {"void mla::decode_kernel<4>(mla::DecodeArgs)": [50.0],
                                                 "mla::(anonymous namespace)::decode_wide_kernel(mla::DecodeArgs)": [4.0],
                                                 "mla::combine_kernel(mla::DecodeArgs)": [5.0, 7.0]})
    d = traffic.summarize(str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), str(tmp_path / "f.csv"),
                          str(tmp_path / "w.csv"), "wide")
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    # the plan is not part of the call
    assert sorted(d["kernels"]) == ["combine_kernel", "decode_kernel<4>", "decode_wide_kernel"]
    assert d["kernels"]["decode_kernel<4>"]["fetch_bytes"] == 200.0 * 1024 * 2
    assert d["kernels"]["combine_kernel"]["write_bytes"] == 6.0 * 1024
    assert d["bytes_per_call"] == (200 * 2 + 50 + 10 * 2 + 6 + 8 * 2 + 4) * 1024
    assert d["source_sha256"] == traffic.source_hash()
    json.dumps(d)


def test_source_hash_is_stable():
    assert traffic.source_hash() == traffic.source_hash()
    assert len(traffic.source_hash()) == 64
