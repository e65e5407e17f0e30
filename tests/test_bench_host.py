"""Host-side checks of bench.py's measurement arithmetic (no GPU): the algorithmic byte and
flop counts of a call, and the conversion of two rocprofv3 counter runs into HBM bytes per
launch, scaled by the calibration copy of known size."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def _names():
    # how the profiler prints the kernels: the full signature around the template name
    return {key: f"void qlr::(anonymous namespace)::{kname}(qlr::(anonymous namespace)::Params, qlr::Levels)"
            for key, (kname, _) in bench.TRAFFIC_KERNELS.items()}


def test_decode_bytes_and_prefill_flops():
    # 4096 x 4096 4-bit, M = 1, r 16: codes + 8-bit scales + group steps + adapters + x + y
    assert bench.decode_bytes(M=1, N=4096, K=4096, r=16) == (8388608 + 262144 + 4096 + 2 * 16 * 4096 * 2
                                                           + 2 * 4096 + 2 * 4096)
    assert bench.decode_bytes(M=1, N=4096, K=4096, r=0) == 8671232
    assert bench.prefill_flops(M=2048, N=4096, K=4096, r=0) == 2 * 2048 * 4096 * 4096
    assert bench.prefill_flops(M=2048, N=4096, K=4096, r=16) == 2 * 2048 * 4096 * 4096 + 2 * 2048 * 16 * 8192


def test_traffic_from_counters_scales_by_the_calibration_copy(tmp_path):
    names = _names()
    copy = "void at::native::vectorized_elementwise_kernel<4, add>(int)"
    # the copy reads 256 MiB and writes 256 MiB; its FETCH reads half (scale 2), its WRITE all (scale 1)
    fetch = [(copy, 131072.0)] + [(names[k], v) for k, v in (("decode", 4300.0), ("decode", 4400.0),
                                                              ("prefill", 42000.0), ("backward", 41000.0))]
    write = [(copy, 262144.0)] + [(names[k], v) for k, v in (("decode", 8.0), ("decode", 8.0),
                                                             ("prefill", 16384.0), ("backward", 16384.0))]
    _write_run(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_run(str(tmp_path / "w"), "WRITE_SIZE", write)
    out = str(tmp_path / "traffic.json")
    bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), out)
    rec = json.load(open(out))
    assert set(rec) == set(bench.TRAFFIC_KERNELS)
    assert rec["decode"]["launches"] == 2
    assert rec["decode"]["bytes_per_launch"] == int(round(4350.0 * 1024 * 2.0 + 8.0 * 1024))
    assert rec["prefill"]["bytes_per_launch"] == int(round(42000.0 * 1024 * 2.0 + 16384.0 * 1024))
    assert rec["prefill"]["calibration"]["fetch_scale"] == 2.0
    # the stored figure is current for the sources as they are
    for key in rec:
        assert rec[key]["sources"] == bench.TRAFFIC_KERNELS[key][1]


def test_traffic_from_counters_refuses_a_missing_kernel(tmp_path):
    names = _names()
    copy = "void at::native::vectorized_elementwise_kernel<4, add>(int)"
    rows = [(copy, 131072.0), (names["prefill"], 1.0), (names["backward"], 1.0)]  # no decode rows
    _write_run(str(tmp_path / "f"), "FETCH_SIZE", rows)
    _write_run(str(tmp_path / "w"), "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.json"))

