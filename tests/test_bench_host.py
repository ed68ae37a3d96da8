"""Host-side logic of bench.py (no GPU): the one-GPU guard, which launches a step takes, which profiled kernels
the roofline's traffic counts, and the per-dispatch counter summary on a synthetic counter file."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_decode_04_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_kinds_from_profiler_names():
    assert bench._kernel_kind("pkv::decode_kernel<128, 16, 8, false, true, false, false>") == (
        "decode_kernel", True, False)
    assert bench._kernel_kind("pkv::decode_kernel<128, 16, 8, true, false, false, true>") == (
        "decode_kernel", False, True)
    assert bench._kernel_kind("pkv::varlen_kernel<128, 16, 8, false, 2, true>") == ("varlen_kernel", True, False)
    assert bench._kernel_kind("pkv::varlen_kernel<128, 16, 8, false, 1>") == ("varlen_kernel", False, False)
    assert bench._kernel_kind("pkv::combine_kernel<128>") == ("combine_kernel", False, False)
    assert bench._kernel_kind("pkv::order_kernel") == ("order_kernel", False, False)


def test_dominant_kernels_follow_the_step_shape():
    one_launch = ["pkv::decode_kernel<128, 16, 8, false, true, false, false>", "pkv::append_kernel"]
    assert bench.dominant_kernels("c2", one_launch) == [one_launch[0]]
    split = ["pkv::decode_kernel<128, 16, 8, true, true, false, false>", "pkv::combine_kernel<128>",
             "pkv::decode_kernel<128, 16, 8, true, false, false, false>", "pkv::append_kernel"]
    assert sorted(bench.dominant_kernels("c3", split)) == sorted([split[1], split[2]])
    rounds = ["pkv::append_newest_kernel", "pkv::order_kernel",
              "pkv::decode_kernel<128, 16, 8, false, false, false, true>", "pkv::append_kernel"]
    assert sorted(bench.dominant_kernels("c4", rounds)) == sorted(rounds[1:3])
    varlen = ["pkv::append_varlen_kernel", "pkv::order_varlen_kernel",
              "pkv::varlen_kernel<128, 16, 8, false, 2, false, true>", "pkv::append_kernel"]
    assert sorted(bench.dominant_kernels("v3", varlen)) == sorted(varlen[1:3])
    assert bench.dominant_kernels("r2", ["pkv::qkv_cache_kernel<128>"]) == ["pkv::qkv_cache_kernel<128>"]


def test_step_launch_count_matches_the_library_routing():
    plan1 = {"num_splits": 1}
    c2 = W.config_c2(with_pools=False)
    assert bench.step_launch_count(c2, plan1, 1, False, 256) == 1  # 256 workgroups: one round
    assert bench.step_launch_count(c2, plan1, 1, False, 128) == 2
    assert bench.step_launch_count(c2, {"num_splits": 8}, 8, False, 256) == 2
    v = W.build_varlen_case("t", 32, 32, 8, 128, 16, np.full(32, 8, np.int32), np.full(32, 100, np.int32), 5)
    assert bench.step_launch_count(v, None, 0, True, 256) == 1  # two tiles of 4 rows in one group
    w = W.build_varlen_case("t", 2, 8, 2, 64, 16, (33, 2), (0, 5), 6)
    assert bench.step_launch_count(w, None, 0, True, 256) == 2  # more than 32 new rows


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for i, (name, value) in enumerate(rows):
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    fused = "void pkv::decode_kernel<128, 16, 8, false, true, false, false>(pkv::DecodeParams)"
    # copy kernel over 512 MiB reads 256 Mi KiB-units as counted (factor 2 for FETCH_SIZE, 1 for WRITE_SIZE)
    write(tmp_path / "f.csv", "FETCH_SIZE", [("neg_kernel", 512 * 1024 / 2), (fused, 100000.0), (fused, 100000.0),
                                             ("pkv::append_kernel(pkv::AppendParams)", 10.0)])
    write(tmp_path / "w.csv", "WRITE_SIZE", [("neg_kernel", 512 * 1024), (fused, 2000.0), (fused, 2000.0),
                                             ("pkv::append_kernel(pkv::AppendParams)", 1000.0)])
    rec = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "c2", 1, 512.0)
    assert rec["scale_factors"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert rec["scale_factors"]["WRITE_SIZE"] == pytest.approx(1.0)
    k = rec["kernels"]["pkv::decode_kernel<128, 16, 8, false, true, false, false>"]
    assert k["fetch_bytes"] == 100000 * 1024 * 2 and k["write_bytes"] == 2000 * 1024 and k["dispatches"] == 2
    assert rec["hbm_bytes_per_step"] == 100000 * 1024 * 2 + 2000 * 1024  # the append is not counted


def test_floor_tiles_follow_the_launch_decomposition():
    """bench.py --floor's tiles: one per (sequence, kv head) in id order for one round of CUs, longest first with the
    pieces rule for more (c4's 16384-row sequence in two pieces of 8192 rows), fixed splits for c3; every tile reads
    its rows' K and V (D * 4 bytes a row) and writes G * D * 2 bytes."""
    import numpy as np
    from paged_kv_decode_04_amd import workloads as W
    c = W.config_c2(with_pools=False)
    t = bench.floor_tiles(c, 0, 1, False, 256)
    assert len(t) == 32 * 8
    assert [b for b, _ in t[:8]] == [int(c.context_lens[0]) * 128 * 4] * 8  # id order: sequence 0's heads first
    assert sum(b for b, _ in t) == int(c.context_lens.sum()) * 8 * 128 * 4 and {o for _, o in t} == {4 * 128 * 2}
    c = W.config_c4(with_pools=False)
    t = bench.floor_tiles(c, 0, 1, False, 256)
    L = np.sort(c.context_lens)[::-1]
    assert L[0] == 16384 and len(t) == (256 + 1) * 8
    assert [b for b, _ in t[:16]] == [8192 * 512] * 16  # the two pieces of the longest sequence lead
    assert sum(b for b, _ in t) == int(c.context_lens.sum()) * 8 * 512
    assert all(t[i][0] >= t[i + 8][0] for i in range(16, len(t) - 8, 8))  # longest first after them
    c = W.config_c3(with_pools=False)
    t = bench.floor_tiles(c, 0, 8, False, 256)
    assert len(t) == 4 * 8 * 8 and {b for b, _ in t} == {32768 // 8 * 512}
    t = bench.floor_tiles(W.config_c2(with_pools=False), 512, 1, False, 256)
    assert {b for b, _ in t} == {512 * 512}  # a window of 512 rows
