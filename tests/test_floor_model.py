"""The benchmark's work model reproduces the bandwidth floors the pages print.

The pages' floor assumes each declared input and output tensor moves through HBM
one time, at a datasheet bandwidth; ``bench.tensor_bytes`` / ``xent_bytes`` / ``fused_bytes`` must give exactly
the bytes behind each printed floor (tests/golden/page_floors.json, cited there)."""
import json
import math
import os
import subprocess
import sys

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_floors.json")
ITEMSIZE = {"f32": 4, "bf16": 2, "int64": 8}


def floors():
    with open(GOLDEN) as fh:
        return json.load(fh)["floors"]


@pytest.mark.parametrize("f", floors(), ids=lambda f: f["page"])
def test_floor_reproduced(f):
    b = bench.tensor_bytes([(math.prod(shape), ITEMSIZE[dt]) for _, dt, shape in f["tensors"]])
    us = b / (f["bandwidth_gbs"] * 1e9) * 1e6
    assert round(us, 1) == f["floor_us"]
    # the printed ratio is record / floor, up to the rounding of the printed record
    lo, hi = f["record_us"] - 0.05 * (1000 if f["record_us"] > 1000 else 1), \
        f["record_us"] + 0.05 * (1000 if f["record_us"] > 1000 else 1)
    assert lo / us <= f["ratio"] + 0.005 and hi / us >= f["ratio"] - 0.005


def test_named_models_match_generic_sum():
    assert bench.xent_bytes(16384, 4096, 4, "mean") == 268_566_532
    assert bench.xent_bytes(8192, 4096, 2, "none") == 67_207_168
    assert bench.fused_bytes(2048, 4096, 128256, "mean") == 1_067_466_756
    assert bench.xent_bytes(16384, 131072, 4, "mean") == 8_590_065_668
    assert bench.xent_bytes(8192, 131072, 2, "none") == 2_147_581_952
    assert bench.fused_flops(2048, 4096, 128256) == 2 * 2048 * 4096 * 128256


def test_bench_refuses_several_gpus():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stream_read_probe_exports():
    """bench_probe.so (the plain-read, VALU-rate and fused-loop skeleton probes bench.py reports)
    exports their entries."""
    import ctypes
    if not os.path.exists(bench.PROBE_LIB):
        pytest.skip("bench_probe.so not built (__graft_entry__.build() builds it)")
    lib = ctypes.CDLL(bench.PROBE_LIB)
    assert hasattr(lib, "bench_stream_read")
    assert hasattr(lib, "bench_valu_rate")
    assert hasattr(lib, "bench_mfma_lds")
    assert hasattr(lib, "bench_lds_read")
