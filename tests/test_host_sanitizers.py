"""liblce's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host sources (validation, scratch pool, GEMM plans, error strings) are compiled with
both sanitizers and linked, with the kernel objects of the regular build, into a small
driver (host_sanitize_driver.cpp).  The driver replays every argument-error case of
test_abi.py, the empty no-op calls and a two-thread check of the per-thread error
message; a sanitizer report, a wrong status or a missing detail fails the test.  None of
these calls reaches a HIP API, so no device is used.
"""
import inspect
import os
import subprocess

import pytest

import test_abi as abi
import vocab_cross_entropy_row_amd as lce
from vocab_cross_entropy_row_amd import build as lce_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SOURCES = ["lce_api.cpp", "lce_host.cpp", "lce_gemm.cpp", "lce_fused_paths.cpp"]
# noalloc.hip holds a device array and its entry point in one file: it is linked as built
KERNEL_SOURCES = [s for s in lce_build.SOURCES if s.endswith(".hip")]
OUT = os.path.join(ROOT, "_build", "host_sanitize")


# The fused backward's chunk planner, (tokens, vocab, cap) -> (chunk, stored).  The
# stored path writes a token tile's fp32 logits (256 * ld * 4 bytes) through one
# buffer resource with 32-bit offsets, so it is never chosen once ld reaches 2^22,
# however large the cap.
PLANS = [
    ((2048, 128256, 2 << 30), (2048, True)),        # the page shape: one stored chunk
    ((8192, 128256, 2 << 30), (2560, True)),        # chunks of 2560 tokens
    ((4096, (1 << 22) - 256, 16 << 30), (512, True)),   # ld = 2^22 - 256: still addressable
    ((4096, (1 << 22) - 255, 16 << 30), (2048, False)),  # ld = 2^22: recompute, 2 B per logit
    ((8192, (1 << 23) - 512, 64 << 30), (4096, False)),
    ((4096, (1 << 23) - 512, 2 << 30), (256, False)),   # not even 256 tokens: one tile
    ((300, 1000, 0), (256, False)),                      # no cap: recompute
    ((100, 1000, 2 << 30), (100, True)),                 # fewer tokens than a chunk
]


def _flags():
    san = []
    for kind in ("address", "undefined"):  # host only: the device code is not instrumented
        san += ["-Xarch_host", "-fsanitize=" + kind]
    return ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
            "-I", os.path.join(ROOT, "include")] + san


def _build_driver() -> str:
    cc = lce_build.hipcc()
    kernel_objs = [os.path.join(lce_build.BUILD, s.replace(".", "_") + ".o") for s in KERNEL_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        lce_build.build()
    os.makedirs(OUT, exist_ok=True)
    jobs, objs = [], []
    srcs = [os.path.join(lce_build.CSRC, s) for s in HOST_SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"))
    for src in srcs:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [cc, "-x", "hip", "--cuda-host-only", *_flags(), "-I", lce_build.CSRC, "-c", src, "-o", obj]
        jobs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in jobs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{src}:\n{out.decode(errors='replace')[-3000:]}"
    exe = os.path.join(OUT, "host_sanitize_driver")
    link = [cc, f"--offload-arch={lce_build.ARCH}", *_flags()[5:], *objs, *kernel_objs, "-o", exe,
            "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _line(fn_name, helper, kw, status, needle):
    bound = inspect.signature(helper).bind(**kw)
    bound.apply_defaults()
    args = [repr(float(v)) if isinstance(v, float) else str(int(v)) for v in bound.arguments.values()]
    return f"{fn_name} {int(status)} {len(args)} {' '.join(args)} {needle}"


CASE_TABLES = [
    ("lce_xent_fwd", abi._xent, abi.XENT_CASES),
    ("lce_xent_fwd_noalloc", abi._xent_noalloc, abi.XENT_CASES),
    ("lce_fused_linear_xent_fwd", abi._fused, abi.FUSED_CASES),
    ("lce_xent_partial_fwd", abi._partial, abi.PARTIAL_CASES),
    ("lce_xent_merge", abi._merge, abi.MERGE_CASES),
    ("lce_xent_bwd", abi._bwd, abi.BWD_CASES),
    ("lce_fused_linear_logprob_sums", abi._sums, abi.SUMS_CASES),
    ("lce_fused_linear_jsd_fwd", abi._jsd, abi.JSD_CASES),
    ("lce_fused_linear_xent_bwd", abi._fbwd, abi.FBWD_CASES),
    ("lce_xent_fwd_bwd", abi._fwd_bwd, abi.FWD_BWD_CASES),
    ("lce_fused_linear_xent_fwd_bwd", abi._ffb, abi.FUSED_FWD_BWD_CASES),
]

# Empty calls that are no-ops: status LCE_OK and an empty detail message.
EMPTY = [
    "lce_xent_fwd 0 7 0 0 0 32 0 1 0 ",
    "lce_xent_fwd_noalloc 0 7 0 1 0 32 0 1 0 ",
    "lce_xent_partial_fwd 0 7 0 1 0 8 0 0 0 ",
    "lce_xent_merge 0 7 0 3 0 0 10 1 0 ",
    "lce_xent_bwd 0 8 0 0 0 8 0 1 0 0 ",
    "lce_xent_fwd_bwd 0 9 0 0 0 8 0 1 0 0 0 ",
    f"lce_fused_linear_jsd_fwd 0 10 0 {abi.FAKE} 0 {abi.FAKE} 0 64 100 0.5 1 0 ",
]


def test_host_code_is_clean_under_sanitizers():
    exe = _build_driver()
    lines = [_line(fn, helper, kw, st, needle)
             for fn, helper, table in CASE_TABLES for kw, st, needle in table]
    lines += EMPTY
    lines += [f"plan_fused_bwd {2 * chunk + int(stored)} 3 {t} {v} {cap} "
              for (t, v, cap), (chunk, stored) in PLANS]
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main: leak reports would be about it
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert f"cases {len(lines)} failed 0" in r.stdout, report[-4000:]
    assert lce.LCE_OK == 0
