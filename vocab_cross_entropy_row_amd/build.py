"""Build liblce.so in-tree with hipcc for gfx950 only.

    python -m vocab_cross_entropy_row_amd.build

Each source is compiled to an object under ``_build/`` in parallel, then linked
into ``vocab_cross_entropy_row_amd/liblce.so``.  Packed fp32 instructions are
disabled for all device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblce.so")

SOURCES = ["lce_api.cpp", "lce_host.cpp", "lce_gemm.cpp", "lce_fused_paths.cpp", "xent_kernels.hip", "fused_kernel.hip", "bwd_kernels.hip", "seq_kernels.hip",
           "jsd_kernel.hip", "fused_grad_kernel.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblce)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        # Only the C ABI (LCE_API in lce.h) is exported: host code, and the
        # host side of the kernel sources (launchers, stubs), is hidden.
        vis = ["-fvisibility=hidden"] if src.endswith(".cpp") else ["-Xarch_host", "-fvisibility=hidden"]
        cmd = [cc, *lang, *common_flags(), *vis, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 target feature and says so; harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines and (verbose or p.returncode != 0):
            print(f"--- {src}\n" + "\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"liblce build failed: {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
