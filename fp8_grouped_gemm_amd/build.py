"""Build the HIP libraries in-tree for gfx950 with hipcc: libmoe_fp8.so (the
MoE forward) and libmoe_peaks.so (the ceiling-measurement kernels)."""
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_fp8.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["moe_api.cpp", "route.hip", "gemm_direct.hip", "gemm_lds.hip", "gemm_lds160.hip", "gemm_sa.hip",
           "gemm_mx.hip", "pack.hip", "quant.hip"]
PEAKS_LIB = os.path.join(HERE, "libmoe_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 instructions are disabled for every device pass.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(HERE, "..", "include"), "-Wall"]


# The 128-row kernels count their copy waits by hand (vmcnt) on the premise
# that their loop holds no other vector memory access; a register spill to
# scratch would add such accesses (each wait then over-waits), so this
# source is compiled with the resource-usage report and the build fails if
# any of its kernels uses scratch.
NO_SCRATCH = ("gemm_lds.hip", "gemm_lds160.hip")


def _scratch_users(report):
    """(kernel, bytes) of every kernel in a resource-usage report with scratch."""
    out = []
    for block in report.split("remark: Function Name: ")[1:]:
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        if m and int(m.group(1)) > 0:
            out.append((block.split()[0], int(m.group(1))))
    return out


def _compile(sources, verbose):
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if src in NO_SCRATCH:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    return objs, procs


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source (all in parallel) and link both libraries."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = _compile(SOURCES, verbose)
    peak_objs, peak_procs = _compile(PEAKS_SOURCES, verbose)
    failed = False
    for src, p in procs + peak_procs:
        out, _ = p.communicate()
        if src in NO_SCRATCH:
            users = _scratch_users(out)
            out = "\n".join(l for l in out.splitlines() if "kernel-resource-usage" not in l)
            if users:
                failed = True
                sys.stdout.write(f"{src}: kernels spill to scratch: {users}\n")
        if out.strip() and (verbose or p.returncode):
            sys.stdout.write(out)
        if p.returncode:
            failed = True
            sys.stdout.write(f"hipcc failed on {src}\n")
    if failed:
        raise RuntimeError("HIP build failed")
    _link(objs, LIB, verbose)
    _link(peak_objs, PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
