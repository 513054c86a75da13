"""Builds libvq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every translation unit is compiled with -ffp-contract=off (no multiply-add is
fused unless written as one) and with packed fp32 instructions disabled.  The
assignment search is compiled with -fno-honor-nans: its inputs are finite by
contract, and without NaNs a minimum of accumulator values needs no quieting
step (two VALU instructions fewer per tile in the search's inner loop).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvq.so")
SOURCES = ["vq_assign.hip", "vq_update.hip", "vq_select.hip", "vq_elem.hip", "vq_qgemv.hip", "vq_vptq.hip", "vq_hfactor.hip", "vq_groups.hip", "vq_host.hip",
           "vq_timing.hip", "vq_check.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-Wno-unused-result"]
EXTRA = {"vq_assign.hip": ["-fno-honor-nans"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, p.stderr))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n%s" % p.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
