"""Build libgdr.so (the HIP kernels and the C ABI of include/gdr.h) for gfx950.

Each .hip source is compiled with hipcc into an object in _build/, then
linked into gated_delta_rule_85_amd/libgdr.so.  Packed-fp32 instruction
selection is switched off for the device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libgdr.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]
# MFMA operands and results in VGPRs rather than AGPRs (fewer copies in the
# register-resident loops of every kernel that keeps its work in registers).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# The scans run one wave per SIMD, so nothing hides an LDS read's latency but
# the wave's own later instructions: the ILP-seeking scheduler issues the
# operand reads well ahead of their MFMAs (the default one waits on each).
ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
# The backward's chunk-local kernel (also one wave per SIMD, at the register
# limit) spills under the iterative ILP scheduler; with the max-ILP one and
# VGPR-form MFMAs it spills nothing (default scheduler: 17 registers) and runs 8%
# faster.  On the scans the max-ILP scheduler costs 30%.
MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
# The reverse scan runs eight waves (two per SIMD, 256 registers each); the ILP
# scheduler's schedule of it does not survive register allocation in this
# compiler, and the default scheduler with its operand reads pipelined by hand
# serves it.
SOURCES = {"gdr_api.hip": VGPR_FORM, "gdr_prep.hip": VGPR_FORM, "gdr_scan.hip": VGPR_FORM + ILP,
           "gdr_bwd.hip": VGPR_FORM, "gdr_bwd_scan.hip": VGPR_FORM,
           "gdr_bwd_mfma.hip": VGPR_FORM + MAX_ILP, "gdr_noalloc.hip": []}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCES[src] + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                   check=True)
    os.replace(tmp, OUT)
    if verbose:
        print(OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
