"""Build libfbd.so (the HIP kernels and the C ABI) for gfx950, in place.

    python -m fwd_bwd_double_amd.build            # from the repository root

Each source is compiled by hipcc into an object under _build/, then linked
into fwd_bwd_double_amd/libfbd.so next to this file.  Packed fp32 VALU
instructions are disabled in device code (-packed-fp32-ops)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfbd.so")
SOURCES = ["api.cpp", "fwd.hip", "bwd.hip", "bob.hip", "bob_f32.hip", "fp8.hip"]
# MFMA results are kept in the architectural VGPRs, so the element-wise work
# between products needs no accumulator-register moves (not for bob_f32.hip:
# the compiler fails on the fp32 BoB row kernel with it).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PER_SOURCE = {"fwd.hip": VGPR_FORM, "bwd.hip": VGPR_FORM, "bob.hip": VGPR_FORM,
              "fp8.hip": VGPR_FORM}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-mcode-object-version=5",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def compile_one(src: str, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *PER_SOURCE.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
