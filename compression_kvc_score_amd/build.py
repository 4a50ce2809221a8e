"""Build libkvc.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every source is compiled by hipcc to an object in parallel, then linked into
one shared library next to this file. Usage: ``python -m
compression_kvc_score_amd.build``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libkvc.so"
OFFLOAD_ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={OFFLOAD_ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Per-source additions. The chunk attention keeps its output accumulators in
# ordinary VGPRs (the MFMA's VGPR form): with accumulation registers the
# compiler copies them to VGPRs and back around the softmax rescale.
EXTRA_FLAGS = {
    "prefill_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = shutil.which("hipcc") or os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libkvc)")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    jobs = jobs or min(16, max(1, len(srcs)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(compile_one, srcs))
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
