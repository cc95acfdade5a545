"""Build libpingala.so in-tree: host C++ with g++, HIP kernels with hipcc for
gfx950, linked by hipcc.  Every call rebuilds from source."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpingala.so")
ARCH = "gfx950"

HOST_SOURCES = ["pg_host.cpp", "pg_api.cpp"]
HIP_SOURCES = ["pg_kernels.hip", "pg_fused.hip", "pg_fused1.hip", "pg_fused1_r23.hip", "pg_fused_carry.hip", "pg_fused_mma.hip", "pg_qgemm.hip", "pg_qgemv_mma.hip", "pg_encode.hip"]


def _hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="pg_build_")
    objs, procs = [], []
    try:
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            # host code: strict IEEE evaluation (the encoder must match the
            # oracle's rounding), no fused multiply-add
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
                   "-Wall", "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd)))
            objs.append(obj)
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            # kernel arguments preloaded into scalar registers (the first 16
            # dwords): a launch's first instructions need not wait for the
            # argument segment (0.4% per token on the batch-1 stack)
            cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-mllvm", "-amdgpu-kernarg-preload-count=16",
                   "-Wall", "-Wno-unused-function", "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, p in procs:
            _, err = p.communicate()
            if err:
                err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
                if err.strip():
                    print(err)
            if p.returncode != 0:
                raise RuntimeError("build step failed: " + " ".join(cmd))
            if verbose:
                print(" ".join(cmd))
        link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp", "-lpthread"]
        if verbose:
            print(" ".join(link))
        subprocess.run(link, check=True)
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
