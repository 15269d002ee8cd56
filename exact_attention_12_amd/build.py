"""Build libattn.so (HIP kernels + C ABI) for gfx950, in the package directory.

Every source is compiled by hipcc for --offload-arch=gfx950 (cross-compiles
without a GPU), then linked into one shared library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# Sources and their extra flags.
SOURCES = {
    "attn_api.cpp": [],
    "attn_fwd.hip": [],
    "attn_bwd.hip": [],
    "attn_bwd_dq.hip": [],
    "attn_decode.hip": [],
    "mfma_probe.hip": [],
}

# Packed fp32 VALU forms are turned off for all device code. MFMA results
# and accumulators are kept in the VGPR form: otherwise, above 256 live
# registers, the backend places the score tiles in AGPRs and shuttles the
# gradient accumulators between AGPRs and VGPRs on every loop step.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libattn.so")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCES[src], "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


# Sources with inline-assembly MFMAs, whose VALU -> MFMA wait states the
# compiler does not track: their device assembly is checked (hazards.py).
HAZARD_CHECKED = ["attn_bwd.hip"]


def _check_hazards(src: str) -> None:
    asm = os.path.join(BUILD_DIR, os.path.basename(src) + ".gfx950.s")
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCES[src], "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{res.stdout}{res.stderr}")
    sys.path.insert(0, PKG)
    try:
        import hazards
    finally:
        sys.path.pop(0)
    with open(asm) as f:
        found = hazards.check(f.read())
    if found:
        name, seq = found[0]
        raise RuntimeError(f"{src}: {len(found)} VALU -> MFMA operand hazard(s) in the generated code, "
                           f"first in {name}:\n  " + "\n  ".join(seq))


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [("c", s) for s in SOURCES] + [("h", s) for s in HAZARD_CHECKED]

    def run(job):
        kind, src = job
        return _compile(src, verbose) if kind == "c" else _check_hazards(src)

    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(run, jobs))
    objs = [r for (kind, _), r in zip(jobs, results) if kind == "c"]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
