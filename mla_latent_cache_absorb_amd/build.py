"""Build libmla_absorb.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

python -m mla_latent_cache_absorb_amd.build   (or __graft_entry__.build())
Objects go to _build/ at the repository root; the library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["mla_api.hip", "latent_attn.hip", "absorb_q.hip", "up_v.hip", "kpool_indexer.hip",
           "latent_down.hip", "naive_attn.hip", "check_inputs.hip", "stream_probe.hip"]
LIB_NAME = "libmla_absorb.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for every kernel: the compiler would otherwise form them
# from ordinary float code.  The host pass warns that it does not know the feature (harmless).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA accumulators in VGPRs: accumulators and operands share one register
                # budget (168 per wave in the attention kernel, three waves per SIMD) instead of
                # being split between VGPRs and AGPRs with copies between them
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmla_absorb.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object (in parallel) and link the shared library. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = COMMON + DEVICE_FLAGS + list(extra_flags or [])
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(k):
        return _run([cc, *flags, "-c", os.path.join(CSRC, SOURCES[k]), "-o", objs[k]])

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
