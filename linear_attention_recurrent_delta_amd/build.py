"""Build libkdn.so (the gfx950 HIP library behind include/kdn.h) in-tree.

    python -m linear_attention_recurrent_delta_amd.build

Each source is compiled with hipcc for gfx950 in parallel, then linked into
``linear_attention_recurrent_delta_amd/libkdn.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkdn.so")
OBJDIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS

# (source, extra defines, object name).  The prefill source is compiled once
# per variant so the template instantiations build in parallel.
UNITS = [("kdn_abi.cpp", [], "kdn_abi.o"),
         ("kdn_decode.hip", [], "kdn_decode.o")]
UNITS += [("kdn_prefill.hip", [f"-DKDN_PREFILL_VARIANT={v}"], f"kdn_prefill_{v}.o")
          for v in range(5)]
UNITS += [("kdn_prefill.hip", ["-DKDN_PREFILL_DISPATCH"], "kdn_prefill_dispatch.o"),
          ("kdn_prefill_state.hip", [], "kdn_prefill_state.o"),
          # MFMA accumulators in VGPRs: the chain applies VALU work (decay,
          # subtraction, bf16 rounding) to every accumulator it produces
          ("kdn_prefill_chain.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"], "kdn_prefill_chain.o"),
          ("kdn_prefill_short.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"], "kdn_prefill_short.o"),
          ("kdn_variance.hip", [], "kdn_variance.o"),
          ("kdn_noalloc.hip", [], "kdn_noalloc.o"),
          ("kdn_backward.hip", [], "kdn_backward.o")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(unit):
    src, defs, obj = unit
    out = os.path.join(OBJDIR, obj)
    cmd = [hipcc()] + COMMON + defs + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {defs}:\n{err}")
    return out


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
