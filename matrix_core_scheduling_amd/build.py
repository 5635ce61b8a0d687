"""Build libmcs_gemm.so (the gfx950 GEMM kernels and their C ABI) in-tree with hipcc.

    python -m matrix_core_scheduling_amd.build            # build the library
    python -m matrix_core_scheduling_amd.build --asm DIR  # also write device assembly
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmcs_gemm.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["gemm_pipelined.hip", "gemm_interleaved.hip", "gemm_tile128.hip", "gemm_generic.hip",
           "gemm_api.hip", "attention_fwd.hip"]

# Packed-FP32 instructions stay off: hipcc would otherwise form v_pk_* FP32
# arithmetic from ordinary float code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def device_asm(src: str, out: str) -> str:
    """Write the gfx950 assembly of one source file of csrc/ to ``out``."""
    _run([HIPCC, *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out])
    return out


def build(asm_dir: str | None = None, jobs: int = 4) -> str:
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        _run([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        if asm_dir:
            os.makedirs(asm_dir, exist_ok=True)
            device_asm(src, os.path.join(asm_dir, src.replace(".hip", f"-{ARCH}.s")))
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="directory for device assembly (.s) files")
    a = ap.parse_args(argv)
    print(build(a.asm))


if __name__ == "__main__":
    sys.exit(main())
