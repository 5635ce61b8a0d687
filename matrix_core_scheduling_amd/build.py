"""Build libmcs_gemm.so (the gfx950 GEMM kernels and their C ABI) in-tree with hipcc.

    python -m matrix_core_scheduling_amd.build            # build the libraries
    python -m matrix_core_scheduling_amd.build --asm DIR  # also write device assembly

Two libraries come out of the same sources: libmcs_gemm.so, the product, and
libmcs_gemm_stagger.so, the race-stress build (compiled with MCS_STAGGER:
random sleeps at every workgroup barrier and NaN-filled LDS at kernel start),
which only the tests load.
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
STAGGER_LIB = os.path.join(PKG, "libmcs_gemm_stagger.so")
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


# Per-source options.  The attention kernel's scores are finite or -inf (a
# masked key) for finite inputs, so its maxima need no NaN quieting: without
# it each fmaxf is one v_max instead of a max plus canonicalising copies.
# The compiler's own MFMAs in it keep their accumulators in VGPRs (the 4-wave
# form writes its O products itself, with AGPR accumulators).
EXTRA = {"attention_fwd.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def device_asm(src: str, out: str, defines=()) -> str:
    """Write the gfx950 assembly of one source file of csrc/ to ``out``
    (``defines``: extra -D options, e.g. ["-DMCS_STAGGER=1"] for the race-stress build)."""
    _run([HIPCC, *COMMON, *EXTRA.get(src, []), *defines, "--cuda-device-only", "-S", os.path.join(CSRC, src),
          "-o", out])
    return out


def build(asm_dir: str | None = None, jobs: int = 4) -> str:
    """Compile both libraries; return the product library's path."""
    variants = [(LIB, OBJDIR, []), (STAGGER_LIB, os.path.join(OBJDIR, "stagger"), ["-DMCS_STAGGER=1"])]
    for _, objdir, _ in variants:
        os.makedirs(objdir, exist_ok=True)

    def compile_one(job):
        src, objdir, defs = job
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        _run([HIPCC, *COMMON, *EXTRA.get(src, []), *defs, "-c", os.path.join(CSRC, src), "-o", obj])
        if asm_dir and not defs:
            os.makedirs(asm_dir, exist_ok=True)
            device_asm(src, os.path.join(asm_dir, src.replace(".hip", f"-{ARCH}.s")))
        return obj

    jobs_list = [(src, objdir, defs) for _, objdir, defs in variants for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, jobs_list))
    for i, (lib, _, _) in enumerate(variants):
        tmp = lib + f".tmp{os.getpid()}"
        mine = objs[i * len(SOURCES):(i + 1) * len(SOURCES)]
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *mine, "-o", tmp])
        os.replace(tmp, lib)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="directory for device assembly (.s) files")
    a = ap.parse_args(argv)
    print(build(a.asm))


if __name__ == "__main__":
    sys.exit(main())
