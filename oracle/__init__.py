"""CPU oracle for the FP16/BF16/FP8 GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU package.

The arithmetic lives in ``gemm_oracle.c`` (a plain binary64 triple loop with
hand-written binary16/bfloat16/FP8-E4M3 decoders and round-to-nearest-even
encoders for the 16-bit outputs);
this file compiles it with gcc on first use and marshals numpy arrays.

Pins (the tests that tie the oracle to something other than itself):
  * decoders: exhaustive over all 65536 bit patterns against numpy (binary16)
    and torch (bfloat16) widening, and over all 256 FP8 E4M3 patterns against
    torch's float8_e4m3fn widening;
  * encoders: against numpy's float64->float16 rounding on random and edge
    values, and bfloat16 ties worked by hand;
  * product: exact rational brute force (fractions.Fraction) on tiny shapes,
    numpy.matmul in float64 at moderate sizes, identity / permutation /
    all-ones / rank-1 closed forms, and the exact-integer regime.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "libgemm_oracle.so")
_lock = threading.Lock()
_lib = None

ELEM = {"f16": 0, "bf16": 1, "fp8": 2}
# numpy dtype of an operand's bit patterns
BITS = {"f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def build(force: bool = False, src: str = _SRC, out: str = _LIB, defines=()) -> str:
    """Compile gemm_oracle.c into libgemm_oracle.so (gcc, no fast-math, no FP contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", "-pthread", *[f"-D{d}" for d in defines], src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, u16p, f64p, i64p, vp = (ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                 ctypes.c_void_p)
    lib.oracle_gemm_rows.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, i64,
                                     ctypes.c_int, i64, i64, f64p, f64p, ctypes.c_int]
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm_points.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, i64,
                                       ctypes.c_int, i64, i64p, i64p, f64p, f64p]
    lib.oracle_gemm_points.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [ctypes.c_int, i64, vp, f64p]
    lib.oracle_decode.restype = None
    lib.oracle_round.argtypes = [ctypes.c_int, i64, f64p, u16p]
    lib.oracle_round.restype = None
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits(a, elem: str) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != BITS[elem]:
        raise TypeError(f"{elem} operands are passed as {np.dtype(BITS[elem]).name} bit patterns")
    return a


def _shape_args(A, B, trans_b, elem, K=None):
    A = _bits(A, elem)
    B = _bits(B, elem)
    if A.ndim != 2 or B.ndim != 2 or not A.flags.c_contiguous or not B.flags.c_contiguous:
        raise ValueError("A and B must be 2-D C-contiguous arrays (row stride = shape[1])")
    M, lda = A.shape
    K = lda if K is None else K
    if trans_b:
        N, ldb = B.shape
        if ldb < K:
            raise ValueError("B (N x K) too narrow")
    else:
        if B.shape[0] < K:
            raise ValueError("B (K x N) too short")
        N = ldb = B.shape[1]
    return A, B, M, N, K, lda, ldb


class Oracle:
    """The oracle bound to one compiled library (the default one, or a test's own build)."""

    def __init__(self, path: str):
        self.lib = _bind(path)

    def decode(self, bits, elem: str) -> np.ndarray:
        """Exact float64 values of FP16/BF16 (uint16) or FP8 E4M3 (uint8) bit patterns."""
        b = np.ascontiguousarray(_bits(bits, elem))
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode(ELEM[elem], b.size, b.ctypes.data, _ptr(out, ctypes.c_double))
        return out

    def round_to(self, values, elem: str) -> np.ndarray:
        """Round-to-nearest-even of float64 values into FP16/BF16 bit patterns."""
        if elem not in ("f16", "bf16"):
            raise ValueError("results round to f16 or bf16")
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_round(ELEM[elem], v.size, _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16))
        return out

    def gemm(self, A, B, elem: str, trans_b: int, K: int | None = None, N: int | None = None,
             rows: tuple[int, int] | None = None, nthreads: int | None = None, with_sabs: bool = True):
        """Cref (and Sabs) = rows of A.B in float64.

        A: M x lda bit patterns (uint16, or uint8 for fp8; first K columns
        used); B: K x ldb (trans_b=0, first N columns used) or N x ldb
        (trans_b=1, first K columns used)."""
        A, B, M, Nb, K, lda, ldb = _shape_args(A, B, trans_b, elem, K)
        N = Nb if N is None else N
        r0, r1 = (0, M) if rows is None else rows
        nthreads = nthreads or min(os.cpu_count() or 1, 16)
        C = np.empty((r1 - r0, N), dtype=np.float64)
        S = np.empty((r1 - r0, N), dtype=np.float64) if with_sabs else None
        rc = self.lib.oracle_gemm_rows(ELEM[elem], M, N, K, A.ctypes.data, lda,
                                       B.ctypes.data, ldb, int(trans_b), r0, r1,
                                       _ptr(C, ctypes.c_double),
                                       _ptr(S, ctypes.c_double) if S is not None else None, nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_rows rejected its arguments")
        return (C, S) if with_sabs else C

    def gemm_points(self, A, B, elem: str, trans_b: int, ii, jj, K: int | None = None,
                    N: int | None = None):
        """Cref and Sabs at the points (ii[p], jj[p])."""
        A, B, M, Nb, K, lda, ldb = _shape_args(A, B, trans_b, elem, K)
        N = Nb if N is None else N
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        C = np.empty(ii.shape, dtype=np.float64)
        S = np.empty(ii.shape, dtype=np.float64)
        rc = self.lib.oracle_gemm_points(ELEM[elem], M, N, K, A.ctypes.data, lda,
                                         B.ctypes.data, ldb, int(trans_b), ii.size,
                                         _ptr(ii, ctypes.c_int64), _ptr(jj, ctypes.c_int64),
                                         _ptr(C, ctypes.c_double), _ptr(S, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_gemm_points rejected its arguments")
        return C, S


def default() -> Oracle:
    global _lib
    with _lock:
        if _lib is None:
            _lib = Oracle(build())
    return _lib


def decode(bits, elem: str) -> np.ndarray:
    return default().decode(bits, elem)


def round_to(values, elem: str) -> np.ndarray:
    return default().round_to(values, elem)


def gemm(*args, **kw):
    return default().gemm(*args, **kw)


def gemm_points(*args, **kw):
    return default().gemm_points(*args, **kw)


def bf16_half_ulp(x) -> np.ndarray:
    """Half the spacing of bfloat16 values at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def within_tolerance(c, cref, sabs, out: str = "f16") -> np.ndarray:
    """Per-element acceptance: |c - Cref| <= 2e-3 * Sabs + 2^-10 * |Cref|.

    The 2^-10 |Cref| term covers rounding the FP32 sum to an FP16 (or FP32)
    output, whose half-spacing is at most 2^-11 |C|.  A BF16 output has 8
    significant bits, so a correctly rounded BF16 result can sit up to 2^-8 |C|
    from Cref; for out="bf16" that half-spacing is added to the bound."""
    c = np.asarray(c, dtype=np.float64)
    bound = 2e-3 * sabs + (2.0 ** -10) * np.abs(cref)
    if out == "bf16":
        bound = bound + bf16_half_ulp(cref)
    return np.abs(c - cref) <= bound
