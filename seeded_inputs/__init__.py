"""Seeded synthetic operands for the FP16/BF16/FP8 GEMM and for its CPU oracle.

This module is the only code shared by the GPU path's tests/bench and the
oracle.  It produces *input bit patterns* and the workload table; it holds
none of the GEMM arithmetic (no products, sums or output rounding).

Generator (counter-based, so any element can be regenerated on its own):

    key(seed, stream) = seed * 0x9E3779B97F4A7C15 + stream * 2**40      (mod 2**64)
    x(seed, stream, i) = mix64(key(seed, stream) + i)
    mix64(z) = the SplitMix64 output function (Steele, Lea and Flood,
               "Fast splittable pseudorandom number generators", OOPSLA 2014):
               z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
               z ^= z >> 27; z *= 0x94D049BB133111EB;
               z ^= z >> 31

Distributions, for the element at flat index i = row * ld + col (ld = the
row stride in elements; padding elements get values too):

    uniform[-1,1)  : u(i) = (x >> 11) * 2**-53;  v = 2 u - 1
    normal(0,1)    : Box-Muller on the two uniforms drawn at 2i and 2i+1:
                     v = sqrt(-2 ln(1 - u(2i))) * cos(2 pi u(2i+1))
    integers [-2,2]: v = (x mod 5) - 2
    integers {1,2} : v = (x mod 2) + 1      ("int12": same-sign sums that grow
                     like 2.25 K, past FP16's exact-integer range)

The double v is rounded once to the operand type: FP16 by numpy's
float64->float16 cast (round to nearest even), BF16 by float64->float32
(numpy) then float32->bfloat16 (torch), FP8 E4M3 by float64->float32 then
float32->float8_e4m3fn (torch), all round-to-nearest-even.  FP16/BF16 bit
patterns are uint16, FP8 bit patterns uint8.
Stream 2r holds A and 2r+1 holds B of rotation set r (r = 0 is the set
that is checked).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


_CHUNK = 1 << 20


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> int:
    return (int(seed) * 0x9E3779B97F4A7C15 + int(stream) * (1 << 40)) & ((1 << 64) - 1)


class _Scratch:
    """Chunk buffers reused across calls (fresh pages are slow on some hosts)."""

    def __init__(self):
        self.base = np.arange(2 * _CHUNK, dtype=np.uint64)
        self.z = np.empty(2 * _CHUNK, dtype=np.uint64)
        self.t = np.empty(2 * _CHUNK, dtype=np.uint64)
        self.f = np.empty(2 * _CHUNK, dtype=np.float64)
        self.g = np.empty(_CHUNK, dtype=np.float64)


_scratch = None


def _mix_chunk(key: int, start: int, m: int, sc: _Scratch) -> np.ndarray:
    """mix64(key + start + i) for i < m, in sc.z[:m] (in place, no allocation)."""
    z, t = sc.z[:m], sc.t[:m]
    with np.errstate(over="ignore"):
        np.add(sc.base[:m], np.uint64((key + start) & ((1 << 64) - 1)), out=z)
        for shift, mul in ((30, _M1), (27, _M2)):
            np.right_shift(z, np.uint64(shift), out=t)
            np.bitwise_xor(z, t, out=z)
            np.multiply(z, mul, out=z)
        np.right_shift(z, np.uint64(31), out=t)
        np.bitwise_xor(z, t, out=z)
    return z


def raw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """SplitMix64 outputs for counters start .. start+count-1."""
    key = _key(seed, stream)
    with np.errstate(over="ignore"):
        idx = np.arange(start, start + count, dtype=np.uint64)
        return _mix64(np.uint64(key) + idx)


def _values_into(dist: str, seed: int, stream: int, start: int, out: np.ndarray, scale: float = 1.0):
    """Write float64 draws for flat indices start .. start+len(out)-1 into out
    (any float dtype: the float64 draw is cast once on assignment)."""
    global _scratch
    if _scratch is None:
        _scratch = _Scratch()
    sc = _scratch
    key = _key(seed, stream)
    count = out.size
    for c0 in range(0, count, _CHUNK):
        m = min(_CHUNK, count - c0)
        f = sc.f[:m]
        if dist == "uniform":
            z = _mix_chunk(key, start + c0, m, sc)
            np.right_shift(z, np.uint64(11), out=z)
            np.multiply(z, 2.0 ** -52, out=f, casting="unsafe")       # 2u, u = (x >> 11) 2^-53
            np.subtract(f, 1.0, out=f)
        elif dist == "normal":
            z = _mix_chunk(key, 2 * (start + c0), 2 * m, sc)
            np.right_shift(z, np.uint64(11), out=z)
            u = sc.f[:2 * m]
            np.multiply(z, 2.0 ** -53, out=u, casting="unsafe")
            g = sc.g[:m]
            np.multiply(u[1::2], 2.0 * math.pi, out=g)              # 2 pi u(2i+1)
            np.cos(g, out=g)
            r = u[0::2]                                              # -> sqrt(-2 ln(1 - u(2i)))
            np.negative(r, out=r)
            np.log1p(r, out=r)
            np.multiply(r, -2.0, out=r)
            np.sqrt(r, out=r)
            np.multiply(r, g, out=g)
            f = g
        elif dist == "int12":
            z = _mix_chunk(key, start + c0, m, sc)
            np.bitwise_and(z, np.uint64(1), out=z)
            np.add(z, np.uint64(1), out=z)
            np.copyto(f, z, casting="unsafe")
        elif dist == "int5":
            z = _mix_chunk(key, start + c0, m, sc)
            np.remainder(z, np.uint64(5), out=z)
            np.subtract(z, np.uint64(2), out=z)                     # 0, 1 wrap around ...
            np.copyto(f, z.view(np.int64), casting="unsafe")         # ... and read back as -2, -1
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        if scale != 1.0:
            np.multiply(f, scale, out=f)
        out[c0:c0 + m] = f


def values(dist: str, seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    """float64 draws for flat indices start .. start+count-1."""
    out = np.empty(count, dtype=np.float64)
    _values_into(dist, seed, stream, start, out)
    return out


def to_bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to FP16/BF16 (uint16 bit patterns) or FP8 E4M3
    (uint8 bit patterns)."""
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    if dtype in ("bf16", "fp8"):
        import torch

        f32 = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
        if dtype == "bf16":
            return f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return f32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(f"unknown operand type {dtype!r}")


def matrix_bits(dtype: str, dist: str, rows: int, cols: int, ld: int | None = None,
                seed: int = 1, stream: int = 0, scale: float = 1.0) -> np.ndarray:
    """A rows x ld array (row-major, row stride ld) of seeded operand bits
    (uint16 for f16/bf16, uint8 for fp8).

    Only the first ``cols`` columns are meant to be read; the padding columns
    hold draws too (they must never influence a result)."""
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    n = rows * ld
    if dtype == "f16":
        out = np.empty(n, dtype=np.float16)
        _values_into(dist, seed, stream, 0, out, scale)
        return out.view(np.uint16).reshape(rows, ld)
    out = np.empty(n, dtype=np.uint8 if dtype == "fp8" else np.uint16)
    buf = np.empty(min(n, _CHUNK), dtype=np.float32)
    for c0 in range(0, n, _CHUNK):
        m = min(_CHUNK, n - c0)
        _values_into(dist, seed, stream, c0, buf[:m], scale)
        out[c0:c0 + m] = to_bits(buf[:m], dtype)
    return out.reshape(rows, ld)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic GEMM workload: C (MxN) = A (MxK) . B, B given KxN (trans_b=0) or NxK (trans_b=1)."""
    name: str
    dtype: str          # "f16" | "bf16" | "fp8" (E4M3) operands
    M: int
    N: int
    K: int
    trans_b: int
    dist: str           # "uniform" | "normal" | "normal_scaled" (normal / sqrt(K))
    out: str            # "same" | "f32" | "bf16" (fp8 operands: "f32" or "bf16")
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 1 if self.dtype == "fp8" else 2

    @property
    def out_type(self) -> str:
        """Element type of C: "f16", "bf16" or "f32"."""
        return self.dtype if self.out == "same" else self.out

    def algorithmic_bytes(self) -> int:
        out_bytes = 4 if self.out_type == "f32" else 2
        return self.elem_bytes * (self.M * self.K + self.K * self.N) + out_bytes * self.M * self.N

    def operands(self, rotation: int = 0):
        """(A bits MxK, B bits) for rotation set ``rotation``."""
        dist, scale = self.dist, 1.0
        if dist == "normal_scaled":
            dist, scale = "normal", 1.0 / math.sqrt(self.K)
        a = matrix_bits(self.dtype, dist, self.M, self.K, seed=self.seed,
                        stream=2 * rotation, scale=scale)
        if self.trans_b:
            b = matrix_bits(self.dtype, dist, self.N, self.K, seed=self.seed,
                            stream=2 * rotation + 1, scale=scale)
        else:
            b = matrix_bits(self.dtype, dist, self.K, self.N, seed=self.seed,
                            stream=2 * rotation + 1, scale=scale)
        return a, b


# The workloads: a 256^3 case the oracle finishes in seconds, a 1024^3 case
# with B given transposed, the 4096x4096x8192 FP16 compute-bound shape the
# MI355X figures are quoted on, an 8192^3 BF16 case, a tall-skinny
# 16384x2048x8192 case with FP32 output, the 8192^3 FP8 E4M3 shape (B given
# N x K, normally distributed values) an MI355X FP8 figure is quoted on, and
# one GPU's row block (512x4096x8192) of an 8-way row split of the FP16 shape,
# and the FP16 shape at twice the K (4096x4096x16384), the second MI355X point.
WORKLOADS = {
    "f16_256": Workload("f16_256", "f16", 256, 256, 256, 0, "uniform", "same", 1001),
    "f16_1024_bt": Workload("f16_1024_bt", "f16", 1024, 1024, 1024, 1, "normal_scaled", "same", 1002),
    "f16_4096x4096x8192": Workload("f16_4096x4096x8192", "f16", 4096, 4096, 8192, 1, "uniform", "same", 1003),
    "bf16_8192": Workload("bf16_8192", "bf16", 8192, 8192, 8192, 1, "normal", "same", 1004),
    "f16_16384x2048x8192_f32out": Workload("f16_16384x2048x8192_f32out", "f16", 16384, 2048, 8192, 0,
                                           "uniform", "f32", 1005),
    "fp8_8192": Workload("fp8_8192", "fp8", 8192, 8192, 8192, 1, "normal", "bf16", 1006),
    "f16_512x4096x8192": Workload("f16_512x4096x8192", "f16", 512, 4096, 8192, 1, "uniform", "same", 1007),
    "f16_4096x4096x16384": Workload("f16_4096x4096x16384", "f16", 4096, 4096, 16384, 1, "uniform", "same", 1008),
}
HEADLINE = "f16_4096x4096x8192"


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One synthetic attention workload: Q (B,H,Sq,D), K and V (B,H,Sk,D), all
    of one operand type, row-major with D contiguous; scale 1/sqrt(D)."""
    name: str
    dtype: str          # "f16" | "bf16"
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    dist: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> int:
        """2 products of 2*Sq*Sk*D each per head; causal counts the allowed
        (query, key) pairs only."""
        pairs = self.Sq * self.Sk
        if self.causal:
            off = self.Sk - self.Sq
            pairs = sum(max(0, min(self.Sk, i + off + 1)) for i in range(self.Sq))
        return 4 * self.B * self.H * pairs * self.D

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and O written once (operand type), plus the FP32 lse."""
        return 2 * self.B * self.H * self.D * (2 * self.Sq + 2 * self.Sk) + 4 * self.B * self.H * self.Sq

    def operands(self, rotation: int = 0):
        """(Q, K, V) bit patterns for rotation set ``rotation``."""
        q = matrix_bits(self.dtype, self.dist, self.B * self.H * self.Sq, self.D, seed=self.seed,
                        stream=3 * rotation).reshape(self.B, self.H, self.Sq, self.D)
        k = matrix_bits(self.dtype, self.dist, self.B * self.H * self.Sk, self.D, seed=self.seed,
                        stream=3 * rotation + 1).reshape(self.B, self.H, self.Sk, self.D)
        v = matrix_bits(self.dtype, self.dist, self.B * self.H * self.Sk, self.D, seed=self.seed,
                        stream=3 * rotation + 2).reshape(self.B, self.H, self.Sk, self.D)
        return q, k, v


# Attention workloads: a small case the oracle finishes in seconds, and
# 4 sequences x 32 heads x 4096 tokens at head size 128 (16k tokens of a
# 4096-wide model), plain, causal and BF16.  Values normal(0, 1).
ATTN_WORKLOADS = {
    "attn_f16_b1h4s512d128": AttnWorkload("attn_f16_b1h4s512d128", "f16", 1, 4, 512, 512, 128, False, "normal", 2001),
    "attn_f16_b4h32s4096d128": AttnWorkload("attn_f16_b4h32s4096d128", "f16", 4, 32, 4096, 4096, 128, False,
                                            "normal", 2002),
    "attn_f16_b4h32s4096d128_causal": AttnWorkload("attn_f16_b4h32s4096d128_causal", "f16", 4, 32, 4096, 4096,
                                                   128, True, "normal", 2003),
    "attn_bf16_b4h32s4096d128": AttnWorkload("attn_bf16_b4h32s4096d128", "bf16", 4, 32, 4096, 4096, 128, False,
                                             "normal", 2004),
}
