"""Helpers for the GPU tests: upload seeded operand bits, run the library
through its C ABI, and read results back as float64."""
from __future__ import annotations

import numpy as np

import matrix_core_scheduling_amd as mcs
import oracle

TORCH_DT = {}


def _torch():
    import torch
    if not TORCH_DT:
        TORCH_DT.update({"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn,
                         "f32": torch.float32})
    return torch


def out_elem(elem: str, out: str) -> str:
    """Element type of C for operand type elem and output choice out ("same", "f32", "bf16")."""
    return elem if out == "same" else out


def upload(bits: np.ndarray, elem: str, pad_front: int = 0):
    """Bit patterns (rows x ld; uint16, or uint8 for fp8) -> device tensor of the
    operand dtype.  With pad_front > 0 the data starts pad_front elements into
    the allocation (to build misaligned operands)."""
    torch = _torch()
    if elem == "fp8":
        flat, tdt = np.ascontiguousarray(bits).reshape(-1), torch.uint8
    else:
        flat, tdt = np.ascontiguousarray(bits).reshape(-1).view(np.int16), torch.int16
    t = torch.empty(flat.size + pad_front, dtype=tdt, device="cuda")
    t[pad_front:].copy_(torch.from_numpy(flat.copy()))
    return t.view(TORCH_DT[elem]), pad_front


def run(elem: str, M: int, N: int, K: int, a_bits, b_bits, trans_b: int, out: str = "same",
        schedule: int = mcs.GEMM_SCHED_AUTO, ldc: int | None = None, c_fill: float | None = None,
        a_offset: int = 0, entry: str = "ex", return_raw: bool = False, allow_refusal: bool = False):
    """C = A.B on the GPU through the C ABI; returns (C float64 M x N, raw C bits).
    out: "same" (the operand type; not for fp8), "f32" or "bf16".

    With allow_refusal, a GEMM_EALIGN or GEMM_EUNSUPPORTED answer (the MFMA
    kernels cannot take these operands; nothing was launched) returns None
    instead."""
    torch = _torch()
    print(f"[gpu] {entry} elem={elem} M={M} N={N} K={K} trans_b={trans_b} out={out} "
          f"sched={schedule} ldc={ldc} a_off={a_offset}", flush=True)
    lda = a_bits.shape[1]
    ldb = b_bits.shape[1]
    A, off = upload(a_bits, elem, a_offset)
    B, _ = upload(b_bits, elem)
    ldc = N if ldc is None else ldc
    oe = out_elem(elem, out)
    C = torch.empty(max(M, 1) * ldc, dtype=TORCH_DT[oe], device="cuda")
    if c_fill is not None:
        C.fill_(c_fill)
    out_type = {"same": mcs.GEMM_OUT_SAME, "f32": mcs.GEMM_OUT_F32, "bf16": mcs.GEMM_OUT_BF16}[out]
    stream = torch.cuda.current_stream().cuda_stream
    a_ptr = A.data_ptr() + (1 if elem == "fp8" else 2) * off
    if entry == "ex":
        dt = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16, "fp8": mcs.GEMM_DTYPE_FP8_E4M3}[elem]
        st = mcs.gemm_ex(dt, M, N, K, a_ptr, lda, B.data_ptr(), ldb, trans_b, C.data_ptr(), ldc,
                         out_type, schedule, stream)
    else:
        fn = {"f16": mcs.gemm_f16, "bf16": mcs.gemm_bf16, "fp8": mcs.gemm_fp8}[elem]
        st = fn(M, N, K, a_ptr, lda, B.data_ptr(), ldb, trans_b, C.data_ptr(), ldc, out_type, stream)
    if allow_refusal and st in (mcs.GEMM_EALIGN, mcs.GEMM_EUNSUPPORTED):
        return None
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    full = C.view(max(M, 1), ldc)
    raw = full.cpu()
    if oe == "f32":
        vals = raw.double().numpy()
        bits = raw.numpy().view(np.uint32)
    else:
        bits = raw.view(torch.int16).numpy().view(np.uint16)
        vals = oracle.decode(bits, oe)
    if return_raw:
        return vals[:M, :N], bits, vals
    return vals[:M, :N], bits[:M, :N]


def assert_within_tolerance(c, cref, sabs, what="", out="f16"):
    """out: the output element type ("f16", "bf16" or "f32")."""
    ok = oracle.within_tolerance(c, cref, sabs, out=out)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} elements outside tolerance; first at "
                             f"({i},{j}): got {c[i, j]!r}, oracle {cref[i, j]!r}, Sabs {sabs[i, j]!r}")


def assert_bit_exact(c_bits, cref, elem, out, what=""):
    """Integer regime: C must be the round-to-nearest-even of the exact value."""
    oe = out_elem(elem, out)
    if oe == "f32":
        want = cref.astype(np.float32)
        got = c_bits.view(np.float32)
        eq = got.astype(np.float64) == want.astype(np.float64)
    else:
        want = oracle.round_to(cref, oe)
        eq = oracle.decode(c_bits, oe) == oracle.decode(want, oe)         # +0 == -0
    if not eq.all():
        bad = np.argwhere(~eq)
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} elements differ; first at ({i},{j}) oracle {cref[i, j]}")


# FP16 values whose sums land at the top of the FP16 range.  Each sum is an
# integer below 2^24, so the FP32 accumulator holds it exactly.
OVERFLOW_SUMS = [(32768, 32704, 31),          # 65503 -> 65504
                 (32768, 32736),              # 65504, the largest finite FP16
                 (32768, 32736, 15),          # 65519 -> 65504
                 (32768, 32736, 16),          # 65520: the tie with 65536 goes to even, +inf
                 (32768, 32768),              # 65536 -> +inf
                 (32768,) * 32,               # 2^20 -> +inf
                 (2048, 1, 0.5)]              # 2049.5 -> 2050 (a tie, to even)


def overflow_operand(M: int, K: int, spread: bool = False) -> np.ndarray:
    """A (M x K FP16 bits) whose row i holds the terms of OVERFLOW_SUMS[i % 7],
    negated on every other block of 7 rows; with B all ones, C[i, :] is that
    sum.  The terms sit at k = 0, 1, 2 ..., or with spread as far apart as K
    allows (a quarter of K for up to four terms), so that a product split along
    K over up to four slices adds them in its reduction."""
    a = np.zeros((M, K), np.float64)
    for i in range(M):
        vals = OVERFLOW_SUMS[i % len(OVERFLOW_SUMS)]
        sign = -1.0 if (i // len(OVERFLOW_SUMS)) % 2 else 1.0
        step = (K // max(4, len(vals))) if spread else 1
        a[i, np.arange(len(vals)) * step] = sign * np.asarray(vals, np.float64)
    bits = oracle.round_to(a, "f16")
    assert np.array_equal(oracle.decode(bits, "f16"), a)              # every term is an FP16 value
    return bits


# Sums of FP16 terms at the bottom of the FP16 range, in units of 2^-24 (the
# smallest subnormal).  With B = 0.5 the products are exact FP32 values and
# C = sum / 2 in units of 2^-24: odd sums fall halfway between two FP16
# subnormals.
SUBNORMAL_SUMS = [(1,),                # 2^-25: tie between 0 and 2^-24 -> +0
                  (3,),                # 1.5 * 2^-24: tie -> 2 * 2^-24 (even)
                  (5,),                # 2.5 * 2^-24: tie -> 2 * 2^-24
                  (1024, 1),           # 2^-15 + 2^-25: tie -> 2^-15 (512 units, even)
                  (1023, 1023, 1),     # 1023.5 units: tie between 1023 (odd) and 1024 = 2^-14, normal
                  (7, 9, 1024, 512),   # 776 units, exact
                  (2047,)]             # 1023.5 units again, from one subnormal term


def subnormal_operand(M: int, K: int) -> np.ndarray:
    """A (M x K FP16 bits) whose row i holds the terms of SUBNORMAL_SUMS[i % 7]
    times 2^-24 (subnormal or small normal FP16 values), negated on every
    other block of 7 rows."""
    a = np.zeros((M, K), np.float64)
    for i in range(M):
        vals = SUBNORMAL_SUMS[i % len(SUBNORMAL_SUMS)]
        sign = -1.0 if (i // len(SUBNORMAL_SUMS)) % 2 else 1.0
        a[i, :len(vals)] = sign * np.asarray(vals, np.float64) * 2.0 ** -24
    bits = oracle.round_to(a, "f16")
    assert np.array_equal(oracle.decode(bits, "f16"), a)              # every term is an FP16 value
    return bits


# BF16 terms in units of 2^-133 (the smallest BF16 subnormal; 2^-126 is the
# smallest normal).  With B = 0.5 every product is an FP32 denormal and C is
# the sum / 2 in units of 2^-133: odd sums fall halfway between two BF16
# subnormals.
BF16_SUBNORMAL_SUMS = [(1,), (3,), (5,), (255, 1), (127, 127, 1), (7, 9, 100), (300,)]


def bf16_subnormal_operand(M: int, K: int) -> np.ndarray:
    """A (M x K BF16 bits), row i the terms of BF16_SUBNORMAL_SUMS[i % 7] times
    2^-133, negated on every other block of 7 rows."""
    a = np.zeros((M, K), np.float64)
    for i in range(M):
        vals = BF16_SUBNORMAL_SUMS[i % len(BF16_SUBNORMAL_SUMS)]
        sign = -1.0 if (i // len(BF16_SUBNORMAL_SUMS)) % 2 else 1.0
        a[i, :len(vals)] = sign * np.asarray(vals, np.float64) * 2.0 ** -133
    bits = oracle.round_to(a, "bf16")
    assert np.array_equal(oracle.decode(bits, "bf16"), a)
    return bits


def fp8_subnormal_operand(M: int, K: int) -> np.ndarray:
    """A (M x K FP8 E4M3 bytes): row i holds the E4M3 subnormals m * 2^-9,
    m = 1 .. 7 (bit pattern m, exponent field 0), in a pattern that varies
    with i, plus the smallest normal 2^-6 (pattern 8) on every third row, and
    negated rows (sign bit) on every other block of 7 rows."""
    a = np.zeros((M, K), np.uint8)
    for i in range(M):
        n = 1 + i % 7
        ms = [(i + 3 * t) % 7 + 1 for t in range(n)]
        if i % 3 == 0:
            ms.append(8)
        a[i, :len(ms)] = np.asarray(ms, np.uint8) | (0x80 if (i // 7) % 2 else 0)
    return a
