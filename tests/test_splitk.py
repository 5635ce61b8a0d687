"""GPU parity of the split-K entry point (gemm_ex_splitk): the same product as
gemm_ex, through a caller-owned FP32 workspace and a reduction kernel, to the
same bar (every element within the tolerance; bit-exact in the exact-integer
regime, where any summation order is exact)."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import (TORCH_DT, _torch, assert_bit_exact, assert_within_tolerance, out_elem, overflow_operand,
                             run, upload)

pytestmark = pytest.mark.gpu

DT = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16, "fp8": mcs.GEMM_DTYPE_FP8_E4M3}
OUT = {"same": mcs.GEMM_OUT_SAME, "f32": mcs.GEMM_OUT_F32, "bf16": mcs.GEMM_OUT_BF16}


def run_splitk(elem, M, N, K, a_bits, b_bits, trans_b, out, schedule, splits, ldc=None, c_fill=None):
    """C through gemm_ex_splitk; returns (C float64 M x N, raw bits, full padded C)."""
    torch = _torch()
    print(f"[gpu] splitk elem={elem} M={M} N={N} K={K} trans_b={trans_b} out={out} sched={schedule} "
          f"splits={splits} ldc={ldc}", flush=True)
    A, _ = upload(a_bits, elem)
    B, _ = upload(b_bits, elem)
    ldc = N if ldc is None else ldc
    oe = out_elem(elem, out)
    C = torch.empty(max(M, 1) * ldc, dtype=TORCH_DT[oe], device="cuda")
    if c_fill is not None:
        C.fill_(c_fill)
    nbytes = mcs.gemm_splitk_workspace_bytes(DT[elem], M, N, K, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    st = mcs.gemm_ex_splitk(DT[elem], M, N, K, A.data_ptr(), a_bits.shape[1], B.data_ptr(), b_bits.shape[1],
                            trans_b, C.data_ptr(), ldc, OUT[out], schedule, splits, ws.data_ptr(), nbytes,
                            torch.cuda.current_stream().cuda_stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    raw = C.view(max(M, 1), ldc).cpu()
    if oe == "f32":
        vals, bits = raw.double().numpy(), raw.numpy().view(np.uint32)
    else:
        bits = raw.view(torch.int16).numpy().view(np.uint16)
        vals = oracle.decode(bits, oe)
    return vals[:M, :N], bits[:M, :N], vals


def operands(elem, dist, M, N, K, trans_b, seed, lda=None, ldb=None):
    a = si.matrix_bits(elem, dist, M, K, ld=lda, seed=seed, stream=0)
    b = (si.matrix_bits(elem, dist, N, K, ld=ldb, seed=seed, stream=1) if trans_b
         else si.matrix_bits(elem, dist, K, N, ld=ldb, seed=seed, stream=1))
    return a, b


CASES = [  # (elem, trans_b, out, M, N, K, splits)
    ("f16", 1, "same", 1024, 1024, 1024, 4),
    ("f16", 0, "f32", 300, 520, 1000, 3),
    ("bf16", 1, "same", 513, 264, 2000, 7),
    ("bf16", 0, "same", 256, 256, 4096, 16),
    ("f16", 1, "same", 200, 136, 136, 8),          # 3 K-steps: slices of one step
    ("fp8", 1, "bf16", 512, 520, 2048, 5),
    ("fp8", 1, "f32", 258, 130, 1008, 3),
]


@pytest.mark.parametrize("sched", ["pipelined", "in_phase", "interleaved", "tile128"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_splitk_every_element(case, sched):
    elem, trans_b, out, M, N, K, splits = case
    schedule = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
                "interleaved": mcs.GEMM_SCHED_INTERLEAVED, "tile128": mcs.GEMM_SCHED_TILE128}[sched]
    a, b = operands(elem, "normal", M, N, K, trans_b, seed=300 + M + K + splits)
    cref, sabs = oracle.gemm(a, b, elem, trans_b)
    ldc = (N + 7) // 8 * 8 + 8
    c, _, full = run_splitk(elem, M, N, K, a, b, trans_b, out, schedule, splits, ldc=ldc, c_fill=-3.0)
    assert_within_tolerance(c, cref, sabs, f"splitk {case} {sched}", out=out_elem(elem, out))
    assert np.all(full[:, N:] == -3.0)


@pytest.mark.parametrize("elem,out", [("f16", "same"), ("bf16", "same"), ("bf16", "f32"), ("fp8", "bf16")])
def test_splitk_integer_regime_bit_exact(elem, out):
    M, N, K = 512, 768, 512
    a, b = operands(elem, "int5", M, N, K, 1, seed=41)
    cref = oracle.gemm(a, b, elem, 1, with_sabs=False)
    for splits in (2, 3, 4):
        _, bits, _ = run_splitk(elem, M, N, K, a, b, 1, out, mcs.GEMM_SCHED_AUTO, splits)
        assert_bit_exact(bits, cref, elem, out, f"splitk int {elem} {out} splits={splits}")


def test_one_split_is_gemm_ex_bitwise():
    M, N, K = 1024, 512, 2048
    a, b = operands("f16", "normal", M, N, K, 1, seed=5)
    _, bits1, _ = run_splitk("f16", M, N, K, a, b, 1, "same", mcs.GEMM_SCHED_AUTO, 1)
    bits0 = run("f16", M, N, K, a, b, 1)[1]
    assert np.array_equal(bits1, bits0)


def test_splitk_schedules_agree_bitwise():
    """Each slice's partial is computed by the same MFMA sequence in all three
    schedules, so the results agree bit for bit."""
    M, N, K = 768, 1024, 3072
    a, b = operands("bf16", "normal", M, N, K, 1, seed=9)
    outs = [run_splitk("bf16", M, N, K, a, b, 1, "same", s, 6)[1]
            for s in (mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_IN_PHASE, mcs.GEMM_SCHED_INTERLEAVED,
                      mcs.GEMM_SCHED_TILE128)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_splitk_shard_workload_every_element():
    """One GPU's row block of the 8-way split of the 4096x4096x8192 product
    (512x4096x8192), split two and four ways: every element."""
    M, N, K = 512, 4096, 8192
    a, b = operands("f16", "uniform", M, N, K, 1, seed=1003)
    cref, sabs = oracle.gemm(a, b, "f16", 1)
    for splits in (2, 4):
        c, _, _ = run_splitk("f16", M, N, K, a, b, 1, "same", mcs.GEMM_SCHED_AUTO, splits)
        assert_within_tolerance(c, cref, sabs, f"shard splitk {splits}")


@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("K", [1024, 2048, 4096])
def test_splitk_output_rounds_to_nearest_even(K, elem):
    """The reduction kernel rounds the summed FP32 partials to nearest even:
    same-sign integer sums past FP16's exact-integer range (ties included),
    exact in FP32 in any order, must equal RNE of the exact value bit for bit."""
    M, N = 512, 520
    a, b = operands(elem, "int12", M, N, K, 1, seed=80 + K)
    a[1::2] |= np.uint16(0x8000)                # odd rows of A negative
    cref = oracle.gemm(a, b, elem, 1, with_sabs=False)
    assert int((oracle.decode(oracle.round_to(cref, elem), elem) != cref).sum()) > M * N // 4
    for splits in (2, 3, 4):
        _, bits, _ = run_splitk(elem, M, N, K, a, b, 1, "same", mcs.GEMM_SCHED_AUTO, splits)
        assert_bit_exact(bits, cref, elem, "same", f"splitk RNE K={K} {elem} splits={splits}")


@pytest.mark.parametrize("splits", [2, 4])
@pytest.mark.parametrize("sched", ["pipelined", "tile128"])
def test_splitk_fp16_overflow_rounds_to_nearest_even(sched, splits):
    """The reduction's FP16 conversion at the end of the range, bit for bit:
    each row's terms sit in different K slices, so the sums that reach 65520
    and beyond (+inf / -inf) or stay at 65519 and below (65504) are formed in
    the reduction itself."""
    M, N, K = 256, 264, 2048
    a = overflow_operand(M, K, spread=True)
    ones = np.full((N, K), 0x3C00, np.uint16)
    cref = oracle.gemm(a, ones, "f16", 1, with_sabs=False)
    schedule = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "tile128": mcs.GEMM_SCHED_TILE128}[sched]
    _, bits, _ = run_splitk("f16", M, N, K, a, ones, 1, "same", schedule, splits)
    assert_bit_exact(bits, cref, "f16", "same", f"split-K FP16 overflow {sched} S={splits}")
