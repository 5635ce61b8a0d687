"""GPU parity of the FP8 (E4M3) GEMM: the HIP path through the C ABI against the
CPU oracle, to the same bar as the FP16/BF16 product (every element within
|C - Cref| <= 2e-3 Sabs + 2^-10 |Cref|, plus half a BF16 spacing for BF16
output; bit-exact in the exact-integer regime)."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import assert_bit_exact, assert_within_tolerance, fp8_subnormal_operand, run

pytestmark = pytest.mark.gpu

FP8_NAN = 0x7F
SCHEDS = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
          "interleaved": mcs.GEMM_SCHED_INTERLEAVED, "tile128": mcs.GEMM_SCHED_TILE128}


def operands(dist, M, N, K, trans_b, seed, lda=None, ldb=None, nan_pad=False):
    a = si.matrix_bits("fp8", dist, M, K, ld=lda, seed=seed, stream=0)
    b = (si.matrix_bits("fp8", dist, N, K, ld=ldb, seed=seed, stream=1) if trans_b
         else si.matrix_bits("fp8", dist, K, N, ld=ldb, seed=seed, stream=1))
    if nan_pad:
        a[:, K:] = FP8_NAN
        if trans_b:
            b[:, K:] = FP8_NAN
        else:
            b[:, N:] = FP8_NAN
    return a, b


def rup16(x):
    return (x + 15) // 16 * 16


def fast_eligible(K, trans_b):
    """The documented FP8 conditions, given 16-byte aligned buffers and leading
    dimensions whose rows are whole 16-byte chunks: K % 16 == 0, B given N x K."""
    return K % 16 == 0 and trans_b == 1


SHAPES = [(256, 256, 256), (1, 1, 16), (17, 33, 16), (300, 520, 208), (513, 257, 144), (64, 640, 1008),
          (258, 130, 136), (200, 96, 1000)]


@pytest.mark.parametrize("sched", ["pipelined", "in_phase", "interleaved", "tile128"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_every_element(shape, trans_b, out, sched):
    M, N, K = shape
    lda = rup16(K) + 16                     # padded rows, padding filled with NaN
    ldb = (rup16(K) + 16) if trans_b else (rup16(N) + 16)
    ldc = (N + 7) // 8 * 8 + 8              # padded output rows must stay untouched
    a, b = operands("normal", M, N, K, trans_b, seed=200 + M + N + K, lda=lda, ldb=ldb, nan_pad=True)
    cref, sabs = oracle.gemm(a, b, "fp8", trans_b, K=K, N=N)
    got = run("fp8", M, N, K, a, b, trans_b, out=out, schedule=SCHEDS[sched], ldc=ldc, c_fill=-3.0,
              return_raw=True, allow_refusal=True)
    if got is None:
        assert not fast_eligible(K, trans_b)
        assert run("fp8", M, N, K, a, b, trans_b, out=out, ldc=ldc, allow_refusal=True) is None
        got = run("fp8", M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_GENERIC, ldc=ldc,
                  c_fill=-3.0, return_raw=True)
    else:
        assert fast_eligible(K, trans_b)
    c, _, full = got
    assert_within_tolerance(c, cref, sabs, f"{shape} tb={trans_b} {out} {sched}", out=out)
    assert np.all(full[:, N:] == -3.0)


INT_SHAPES = [(256, 256, 32), (512, 256, 128), (256, 512, 192), (512, 512, 448), (1024, 1024, 512)]


@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("shape", INT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_regime_bit_exact(shape, out, sched):
    M, N, K = shape
    a, b = operands("int5", M, N, K, 1, seed=9 + K)
    cref = oracle.gemm(a, b, "fp8", 1, with_sabs=False)
    schedule = mcs.GEMM_SCHED_GENERIC if sched == "generic" else SCHEDS[sched]
    _, bits = run("fp8", M, N, K, a, b, 1, out=out, schedule=schedule)
    assert_bit_exact(bits, cref, "fp8", out, f"int {shape} {out} {sched}")


def test_b_given_k_by_n_runs_generic_and_matches_n_by_k():
    M, N, K = 384, 320, 528
    a, b = operands("normal", M, N, K, 0, seed=61)
    assert run("fp8", M, N, K, a, b, 0, out="f32", entry="abi", allow_refusal=True) is None
    c0 = run("fp8", M, N, K, a, b, 0, out="f32", schedule=mcs.GEMM_SCHED_GENERIC)[0]
    cref, sabs = oracle.gemm(a, b, "fp8", 0)
    assert_within_tolerance(c0, cref, sabs, "fp8 B K x N", out="f32")
    c1 = run("fp8", M, N, K, a, np.ascontiguousarray(b.T), 1, out="f32")[0]
    assert_within_tolerance(c1, cref, sabs, "fp8 B N x K", out="f32")


def test_fp8_equals_fp16_on_the_same_values_in_the_integer_regime():
    """Every E4M3 value is exactly an FP16 value: the FP8 kernel and the FP16
    kernel on the widened operands must agree bit for bit where FP32
    accumulation is exact."""
    M, N, K = 512, 768, 512
    a, b = operands("int5", M, N, K, 1, seed=77)
    a16 = si.to_bits(oracle.decode(a, "fp8"), "f16")
    b16 = si.to_bits(oracle.decode(b, "fp8"), "f16")
    c8 = run("fp8", M, N, K, a, b, 1, out="f32")[1]
    c16 = run("f16", M, N, K, a16, b16, 1, out="f32")[1]
    assert np.array_equal(c8, c16)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_interleaved_matches_pipelined_bitwise(out):
    for (M, N, K) in [(1024, 768, 2048), (300, 520, 208), (513, 264, 1008)]:
        a, b = operands("normal", M, N, K, 1, seed=M + K)
        p = run("fp8", M, N, K, a, b, 1, out=out, schedule=mcs.GEMM_SCHED_PIPELINED)[1]
        i = run("fp8", M, N, K, a, b, 1, out=out, schedule=mcs.GEMM_SCHED_INTERLEAVED)[1]
        assert np.array_equal(p, i), (M, N, K)
        t = run("fp8", M, N, K, a, b, 1, out=out, schedule=mcs.GEMM_SCHED_TILE128)[1]
        assert np.array_equal(p, t), (M, N, K)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
def test_fp8_subnormal_operands(sched, out):
    """E4M3 subnormal operands (m * 2^-9, m = 1 .. 7) enter the products at
    their value: the sums are exact in FP32 and in BF16, so every element must
    match the oracle bit for bit."""
    M, N, K = 256, 264, 128
    a = fp8_subnormal_operand(M, K)
    assert ((a & 0x78) == 0).sum() > M and (a & 0x07).any()             # subnormal patterns present
    one = np.full((N, K), 0x38, np.uint8)                              # B = 1.0, given N x K
    cref = oracle.gemm(a, one, "fp8", 1, with_sabs=False)
    schedule = mcs.GEMM_SCHED_GENERIC if sched == "generic" else SCHEDS[sched]
    _, bits = run("fp8", M, N, K, a, one, 1, out=out, schedule=schedule)
    assert_bit_exact(bits, cref, "fp8", out, f"FP8 subnormals out={out} {sched}")


def test_nan_operand_propagates():
    M, N, K = 256, 256, 256
    a, b = operands("normal", M, N, K, 1, seed=5)
    a[7, 100] = FP8_NAN                     # row 7 of C depends on it at every column
    b[9, 3] = FP8_NAN | 0x80                # column 9 of C depends on it at every row
    c = run("fp8", M, N, K, a, b, 1, out="f32")[0]
    assert np.isnan(c[7, :]).all() and np.isnan(c[:, 9]).all()
    c[7, :] = 0
    c[:, 9] = 0
    assert np.isfinite(c).all()


def test_misaligned_operand_is_refused_and_runs_on_request_in_the_plain_kernel():
    M, N, K = 100, 70, 64
    a, b = operands("normal", M, N, K, 1, seed=17)
    cref, sabs = oracle.gemm(a, b, "fp8", 1, K=K, N=N)
    # A starts 1 byte into its buffer: gemm_fp8 says GEMM_EALIGN and launches nothing
    assert run("fp8", M, N, K, a, b, 1, out="bf16", a_offset=1, entry="abi", allow_refusal=True) is None
    c, _ = run("fp8", M, N, K, a, b, 1, out="bf16", a_offset=1, schedule=mcs.GEMM_SCHED_GENERIC)
    assert_within_tolerance(c, cref, sabs, "misaligned A", out="bf16")


def test_fp8_kernels_have_no_spills():
    for out in (mcs.GEMM_OUT_BF16, mcs.GEMM_OUT_F32):
        for sched, threads in ((mcs.GEMM_SCHED_PIPELINED, 512), (mcs.GEMM_SCHED_INTERLEAVED, 256),
                               (mcs.GEMM_SCHED_TILE128, 256)):
            info = mcs.gemm_kernel_info(mcs.GEMM_DTYPE_FP8_E4M3, 1, out, sched)
            assert info["local_bytes"] == 0, info
            assert info["shared_bytes"] == 128 * 1024, info
            assert info["block_threads"] == threads and info["tile_k"] == 128
