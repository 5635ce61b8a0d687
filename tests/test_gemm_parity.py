"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: every element within |C - Cref| <= 2e-3 * Sabs + 2^-10 * |Cref|, and
bit-exact (round-to-nearest-even of the exact value) for integer operands in
[-2, 2] with K <= 512, where FP32 accumulation is exact in any order.
"""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import (assert_bit_exact, assert_within_tolerance, bf16_subnormal_operand, overflow_operand,
                             run, subnormal_operand, upload)

pytestmark = pytest.mark.gpu

SCHEDS = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
          "interleaved": mcs.GEMM_SCHED_INTERLEAVED, "generic": mcs.GEMM_SCHED_GENERIC,
          "tile128": mcs.GEMM_SCHED_TILE128}


def operands(elem, dist, M, N, K, trans_b, seed, lda=None, ldb=None, nan_pad=False):
    a = si.matrix_bits(elem, dist, M, K, ld=lda, seed=seed, stream=0)
    if trans_b:
        b = si.matrix_bits(elem, dist, N, K, ld=ldb, seed=seed, stream=1)
    else:
        b = si.matrix_bits(elem, dist, K, N, ld=ldb, seed=seed, stream=1)
    if nan_pad:
        nan = 0x7E00 if elem == "f16" else 0x7FC0
        a[:, K:] = nan
        if trans_b:
            b[:, K:] = nan
        else:
            b[:, N:] = nan
    return a, b


def ref(a, b, elem, trans_b, K, N):
    return oracle.gemm(a, b, elem, trans_b, K=K, N=N)


def rup8(x):
    return (x + 7) // 8 * 8


# ---- small and ragged shapes: every element --------------------------------

SHAPES = [(256, 256, 256), (1, 1, 8), (17, 33, 8), (300, 520, 200), (513, 257, 72), (64, 640, 1000),
          (258, 130, 136)]


def pipelined_eligible(N, K, trans_b):
    """The documented conditions, given 16-byte aligned buffers and leading
    dimensions that are multiples of 8: K % 8 == 0, and an even N when B is K x N."""
    return K % 8 == 0 and (trans_b or N % 2 == 0)


@pytest.mark.parametrize("sched", ["pipelined", "in_phase", "interleaved", "tile128"])
@pytest.mark.parametrize("out", ["same", "f32"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_every_element(shape, elem, trans_b, out, sched):
    M, N, K = shape
    lda = rup8(K) + 8                      # padded rows, padding filled with NaN
    ldb = (rup8(K) + 8) if trans_b else (rup8(N) + 8)
    ldc = rup8(N) + 8                      # padded output rows must stay untouched
    a, b = operands(elem, "uniform", M, N, K, trans_b, seed=100 + M + N + K, lda=lda, ldb=ldb,
                    nan_pad=True)
    cref, sabs = ref(a, b, elem, trans_b, K, N)
    got = run(elem, M, N, K, a, b, trans_b, out=out, schedule=SCHEDS[sched], ldc=ldc, c_fill=-3.0,
              return_raw=True, allow_refusal=True)
    if got is None:
        # refused before launch, as documented (and so is AUTO, the entry points'
        # schedule); the plain kernel, asked for explicitly, must still be right
        assert not pipelined_eligible(N, K, trans_b)
        assert run(elem, M, N, K, a, b, trans_b, out=out, ldc=ldc, allow_refusal=True) is None
        got = run(elem, M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_GENERIC, ldc=ldc,
                  c_fill=-3.0, return_raw=True)
    else:
        assert pipelined_eligible(N, K, trans_b)
    c, _, full = got
    assert_within_tolerance(c, cref, sabs, f"{shape} {elem} tb={trans_b} {out} {sched}",
                            out=elem if out == "same" else "f32")
    assert np.all(full[:, N:] == -3.0)


@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_generic_kernel_every_element(elem, trans_b):
    M, N, K = 130, 77, 45                  # K % 8 != 0 and odd sizes: only the generic kernel
    a, b = operands(elem, "normal", M, N, K, trans_b, seed=3)
    cref, sabs = ref(a, b, elem, trans_b, K, N)
    # the entry points' AUTO schedule refuses the shape instead of switching kernels
    assert run(elem, M, N, K, a, b, trans_b, entry="abi", allow_refusal=True) is None
    c, _ = run(elem, M, N, K, a, b, trans_b, schedule=mcs.GEMM_SCHED_GENERIC)
    assert_within_tolerance(c, cref, sabs, "generic", out=elem)
    c, _ = run(elem, M, N, K, a, b, trans_b, schedule=mcs.GEMM_SCHED_GENERIC, out="f32")
    assert_within_tolerance(c, cref, sabs, "generic f32")


# ---- exact-integer regime: bit-exact ------------------------------------------

INT_SHAPES = [(256, 256, 32), (512, 256, 64), (256, 512, 192), (512, 512, 448), (1024, 1024, 512)]


@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128"])
@pytest.mark.parametrize("out", ["same", "f32"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("shape", INT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_regime_bit_exact(shape, elem, trans_b, out, sched):
    M, N, K = shape
    a, b = operands(elem, "int5", M, N, K, trans_b, seed=7 + K)
    cref = oracle.gemm(a, b, elem, trans_b, with_sabs=False)
    _, bits = run(elem, M, N, K, a, b, trans_b, out=out, schedule=SCHEDS[sched])
    assert_bit_exact(bits, cref, elem, out, f"int {shape} {elem} tb={trans_b} {out} {sched}")


# ---- output rounding beyond FP16's exact-integer range: round to nearest even ---

def same_sign_integer_operands(elem, M, N, K, trans_b, seed):
    """Integers in {1, 2}, with every odd row of A negated: the sums grow like
    +-2.25 K, so for K >= 1024 most of them lie past 2048, where FP16 has no
    integer spacing left and the output must round -- ties included (an odd
    sum in [2048, 4096) sits exactly between two FP16 values).  Every partial
    sum stays below 4 K <= 2^14 in magnitude, so FP32 accumulation is exact in
    any order and the only rounding is the conversion to the output type."""
    a, b = operands(elem, "int12", M, N, K, trans_b, seed=seed)
    a[1::2] |= np.uint16(0x8000)                # sign bit: odd rows of A negative
    return a, b


def rounding_cases(cref, elem):
    """Counts of results that are not representable in the output type and of
    exact ties between two neighbours (so the test can tell RNE from
    round-toward-zero and round-half-away)."""
    lo = oracle.decode(oracle.round_to(cref, elem), elem)
    inexact = lo != cref
    # a tie: the value is the midpoint of the rounded result and its neighbour
    # one spacing away (the spacing of FP16 at |x| in [2^e, 2^(e+1)) is 2^(e-10))
    mant = 10 if elem == "f16" else 7
    e = np.floor(np.log2(np.maximum(np.abs(cref), 1.0)))
    ulp = np.ldexp(1.0, (e - mant).astype(np.int64))
    tie = np.abs(cref / ulp - np.round(cref / ulp)) == 0.5
    return int(inexact.sum()), int(tie.sum())


@pytest.mark.parametrize("sched", ["pipelined", "in_phase", "interleaved", "tile128"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("K", [1024, 2048, 4096])
def test_output_rounds_to_nearest_even(K, elem, trans_b, sched):
    """The FP32 -> FP16/BF16 epilogue is round-to-nearest-even, bit for bit:
    the exact sums here need rounding (and hit ties) in the output type."""
    M, N = 512, 520
    a, b = same_sign_integer_operands(elem, M, N, K, trans_b, seed=60 + K)
    cref = oracle.gemm(a, b, elem, trans_b, with_sabs=False)
    inexact, ties = rounding_cases(cref, elem)
    assert inexact > M * N // 4 and ties > 1000, (inexact, ties)
    _, bits = run(elem, M, N, K, a, b, trans_b, schedule=SCHEDS[sched])
    assert_bit_exact(bits, cref, elem, "same", f"RNE K={K} {elem} tb={trans_b} {sched}")


@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
@pytest.mark.parametrize("trans_b", [0, 1])
def test_fp16_output_overflow_rounds_to_nearest_even(sched, trans_b):
    """The FP16 epilogue at the end of the range, bit for bit: round to
    nearest even carries 65520 and above to infinity with the sign of the sum
    and keeps 65519 and below finite; the negatives mirror it."""
    M, N, K = 256, 264, 64
    a_bits = overflow_operand(M, K)
    ones = np.full((N, K) if trans_b else (K, N), 0x3C00, np.uint16)
    cref = oracle.gemm(a_bits, ones, "f16", trans_b, with_sabs=False)
    want = oracle.decode(oracle.round_to(cref, "f16"), "f16")
    assert np.isposinf(want).any() and np.isneginf(want).any()
    assert (want == 65504.0).any() and (want == -65504.0).any() and (want == 2050.0).any()
    _, bits = run("f16", M, N, K, a_bits, ones, trans_b, schedule=SCHEDS[sched])
    assert_bit_exact(bits, cref, "f16", "same", f"FP16 overflow tb={trans_b} {sched}")


@pytest.mark.parametrize("out", ["f32", "same"])
@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
def test_fp16_subnormal_operands_and_outputs(sched, out):
    """The bottom of the FP16 range, bit for bit: subnormal operands enter the
    products at their value (FP32 output: the exact sums), and subnormal FP16
    outputs round to nearest even, ties included (2^-25 -> 0, 1.5 * 2^-24 ->
    2^-23, 1023.5 * 2^-24 -> 2^-14)."""
    M, N, K = 256, 264, 64
    a = subnormal_operand(M, K)
    half = np.full((N, K), 0x3800, np.uint16)                          # B = 0.5, given N x K
    cref = oracle.gemm(a, half, "f16", 1, with_sabs=False)
    _, bits = run("f16", M, N, K, a, half, 1, out=out, schedule=SCHEDS[sched])
    assert_bit_exact(bits, cref, "f16", out, f"FP16 subnormals out={out} {sched}")


@pytest.mark.parametrize("out", ["f32", "same"])
@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
def test_bf16_subnormal_operands_and_outputs(sched, out):
    """BF16 subnormal operands whose products and sums are FP32 denormals, bit
    for bit: FP32 output keeps the exact denormal sums, BF16 output rounds them
    to nearest even (ties included)."""
    M, N, K = 256, 264, 64
    a = bf16_subnormal_operand(M, K)
    half = np.full((N, K), 0x3F00, np.uint16)                          # B = 0.5, given N x K
    cref = oracle.gemm(a, half, "bf16", 1, with_sabs=False)
    assert (cref != 0).any() and (np.abs(cref) < 2.0 ** -126).any()
    _, bits = run("bf16", M, N, K, a, half, 1, out=out, schedule=SCHEDS[sched])
    assert_bit_exact(bits, cref, "bf16", out, f"BF16 subnormals out={out} {sched}")


@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("sched", ["pipelined", "interleaved", "tile128", "generic"])
def test_infinities_and_nan_reach_the_ieee_outputs(elem, sched):
    """Special operands through the FP32 accumulator and the epilogue, class
    for class against the oracle (IEEE binary64 products and sums): an
    infinity times positive, negative and zero partners gives +inf, -inf and
    NaN; +inf and -inf in one dot product give NaN; a NaN spoils its column.
    The other outputs are integer sums below 2048, exact and bit for bit."""
    M, N, K = 256, 264, 256
    a = si.matrix_bits(elem, "int5", M, K, seed=70, stream=0)
    b = si.matrix_bits(elem, "int5", N, K, seed=70, stream=1)                # N x K
    pinf, ninf, nan = (0x7C00, 0xFC00, 0x7E00) if elem == "f16" else (0x7F80, 0xFF80, 0x7FC0)
    a[3, 10] = pinf                     # row 3: sign of B[:, 10], NaN where it is 0
    a[5, 20], a[5, 21] = pinf, ninf     # row 5: NaN where B[:, 20] and B[:, 21] have one sign
    a[9, 40] = ninf                     # row 9: the opposite sign of B[:, 40], NaN where it is 0
    b[7, 30] = nan                      # column 7: NaN in every row
    cref = oracle.gemm(a, b, elem, 1, with_sabs=False)
    want = oracle.decode(oracle.round_to(cref, elem), elem)
    assert np.isnan(want).any() and np.isposinf(want).any() and np.isneginf(want).any()
    c, _ = run(elem, M, N, K, a, b, 1, schedule=SCHEDS[sched])
    for name, cls in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        assert np.array_equal(cls(c), cls(want)), (name, sched, np.argwhere(cls(c) != cls(want))[:3].tolist())
    fin = np.isfinite(want)
    assert np.array_equal(c[fin], want[fin]), sched


# ---- closed forms ---------------------------------------------------------------

@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_identity_gives_b(elem):
    n, m = 512, 384
    one = 0x3C00 if elem == "f16" else 0x3F80
    eye = np.zeros((n, n), np.uint16)
    eye[np.arange(n), np.arange(n)] = one
    b = si.matrix_bits(elem, "normal", n, m, seed=11, stream=1)               # K x N
    _, bits = run(elem, n, m, n, eye, b, 0)
    assert np.array_equal(oracle.decode(bits, elem), oracle.decode(b, elem))
    bt = np.ascontiguousarray(b.T)                                            # N x K
    _, bits = run(elem, n, m, n, eye, bt, 1)
    assert np.array_equal(oracle.decode(bits, elem), oracle.decode(b, elem))


@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_permutation_permutes_rows(elem):
    n, m = 256, 320
    one = 0x3C00 if elem == "f16" else 0x3F80
    perm = np.random.default_rng(5).permutation(n)
    P = np.zeros((n, n), np.uint16)
    P[np.arange(n), perm] = one
    b = si.matrix_bits(elem, "uniform", n, m, seed=12, stream=1)
    _, bits = run(elem, n, m, n, P, b, 0)
    assert np.array_equal(oracle.decode(bits, elem), oracle.decode(b[perm], elem))


@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_all_ones_gives_k(elem):
    M, N, K = 256, 512, 8192                   # 8192 = 2^13: exact in both output types
    one = 0x3C00 if elem == "f16" else 0x3F80
    a = np.full((M, K), one, np.uint16)
    b = np.full((N, K), one, np.uint16)
    c, _ = run(elem, M, N, K, a, b, 1)
    assert np.all(c == K)


def test_rank_one_integer():
    rng = np.random.default_rng(8)
    M, N, K = 300, 264, 96
    u = rng.integers(-3, 4, M).astype(np.float16)
    v = rng.integers(-3, 4, N).astype(np.float16)
    a = np.repeat(u[:, None], K, axis=1).view(np.uint16)
    b = np.repeat(v[None, :], K, axis=0).view(np.uint16)
    c, _ = run("f16", M, N, K, np.ascontiguousarray(a), np.ascontiguousarray(b), 0, out="f32")
    assert np.array_equal(c, K * np.outer(u.astype(np.float64), v.astype(np.float64)))


# ---- the workloads, in the configuration the benchmark launches: every element ----

_ORACLE = {}


def workload_reference(name):
    """(A bits, B bits, Cref, Sabs) of a workload's first input set: the full
    oracle over every output element (threaded over the host's cores; about
    20 s for the 8192^3 products on 16 threads), computed once per session."""
    if name not in _ORACLE:
        w = si.WORKLOADS[name]
        print(f"[gpu] oracle for workload {name} ({w.M}x{w.N}x{w.K})", flush=True)
        a, b = w.operands(0)
        cref, sabs = oracle.gemm(a, b, w.dtype, w.trans_b)
        _ORACLE[name] = (a, b, cref, sabs)
    return _ORACLE[name]


def sample_points(M, N, count, seed):
    rng = np.random.default_rng(seed)
    ii = list(rng.integers(0, M, count))
    jj = list(rng.integers(0, N, count))
    # tile corners and edges of the 256x256 output tiles and of the matrix
    for i in sorted({0, 127, 128, 255, 256, M // 2, M - 1} & set(range(M))):
        for j in sorted({0, 127, 128, 255, 256, N // 2, N - 1} & set(range(N))):
            ii.append(i)
            jj.append(j)
    return np.array(ii), np.array(jj)


def check_workload(name, c, what):
    """Sampled points first (a quick, independent recomputation at single
    elements), then every element against the full oracle."""
    w = si.WORKLOADS[name]
    a, b, cref, sabs = workload_reference(name)
    ii, jj = sample_points(w.M, w.N, 500, seed=w.seed)
    cp, sp = oracle.gemm_points(a, b, w.dtype, w.trans_b, ii, jj)
    assert np.array_equal(cp, cref[ii, jj]) and np.array_equal(sp, sabs[ii, jj])
    assert_within_tolerance(c[ii, jj][None, :], cp[None, :], sp[None, :], f"{what} (points)", out=w.out_type)
    assert_within_tolerance(c, cref, sabs, what, out=w.out_type)


@pytest.mark.parametrize("name", list(si.WORKLOADS))
def test_workload(name):
    """Every workload through the entry point (gemm_f16 / gemm_bf16 /
    gemm_fp8, AUTO), every element against the oracle."""
    w = si.WORKLOADS[name]
    a, b, _, _ = workload_reference(name)
    c, _ = run(w.dtype, w.M, w.N, w.K, a, b, w.trans_b, out=w.out, entry="abi")
    check_workload(name, c, name)


# ---- invariants --------------------------------------------------------------

def test_deterministic_and_schedules_agree_bitwise():
    w = si.WORKLOADS["f16_1024_bt"]
    a, b = w.operands(0)
    outs = [run("f16", w.M, w.N, w.K, a, b, 1, schedule=s)[1]
            for s in (mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_IN_PHASE)]
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("out", ["same", "f32"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_interleaved_matches_pipelined_bitwise(elem, trans_b, out):
    """Both 256x256x64 kernels give every output element the same sequence of
    MFMAs (K-steps in order, two k-slices each, same operand roles), so their
    results agree bit for bit, ragged edges and K tail included."""
    for (M, N, K) in [(1024, 768, 2048), (300, 520, 200), (513, 264, 1000)]:
        a, b = operands(elem, "normal", M, N, K, trans_b, seed=M + K)
        p = run(elem, M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_PIPELINED)[1]
        i = run(elem, M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_INTERLEAVED)[1]
        assert np.array_equal(p, i), (M, N, K)


@pytest.mark.parametrize("out", ["same", "f32"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_tile128_matches_pipelined_bitwise(elem, trans_b, out):
    """The 128x128-tile kernel runs the same MFMA sequence per output element
    as the 256x256 kernels (K-steps in order, two k-chunks each), so the
    results agree bit for bit."""
    for (M, N, K) in [(1024, 768, 2048), (300, 520, 200), (513, 264, 1000), (129, 136, 64)]:
        a, b = operands(elem, "normal", M, N, K, trans_b, seed=M + K)
        p = run(elem, M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_PIPELINED)[1]
        t = run(elem, M, N, K, a, b, trans_b, out=out, schedule=mcs.GEMM_SCHED_TILE128)[1]
        assert np.array_equal(p, t), (M, N, K)


@pytest.mark.parametrize("name", [n for n, w in si.WORKLOADS.items() if w.M * w.N * w.K <= 2 ** 31
                                  or w.M <= 512])
def test_workload_tile128(name):
    """Workloads with few 256x256 tiles through the 128x128-tile kernel:
    every element."""
    w = si.WORKLOADS[name]
    a, b, _, _ = workload_reference(name)
    c, _ = run(w.dtype, w.M, w.N, w.K, a, b, w.trans_b, out=w.out, schedule=mcs.GEMM_SCHED_TILE128)
    check_workload(name, c, f"{name} tile128")


@pytest.mark.parametrize("name", [n for n, w in si.WORKLOADS.items() if w.M * w.N >= 4096 * 4096])
def test_workload_interleaved(name):
    """Full-size workloads through the 4-wave and the 8-wave kernel: every
    element against the oracle, and the two bitwise equal."""
    w = si.WORKLOADS[name]
    a, b, _, _ = workload_reference(name)
    c, bits = run(w.dtype, w.M, w.N, w.K, a, b, w.trans_b, out=w.out, schedule=mcs.GEMM_SCHED_INTERLEAVED)
    check_workload(name, c, f"{name} interleaved")
    _, bits_p = run(w.dtype, w.M, w.N, w.K, a, b, w.trans_b, out=w.out, schedule=mcs.GEMM_SCHED_PIPELINED)
    assert np.array_equal(bits, bits_p)


def test_repeated_runs_are_bitwise_identical():
    M, N, K = 2048, 2048, 4096
    a, b = operands("bf16", "normal", M, N, K, 1, seed=99)
    first = run("bf16", M, N, K, a, b, 1)[1]
    for _ in range(5):
        assert np.array_equal(run("bf16", M, N, K, a, b, 1)[1], first)


@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_b_layouts_agree_bitwise(elem):
    M, N, K = 384, 640, 1216
    a, b = operands(elem, "uniform", M, N, K, 0, seed=41)
    c0 = run(elem, M, N, K, a, b, 0, out="f32")[1]
    c1 = run(elem, M, N, K, a, np.ascontiguousarray(b.T), 1, out="f32")[1]
    assert np.array_equal(c0, c1)


# ---- edge cases ----------------------------------------------------------------

def test_k_zero_writes_zeros():
    a = np.zeros((64, 8), np.uint16)
    b = np.zeros((64, 8), np.uint16)
    c, _ = run("f16", 64, 48, 0, a, b, 1, c_fill=7.0)
    assert np.all(c == 0)


def test_m_zero_is_a_no_op():
    torch = pytest.importorskip("torch")
    C = torch.full((4, 8), 3.0, dtype=torch.float16, device="cuda")
    st = mcs.gemm_f16(0, 8, 16, 0, 16, 0, 16, 1, C.data_ptr(), 8, 0, 0)
    torch.cuda.synchronize()
    assert st == mcs.GEMM_OK and bool((C == 3).all())


@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_output_padding_untouched(elem):
    M, N, K, ldc = 200, 100, 136, 136
    a, b = operands(elem, "uniform", M, N, K, 1, seed=13)
    c, bits, full = run(elem, M, N, K, a, b, 1, ldc=ldc, c_fill=5.0, return_raw=True)
    assert np.all(full[:, N:] == 5.0)
    cref, sabs = ref(a, b, elem, 1, K, N)
    assert_within_tolerance(c, cref, sabs, "ldc > N", out=elem)


def test_misaligned_operand_is_refused_and_runs_on_request_in_the_plain_kernel():
    M, N, K = 100, 70, 64
    a, b = operands("f16", "uniform", M, N, K, 1, seed=17)
    cref, sabs = ref(a, b, "f16", 1, K, N)
    # A starts 2 bytes into its buffer: gemm_f16 says GEMM_EALIGN and launches nothing
    assert run("f16", M, N, K, a, b, 1, a_offset=1, entry="abi", allow_refusal=True) is None
    c, _ = run("f16", M, N, K, a, b, 1, a_offset=1, schedule=mcs.GEMM_SCHED_GENERIC)
    assert_within_tolerance(c, cref, sabs, "misaligned A")


def test_kernels_have_no_spills():
    for dt in (mcs.GEMM_DTYPE_F16, mcs.GEMM_DTYPE_BF16):
        for out in (mcs.GEMM_OUT_SAME, mcs.GEMM_OUT_F32):
            for tb in (0, 1):
                for sched, threads in ((mcs.GEMM_SCHED_PIPELINED, 512), (mcs.GEMM_SCHED_INTERLEAVED, 256),
                                       (mcs.GEMM_SCHED_TILE128, 256)):
                    info = mcs.gemm_kernel_info(dt, tb, out, sched)
                    assert info["local_bytes"] == 0, info
                    assert info["shared_bytes"] == 128 * 1024, info
                    assert info["block_threads"] == threads


@pytest.mark.parametrize("elem", ["f16", "fp8"])
def test_longest_rows_the_tiled_kernels_take(elem):
    """Rows of 2^24 - 16 bytes, the most the tiled kernels accept (their 128-row
    copy windows then span ~2 GiB of 32-bit buffer offsets): M = 130, N = 24,
    K = 8,388,600 FP16 or 16,777,200 FP8 (a partial last K-step either way),
    B given N x K.  Sparse integer operands put their nonzeros in the first,
    middle and last K-steps, so every product is a short exact sum: each
    output must equal it bit for bit (and the oracle at sampled points)."""
    torch = pytest.importorskip("torch")
    M, N = 130, 24
    eb = 1 if elem == "fp8" else 2
    K = (2 ** 24 - 16) // eb
    if elem == "fp8":
        enc, dt, oe = {-2: 0xC0, -1: 0xB8, 0: 0, 1: 0x38, 2: 0x40}, np.uint8, "bf16"
    else:
        enc, dt, oe = {-2: 0xC000, -1: 0xBC00, 0: 0, 1: 0x3C00, 2: 0x4000}, np.uint16, "f16"
    a = np.zeros((M, K), dt)
    b = np.zeros((N, K), dt)
    r = np.arange(M)
    a[r, K - 1 - r] = enc[1]
    a[r, 8 * r + 3] = enc[2]
    a[r, K // 2 + r] = enc[-1]
    for j in range(N):
        b[j, K - 1 - r] = [enc[(j + x) % 5 - 2] for x in r]
        b[j, 8 * r + 3] = [enc[(j * x) % 3 - 1] for x in r]
        b[j, K // 2 + r] = [enc[(j + x) % 2] for x in r]
    cols = np.unique(np.concatenate([K - 1 - r, 8 * r + 3, K // 2 + r]))
    exact = oracle.decode(a[:, cols], elem) @ oracle.decode(b[:, cols], elem).T
    ii = np.array([0, 1, 64, 127, 128, 129, 129])
    jj = np.array([0, 23, 5, 17, 0, 23, 11])
    cpts, _ = oracle.gemm_points(a, b, elem, 1, ii, jj)
    assert np.array_equal(cpts, exact[ii, jj])
    A, _ = upload(a, elem)
    B, _ = upload(b, elem)
    del a, b
    stream = torch.cuda.current_stream().cuda_stream
    dtype = mcs.GEMM_DTYPE_FP8_E4M3 if elem == "fp8" else mcs.GEMM_DTYPE_F16
    out_type = mcs.GEMM_OUT_BF16 if elem == "fp8" else mcs.GEMM_OUT_SAME
    cdt = torch.bfloat16 if elem == "fp8" else torch.float16
    for sched in (mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_INTERLEAVED, mcs.GEMM_SCHED_TILE128):
        print(f"[gpu] longest rows {elem} M={M} N={N} K={K} sched={sched}", flush=True)
        C = torch.full((M, N), 7.0, dtype=cdt, device="cuda")
        st = mcs.gemm_ex(dtype, M, N, K, A.data_ptr(), K, B.data_ptr(), K, 1, C.data_ptr(), N, out_type, sched,
                         stream)
        assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
        torch.cuda.synchronize()
        got = oracle.decode(C.cpu().view(torch.int16).numpy().view(np.uint16), oe)
        bad = np.argwhere(got != exact)
        assert bad.size == 0, f"sched {sched}: {len(bad)} wrong, first {bad[0].tolist()}"
