"""Checks that tie the CPU oracle to facts outside itself.

Each check takes an ``oracle.Oracle`` and raises AssertionError on failure, so
the same checks run against the real oracle (tests/test_oracle_pins.py) and
against deliberately broken builds of it (tests/test_oracle_mutants.py).

Sources of truth used here, none of which is the oracle's own code:
  * numpy's binary16 <-> float64 conversions and torch's bfloat16 and
    float8_e4m3fn widening;
  * exact rational arithmetic (fractions.Fraction);
  * numpy.matmul in float64 and int64;
  * closed forms of special matrices (identity, permutation, all-ones,
    rank-1) and hand-worked round-to-nearest-even ties.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from seeded_inputs import matrix_bits

F16_NAN = 0x7E00


# ---------------------------------------------------------------- decoders

def check_f16_decode_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_bf16_decode_exhaustive(o):
    import torch

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_fp8_decode_exhaustive(o):
    import torch

    bits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    got = o.decode(bits, "fp8")
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2                                 # 0x7F and 0xFF only: no infinities
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_decode_worked_values(o):
    # IEEE 754 binary16 / bfloat16 encodings of a few textbook values.
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24,
           0x3555: 0.333251953125, 0x8000: -0.0}
    bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x4380: 256.0, 0x4382: 260.0, 0x0080: 2.0 ** -126,
            0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    # FP8 E4M3 (bias 7, 3 fraction bits, no infinities): 1.0, -2.0, the
    # largest value 448 = 1.75 * 2^8, the smallest normal 2^-6, the smallest
    # subnormal 2^-9, 13/16 and -0.
    fp8 = {0x38: 1.0, 0xC0: -2.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x35: 0.8125,
           0x80: -0.0}
    for elem, table in (("f16", f16), ("bf16", bf16), ("fp8", fp8)):
        k = np.array(list(table), dtype=np.uint8 if elem == "fp8" else np.uint16)
        got = o.decode(k, elem)
        assert np.array_equal(got, np.array(list(table.values())))
        assert np.array_equal(np.signbit(got), np.signbit(np.array(list(table.values()))))


# ---------------------------------------------------------------- encoders

def _f16_grid():
    """All finite non-negative binary16 values, ascending."""
    b = np.arange(0, 0x7C00, dtype=np.uint16)
    return b, b.view(np.float16).astype(np.float64)


def check_f16_round_vs_numpy(o):
    rng = np.random.default_rng(7)
    b, v = _f16_grid()
    mids = (v[:-1] + v[1:]) / 2                      # exact ties in binary64
    near = np.concatenate([mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40)])
    rand = np.concatenate([rng.uniform(-1, 1, 20000), rng.normal(0, 300, 20000),
                           rng.uniform(-1e-6, 1e-6, 5000), rng.uniform(6.5e4, 6.6e4, 2000),
                           np.array([65519.0, 65520.0, 65535.0, 1e300, -1e300, 0.0, -0.0])])
    for x in (v, mids, -mids, near, rand):
        got = o.round_to(x, "f16")
        ref = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref)


def check_round_worked_ties(o):
    # binary16: 2048..4096 has spacing 2, so odd integers are ties.
    assert list(o.round_to(np.array([2049.0, 2051.0, 2053.0]), "f16").view(np.float16)) == [2048, 2052, 2052]
    # bfloat16: 256..512 has spacing 2 (8 significant bits).
    r = o.round_to(np.array([257.0, 259.0, 261.0, 257.0000001, -259.0]), "bf16")
    assert [int(x) for x in r] == [0x4380, 0x4382, 0x4382, 0x4381, 0xC382]
    # overflow / max finite
    assert int(o.round_to(np.array([65519.9]), "f16")[0]) == 0x7BFF
    assert int(o.round_to(np.array([65520.0]), "f16")[0]) == 0x7C00


def check_bf16_round_ties(o):
    """Midpoints between neighbouring bfloat16 values go to the one with an even last bit."""
    import torch

    b = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    mids = (v[:-1] + v[1:]) / 2
    got = o.round_to(mids, "bf16")
    lo = b[:-1]
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # off-tie values round to the nearer neighbour; compare with torch's
    # float32 -> bfloat16 (round to nearest even), exact here because every
    # test value is a binary32 value.
    x = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)]).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.round_to(x.astype(np.float64), "bf16"), ref)


# ---------------------------------------------------------------- product

def _decode_ref(bits, elem):
    """Independent widening (numpy / torch), used only by the checks."""
    if elem == "f16":
        return bits.view(np.float16).astype(np.float64)
    import torch
    if elem == "fp8":
        return torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def _bhat(b, trans_b, K, N):
    """b(k, j) as a K x N float64 matrix."""
    return b[:N, :K].T if trans_b else b[:K, :N]


def check_bruteforce_fraction(o):
    rng_shapes = [(1, 1, 1), (2, 3, 7), (3, 7, 2), (7, 2, 33), (16, 3, 16), (3, 33, 16), (33, 16, 3)]
    for elem in ("f16", "bf16", "fp8"):
        for trans_b in (0, 1):
            for s, (M, N, K) in enumerate(rng_shapes):
                a = matrix_bits(elem, "uniform", M, K, ld=K + 3, seed=11 + s, stream=0)
                b = (matrix_bits(elem, "uniform", N, K, ld=K + 1, seed=11 + s, stream=1) if trans_b
                     else matrix_bits(elem, "uniform", K, N, seed=11 + s, stream=1))
                C, S = o.gemm(a, b, elem, trans_b, K=K, N=N)
                av, bv = _decode_ref(a, elem), _bhat(_decode_ref(b, elem), trans_b, K, N)
                for i in range(M):
                    for j in range(N):
                        terms = [Fraction(float(av[i, k])) * Fraction(float(bv[k, j])) for k in range(K)]
                        exact = sum(terms, Fraction(0))
                        sab = sum((abs(t) for t in terms), Fraction(0))
                        bound = K * 2.0 ** -53 * float(sab)
                        assert abs(Fraction(C[i, j]) - exact) <= Fraction(bound), (elem, trans_b, M, N, K, i, j)
                        assert abs(Fraction(S[i, j]) - sab) <= Fraction(bound)


def check_numpy_matmul(o):
    for elem in ("f16", "bf16", "fp8"):
        for trans_b in (0, 1):
            M, N, K = 67, 45, 301
            a = matrix_bits(elem, "normal", M, K, ld=K + 11, seed=5, stream=0)
            if trans_b:
                b = matrix_bits(elem, "normal", N, K, ld=K + 5, seed=5, stream=1)
            else:
                b = matrix_bits(elem, "normal", K, N + 9, seed=5, stream=1)
            C, S = o.gemm(a, b, elem, trans_b, K=K, N=N)
            av = _decode_ref(a, elem)[:, :K]
            bv = _bhat(_decode_ref(b, elem), trans_b, K, N)
            ref = av @ bv
            sref = np.abs(av) @ np.abs(bv)
            assert np.all(np.abs(C - ref) <= 1e-12 * sref)
            assert np.all(np.abs(S - sref) <= 1e-12 * sref)


def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def check_identity_and_permutation(o):
    rng = np.random.default_rng(3)
    n, m = 24, 19
    eye = _f16(np.eye(n))
    b = matrix_bits("f16", "uniform", n, m, seed=3, stream=1)           # K x N
    C = o.gemm(eye, b, "f16", 0, with_sabs=False)
    assert np.array_equal(o.round_to(C, "f16"), b)                        # I.B = B
    bt = matrix_bits("f16", "uniform", m, n, seed=3, stream=2)           # N x K
    C = o.gemm(eye, bt, "f16", 1, with_sabs=False)
    assert np.array_equal(o.round_to(C, "f16"), bt.T)                     # I.(Bt)^T = B
    a = matrix_bits("f16", "uniform", m, n, seed=3, stream=3)            # M x K
    C = o.gemm(a, eye, "f16", 0, with_sabs=False)
    assert np.array_equal(o.round_to(C, "f16"), a)                        # A.I = A
    perm = rng.permutation(n)
    P = np.zeros((n, n)); P[np.arange(n), perm] = 1.0                     # (P.B)[i] = B[perm[i]]
    C = o.gemm(_f16(P), b, "f16", 0, with_sabs=False)
    assert np.array_equal(o.round_to(C, "f16"), b[perm])
    Q = np.zeros((m, m)); Q[np.arange(m), rng.permutation(m)] = 1.0
    sigma = Q.argmax(axis=1)                                              # (B.Q)[:, sigma[i]] = B[:, i]
    C = o.gemm(b, _f16(Q), "f16", 0, with_sabs=False)
    want = np.empty_like(b); want[:, sigma] = b
    assert np.array_equal(o.round_to(C, "f16"), want)


def check_all_ones(o):
    for elem, K in (("f16", 5), ("f16", 2048), ("bf16", 256), ("bf16", 300)):
        one = 0x3C00 if elem == "f16" else 0x3F80
        a = np.full((3, K), one, dtype=np.uint16)
        b = np.full((K, 4), one, dtype=np.uint16)
        C, S = o.gemm(a, b, elem, 0)
        assert np.all(C == K) and np.all(S == K)
    # bfloat16 has 8 significant bits: 300 rounds to 300 (=0x4396), 257 to 256
    assert int(o.round_to(np.array([300.0]), "bf16")[0]) == 0x4396


def check_rank_one(o):
    rng = np.random.default_rng(9)
    u = rng.integers(-3, 4, 13).astype(np.float64)
    v = rng.integers(-3, 4, 10).astype(np.float64)
    for K in (1, 7, 64):
        a = _f16(np.repeat(u[:, None], K, axis=1))                      # A = u 1^T
        b = _f16(np.repeat(v[None, :], K, axis=0))                      # B = 1 v^T
        C = o.gemm(a, b, "f16", 0, with_sabs=False)
        assert np.array_equal(C, K * np.outer(u, v))
    x = matrix_bits("f16", "uniform", 9, 1, seed=4, stream=0)
    y = matrix_bits("f16", "uniform", 1, 8, seed=4, stream=1)
    C = o.gemm(x, y, "f16", 0, with_sabs=False)
    assert np.array_equal(C, np.outer(x.view(np.float16).astype(np.float64),
                                      y.view(np.float16).astype(np.float64)))


def check_integer_regime(o):
    for elem in ("f16", "bf16", "fp8"):
        for trans_b in (0, 1):
            M, N, K = 40, 33, 512
            a = matrix_bits(elem, "int5", M, K, seed=21, stream=0)
            b = matrix_bits(elem, "int5", N, K, seed=21, stream=1) if trans_b else \
                matrix_bits(elem, "int5", K, N, seed=21, stream=1)
            C, S = o.gemm(a, b, elem, trans_b)
            ai = _decode_ref(a, elem).astype(np.int64)
            bi = _bhat(_decode_ref(b, elem), trans_b, K, N).astype(np.int64)
            assert np.array_equal(C, (ai @ bi).astype(np.float64))
            assert np.array_equal(S, (np.abs(ai) @ np.abs(bi)).astype(np.float64))


def check_layouts_agree(o):
    """trans_b=0 with B and trans_b=1 with B^T are the same product, term for term."""
    a = matrix_bits("bf16", "normal", 21, 77, seed=8, stream=0)
    b = matrix_bits("bf16", "normal", 77, 30, seed=8, stream=1)
    C0 = o.gemm(a, b, "bf16", 0, with_sabs=False)
    C1 = o.gemm(a, np.ascontiguousarray(b.T), "bf16", 1, with_sabs=False)
    assert np.array_equal(C0, C1)
    ii = np.array([0, 20, 5, 13]); jj = np.array([0, 29, 17, 3])
    Cp, _ = o.gemm_points(a, b, "bf16", 0, ii, jj)
    assert np.array_equal(Cp, C0[ii, jj])


ALL_CHECKS = [check_f16_decode_exhaustive, check_bf16_decode_exhaustive, check_fp8_decode_exhaustive,
              check_decode_worked_values,
              check_f16_round_vs_numpy, check_round_worked_ties, check_bf16_round_ties,
              check_bruteforce_fraction, check_numpy_matmul, check_identity_and_permutation,
              check_all_ones, check_rank_one, check_integer_regime, check_layouts_agree]
