"""The CPU oracle against its pins (decoders, encoders, brute force, closed forms)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.default())


def test_thread_count_does_not_change_results():
    import numpy as np
    from seeded_inputs import matrix_bits
    a = matrix_bits("f16", "uniform", 37, 130, seed=2, stream=0)
    b = matrix_bits("f16", "uniform", 130, 29, seed=2, stream=1)
    c1 = oracle.gemm(a, b, "f16", 0, nthreads=1, with_sabs=False)
    c7 = oracle.gemm(a, b, "f16", 0, nthreads=7, with_sabs=False)
    assert np.array_equal(c1, c7)
    part = oracle.gemm(a, b, "f16", 0, rows=(5, 20), with_sabs=False)
    assert np.array_equal(part, c1[5:20])


def test_tolerance_formula():
    import numpy as np
    cref = np.array([1.0, -2.0, 100.0])
    sabs = np.array([1.0, 10.0, 100.0])
    lim = 2e-3 * sabs + 2.0 ** -10 * np.abs(cref)
    assert oracle.within_tolerance(cref + 0.999 * lim, cref, sabs).all()
    assert not oracle.within_tolerance(cref + 1.001 * lim, cref, sabs).any()


def test_bf16_output_bound_admits_exactly_the_rounding():
    """For a BF16 output the bound grows by half a BF16 spacing: a correctly
    rounded value passes, the neighbour beyond it fails."""
    import numpy as np
    cref = np.array([-1.027321845293045, 300.7, 1e-3])
    sabs = np.abs(cref)                       # same-sign sums: Sabs = |Cref|
    r = oracle.decode(oracle.round_to(cref, "bf16"), "bf16")
    assert oracle.within_tolerance(r, cref, sabs, out="bf16").all()
    assert not oracle.within_tolerance(r, cref, sabs, out="f16")[0]
    step = 2 * oracle.bf16_half_ulp(cref)
    far = r + np.sign(r - cref) * step        # next bfloat16 away from Cref
    assert not oracle.within_tolerance(far, cref, sabs, out="bf16").any()


def test_rejects_bad_arguments():
    import numpy as np
    a = np.zeros((2, 3), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(a, a, "f16", 0, rows=(0, 5))
    with pytest.raises(TypeError):
        oracle.gemm(a.astype(np.float32), a, "f16", 1)
