"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle (built on the CPU into a temporary directory) fails at least one pin."""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")

# (name, exact text in gemm_oracle.c, replacement)
MUTANTS = [
    ("dropped_last_term", "double p = arow[k] * bcol[k];",
     "double p = (k == jb->K - 1) ? 0.0 : arow[k] * bcol[k];"),
    ("transposed_B_operand", "bt[j * K + k] = load(elem, B, trans_b ? j * ldb + k : k * ldb + j);",
     "bt[j * K + k] = load(elem, B, trans_b ? k * ldb + j : j * ldb + k);"),
    ("ignores_lda_padding", "arow[k] = load(jb->elem, jb->A, i * jb->lda + k);",
     "arow[k] = load(jb->elem, jb->A, i * jb->K + k);"),
    ("f16_exponent_bias_off_by_one", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);"),
    ("bf16_sign_dropped", "        v = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) * 2^(e-127) */\n    return sign ? -v : v;",
     "        v = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) * 2^(e-127) */\n    return v;"),
    ("ties_away_from_zero", "if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))",
     "if (rem >= 0.5)"),
    ("sabs_without_abs", "sa += fabs(p);", "sa += p;"),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("points_wrong_row", "double a = load(elem, A, i * lda + k);", "double a = load(elem, A, j * lda + k);"),
    ("fp8_exponent_bias_off_by_one", "v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 11);"),
    ("fp8_top_binade_as_nan", "else if (e == 15 && f == 7)", "else if (e == 15)"),
    ("fp8_read_as_two_bytes", "if (elem == 2)\n        return oracle_fp8e4m3_to_f64(((const uint8_t *)p)[idx]);",
     "if (elem == 2)\n        return oracle_fp8e4m3_to_f64(((const uint8_t *)p)[2 * idx]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mpath), out=str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(lib)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            failed.append(check.__name__)
        except (ValueError, TypeError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"
