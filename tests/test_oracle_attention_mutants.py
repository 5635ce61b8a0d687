"""Plausible mistakes planted in copies of the attention oracle: each must
fail at least one pin, so a pin set that passes says something."""
import importlib.util
import os
import sys

import pytest

from tests import oracle_attention_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = [
    ("no scale", "s = scale * (qr @ k.T)", "s = (qr @ k.T)"),
    ("keys shifted against values", "s = scale * (qr @ k.T)", "s = scale * (qr @ np.roll(k, 1, axis=0).T)"),
    ("values reversed", "o = p @ v\n", "o = p @ v[::-1]\n"),
    ("row sum over queries", "tot = e.sum(axis=1, keepdims=True)", "tot = e.sum(axis=0, keepdims=True)"),
    ("causal off by one", "return j <= i + (Sk - Sq)", "return j < i + (Sk - Sq)"),
    ("causal aligned top-left", "return j <= i + (Sk - Sq)", "return j <= i"),
    ("lse without the shift", "shift[:, 0] + np.log(", "np.log("),
    ("exp without the shift", "np.exp(s - shift)", "np.exp(s)"),
    ("square instead of exp", "np.exp(s - shift)", "np.square(s - shift)"),
]


def load_mutant(tmp_path, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, old
    text = text.replace(old, new).replace("from . import decode", "from oracle import decode")
    path = tmp_path / "attention_mutant.py"
    path.write_text(text)
    spec = importlib.util.spec_from_file_location(f"attention_mutant_{abs(hash(new))}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_attention_mutant_is_caught(tmp_path, name, old, new):
    mod = load_mutant(tmp_path, old, new)
    failed = []
    for check in pins.ALL:
        try:
            check(mod)
        except Exception as e:               # an AssertionError, or the mistake breaking a shape
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"no pin caught mutant {name}"
