"""Mutation tests for the oracle's pins.

Each case plants one plausible mistake (a dropped term, a wrong sign or
index, a swapped operand, a wrong divisor) into a copy of the oracle's source,
loads that copy as a separate module on the CPU, and requires at least one pin
to fail on it.  The real oracle is never modified.
"""

import os
import sys
import types

import pytest

from oracle_pins import CHECKS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC_PATH = os.path.join(ROOT, "oracle", "adaln_ref.py")

MUTANTS = [
    ("mean divisor", "mean = x.sum(axis=-1) / D ", "mean = x.sum(axis=-1) / (D + 1) "),
    ("unbiased variance", "var = (dev * dev).sum(axis=-1) / D ", "var = (dev * dev).sum(axis=-1) / (D - 1) "),
    ("eps outside the root", "rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / (np.sqrt(var) + eps)"),
    ("eps dropped", "rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / np.sqrt(var)"),
    ("xhat sign (fwd)", "xhat = (xr - mean[:, None]) * rstd[:, None]", "xhat = (mean[:, None] - xr) * rstd[:, None]"),
    ("modulation without 1+", "y = xhat * (1.0 + scale[b]) + shift[b]", "y = xhat * scale[b] + shift[b]"),
    ("shift and scale swapped", "y = xhat * (1.0 + scale[b]) + shift[b]", "y = xhat * (1.0 + shift[b]) + scale[b]"),
    ("sample lookup off by one", 'side="right") - 1', 'side="left") - 1'),
    ("g without modulation", "g = dy_r * (1.0 + scale_b)", "g = dy_r"),
    ("dx drops a", "(g - a[:, None] - xhat * c[:, None])", "(g - xhat * c[:, None])"),
    ("dx drops xhat*c", "(g - a[:, None] - xhat * c[:, None])", "(g - a[:, None])"),
    ("dx sign of xhat*c", "(g - a[:, None] - xhat * c[:, None])", "(g - a[:, None] + xhat * c[:, None])"),
    ("dx without rstd", "dx = rstd[:, None] * (g", "dx = (g"),
    ("c from x not xhat", "c = (g * xhat).sum(axis=-1) / D", "c = (g * x_r).sum(axis=-1) / D"),
    ("c transposed reduction", "c = (g * xhat).sum(axis=-1) / D", "c = (g * xhat).sum(axis=0).sum() / D + 0 * xhat[:, 0]"),
    ("dshift mean not sum", "dshift[i] = dy[lo:hi].sum(axis=0)", "dshift[i] = dy[lo:hi].mean(axis=0)"),
    ("dscale from x not xhat", "dscale[i] = (dy[lo:hi] * xhat).sum(axis=0)", "dscale[i] = (dy[lo:hi] * xb).sum(axis=0)"),
    ("dscale with modulation", "dscale[i] = (dy[lo:hi] * xhat).sum(axis=0)",
     "dscale[i] = (dy[lo:hi] * (1.0 + scale[b]) * xhat).sum(axis=0)"),
    ("sample range drops last row", "lo, hi = int(off[b]), int(off[b + 1])", "lo, hi = int(off[b]), max(int(off[b]), int(off[b + 1]) - 1)"),
    ("bf16 decode shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("bucket rule max not min", "max(1, min(by_mem, by_comp))", "max(1, max(by_mem, by_comp))"),
    ("bucket rule floor lost", "by_mem = m_mem // S", "by_mem = -(-m_mem // S)"),
]


def _load_mutant(name, old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutant {name!r}: pattern not found in the oracle"
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{abs(hash(name))}")
    mod.__file__ = SRC_PATH
    sys.modules[mod.__name__] = mod
    try:
        exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        sys.modules.pop(mod.__name__, None)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    mod = _load_mutant(name, old, new)
    failed = []
    for check in CHECKS:
        try:
            check(mod)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
