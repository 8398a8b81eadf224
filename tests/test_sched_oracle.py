"""The scheduler oracle (oracle/sched_ref.py, oracle.b_shape) against pins
that do not restate its formulas: brute-force search for the largest batch,
the hand-worked bucket example, partition invariants, exact recovery of a
known cost model, and coefficients of variation worked by hand."""

import itertools
import math
import os
import sys
import types

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_batch(S, m_mem, m_comp, p):
    """Largest B >= 1 with B*S <= m_mem and B*S^p <= m_comp, found by trying
    every B (integer p only, so S^p is exact); 1 when no B fits."""
    best = 1
    B = 1
    while B * S <= m_mem and B * S ** p <= m_comp:
        best = B
        B += 1
    return best


def check_b_shape_is_the_largest_feasible_batch(impl):
    for S, m_mem, m_comp, p in itertools.product((1, 2, 3, 7, 16, 100, 513), (0, 5, 64, 1000),
                                                  (0, 9, 300, 10 ** 5), (1, 2, 3)):
        assert impl.b_shape(S, m_mem, m_comp, p) == brute_batch(S, m_mem, m_comp, p), (S, m_mem, m_comp, p)


def check_plan_worked_buckets(impl):
    """The mixed-length corpus of four lengths (256 x 256, 4096 x 16,
    16384 x 4, 32760 x 1) under M_mem = 65536, M_comp = 2^30, p = 2 is
    exactly one group per length, of 256, 16, 4 and 1 samples (the same
    numbers worked by hand for b_shape)."""
    lengths = [32760] + [4096] * 16 + [256] * 256 + [16384] * 4
    groups = impl.plan_groups(lengths, 65536, 2 ** 30, 2)
    assert [len(g) for g in groups] == [256, 16, 4, 1]
    assert [lengths[g[0]] for g in groups] == [256, 4096, 16384, 32760]


def check_plan_partition_invariants(impl):
    for seed in range(6):
        _plan_invariants(impl, seed)


def _plan_invariants(impl, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.choice([1, 17, 256, 300, 4096, 9000], size=int(rng.integers(0, 60))).tolist()
    m_mem, m_comp, p = int(rng.integers(1, 20000)), int(rng.integers(1, 10 ** 7)), float(rng.choice([1, 1.5, 2]))
    groups = impl.plan_groups(lengths, m_mem, m_comp, p)
    flat = sorted(i for g in groups for i in g)
    assert flat == list(range(len(lengths)))                     # every sample exactly once
    prev = (0, -1)
    for g in groups:
        S = lengths[g[0]]
        assert all(lengths[i] == S for i in g)                   # one length per group
        assert g == sorted(g)                                    # input order inside a group
        assert (S, g[0]) > prev                                  # ascending length, then input order
        prev = (S, g[0])
        if len(g) > 1:                                           # both constraints hold
            assert len(g) * S <= m_mem and len(g) * S ** p <= m_comp
    for S in set(lengths):                                       # full groups except the last
        sizes = [len(g) for g in groups if lengths[g[0]] == S]
        full = brute_batch(S, m_mem, m_comp, int(p)) if float(p).is_integer() else sizes[0]
        assert all(n == full for n in sizes[:-1]) and 1 <= sizes[-1] <= full


def check_plan_rejects_bad_lengths(impl):
    with pytest.raises(ValueError):
        impl.plan_groups([4, 0], 10, 10, 2)


def check_cost_fit_recovers_a_known_model(impl):
    """Noise-free timings of a known model are fitted back exactly."""
    Bs, Ss = np.meshgrid([1, 2, 4, 8], [256, 1024, 4096, 16384])
    B, S = Bs.ravel().astype(float), Ss.ravel().astype(float)
    for a, b, p in ((35.0, 2e-6, 2.0), (10.0, 3e-4, 1.0), (5.0, 7e-5, 1.4)):
        t = a + b * B * S ** p
        fa, fb, fp, rss = impl.fit_cost_model(B, S, t)
        assert abs(fp - p) < 1e-6 and abs(fa - a) < 1e-6 * max(1.0, a) and abs(fb / b - 1) < 1e-5
        assert rss < 1e-12 * float(np.sum(t * t))


def check_cost_fit_is_a_least_squares_minimum(impl):
    """With noise, no nearby (a, b, p) has a smaller squared residual."""
    rng = np.random.default_rng(3)
    Bs, Ss = np.meshgrid([1, 2, 3, 4, 6, 8], [512, 1024, 2048, 4096, 8192])
    B, S = Bs.ravel().astype(float), Ss.ravel().astype(float)
    t = (20.0 + 4e-6 * B * S ** 1.8) * (1 + 0.02 * rng.standard_normal(B.size))
    fa, fb, fp, rss = impl.fit_cost_model(B, S, t)
    # the model and residual are evaluated here, independently of impl
    assert abs(rss - float(np.sum((fa + fb * B * S ** fp - t) ** 2))) <= 1e-9 * rss
    for da, db, dp in itertools.product((-1e-3, 0, 1e-3), repeat=3):
        v = (fa * (1 + da), fb * (1 + db), fp + dp)
        assert float(np.sum((v[0] + v[1] * B * S ** v[2] - t) ** 2)) >= rss * (1 - 1e-12)


def check_load_cv_worked(impl):
    assert impl.load_cv([3.0, 3.0, 3.0]) == 0.0
    assert impl.load_cv([1.0, 3.0]) == 0.5                        # std 1, mean 2
    assert math.isclose(impl.load_cv([1.0, 2.0, 3.0, 4.0]), math.sqrt(1.25) / 2.5, rel_tol=1e-15)
    with pytest.raises(ValueError):
        impl.load_cv([])


def check_cost_model_form(impl):
    """The model a + b*B*S^p at hand-computed points."""
    assert impl.cost_model(2.0, 4.0, 1.0, 3.0, 2.0) == 1.0 + 3.0 * 2.0 * 16.0
    assert impl.cost_model(1.0, 9.0, 0.0, 1.0, 0.5) == 3.0


CHECKS = [check_b_shape_is_the_largest_feasible_batch, check_plan_worked_buckets,
          check_plan_partition_invariants, check_plan_rejects_bad_lengths,
          check_cost_fit_recovers_a_known_model, check_cost_fit_is_a_least_squares_minimum,
          check_load_cv_worked, check_cost_model_form]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_sched_oracle_pin(check):
    check(oracle)


# Mutation tests: each plants one plausible mistake in a copy of the
# scheduler oracle's source and requires at least one pin to fail on it.
SCHED_SRC = os.path.join(ROOT, "oracle", "sched_ref.py")
MUTANTS = [
    ("groups by descending length", "for S in sorted(set(lengths)):", "for S in sorted(set(lengths), reverse=True):"),
    ("group one sample short", "members[start:start + size]", "members[start:start + size - 1] or members[start:start + 1]"),
    ("group size from S not B_shape", "size = b_shape(S, m_mem, m_comp, p)", "size = max(1, m_mem // S)"),
    ("model without the batch", "return a + b * B * S ** p", "return a + b * S ** p"),
    ("fit model without the batch", "return (a + b * B * S ** p - t) / scale_t", "return (a + b * S ** p - t) / scale_t"),
    ("fit p fixed at the first start", "x0=[a0, b0, p0], bounds=([-np.inf, -np.inf, p_lo], [np.inf, np.inf, p_hi])",
     "x0=[a0, b0, p0], bounds=([-np.inf, -np.inf, p0], [np.inf, np.inf, p0 + 1e-12])"),
    ("cv with the sample deviation", "var = ((x - mean) ** 2).sum() / x.size", "var = ((x - mean) ** 2).sum() / max(1, x.size - 1)"),
    ("cv over the variance", "return float(np.sqrt(var) / mean)", "return float(var / mean)"),
]


def _load_sched_mutant(name, old, new):
    src = open(SCHED_SRC).read()
    assert src.count(old) >= 1, f"mutant {name!r}: pattern not found"
    src = src.replace(old, new).replace("from .adaln_ref import b_shape", "from oracle import b_shape")
    mod = types.ModuleType(f"sched_mutant_{abs(hash(name))}")
    sys.modules[mod.__name__] = mod
    try:
        exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        sys.modules.pop(mod.__name__, None)
    mod.b_shape = oracle.b_shape
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_sched_pins_catch_mutant(name, old, new):
    mod = _load_sched_mutant(name, old, new)
    failed = []
    for check in CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, TypeError, IndexError) as e:
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"no pin caught the mutant {name!r}"
