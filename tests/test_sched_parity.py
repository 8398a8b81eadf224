"""The library's host scheduler (include/adaln_sched.h) against the oracle.

Batch sizes and groupings are integers: bit-exact.  The cost fit is a
different algorithm from the oracle's (closed-form (a, b) with a search over
p, against a trust-region solve over all three): both must reach the same
least-squares minimum.  The coefficient of variation agrees to rounding.
These are host functions, so the tests run on the CPU.
"""

import itertools
import math

import numpy as np
import pytest

import diffusion_transformer_adaln_amd as adaln
import oracle


def test_batch_size_matches_oracle():
    Ss = (1, 2, 3, 7, 255, 256, 4096, 16384, 32760, 70000, 10 ** 6)
    mems = (0, 1, 65536, 10 ** 9, 2 ** 62)
    comps = (0, 1, 2 ** 30, 10 ** 12, 2 ** 62)
    ps = (1, 2, 3, 4, 0.5, 1.5, 1.8, 2.5, 3.3)
    for S, m_mem, m_comp, p in itertools.product(Ss, mems, comps, ps):
        want = oracle.b_shape(S, m_mem, m_comp, p)
        assert adaln.adaln_sched_batch_size(S, m_mem, m_comp, p) == want, (S, m_mem, m_comp, p)


def test_batch_size_rejects_bad_arguments():
    for args in ((0, 10, 10, 2.0), (5, -1, 10, 2.0), (5, 10, -1, 2.0), (5, 10, 10, 0.0), (5, 10, 10, float("nan")),
                 (5, 10, 10, float("inf"))):
        with pytest.raises(adaln.AdaLNError):
            adaln.adaln_sched_batch_size(*args)


def _groups(group_of, n_groups):
    out = [[] for _ in range(n_groups)]
    for i, g in enumerate(group_of):
        out[g].append(i)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_plan_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(0, 400))
    lengths = rng.choice([1, 64, 256, 1000, 4096, 16384, 32760], size=n)
    m_mem = int(rng.choice([1, 4096, 65536, 10 ** 6]))
    m_comp = int(rng.choice([1, 2 ** 20, 2 ** 30, 10 ** 12]))
    p = float(rng.choice([1.0, 1.5, 2.0, 2.2]))
    group_of, n_groups = adaln.adaln_sched_plan(lengths, m_mem, m_comp, p)
    assert _groups(group_of, n_groups) == oracle.plan_groups(lengths.tolist(), m_mem, m_comp, p)


def test_plan_worked_buckets_and_edges():
    lengths = [32760] + [4096] * 16 + [256] * 256 + [16384] * 4
    group_of, n = adaln.adaln_sched_plan(lengths, 65536, 2 ** 30, 2)
    assert n == 4 and [int((group_of == g).sum()) for g in range(n)] == [256, 16, 4, 1]
    assert adaln.adaln_sched_plan([], 10, 10, 2.0)[1] == 0
    g, n = adaln.adaln_sched_plan([7], 0, 0, 2.0)                 # budgets too small: still one sample
    assert n == 1 and g.tolist() == [0]
    with pytest.raises(adaln.AdaLNError):
        adaln.adaln_sched_plan([5, 0, 3], 10, 10, 2.0)


def _grid():
    Bs, Ss = np.meshgrid([1, 2, 3, 4, 6, 8], [256, 512, 1024, 2048, 4096, 8192, 16384])
    return Bs.ravel().astype(float), Ss.ravel().astype(float)


@pytest.mark.parametrize("a,b,p", [(35.0, 2e-6, 2.0), (10.0, 3e-4, 1.0), (5.0, 7e-5, 1.4), (0.0, 1e-9, 2.7)])
def test_cost_fit_noise_free(a, b, p):
    B, S = _grid()
    t = a + b * B * S ** p
    fa, fb, fp, rss = adaln.adaln_cost_fit(B, S, t)
    assert abs(fp - p) < 1e-7
    assert abs(fa - a) < 1e-6 * max(1.0, abs(a)) + 1e-9 * float(t.max())
    assert abs(fb / b - 1) < 1e-6
    assert rss < 1e-14 * float(np.sum(t * t))


@pytest.mark.parametrize("seed", range(5))
def test_cost_fit_matches_oracle_with_noise(seed):
    rng = np.random.default_rng(seed)
    B, S = _grid()
    p_true = float(rng.uniform(1.0, 2.2))
    t = (float(rng.uniform(5, 50)) + float(rng.uniform(1e-7, 1e-5)) * B * S ** p_true)
    t = t * (1 + 0.03 * rng.standard_normal(t.size))
    fa, fb, fp, rss = adaln.adaln_cost_fit(B, S, t)
    oa, ob, op, orss = oracle.fit_cost_model(B, S, t)
    # the same minimum: equal residuals, and parameters within the flatness of the optimum
    assert rss <= orss * (1 + 1e-9)
    assert abs(rss - orss) <= 1e-7 * orss
    assert abs(fp - op) < 1e-4 and abs(fb / ob - 1) < 1e-3 and abs(fa - oa) <= 1e-3 * float(np.abs(t).max())
    # the reported rss is the residual of the reported parameters
    assert abs(rss - float(np.sum((fa + fb * B * S ** fp - t) ** 2))) <= 1e-9 * rss


def test_cost_fit_rejects_bad_input():
    B, S = _grid()
    t = 1.0 + B * S
    for args in ((B[:2], S[:2], t[:2]), (np.ones(5), np.full(5, 7.0), np.arange(5.0)),      # too few; no slope
                 (np.where(B == 1, -1.0, B), S, t), (B, S, np.where(B == 2, np.nan, t))):
        with pytest.raises(adaln.AdaLNError):
            adaln.adaln_cost_fit(*args)
    with pytest.raises(adaln.AdaLNError):
        adaln.adaln_cost_fit(B, S, t, p_lo=2.0, p_hi=1.0)


def test_load_cv_matches_oracle():
    rng = np.random.default_rng(9)
    for n in (1, 2, 5, 64, 1000):
        x = rng.uniform(0.1, 10.0, n)
        assert math.isclose(adaln.adaln_load_cv(x), oracle.load_cv(x), rel_tol=1e-13, abs_tol=1e-16)
    assert math.isnan(adaln.adaln_load_cv([]))
    assert math.isnan(adaln.adaln_load_cv([1.0, -1.0]))
