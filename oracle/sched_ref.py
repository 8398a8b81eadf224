"""Plain CPU oracle for the dual-constraint batch scheduler and its cost model.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite and the benchmark's measurement legs
do.  It shares no code with the library's scheduler (csrc/adaln_sched.cpp)
and imports nothing from it.

What it computes
----------------
The AdaptiveLoad technical summary (gist.science, paper 2605.17923), section
2.A "Equilibrio de Carga Adaptativo de Doble Restricción", sizes the batch of
a group of equal-length sequences with two constraints at once: a linear
memory bound B*S <= M_mem and a polynomial compute bound B*S^p <= M_comp
(attention makes the per-sequence cost grow like S^2).  The group's batch is
the largest B meeting both, at least one (`b_shape`, in adaln_ref).  The
"Sistema de Ajuste de Costos" bullet of the same section calibrates p (and
from it M_comp) by timing synthetic shapes and fitting the cost model

    step_time ~= a + b * B * S^p

by nonlinear regression.  Section 4 measures load balance as the coefficient
of variation of per-worker compute load.

Readings where the page is silent:
  * grouping: samples of one length form that length's groups; each group
    takes the next B_shape(S) samples in their input order, the last group of
    a length takes what is left; groups are numbered by ascending length,
    then input order.  (The page sizes one group's batch and says nothing of
    how a corpus is cut into groups; this is the plainest cut.)
  * the fit minimises the ordinary sum of squared residuals of the model
    above over (a, b, p), with p restricted to a stated interval;
  * the coefficient of variation uses the population standard deviation
    (divide by n): the loads are the whole set of workers, not a sample.
No function here is parity unpinned: see tests/test_sched_oracle.py.
"""

from __future__ import annotations

import numpy as np

from .adaln_ref import b_shape


def plan_groups(lengths, m_mem: int, m_comp: int, p: float) -> list:
    """Cut samples into groups of equal length, B_shape(S) samples per group.

    Returns a list of groups; each group is a list of sample indices (into
    `lengths`) in input order.  Groups come by ascending length, then input
    order.
    """
    lengths = [int(v) for v in lengths]
    for v in lengths:
        if v <= 0:
            raise ValueError("sequence lengths must be positive")
    groups = []
    for S in sorted(set(lengths)):
        members = [i for i, v in enumerate(lengths) if v == S]
        size = b_shape(S, m_mem, m_comp, p)
        for start in range(0, len(members), size):
            groups.append(members[start:start + size])
    return groups


def cost_model(B, S, a: float, b: float, p: float):
    """step_time = a + b * B * S^p (section 2.A, cost-fitting bullet)."""
    B = np.asarray(B, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    return a + b * B * S ** p


def fit_cost_model(B, S, t, p_lo: float = 0.5, p_hi: float = 4.0):
    """Nonlinear least-squares fit of the cost model to timings t(B, S).

    A textbook nonlinear regression: scipy's trust-region least squares over
    (a, b, p) with p bounded to [p_lo, p_hi], started from several values of
    p and keeping the smallest residual.  Returns (a, b, p, rss).
    """
    from scipy.optimize import least_squares

    B = np.asarray(B, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    scale_t = float(np.abs(t).max()) or 1.0

    def resid(v):
        a, b, p = v
        return (a + b * B * S ** p - t) / scale_t

    best = None
    for p0 in np.linspace(p_lo, p_hi, 9):
        x0 = B * S ** p0
        b0 = (t.max() - t.min()) / max(float(x0.max() - x0.min()), 1e-300)
        a0 = float(t.min() - b0 * x0.min())
        r = least_squares(resid, x0=[a0, b0, p0], bounds=([-np.inf, -np.inf, p_lo], [np.inf, np.inf, p_hi]),
                          x_scale="jac", xtol=1e-15, ftol=1e-15, gtol=1e-15, max_nfev=20000)
        rss = float(np.sum((r.fun * scale_t) ** 2))
        if best is None or rss < best[3]:
            best = (float(r.x[0]), float(r.x[1]), float(r.x[2]), rss)
    return best


def load_cv(loads) -> float:
    """Coefficient of variation of per-worker loads: population standard
    deviation over the mean (section 4, load-balance bullet)."""
    x = np.asarray(loads, dtype=np.float64)
    if x.size == 0:
        raise ValueError("no loads")
    mean = x.sum() / x.size
    if mean == 0.0:
        raise ValueError("mean load is zero")
    var = ((x - mean) ** 2).sum() / x.size
    return float(np.sqrt(var) / mean)
