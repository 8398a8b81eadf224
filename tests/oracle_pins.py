"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each ``check_*`` takes an implementation namespace (the oracle module, or a
mutated copy of it in the mutation tests) and raises AssertionError when the
implementation disagrees with a fact fixed by the mathematics or by an
independent library routine:

  * torch's fp64 LayerNorm (scale = shift = 0 special case) and autograd,
  * closed forms and invariants of the normalised rows and of dx,
  * central finite differences of L = sum(y * dy), and explicit per-row
    Jacobians of the forward by finite differences against torch's,
  * hand-derived worked examples,
  * exact special cases (scale = -1, dy = 1, constant rows, empty samples),
  * the page's bucket rule evaluated by hand (AdaptiveLoad summary, section 2.A).

None of them retypes the oracle's formulas.
"""

from __future__ import annotations

import math

import numpy as np
import torch

# --------------------------------------------------------------------------
# small seeded inputs (float64 throughout)
# --------------------------------------------------------------------------


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _offsets(lengths):
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    return off


def _case(seed, lengths, D, outliers=True):
    g = _rng(seed)
    R = int(sum(lengths))
    x = g.standard_normal((R, D)) + g.standard_normal((R, 1)) * 2.0
    if outliers and R > 2:
        x[g.choice(R, size=max(1, R // 10), replace=False)] *= 20.0
    shift = g.standard_normal((len(lengths), D)) * 0.1
    scale = g.standard_normal((len(lengths), D)) * 0.1
    dy = g.standard_normal((R, D))
    return x, shift, scale, dy, _offsets(lengths)


def _expand(per_sample, lengths):
    """[B, D] -> [R, D] by repeating sample b's row lengths[b] times (torch, no oracle code)."""
    t = torch.as_tensor(per_sample)
    return torch.repeat_interleave(t, torch.as_tensor(lengths, dtype=torch.int64), dim=0)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim):
        worst = int(np.argmax((err - lim).ravel()))
        raise AssertionError(f"{what}: max err {err.max():.3e}; worst element err {err.ravel()[worst]:.3e} "
                             f"> limit {lim.ravel()[worst]:.3e}")


LENGTHS = (3, 1, 5, 0, 4)   # ragged, with a one-row and an empty sample


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def check_layernorm_library(impl):
    """scale = shift = 0 reduces F1-F5 to plain LayerNorm (torch fp64)."""
    for eps in (1e-6, 1e-2, 0.5):
        for D in (1, 2, 7, 64):
            x, _, _, _, off = _case(11 + D, LENGTHS, D)
            z = np.zeros((len(LENGTHS), D))
            y, mean, rstd = impl.adaln_fwd(x, z, z, eps, off)
            xt = torch.as_tensor(x)
            ref = torch.nn.functional.layer_norm(xt, (D,), None, None, eps).numpy()
            _close(y, ref, 1e-12, 1e-12, f"layer_norm D={D} eps={eps}")
            var_t, mean_t = torch.var_mean(xt, dim=-1, unbiased=False)
            _close(mean, mean_t.numpy(), 1e-12, 1e-12, "mean")
            _close(rstd, (1.0 / torch.sqrt(var_t + eps)).numpy(), 1e-12, 0.0, "rstd")


def check_worked_example(impl):
    """x = [1, 2, 3, 4], eps = 0: mean 5/2, variance 5/4, xhat = [-3, -1, 1, 3]/sqrt(5)."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    scale = np.array([[0.5, -0.5, 1.0, 0.0]])
    shift = np.array([[1.0, 2.0, 3.0, 4.0]])
    y, mean, rstd = impl.adaln_fwd(x, shift, scale, 0.0, np.array([0, 1]))
    s5 = math.sqrt(5.0)
    xhat = np.array([-3.0, -1.0, 1.0, 3.0]) / s5
    _close(mean, [2.5], 1e-15, 0, "mean")
    _close(rstd, [2.0 / s5], 1e-15, 0, "rstd")          # 1/sqrt(5/4)
    # y = xhat * (1 + scale) + shift, entry by entry
    expect = np.array([-4.5 / s5 + 1.0, -0.5 / s5 + 2.0, 2.0 / s5 + 3.0, 3.0 / s5 + 4.0])
    _close(y[0], expect, 1e-15, 1e-15, "y")
    # backward with dy = [1, 0, 0, 0], same modulation, eps = 0:
    # g = [1.5, 0, 0, 0]; a = 3/8; c = 1.5 * (-3/sqrt5) / 4 = -9/(8 sqrt5)
    # dx_j = rstd * (g_j - a - xhat_j * c)
    dy = np.array([[1.0, 0.0, 0.0, 0.0]])
    dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, 0.0, np.array([0, 1]))
    a = 3.0 / 8.0
    c = -9.0 / (8.0 * s5)
    g = np.array([1.5, 0.0, 0.0, 0.0])
    dx_expect = (2.0 / s5) * (g - a - xhat * c)
    # same values written out: [1.5 - 3/8 - 27/40, -3/8 - 9/40, -3/8 + 9/40, -3/8 + 27/40] * 2/sqrt5
    dx_expect2 = np.array([0.45, -0.6, -0.15, 0.3]) * (2.0 / s5)
    _close(dx_expect, dx_expect2, 1e-15, 1e-15, "hand arithmetic")
    _close(dx[0], dx_expect2, 1e-14, 1e-15, "dx")
    _close(dshift[0], [1.0, 0.0, 0.0, 0.0], 0, 0, "dshift")
    _close(dscale[0], [-3.0 / s5, 0.0, 0.0, 0.0], 1e-15, 0, "dscale")


def check_modulation(impl):
    """F5 per sample: y - shift[b] = xhat * (1 + scale[b]); scale = -1 gives y = shift exactly."""
    D = 16
    x, shift, scale, _, off = _case(21, LENGTHS, D)
    eps = 1e-6
    y, _, _ = impl.adaln_fwd(x, shift, scale, eps, off)
    xhat = torch.nn.functional.layer_norm(torch.as_tensor(x), (D,), None, None, eps)
    ref = xhat * (1.0 + _expand(scale, LENGTHS)) + _expand(shift, LENGTHS)
    _close(y, ref.numpy(), 1e-12, 1e-12, "per-sample modulation")
    minus_one = -np.ones_like(scale)
    y2, _, _ = impl.adaln_fwd(x, shift, minus_one, eps, off)
    assert np.array_equal(y2, _expand(shift, LENGTHS).numpy()), "scale=-1 must give y = shift"


def check_fwd_invariants(impl):
    """Each row of xhat has mean 0 and mean square var/(var+eps) (1 at eps = 0)."""
    D = 48
    x, shift, scale, _, off = _case(31, LENGTHS, D)
    for eps in (0.0, 1e-6, 1e-1):
        z = np.zeros_like(shift)
        xhat, _, _ = impl.adaln_fwd(x, z, z, eps, off)
        var = np.var(x, axis=1)             # numpy's own biased variance
        assert np.all(np.abs(xhat.mean(axis=1)) <= 1e-13), "row mean of xhat"
        _close((xhat ** 2).mean(axis=1), var / (var + eps), 1e-12, 0, f"row mean square, eps={eps}")


def check_affine_invariance(impl):
    """At eps = 0 the normalised row is unchanged by x -> alpha*x + beta (alpha > 0)."""
    D = 32
    x, _, _, _, off = _case(41, LENGTHS, D)
    z = np.zeros((len(LENGTHS), D))
    a, _, _ = impl.adaln_fwd(x, z, z, 0.0, off)
    b, _, _ = impl.adaln_fwd(3.5 * x - 7.25, z, z, 0.0, off)
    _close(b, a, 1e-11, 1e-12, "affine invariance")


def check_constant_row(impl):
    """A constant row: rstd = eps^-1/2, xhat = 0, y = shift, dx = rstd * (g - mean(g))."""
    D, eps = 8, 1e-2
    x = np.full((2, D), 3.25)
    shift = np.arange(D, dtype=np.float64)[None, :] * 0.5
    scale = np.linspace(-0.5, 0.5, D)[None, :]
    off = np.array([0, 2])
    y, mean, rstd = impl.adaln_fwd(x, shift, scale, eps, off)
    _close(rstd, np.full(2, 10.0), 1e-15, 0, "rstd")
    _close(mean, np.full(2, 3.25), 0, 0, "mean")
    _close(y, np.repeat(shift, 2, axis=0), 0, 1e-15, "y")
    dy = _rng(5).standard_normal((2, D))
    dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, eps, off)
    g = dy * (1.0 + scale)
    _close(dx, 10.0 * (g - g.mean(axis=1, keepdims=True)), 1e-13, 1e-14, "dx")
    _close(dscale, np.zeros((1, D)), 0, 0, "dscale")


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _loss(impl, x, shift, scale, dy, eps, off):
    y, _, _ = impl.adaln_fwd(x, shift, scale, eps, off)
    return float((y * dy).sum())


def check_finite_differences(impl):
    """Central differences of L = sum(y * dy) match dx, dshift and dscale."""
    lengths = (3, 2)
    for D in (1, 2, 5, 8):
        for eps in (1e-6, 1e-2):
            x, shift, scale, dy, off = _case(51 + D, lengths, D, outliers=False)
            dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, eps, off)
            h = 1e-6
            for name, arr, grad in (("x", x, dx), ("scale", scale, dscale), ("shift", shift, dshift)):
                fd = np.zeros_like(arr)
                for idx in np.ndindex(arr.shape):
                    keep = arr[idx]
                    arr[idx] = keep + h
                    lp = _loss(impl, x, shift, scale, dy, eps, off)
                    arr[idx] = keep - h
                    lm = _loss(impl, x, shift, scale, dy, eps, off)
                    arr[idx] = keep
                    fd[idx] = (lp - lm) / (2 * h)
                _close(grad, fd, 1e-6, 1e-7, f"finite differences d{name} D={D} eps={eps}")


def check_explicit_jacobian(impl):
    """Per row, the D x D Jacobian of y with respect to x, by central
    differences of the oracle's forward, equals torch fp64 autograd's Jacobian
    of layer_norm(x) * (1 + scale) + shift; it sends a constant shift of the
    row to zero (J @ 1 = 0); and the oracle's dx is J^T dy for several dy."""
    D = 6
    lengths = (2, 1)
    one_row = np.array([0, 1], dtype=np.int64)
    g = _rng(82)
    h = 1e-6
    for eps in (1e-6, 1e-2):
        x, shift, scale, _, _ = _case(81, lengths, D, outliers=False)
        for r in range(x.shape[0]):
            b = 0 if r < lengths[0] else 1

            def f(v):
                y, _, _ = impl.adaln_fwd(v[None, :], shift[b:b + 1], scale[b:b + 1], eps, one_row)
                return y[0]

            J = np.zeros((D, D))
            for j in range(D):
                e = np.zeros(D)
                e[j] = h
                J[:, j] = (f(x[r] + e) - f(x[r] - e)) / (2 * h)
            sc_t, sh_t = torch.as_tensor(scale[b]), torch.as_tensor(shift[b])
            Jt = torch.autograd.functional.jacobian(
                lambda v: torch.nn.functional.layer_norm(v, (D,), None, None, eps) * (1.0 + sc_t) + sh_t,
                torch.as_tensor(x[r])).numpy()
            _close(J, Jt, 1e-6, 1e-7, f"Jacobian row {r} eps={eps}")
            _close(J @ np.ones(D), np.zeros(D), 0.0, 1e-6, f"J @ 1 row {r} eps={eps}")
            for _ in range(3):
                dy = g.standard_normal((1, D))
                dx, _, _ = impl.adaln_bwd(dy, x[r:r + 1], scale[b:b + 1], eps, one_row)
                _close(dx[0], Jt.T @ dy[0], 1e-10, 1e-12, f"dx = J^T dy row {r} eps={eps}")


def check_torch_autograd(impl):
    """dx, dscale, dshift equal torch fp64 autograd of layer_norm(x)*(1+scale[b])+shift[b]."""
    D = 24
    for eps in (1e-6, 1e-2):
        x, shift, scale, dy, off = _case(61, LENGTHS, D)
        xt = torch.as_tensor(x).clone().requires_grad_(True)
        st = torch.as_tensor(scale).clone().requires_grad_(True)
        ht = torch.as_tensor(shift).clone().requires_grad_(True)
        xhat = torch.nn.functional.layer_norm(xt, (D,), None, None, eps)
        rep = torch.as_tensor(LENGTHS, dtype=torch.int64)
        y = xhat * (1.0 + torch.repeat_interleave(st, rep, dim=0)) + torch.repeat_interleave(ht, rep, dim=0)
        (y * torch.as_tensor(dy)).sum().backward()
        dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, eps, off)
        _close(dx, xt.grad.numpy(), 1e-10, 1e-12, f"dx eps={eps}")
        _close(dscale, st.grad.numpy(), 1e-10, 1e-12, f"dscale eps={eps}")
        _close(dshift, ht.grad.numpy(), 1e-10, 1e-12, f"dshift eps={eps}")


def check_dx_closed_forms(impl):
    """sum_d dx = 0 and sum_d dx*xhat = eps * rstd^3 * sum_d g*xhat for every row."""
    D = 40
    x, shift, scale, dy, off = _case(71, LENGTHS, D)
    for eps in (0.0, 1e-6, 1e-1):
        dx, _, _ = impl.adaln_bwd(dy, x, scale, eps, off)
        xt = torch.as_tensor(x)
        var, mean = torch.var_mean(xt, dim=-1, unbiased=False)
        rstd = (1.0 / torch.sqrt(var + eps)).numpy()
        xhat = ((xt - mean[:, None]) * torch.as_tensor(rstd)[:, None]).numpy()
        g = dy * (1.0 + _expand(scale, LENGTHS).numpy())
        scale_ref = np.abs(g).sum(axis=1) * rstd
        assert np.all(np.abs(dx.sum(axis=1)) <= 1e-12 * scale_ref), "sum_d dx = 0"
        lhs = (dx * xhat).sum(axis=1)
        rhs = eps * rstd ** 3 * (g * xhat).sum(axis=1)
        assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale_ref * (1 + np.abs(xhat).max())), \
            f"sum_d dx*xhat closed form, eps={eps}"


def check_dy_constant(impl):
    """dy = 1, scale = 0: dx = 0, dshift[b] = N_b, dscale[b] = sum_n xhat."""
    D, eps = 12, 1e-6
    x, shift, _, _, off = _case(81, LENGTHS, D)
    scale = np.zeros_like(shift)
    dy = np.ones_like(x)
    dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, eps, off)
    assert np.all(np.abs(dx) <= 1e-12 * np.sqrt(1.0 / eps)), "dx must vanish"
    for b, n in enumerate(LENGTHS):
        assert np.all(dshift[b] == n), f"dshift[{b}] must be N_b"
    xhat = torch.nn.functional.layer_norm(torch.as_tensor(x), (D,), None, None, eps)
    ref = torch.zeros(len(LENGTHS), D, dtype=torch.float64).index_add_(
        0, torch.repeat_interleave(torch.arange(len(LENGTHS)), torch.as_tensor(LENGTHS)), xhat)
    _close(dscale, ref.numpy(), 1e-12, 1e-12, "dscale = sum xhat")


def check_packed_additivity(impl):
    """A packed call equals each sample computed on its own (and subsets equal the full call)."""
    D, eps = 20, 1e-6
    x, shift, scale, dy, off = _case(91, LENGTHS, D)
    y, mean, rstd = impl.adaln_fwd(x, shift, scale, eps, off)
    dx, dscale, dshift = impl.adaln_bwd(dy, x, scale, eps, off)
    for b, n in enumerate(LENGTHS):
        lo, hi = off[b], off[b + 1]
        one = np.array([0, n])
        yb, mb, rb = impl.adaln_fwd(x[lo:hi], shift[b:b + 1], scale[b:b + 1], eps, one)
        dxb, dsb, dhb = impl.adaln_bwd(dy[lo:hi], x[lo:hi], scale[b:b + 1], eps, one)
        assert np.array_equal(yb, y[lo:hi]) and np.array_equal(mb, mean[lo:hi]) and np.array_equal(rb, rstd[lo:hi])
        assert np.array_equal(dxb, dx[lo:hi])
        assert np.array_equal(dsb[0], dscale[b]) and np.array_equal(dhb[0], dshift[b])
        if n == 0:
            assert not dscale[b].any() and not dshift[b].any(), "empty sample sums to zero"
    rows = np.array([11, 0, 4, 12])
    yr, _, _ = impl.adaln_fwd(x, shift, scale, eps, off, rows=rows)
    assert np.array_equal(yr, y[rows])
    dxr, dsr, dhr = impl.adaln_bwd(dy, x, scale, eps, off, rows=rows, samples=np.array([4, 2]))
    assert np.array_equal(dxr, dx[rows])
    assert np.array_equal(dsr, dscale[[4, 2]]) and np.array_equal(dhr, dshift[[4, 2]])


def check_decode_bf16(impl):
    """bf16 bits widen exactly as torch's bfloat16 -> float64 conversion does."""
    g = _rng(3)
    bits = g.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                                  # finite patterns only
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = impl.decode_bf16(bits)
    assert np.array_equal(got, ref), "bf16 decode"
    f = g.standard_normal(100).astype(np.float32)
    assert np.array_equal(impl.decode(f, "f32"), f.astype(np.float64))


def check_b_shape(impl):
    """The page's bucket rule evaluated by hand for M_mem = 65536, M_comp = 2^30, p = 2.

    S = 256:   65536/256 = 256,   2^30/2^16 = 16384     -> 256
    S = 4096:  65536/4096 = 16,   2^30/2^24 = 64        -> 16
    S = 16384: 65536/16384 = 4,   2^30/2^28 = 4         -> 4
    S = 32760: floor(2.0005) = 2, floor(1.00049) = 1    -> 1
    S = 70000: floor(0.936) = 0 (memory bound binds)    -> max(1, 0) = 1
    S = 3000:  floor(21.85) = 21, floor(119.3) = 119    -> 21 (memory bound)
    S = 20000: floor(3.28) = 3,   floor(2.68) = 2       -> 2  (compute bound)
    """
    m_mem, m_comp = 65536, 2 ** 30
    for S, want in ((256, 256), (4096, 16), (16384, 4), (32760, 1), (70000, 1), (1, 65536), (2048, 32),
                    (3000, 21), (20000, 2)):
        got = impl.b_shape(S, m_mem, m_comp, 2)
        assert got == want, f"B_shape({S}) = {got}, expected {want}"
    # with a weaker exponent the compute bound stops binding at S = 4096
    assert impl.b_shape(4096, m_mem, m_comp, 1.5) == 16


CHECKS = [
    check_layernorm_library,
    check_worked_example,
    check_modulation,
    check_fwd_invariants,
    check_affine_invariance,
    check_constant_row,
    check_finite_differences,
    check_explicit_jacobian,
    check_torch_autograd,
    check_dx_closed_forms,
    check_dy_constant,
    check_packed_additivity,
    check_decode_bf16,
    check_b_shape,
]
