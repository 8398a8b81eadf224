"""The unfused eager-PyTorch baseline that bench.py --impl torch times.

It is a comparison leg, not part of the HIP path: these tests check that it
computes the same operator as the oracle (so the timing compares like with
like) and that its activation accounting counts what autograd really keeps.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads


def _problem(dtype, B, N, D, seed):
    pd = workloads.make_problem_data(workloads.custom_problem(dtype, D, [N] * B, dy_sigma=1.0), seed)
    p = pd.problem
    dec = lambda a: oracle.decode(a, p.dtype)
    return pd, dec(pd.x).reshape(B, N, D), dec(pd.dy).reshape(B, N, D), dec(pd.shift), dec(pd.scale)


def test_eager_chain_is_the_operator_fp64():
    """In fp64 on the CPU the eager chain and its autograd backward agree with
    the oracle to rounding: the same forward and the same three gradients."""
    B, N, D = 3, 7, 24
    pd, x, dy, sh, sc = _problem("f32", B, N, D, seed=3)
    xt = torch.tensor(x, requires_grad=True)
    sht = torch.tensor(sh, requires_grad=True)
    sct = torch.tensor(sc, requires_grad=True)
    y = bench.eager_adaln(xt, sht, sct, 1e-6)
    gx, gsc, gsh = torch.autograd.grad(y, (xt, sct, sht), torch.tensor(dy))
    off = pd.offsets
    y_ref, _, _ = oracle.adaln_fwd(x.reshape(-1, D), sh, sc, 1e-6, off)
    dx_ref, ds_ref, dh_ref = oracle.adaln_bwd(dy.reshape(-1, D), x.reshape(-1, D), sc, 1e-6, off)
    assert np.abs(y.detach().numpy().reshape(-1, D) - y_ref).max() < 1e-12
    assert np.abs(gx.numpy().reshape(-1, D) - dx_ref).max() < 1e-10
    assert np.abs(gsc.numpy() - ds_ref).max() < 1e-10
    assert np.abs(gsh.numpy() - dh_ref).max() < 1e-10


def test_saved_activation_accounting_cpu():
    """fp32 on the CPU: autograd keeps the normalised tensor (R*D), the row
    mean and rstd (R each) and 1 + scale (B*D), all fp32; the inputs x,
    shift and scale are not counted."""
    B, N, D = 2, 33, 40
    x = torch.randn(B, N, D, requires_grad=True)
    sh = torch.randn(B, D, requires_grad=True)
    sc = torch.randn(B, D, requires_grad=True)
    _, n = bench.saved_activation_bytes(bench.eager_adaln, x, sh, sc, 1e-6)
    R = B * N
    assert n == 4 * (R * D + 2 * R + B * D)
    with torch.no_grad():   # nothing is saved without a graph
        _, n0 = bench.saved_activation_bytes(bench.eager_adaln, x, sh, sc, 1e-6)
    assert n0 == 0


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_eager_chain_on_gpu_matches_oracle(dtype):
    """The eager chain on the GPU, against the oracle.  fp32: the operator's
    fp32 tolerances.  bf16: each of its three elementwise steps rounds to
    bf16 (LayerNorm output, the product, the sum), so its forward error is
    bounded by 2e-2 plus 2^-8 of |LN(x)*(1+scale)| twice and of |y| once;
    dx and the column sums are checked normwise."""
    from gpu_helpers import say, to_dev, to_host64

    B, N, D = 2, 300, 1024
    pd, x, dy, sh, sc = _problem(dtype, B, N, D, seed=17)
    p = pd.problem
    say(f"[eager] {dtype} B={B} N={N} D={D}")
    xt = to_dev(pd.x, dtype).view(B, N, D).requires_grad_(True)
    sht = to_dev(pd.shift, dtype).requires_grad_(True)
    sct = to_dev(pd.scale, dtype).requires_grad_(True)
    y = bench.eager_adaln(xt, sht, sct, p.eps)
    gx, gsc, gsh = torch.autograd.grad(y, (xt, sct, sht), to_dev(pd.dy, dtype).view(B, N, D))
    torch.cuda.synchronize()
    off = pd.offsets
    y_ref, _, rstd_ref = oracle.adaln_fwd(x.reshape(-1, D), sh, sc, p.eps, off)
    dx_ref, ds_ref, dh_ref = oracle.adaln_bwd(dy.reshape(-1, D), x.reshape(-1, D), sc, p.eps, off)
    yg = to_host64(y).reshape(-1, D)
    dxg = to_host64(gx).reshape(-1, D)
    if dtype == "f32":
        assert np.abs(yg - y_ref).max() <= 1e-4
        assert np.abs(dxg - dx_ref).max() <= 1e-4
        for got, ref in ((to_host64(gsc), ds_ref), (to_host64(gsh), dh_ref)):
            assert np.abs(got - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())
    else:
        rows = np.repeat(np.arange(B), N)
        mod = y_ref - sh[rows]
        bound = 2e-2 + 2.0 ** -8 * (2 * np.abs(mod) + np.abs(y_ref))
        assert np.all(np.abs(yg - y_ref) <= bound)
        assert np.abs(dxg - dx_ref).max() / np.abs(dx_ref).max() <= 2e-2
        for got, ref in ((to_host64(gsc), ds_ref), (to_host64(gsh), dh_ref)):
            assert np.abs(got - ref).max() / np.abs(ref).max() <= 2e-2
