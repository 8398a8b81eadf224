"""The Python binding refuses tensors whose shape or dtype differs from what
the C entry point will read or write (a wrong-sized output would be written
past its storage), before any device is touched.  CPU tensors suffice: these
checks run ahead of the device checks."""

import pytest
import torch

import diffusion_transformer_adaln_amd as adaln

B, N, D = 2, 8, 64
BF = torch.bfloat16


def _fwd_args(dtype=BF):
    x = torch.zeros(B, N, D, dtype=dtype)
    return x, torch.zeros(B, D, dtype=dtype), torch.zeros(B, D, dtype=dtype)


def _bwd_args(dtype=BF):
    x = torch.zeros(B, N, D, dtype=dtype)
    return (torch.zeros_like(x), x, torch.zeros(B, D, dtype=dtype), torch.zeros(B, N),
            torch.zeros(B, N))


@pytest.mark.parametrize("kw,err,name", [
    ({"y": torch.zeros(B, N, D, dtype=torch.float32)}, TypeError, "y"),
    ({"y": torch.zeros(B, N, D // 2, dtype=BF)}, ValueError, "y"),
    ({"mean": torch.zeros(B * N - 1)}, ValueError, "mean"),
    ({"rstd": torch.zeros(B, N, dtype=torch.float64)}, TypeError, "rstd"),
])
def test_forward_rejects_bad_outputs(kw, err, name):
    with pytest.raises(err, match=name):
        adaln.adaln_fwd(*_fwd_args(), 1e-6, **kw)


def test_forward_accepts_flat_statistics_and_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        adaln.adaln_fwd(*_fwd_args(), 1e-6, mean=torch.zeros(B * N), rstd=torch.zeros(B * N))


@pytest.mark.parametrize("fn", ["adaln_bwd", "adaln_bwd_f32sums", "adaln_bwd_twopass"])
@pytest.mark.parametrize("kw,err,name", [
    ({"dx": torch.zeros(B, N, D)}, TypeError, "dx"),
    ({"dscale": torch.zeros(B, D + 8, dtype=BF)}, ValueError, "dscale"),
    ({"dshift": torch.zeros(B - 1, D, dtype=BF)}, ValueError, "dshift"),
])
def test_backward_rejects_bad_outputs(fn, kw, err, name):
    with pytest.raises(err, match=name):
        getattr(adaln, fn)(*_bwd_args(), **kw)


def test_f32sums_wants_float32_sums():
    # a bf16 buffer would receive 4-byte sums: twice its size
    with pytest.raises(TypeError, match="dscale"):
        adaln.adaln_bwd_f32sums(*_bwd_args(), dscale=torch.zeros(B, D, dtype=BF))
    with pytest.raises(TypeError, match="dshift"):
        adaln.adaln_bwd(*_bwd_args(), dshift=torch.zeros(B, D))
    with pytest.raises(ValueError, match="GPU"):      # right types: only the device check is left
        adaln.adaln_bwd_f32sums(*_bwd_args(), dscale=torch.zeros(B, D), dshift=torch.zeros(B, D))


@pytest.mark.parametrize("i,bad,err,name", [
    (2, torch.zeros(B, D + 1, dtype=BF), ValueError, "scale"),
    (2, torch.zeros(B, D), TypeError, "scale"),
    (3, torch.zeros(B, N + 1), ValueError, "mean"),
    (4, torch.zeros(B, N, dtype=BF), TypeError, "rstd"),
])
def test_backward_rejects_bad_inputs(i, bad, err, name):
    args = list(_bwd_args())
    args[i] = bad
    with pytest.raises(err, match=name):
        adaln.adaln_bwd(*args)


@pytest.mark.parametrize("fn", ["adaln_bwd_varlen", "adaln_bwd_varlen_f32sums"])
def test_varlen_backward_rejects_bad_outputs(fn):
    R = B * N
    x = torch.zeros(R, D, dtype=BF)
    off = torch.tensor([0, N, R], dtype=torch.int64)
    args = (torch.zeros_like(x), x, torch.zeros(B, D, dtype=BF), torch.zeros(R), torch.zeros(R), off)
    with pytest.raises(ValueError, match="dscale"):
        getattr(adaln, fn)(*args, dscale=torch.zeros(B, 2 * D))
    with pytest.raises(ValueError, match="mean"):
        getattr(adaln, fn)(*args[:3], torch.zeros(R - 1), *args[4:])
