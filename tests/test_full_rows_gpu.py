"""Every row of the full-size workloads against the fp64 oracle.

y, dx, mean and rstd of every row of the DiT, MMDiT (both streams, and packed
into one batch) and video workloads, and
of the fuzz grid's 4,097-row batches, are compared element by element (the
oracle runs over row chunks), together with every sample's column sums.  The
persistent forward is also checked in full where each wave carries several
rows (3,000 rows of D = 5120: about three rows per wave, with the next row's
loads in flight while the current one is reduced), and the finish's single
rounding is pinned on values where a rounding of partial sums would change
the result."""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import bits, check_all, check_every_row, check_samples, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _pd(dtype, D, lengths, seed=0, dense=None, **kw):
    p = workloads.custom_problem(dtype, D, lengths, dense=dense, **kw)
    return workloads.make_problem_data(p, seed)


@pytest.mark.parametrize("name", ["dit_bf16", "mmdit_bf16", "mmdit_packed_bf16", "video_bf16"])
def test_full_size_every_row(name):
    for pd in workloads.make_config(name):
        p = pd.problem
        say(f"[every-row] {name}/{p.name} B={p.B} R={p.R} D={p.D}")
        out = run_gpu(pd)
        res = check_every_row(pd, out)
        res.update(check_samples(pd, out, np.arange(p.B)))
        say(f"  {res}")
        del out
        torch.cuda.empty_cache()


FUZZ_D = [1, 7, 64, 127, 768, 1152, 3072, 4096, 5120, 8192]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", FUZZ_D)
def test_fuzz_4097_every_row(dtype, D):
    """The fuzz grid's B = 3, N = 4097 batches (same seeds as test_fuzz_grid),
    every row and every sample."""
    B, N = 3, 4097
    pd = _pd(dtype, D, [N] * B, seed=1000 + D + N, dy_sigma=1.0 if dtype == "f32" else 1e-2)
    say(f"[every-row fuzz] {dtype} D={D} B={B} N={N}")
    out = run_gpu(pd)
    res = check_every_row(pd, out)
    res.update(check_samples(pd, out, np.arange(B)))
    say(f"  {res}")


@pytest.mark.parametrize("lengths", [[3000], [1500, 1500], [2999, 1, 700]])
def test_persistent_forward_several_rows_per_wave(lengths):
    """D = 5120 bf16 runs the one-wave-per-row persistent forward; with 3,000
    or more rows each of its ~1,000 waves walks several rows (and crosses
    sample boundaries in the packed cases), every one checked."""
    pd = _pd("bf16", 5120, lengths, seed=23, dy_sigma=1e-3)
    say(f"[persistent fwd] bf16 D=5120 lengths={lengths}")
    res = check_all(pd, run_gpu(pd))
    if len(lengths) > 1 and pd.problem.dense:
        res.update(check_all(pd, run_gpu(pd, dense=False)))
    say(f"  {res}")


def _dense_tiles(R):
    """The dense backward's tile count on this device: tiles of
    max(4, ceil(R / (2 * CUs))) rows, tile k taking rows k, k + T, k + 2T, ...
    and the finish adding tiles t, t + 64, ... of one slice in one thread."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tile_rows = max(4, -(-R // (2 * cus)))
    return -(-R // tile_rows)


def _one_sample(dy_rows, R=2048, D=64, sums_f32=False):
    """dshift of one sample whose dy is zero except the given rows."""
    import diffusion_transformer_adaln_amd as adaln

    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(1, R, D, device="cuda", generator=g).to(torch.bfloat16)
    dy = torch.zeros(1, R, D, device="cuda", dtype=torch.bfloat16)
    for r, v in dy_rows.items():
        dy[0, r] = v
    zero = torch.zeros(1, D, device="cuda", dtype=torch.bfloat16)
    y, mean, rstd = adaln.adaln_fwd(x, zero, zero, 1e-6)
    bwd = adaln.adaln_bwd_f32sums if sums_f32 else adaln.adaln_bwd
    _, _, dshift = bwd(dy, x, zero, mean, rstd)
    torch.cuda.synchronize()
    return dshift


def test_finish_rounds_once_bf16():
    """Tile 0 holds 1 + 2^-8 (rows 0 and T), tile 64 holds 2^-30 (row 64):
    the exact sum lies just above the bf16 midpoint between 1 and 1 + 2^-7, so
    one rounding gives 1 + 2^-7; rounding the slice's sum to fp32 first would
    land on the midpoint and round to 1."""
    R = 2048
    T = _dense_tiles(R)
    if not 129 <= T <= 512:
        pytest.skip(f"{T} tiles: the slice layout this case relies on needs 129..512")
    say(f"[finish rounding] bf16, {T} tiles")
    dshift = _one_sample({0: 1.0, T: 2.0 ** -8, 64: 2.0 ** -30}, R)
    got = dshift.view(torch.int16).cpu().numpy().astype(np.uint16)
    assert np.all(got == 0x3F81), np.unique(got)


def test_finish_rounds_once_f32_sums():
    """Tiles 0, 64 and 128 (one slice of the finish) hold 1, 2^-24 and 2^-24:
    the exact sum 1 + 2^-23 is an fp32 value; adding in fp32 would lose each
    2^-24 to a tie and return 1."""
    R = 2048
    T = _dense_tiles(R)
    if not 129 <= T <= 512:
        pytest.skip(f"{T} tiles: the slice layout this case relies on needs 129..512")
    say(f"[finish rounding] fp32 sums, {T} tiles")
    dshift = _one_sample({0: 1.0, 64: 2.0 ** -24, 128: 2.0 ** -24}, R, sums_f32=True)
    got = dshift.view(torch.int32).cpu().numpy().astype(np.uint32)
    assert np.all(got == 0x3F800001), np.unique(got)


def test_stream_argument_keeps_internal_buffers():
    """Calls that pass stream= and let the binding allocate the outputs and
    the workspace: while the kernels run on that stream, the current stream
    allocates and overwrites memory; the results must be the serial run's
    bits (the binding records the stream on what it allocates, so the
    allocator does not hand those blocks out early)."""
    import diffusion_transformer_adaln_amd as adaln

    pd = _pd("bf16", 5120, [6000], seed=29, dy_sigma=1e-3)
    p = pd.problem
    say("[stream=] internal buffers under a side stream")
    x = to_dev(pd.x, "bf16").view(1, p.R, p.D)
    dy = to_dev(pd.dy, "bf16").view(1, p.R, p.D)
    sh, sc = to_dev(pd.shift, "bf16"), to_dev(pd.scale, "bf16")
    y, mean, rstd = adaln.adaln_fwd(x, sh, sc, p.eps)
    dx, ds, dh = adaln.adaln_bwd(dy, x, sc, mean, rstd)
    torch.cuda.synchronize()
    ref = {k: bits(t) for k, t in (("y", y), ("mean", mean), ("rstd", rstd), ("dx", dx), ("ds", ds), ("dh", dh))}
    ws_bytes = adaln.adaln_bwd_workspace_size(1, p.R, p.D, torch.bfloat16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        y2, m2, r2 = adaln.adaln_fwd(x, sh, sc, p.eps, stream=s)
        dx2, ds2, dh2 = adaln.adaln_bwd(dy, x, sc, m2, r2, stream=s)
        # the current stream reuses whatever the allocator offers, at once
        junk = [torch.full((ws_bytes,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(2)]
        junk += [torch.full((p.R, p.D), 3.0, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        del junk
        torch.cuda.synchronize()
        got = {k: bits(t) for k, t in (("y", y2), ("mean", m2), ("rstd", r2), ("dx", dx2), ("ds", ds2),
                                       ("dh", dh2))}
        assert got == ref, f"repeat {rep}: results under stream= differ from the serial run"
