"""adaln_bwd_noalloc, the backward entry point that allocates nothing (its
workspace is the library's static device array), against adaln_bwd through
the C ABI: bit for bit on two calls in a row, the second with a smaller
problem (the array keeps the first call's contents), and against the oracle;
problems whose workspace exceeds the array are refused before any launch."""

import ctypes

import pytest
import torch

import workloads
from gpu_helpers import bits, check_all, say, to_dev

pytestmark = pytest.mark.gpu


def _pd(dtype, D, lengths, seed, **kw):
    return workloads.make_problem_data(workloads.custom_problem(dtype, D, lengths, **kw), seed)


def _run_both(pd):
    import diffusion_transformer_adaln_amd as adaln

    p = pd.problem
    v = lambda t: t.view(p.B, p.N, p.D)
    x, dy = v(to_dev(pd.x, p.dtype)), v(to_dev(pd.dy, p.dtype))
    sh, sc = to_dev(pd.shift, p.dtype), to_dev(pd.scale, p.dtype)
    y, mean, rstd = adaln.adaln_fwd(x, sh, sc, p.eps)
    ref = adaln.adaln_bwd(dy, x, sc, mean, rstd)
    out = (torch.full_like(x, 7.0), torch.full_like(sc, 7.0), torch.full_like(sc, 7.0))
    got = adaln.adaln_bwd_noalloc(dy, x, sc, mean, rstd, *out)
    torch.cuda.synchronize()
    return {"y": y, "mean": mean, "rstd": rstd}, ref, got


def test_noalloc_matches_adaln_bwd_on_two_calls():
    big = _pd("bf16", 5120, [3000], seed=71, dy_sigma=1e-3)        # ~20 MB of tile partials
    small = _pd("bf16", 3072, [300, 300], seed=72, dy_sigma=1e-2)  # a smaller problem next
    for pd in (big, small):
        p = pd.problem
        say(f"[noalloc] bf16 B={p.B} N={p.N} D={p.D}")
        fwd, ref, got = _run_both(pd)
        for name, a, b in zip(("dx", "dscale", "dshift"), ref, got):
            assert bits(a) == bits(b), f"{name} differs from adaln_bwd"
        check_all(pd, {**fwd, "dx": got[0].view(-1, p.D), "dscale": got[1], "dshift": got[2],
                       "y": fwd["y"].view(-1, p.D), "mean": fwd["mean"].view(-1), "rstd": fwd["rstd"].view(-1)})


def test_noalloc_refuses_problems_beyond_its_array():
    import diffusion_transformer_adaln_amd as adaln

    lib = adaln.load_library()
    B, N, D = 1, 4096, 16384          # needs ~64 MiB of tile partials
    need = adaln.adaln_bwd_workspace_size(B, B * N, D, torch.bfloat16)
    assert need > adaln._lib.NOALLOC_SCRATCH_BYTES, need
    say(f"[noalloc] refuses B={B} N={N} D={D} ({need} bytes)")
    fake = [ctypes.c_void_p((k + 1) << 40) for k in range(8)]   # never dereferenced: refused first
    st = lib.adaln_bwd_noalloc(fake[0], fake[1], fake[2], fake[3], fake[4], B, N, D, 1, None, fake[5],
                               fake[6], fake[7])
    assert st == 4, adaln.adaln_status_str(st)
