"""The measurement probes of include/adaln_probe.h on the GPU: the streaming
probes move exactly the bytes they claim (so the ceilings bench.py reports
are rates of real copies), and the clock probe and marks give plausible,
ordered readings."""

import numpy as np
import pytest
import torch

import diffusion_transformer_adaln_amd as adaln
from gpu_helpers import say

pytestmark = pytest.mark.gpu

# byte sizes: tiny, a ragged tail past a whole grid-stride round, a few MB
SIZES = [16, 16 * 1000 + 16 * 7, (3 << 20) + 16 * 13]
SHAPES = [(1, 1), (1, 4), (2, 8), (16, 2)]


def _rand_bytes(n, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("wg,u", SHAPES)
def test_stream_probes_move_the_bytes(nbytes, wg, u):
    say(f"[probe] bytes={nbytes} wg_per_cu={wg} unroll={u}")
    a = _rand_bytes(nbytes, 1)
    b = _rand_bytes(nbytes, 2)
    out = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    adaln.adaln_probe_stream("copy", a, None, out, wg, u)
    torch.cuda.synchronize()
    assert torch.equal(out, a)
    adaln.adaln_probe_stream("two_to_one", a, b, out, wg, u)
    torch.cuda.synchronize()
    assert torch.equal(out, a ^ b)
    adaln.adaln_probe_stream("write", None, None, out, wg, u)
    torch.cuda.synchronize()
    w = out.view(torch.int32).cpu().numpy().astype(np.int64).reshape(-1, 4)
    assert (w[:, 1:] == [1, 2, 3]).all() and (w[:, 0] == np.arange(len(w))).all()
    # read: every thread xor-reduces its vectors, so the xor of all the
    # outputs is the xor of the whole input
    ro = torch.zeros(adaln.adaln_probe_read_out_bytes(wg), dtype=torch.uint8, device="cuda")
    adaln.adaln_probe_stream("read", a, None, ro, wg, u)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(ro.view(torch.int64).cpu().numpy().reshape(-1, 2), axis=0)
    want = np.bitwise_xor.reduce(a.view(torch.int64).cpu().numpy().reshape(-1, 2), axis=0)
    assert (got == want).all()


def test_clock_probe_and_marks():
    say("[probe] clock and marks")
    khz = adaln.adaln_probe_wall_clock_khz()
    assert khz > 0
    n = 32
    probe = torch.zeros(3 * n, dtype=torch.int64, device="cuda")
    marks = torch.zeros(n, dtype=torch.int64, device="cuda")
    for i in range(n):
        adaln.adaln_probe_mark(marks, i)
        adaln.adaln_probe_clock(probe, i, 4000)
    torch.cuda.synchronize()
    p = probe.cpu().numpy().reshape(n, 3)
    m = marks.cpu().numpy()
    assert (p[:, 1] > 0).all() and (p[:, 2] > 0).all()
    mhz = p[:, 1] / p[:, 2] * khz / 1e3
    say(f"  wall clock {khz} kHz; engine clock {mhz.min():.0f}-{mhz.max():.0f} MHz, "
        f"sample {np.median(p[:, 2]) / khz * 1e3:.1f} us")
    assert (mhz > 100).all() and (mhz < 5000).all()
    # same stream: every mark after the previous sample started, samples in order
    assert (np.diff(m) > 0).all() and (np.diff(p[:, 0]) > 0).all()
    assert (p[:, 0] >= m).all()
