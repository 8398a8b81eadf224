"""HIP path against the fp64 oracle, element by element, through the C ABI.

Small problems (several tiles plus a ragged tail) are checked in full;
the full-size workloads are checked on sampled rows and on whole-sample
column sums.  Edge cases: empty inputs and samples, one-row samples, odd and
tiny D, misaligned pointers (general kernels), the largest supported D,
more than 2^31 elements in one tensor, constant rows, rows far from zero
mean, determinism and dense/packed equivalence.
"""

import hashlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (bits, check_all, check_rows, check_samples, run_gpu, sampled_rows, say,
                         to_dev)

pytestmark = pytest.mark.gpu


def _pd(dtype, D, lengths, seed=0, dense=None, **kw):
    p = workloads.custom_problem(dtype, D, lengths, dense=dense, **kw)
    return workloads.make_problem_data(p, seed)


# ---------------------------------------------------------------------------
# the five workloads at sizes the oracle checks in full
# ---------------------------------------------------------------------------
SMALL = {
    "tiny_fp32": lambda: workloads.make_config("tiny_fp32"),
    "dit_bf16_small": lambda: [_pd("bf16", 1152, [300] * 3, seed=2, dy_sigma=1e-2)],
    "mmdit_bf16_small": lambda: [
        _pd("bf16", 3072, [77] * 2, seed=3, dy_sigma=1e-2, outlier_frac=0.01),
        _pd("bf16", 3072, [513] * 2, seed=4, dy_sigma=1e-2, outlier_frac=0.01)],
    "video_bf16_small": lambda: [_pd("bf16", 5120, [1000], seed=5, dy_sigma=1e-3)],
    "ragged_bf16_small": lambda: [_pd("bf16", 3072, [5, 0, 300, 1, 129, 64], seed=6, dense=False)],
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_full_check(name):
    for pd in SMALL[name]():
        say(f"[parity] {name}/{pd.problem.name} R={pd.problem.R} D={pd.problem.D}")
        out = run_gpu(pd)
        res = check_all(pd, out)
        say(f"  {res}")


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows, whole-sample sums
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["dit_bf16", "mmdit_bf16", "mmdit_packed_bf16", "video_bf16", "ragged_bf16",
                                  "long64k_bf16"])
def test_full_size_workloads_sampled(name):
    for pd in workloads.make_config(name):
        p = pd.problem
        say(f"[parity-full] {name}/{p.name} B={p.B} R={p.R} D={p.D}")
        out = run_gpu(pd)
        rows = sampled_rows(pd)
        res = check_rows(pd, out, rows)
        if p.B <= 8:
            samples = np.arange(p.B)
        else:   # one sample of every distinct length, plus the first and last
            seen, samples = set(), []
            for b, n in enumerate(p.lengths):
                if n not in seen:
                    seen.add(n)
                    samples.append(b)
            samples = np.array(sorted(set(samples) | {0, p.B - 1}))
        res.update(check_samples(pd, out, samples))
        say(f"  rows={rows.size} samples={len(samples)} {res}")
        del out
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# shapes: vector plans, general kernels, extremes
# ---------------------------------------------------------------------------
SHAPES = [
    ("f32", 1, [3, 5]), ("f32", 7, [33]), ("f32", 64, [255]), ("f32", 127, [9, 4]),
    ("f32", 768, [130]), ("f32", 4096, [70]), ("f32", 8192, [17]), ("f32", 12288, [5]),
    ("bf16", 8, [40]), ("bf16", 64, [255]), ("bf16", 127, [9]), ("bf16", 768, [130, 7]),
    ("bf16", 1024, [100]), ("bf16", 2048, [64, 64]), ("bf16", 4096, [97]),
    ("bf16", 8192, [41]), ("bf16", 12288, [9]), ("bf16", 16384, [12]), ("bf16", 20000, [6]),
    ("bf16", 32768, [4]), ("f32", 65536, [3]), ("bf16", 65536, [3]),
    # several rows per wave (16 or 32 lanes per row) with sample boundaries
    # inside a wave's rows, so lanes of one wave use different modulation rows
    ("bf16", 1152, [3, 5, 2, 7]), ("bf16", 1152, [13, 13]), ("f32", 128, [3, 1, 6]),
    ("f32", 128, [5, 5, 5]), ("bf16", 256, [1, 0, 2, 9]),
    # one-wave rows of every width the persistent forward instantiates
    # (64 lanes x 1..10 vectors), with ragged and multi-sample batches
    ("bf16", 512, [33, 2]), ("bf16", 1536, [40]), ("bf16", 2560, [50, 3]), ("bf16", 3584, [33]),
    ("bf16", 4608, [7, 70]), ("f32", 1280, [40]), ("f32", 1792, [9, 9]), ("f32", 2560, [21]),
    # dense batches whose plain tiling would overflow two tiles per CU (3 x 4096 rows: 513
    # tiles of 24 rows), so the planner lengthens the tiles; packed twins take the few-sample rule
    ("bf16", 3072, [4096] * 3), ("f32", 1280, [4096] * 3),
]


@pytest.mark.parametrize("dtype,D,lengths", SHAPES, ids=[f"{d}-D{D}-{'x'.join(map(str, l))}" for d, D, l in SHAPES])
def test_shapes(dtype, D, lengths):
    pd = _pd(dtype, D, lengths, seed=D, dy_sigma=1.0 if dtype == "f32" else 1e-2)
    say(f"[shape] {dtype} D={D} lengths={lengths}")
    check_all(pd, run_gpu(pd))
    if len(set(lengths)) > 1 or len(lengths) > 1:
        check_all(pd, run_gpu(pd, dense=False))


# More samples than the packed backward's one-workgroup prologue scans in one
# pass (1,024), with empty samples at the pass boundaries, so its carried
# prefix sum and the many-sample finish are both exercised.
@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("f32", 128), ("bf16", 3072)])
def test_many_packed_samples(dtype, D):
    g = np.random.Generator(np.random.PCG64(17))
    lengths = g.integers(0, 7, size=2600).tolist()
    for b in (0, 1023, 1024, 2047, 2048, 2599):
        lengths[b] = 0
    lengths[1025] = 40
    pd = _pd(dtype, D, lengths, seed=18, dense=False)
    say(f"[many-samples] {dtype} D={D} B={len(lengths)} R={pd.problem.R}")
    check_all(pd, run_gpu(pd))


# Packed batches of up to 64 samples number their tiles inside the kernels
# (one wave rebuilds the table from the offsets); from 65 on a prologue kernel
# writes it.  Both sides of that switch, with empty samples in the first and
# the last lane and a ragged mix of lengths.
@pytest.mark.parametrize("dtype,D,B", [("bf16", 3072, 64), ("bf16", 3072, 65), ("f32", 128, 64),
                                       ("f32", 128, 65), ("bf16", 1152, 1)])
def test_packed_tile_table_switch(dtype, D, B):
    g = np.random.Generator(np.random.PCG64(23))
    lengths = g.integers(1, 300, size=B).tolist()
    if B > 1:
        lengths[0] = 0
        lengths[min(63, B - 1)] = 0
        lengths[B // 2] = 1500
    pd = _pd(dtype, D, lengths, seed=24, dense=False)
    say(f"[tile-table] {dtype} D={D} B={B} R={pd.problem.R}")
    check_all(pd, run_gpu(pd))


# Many short samples through the dense entry points: B far above the narrow
# finish's 16 samples, tiles of a few rows each.
@pytest.mark.parametrize("dtype,D,B,N", [("bf16", 1152, 3000, 3), ("f32", 128, 2049, 5)])
def test_many_dense_samples(dtype, D, B, N):
    pd = _pd(dtype, D, [N] * B, seed=19, dense=True)
    say(f"[many-dense] {dtype} D={D} B={B} N={N}")
    check_all(pd, run_gpu(pd))


# The fuzz grid: every D here against one-row, tiny, one-wave-plus and
# several-thousand-row batches, both dtypes.  The 4,097-row batches are
# checked on sampled rows and on every sample's full column sums.
FUZZ_D = [1, 7, 64, 127, 768, 1152, 3072, 4096, 5120, 8192]
FUZZ_BN = [(1, 1), (3, 3), (1, 255), (3, 4097)]
FUZZ = [(dt, D, B, N) for dt in ("f32", "bf16") for D in FUZZ_D for B, N in FUZZ_BN]


@pytest.mark.parametrize("dtype,D,B,N", FUZZ, ids=[f"{dt}-D{D}-B{B}xN{N}" for dt, D, B, N in FUZZ])
def test_fuzz_grid(dtype, D, B, N):
    pd = _pd(dtype, D, [N] * B, seed=1000 + D + N, dy_sigma=1.0 if dtype == "f32" else 1e-2)
    say(f"[fuzz] {dtype} D={D} B={B} N={N}")
    out = run_gpu(pd)
    if B * N <= 1024:
        check_all(pd, out)
    else:
        check_rows(pd, out, sampled_rows(pd))
        check_samples(pd, out, np.arange(B))


# eps = 0 (pure LayerNorm scaling; the rows here are never constant) and a
# large eps, on each forward kernel: one wave per row (D = 5120), slots
# (D = 1152), general (D = 100), fp32 slots (D = 768).
EPS_CASES = [("bf16", 5120, [40]), ("bf16", 1152, [3, 30]), ("bf16", 100, [17]), ("f32", 768, [33])]


@pytest.mark.parametrize("eps", [0.0, 1e-2])
@pytest.mark.parametrize("dtype,D,lengths", EPS_CASES, ids=[f"{d}-D{D}" for d, D, _ in EPS_CASES])
def test_eps_values(dtype, D, lengths, eps):
    pd = _pd(dtype, D, lengths, seed=31 + D, dy_sigma=1.0 if dtype == "f32" else 1e-2)
    say(f"[eps] {dtype} D={D} lengths={lengths} eps={eps}")
    check_all(pd, run_gpu(pd, eps=eps), eps=eps)
    if len(lengths) > 1:
        check_all(pd, run_gpu(pd, eps=eps, dense=False), eps=eps)


def test_more_than_2pow31_elements():
    """A dense batch of 700,416 rows x 3072 bf16 (2.15e9 elements per tensor,
    past any 32-bit element index): 684 copies of one seeded 1,024-row block,
    laid out on the device, so the oracle checks rows sampled across the whole
    batch against the block's rows and each column sum against 684 times the
    block's (computed in fp64)."""
    import diffusion_transformer_adaln_amd as adaln
    from gpu_helpers import TOL, assert_rel_floored, to_host64

    D, NB, REP = 3072, 1024, 684
    N = NB * REP
    assert N * D > 2 ** 31
    pd = _pd("bf16", D, [NB], seed=77, dy_sigma=1e-2)
    p = pd.problem
    say(f"[2^31] bf16 B=1 N={N} D={D}")
    x = to_dev(pd.x, "bf16").repeat(REP, 1).view(1, N, D)
    dy = to_dev(pd.dy, "bf16").repeat(REP, 1).view(1, N, D)
    shift, scale = to_dev(pd.shift, "bf16"), to_dev(pd.scale, "bf16")
    y, mean, rstd = adaln.adaln_fwd(x, shift, scale, p.eps)
    dx, ds, dh = adaln.adaln_bwd(dy, x, scale, mean, rstd)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(5))
    big = np.unique(np.concatenate([g.choice(N, 64, replace=False),
                                    [0, 1, N - 1, 2 ** 31 // D, 2 ** 31 // D + 1]])).astype(np.int64)
    idx = torch.from_numpy(big).cuda()
    got = {"y": y.view(N, D).index_select(0, idx), "dx": dx.view(N, D).index_select(0, idx),
           "mean": mean.view(N).index_select(0, idx), "rstd": rstd.view(N).index_select(0, idx)}
    # every repeat of a block row gives the same bits
    blk = big % NB
    for k, v in got.items():
        first = {}
        for i, r in enumerate(blk.tolist()):
            if r in first:
                assert torch.equal(v[i], v[first[r]]), f"{k}: repeats of block row {r} differ"
            else:
                first[r] = i
    # the block's rows against the oracle
    keep = np.array(sorted(first.values()))
    out = {"y": torch.zeros(NB, D, dtype=torch.bfloat16, device="cuda"),
           "dx": torch.zeros(NB, D, dtype=torch.bfloat16, device="cuda"),
           "mean": torch.zeros(NB, device="cuda"), "rstd": torch.zeros(NB, device="cuda")}
    bidx = torch.from_numpy(blk[keep]).cuda()
    kidx = torch.from_numpy(keep).cuda()
    for k in out:
        out[k].index_copy_(0, bidx, got[k].index_select(0, kidx))
    res = check_rows(pd, out, blk[keep])
    # column sums: REP times the block's
    xo, dyo = oracle.decode(pd.x, "bf16"), oracle.decode(pd.dy, "bf16")
    _, ds_ref, dh_ref = oracle.adaln_bwd(dyo, xo, oracle.decode(pd.scale, "bf16"), p.eps, pd.offsets)
    res["dscale_rel"] = assert_rel_floored(to_host64(ds), REP * ds_ref, TOL["bf16"]["rel"], "dscale")
    res["dshift_rel"] = assert_rel_floored(to_host64(dh), REP * dh_ref, TOL["bf16"]["rel"], "dshift")
    say(f"  rows={keep.size} {res}")
    del x, dy, y, dx, mean, rstd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_pointers_take_general_path(dtype):
    import diffusion_transformer_adaln_amd as adaln

    pd = _pd(dtype, 256, [37, 37], seed=9)
    p = pd.problem
    say(f"[misaligned] {dtype}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    n = p.R * p.D

    def shifted(arr):
        t = to_dev(arr.reshape(-1), dtype)
        buf = torch.empty(n + 1, dtype=tdt, device="cuda")
        buf[1:] = t
        return buf[1:]            # 4- or 2-byte offset from a 256-byte-aligned allocation

    x = shifted(pd.x).view(p.B, p.N, p.D)
    dy = shifted(pd.dy).view(p.B, p.N, p.D)
    shift, scale = to_dev(pd.shift, dtype), to_dev(pd.scale, dtype)
    y, mean, rstd = adaln.adaln_fwd(x, shift, scale, p.eps)
    dx, ds, dh = adaln.adaln_bwd(dy, x, scale, mean, rstd)
    out = {"y": y.view(-1, p.D), "mean": mean.view(-1), "rstd": rstd.view(-1), "dx": dx.view(-1, p.D),
           "dscale": ds, "dshift": dh}
    check_all(pd, out)


def test_empty_batch_and_empty_samples():
    import diffusion_transformer_adaln_amd as adaln

    say("[empty] N=0 dense")
    x = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    shift = torch.randn(2, 64, device="cuda").to(torch.bfloat16)
    scale = torch.randn(2, 64, device="cuda").to(torch.bfloat16)
    y, mean, rstd = adaln.adaln_fwd(x, shift, scale, 1e-6)
    assert y.shape == (2, 0, 64)
    ds = torch.full((2, 64), 7.0, device="cuda").to(torch.bfloat16)
    dh = torch.full((2, 64), 7.0, device="cuda").to(torch.bfloat16)
    adaln.adaln_bwd(x, x.clone(), scale, mean, rstd, dscale=ds, dshift=dh)
    torch.cuda.synchronize()
    assert not ds.float().any() and not dh.float().any()
    say("[empty] varlen with empty samples")
    pd = _pd("bf16", 3072, [0, 17, 0, 0, 40, 0], seed=11, dense=False)
    check_all(pd, run_gpu(pd))
    pd = _pd("f32", 96, [0, 0, 0], seed=12, dense=False)
    out = run_gpu(pd)
    assert not out["dscale"].any() and not out["dshift"].any()


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 5120), ("bf16", 100)])
def test_constant_rows(dtype, D):
    """Zero-variance rows: rstd = eps^-1/2, y = shift, dx = rstd*(g - mean(g))."""
    pd = _pd(dtype, D, [40], seed=13)
    const = workloads.encode_bf16_rne(np.full(D, 3.25, np.float32)) if dtype == "bf16" else np.full(D, 3.25, np.float32)
    pd.x[::3] = const
    say(f"[constant rows] {dtype} D={D}")
    for eps in (1e-6, 1e-2):
        # rstd = eps^-1/2 makes |dx| large: outside the workloads' range, where
        # the bf16 format itself sets the error floor
        check_all(pd, run_gpu(pd, eps=eps), eps=eps, strict=False)
    # exactly, for every forward kernel: mean = the value, rstd = 1/sqrt(eps)
    # (fp32, both steps correctly rounded), y = shift bit for bit
    eps = 1e-6
    out = run_gpu(pd, eps=eps)
    mean = out["mean"].cpu().numpy()[::3]
    rstd = out["rstd"].cpu().numpy()[::3]
    assert np.all(mean == np.float32(3.25)), mean
    assert np.all(rstd == np.float32(1.0) / np.sqrt(np.float32(eps))), rstd
    bits_t = torch.int16 if dtype == "bf16" else torch.int32
    y = out["y"][::3].contiguous().view(bits_t).cpu().numpy()
    want = to_dev(pd.shift, dtype)[0].contiguous().view(bits_t).cpu().numpy()   # one sample
    assert np.array_equal(y, np.broadcast_to(want, y.shape)), "y of a constant row is not shift"
    # eps = 0: a zero-variance row has no defined normalisation; its rstd is
    # +inf (1/sqrt(0)), as the formula gives in floating point, and the other
    # rows are untouched by it; dshift (a plain sum of dy) stays finite
    out = run_gpu(pd, eps=0.0)
    rstd = out["rstd"].cpu().numpy()
    assert np.all(np.isposinf(rstd[::3])), rstd[::3]
    keep = np.ones(pd.problem.R, dtype=bool)
    keep[::3] = False
    assert np.all(np.isfinite(rstd[keep]))
    for k in ("y", "dx"):
        assert torch.isfinite(out[k][torch.from_numpy(keep).cuda()].float()).all(), k
    assert torch.isfinite(out["dshift"].float()).all()


# Per-row offsets far above the row's spread (|mean|/std up to ~200 in fp32):
# the statistics must not cancel.  A one-pass E[x^2] - E[x]^2 variance in fp32
# loses most of its digits here (xhat off by ~3e-2 in an fp32 emulation, 300x
# the fp32 bound on y and dx); per-lane two-pass sums merged with Chan's update
# stay near 1e-5.  The dscale bound adds the rounding of the fp32 row mean
# itself (a few u*|mean| per row, common to the whole row), which no fp32
# implementation avoids.  One case per forward kernel: the one-wave-per-row
# kernel (D = 5120 bf16, D = 1280 fp32), the slot kernel (D = 4096 fp32,
# D = 1152 bf16, packed), the general kernel (D = 100).
OFFSET_CASES = [("f32", 1280, [40], 64.0), ("f32", 4096, [70], 64.0), ("f32", 100, [33, 9], 64.0),
                ("bf16", 5120, [300], 32.0), ("bf16", 1152, [3, 50, 7], 32.0)]


@pytest.mark.parametrize("dtype,D,lengths,sigma", OFFSET_CASES,
                         ids=[f"{d}-D{D}-{'x'.join(map(str, l))}" for d, D, l, _ in OFFSET_CASES])
def test_large_row_offsets(dtype, D, lengths, sigma):
    pd = _pd(dtype, D, lengths, seed=17 + D, dy_sigma=1.0 if dtype == "f32" else 1e-2,
             row_offset_sigma=sigma)
    say(f"[row offsets] {dtype} D={D} lengths={lengths} sigma={sigma}")
    check_all(pd, run_gpu(pd), mean_rounding=True)


# ---------------------------------------------------------------------------
# determinism and dense == packed
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,lengths", [("bf16", 5120, [3000]), ("bf16", 1152, [700] * 4), ("f32", 128, [999])])
def test_run_to_run_bitwise(dtype, D, lengths):
    pd = _pd(dtype, D, lengths, seed=21)
    say(f"[determinism] {dtype} D={D} lengths={lengths}")
    ref = None
    for _ in range(20):
        out = run_gpu(pd)
        h = {k: hashlib.sha256(bits(v)).hexdigest() for k, v in out.items()}
        if ref is None:
            ref = h
        assert h == ref, "outputs differ between runs"


@pytest.mark.parametrize("dtype,D,N,B", [("bf16", 3072, 515, 3), ("f32", 128, 300, 2), ("bf16", 100, 33, 2)])
def test_dense_and_packed_agree(dtype, D, N, B):
    """Row outputs are computed identically by both entry points (bitwise);
    the column sums may group tiles differently (packed batches use shorter
    tiles), so they must agree to the accuracy contract."""
    pd = _pd(dtype, D, [N] * B, seed=31)
    say(f"[dense vs packed] {dtype} D={D} N={N} B={B}")
    a = run_gpu(pd, dense=True)
    b = run_gpu(pd, dense=False)
    for k in ("y", "mean", "rstd", "dx"):
        assert bits(a[k]) == bits(b[k]), k
    check_all(pd, a)
    check_all(pd, b)


# ---------------------------------------------------------------------------
# the two-pass (unfused D-tile) backward
# ---------------------------------------------------------------------------
TWOPASS = [("bf16", 5120, [1000]), ("bf16", 1152, [300] * 3), ("bf16", 3072, [77, 77]),
           ("f32", 128, [999]), ("f32", 4096, [70]), ("bf16", 128, [255]), ("bf16", 16384, [5]),
           ("bf16", 3072, [1])]


@pytest.mark.parametrize("dtype,D,lengths", TWOPASS,
                         ids=[f"{d}-D{D}-{'x'.join(map(str, l))}" for d, D, l in TWOPASS])
def test_twopass_backward(dtype, D, lengths):
    """Oracle parity for the two-pass backward; its dx is the fused path's dx
    bit for bit (same row kernel), its column sums add the same terms in
    another fixed order."""
    pd = _pd(dtype, D, lengths, seed=41 + D, dy_sigma=1.0 if dtype == "f32" else 1e-2)
    say(f"[twopass] {dtype} D={D} lengths={lengths}")
    a = run_gpu(pd, twopass=True)
    check_all(pd, a)
    b = run_gpu(pd)
    for k in ("y", "mean", "rstd", "dx"):
        assert bits(a[k]) == bits(b[k]), k
    h = {k: hashlib.sha256(bits(a[k])).hexdigest() for k in ("dscale", "dshift")}
    for _ in range(3):
        c = run_gpu(pd, twopass=True)
        assert {k: hashlib.sha256(bits(c[k])).hexdigest() for k in ("dscale", "dshift")} == h


def test_twopass_full_size_video_sampled():
    pd = workloads.make_config("video_bf16")[0]
    say("[twopass-full] video_bf16")
    out = run_gpu(pd, twopass=True)
    res = check_rows(pd, out, sampled_rows(pd))
    res.update(check_samples(pd, out, np.arange(pd.problem.B)))
    say(f"  {res}")


def test_twopass_rejects_unvectorised_shapes():
    import diffusion_transformer_adaln_amd as adaln

    say("[twopass] unsupported shapes")
    # D = 100 bf16: rows are not whole 16-byte vectors; D = 64 bf16: 8 vectors,
    # fewer than one 16-lane group; D = 127 fp32: odd
    for D, dt in ((100, torch.bfloat16), (64, torch.bfloat16), (127, torch.float32)):
        x = torch.randn(1, 8, D, device="cuda").to(dt)
        sc = torch.zeros(1, D, device="cuda").to(dt)
        y, mean, rstd = adaln.adaln_fwd(x, sc, sc, 1e-6)
        with pytest.raises(adaln.AdaLNError) as e:
            adaln.adaln_bwd_twopass(x, x.clone(), sc, mean, rstd)
        assert e.value.status == 3


# ---------------------------------------------------------------------------
# error codes through the real library
# ---------------------------------------------------------------------------
def test_error_codes_on_device():
    import diffusion_transformer_adaln_amd as adaln

    say("[errors]")
    x = torch.randn(2, 16, 64, device="cuda").to(torch.bfloat16)
    sh = torch.zeros(2, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(adaln.AdaLNError) as e:
        adaln.adaln_fwd(x, sh, sh, 1e-6, y=x)                       # output aliases input
    assert e.value.status == 5
    y, mean, rstd = adaln.adaln_fwd(x, sh, sh, 1e-6)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(adaln.AdaLNError) as e:
        adaln.adaln_bwd(x, x, sh, mean, rstd, workspace=small)
    assert e.value.status == 4
    with pytest.raises(adaln.AdaLNError) as e:
        adaln.adaln_fwd(x, sh, sh, float("nan"))
    assert e.value.status == 1
    assert adaln.adaln_bwd_workspace_size(2, 32, 64, torch.bfloat16) > 0


def test_single_hip_runtime_mapped():
    import diffusion_transformer_adaln_amd as adaln

    adaln.load_library()
    libs = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_concurrent_streams_match_serial():
    """Calls on different streams with disjoint buffers (each its own
    workspace) may run concurrently: two problems interleaved on two streams
    give the bits each gives on its own."""
    import diffusion_transformer_adaln_amd as adaln

    def setup(pd):
        p = pd.problem
        t = {"x": to_dev(pd.x, "bf16"), "dy": to_dev(pd.dy, "bf16"), "sh": to_dev(pd.shift, "bf16"),
             "sc": to_dev(pd.scale, "bf16"), "off": torch.from_numpy(pd.offsets).cuda(),
             "ws": torch.empty(adaln.adaln_bwd_workspace_size(p.B, p.R, p.D, torch.bfloat16),
                               dtype=torch.uint8, device="cuda")}
        t["y"], t["dx"] = torch.empty_like(t["x"]), torch.empty_like(t["x"])
        t["mean"], t["rstd"] = torch.empty(p.R, device="cuda"), torch.empty(p.R, device="cuda")
        t["ds"], t["dh"] = torch.empty_like(t["sc"]), torch.empty_like(t["sc"])
        return t

    def call(pd, t):
        p = pd.problem
        if p.dense:
            v = lambda a: a.view(p.B, p.N, p.D)
            m, r = t["mean"].view(p.B, p.N), t["rstd"].view(p.B, p.N)
            adaln.adaln_fwd(v(t["x"]), t["sh"], t["sc"], p.eps, y=v(t["y"]), mean=m, rstd=r)
            adaln.adaln_bwd(v(t["dy"]), v(t["x"]), t["sc"], m, r, workspace=t["ws"], dx=v(t["dx"]),
                            dscale=t["ds"], dshift=t["dh"])
        else:
            adaln.adaln_fwd_varlen(t["x"], t["sh"], t["sc"], t["off"], p.eps, y=t["y"], mean=t["mean"],
                                   rstd=t["rstd"])
            adaln.adaln_bwd_varlen(t["dy"], t["x"], t["sc"], t["mean"], t["rstd"], t["off"], workspace=t["ws"],
                                   dx=t["dx"], dscale=t["ds"], dshift=t["dh"])

    keys = ("y", "mean", "rstd", "dx", "ds", "dh")
    pa = _pd("bf16", 5120, [2000], seed=61)
    pb = _pd("bf16", 3072, [700, 33, 800], seed=62, dense=False)
    say("[streams] two problems on two streams")
    ta, tb = setup(pa), setup(pb)
    call(pa, ta)
    call(pb, tb)
    torch.cuda.synchronize()
    ref_a = {k: bits(ta[k]) for k in keys}
    ref_b = {k: bits(tb[k]) for k in keys}
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        for k in keys:
            ta[k].zero_()
            tb[k].zero_()
        torch.cuda.synchronize()
        for _ in range(3):
            with torch.cuda.stream(sa):
                call(pa, ta)
            with torch.cuda.stream(sb):
                call(pb, tb)
        torch.cuda.synchronize()
        assert {k: bits(ta[k]) for k in keys} == ref_a, "stream A differs from its serial result"
        assert {k: bits(tb[k]) for k in keys} == ref_b, "stream B differs from its serial result"


# ---------------------------------------------------------------------------
# HIP graph capture
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dense", [True, False])
def test_graph_capture_replays_match_eager(dense):
    """The entry points launch kernels only (no allocation, memset or
    synchronisation), so a caller can capture them in a HIP graph.  Every
    replay, with eager work and synchronisations in between, must give the
    eager call's bits."""
    import diffusion_transformer_adaln_amd as adaln

    pd = _pd("bf16", 3072, [300] * 3 if dense else [300, 129, 64], seed=51, dense=dense)
    p = pd.problem
    say(f"[graph] dense={dense}")
    x, dy = to_dev(pd.x, "bf16"), to_dev(pd.dy, "bf16")
    sh, sc = to_dev(pd.shift, "bf16"), to_dev(pd.scale, "bf16")
    off = torch.from_numpy(pd.offsets).cuda()
    ws = torch.empty(adaln.adaln_bwd_workspace_size(p.B, p.R, p.D, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    y, dx = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(p.R, device="cuda")
    rstd = torch.empty(p.R, device="cuda")
    ds = torch.empty(p.B, p.D, dtype=torch.bfloat16, device="cuda")
    dh = torch.empty_like(ds)

    def call():
        if dense:
            v = lambda t: t.view(p.B, p.N, p.D)
            adaln.adaln_fwd(v(x), sh, sc, p.eps, y=v(y), mean=mean.view(p.B, p.N), rstd=rstd.view(p.B, p.N))
            adaln.adaln_bwd(v(dy), v(x), sc, mean.view(p.B, p.N), rstd.view(p.B, p.N), workspace=ws, dx=v(dx),
                            dscale=ds, dshift=dh)
        else:
            adaln.adaln_fwd_varlen(x, sh, sc, off, p.eps, y=y, mean=mean, rstd=rstd)
            adaln.adaln_bwd_varlen(dy, x, sc, mean, rstd, off, workspace=ws, dx=dx, dscale=ds, dshift=dh)

    outs = lambda: {k: bits(t) for k, t in (("y", y), ("mean", mean), ("rstd", rstd), ("dx", dx),
                                            ("dscale", ds), ("dshift", dh))}
    call()
    torch.cuda.synchronize()
    ref = outs()
    check_all(pd, {"y": y, "mean": mean, "rstd": rstd, "dx": dx, "dscale": ds, "dshift": dh})
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()                          # warm-up on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        for t in (y, dx, mean, rstd, ds, dh, ws):
            t.zero_()                   # eager work between replays; the graph must rewrite it all
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert outs() == ref, f"replay {rep} differs from the eager call"
