"""fp32 column sums (adaln_bwd_f32sums, adaln_bwd_varlen_f32sums) and the
single rounding of every column sum, through the C ABI.

- The fp32-sum entry points return the same dx as adaln_bwd / adaln_bwd_varlen
  (bitwise), and column sums that match the fp64 oracle to the fp32 bound
  (1e-4, floored relative) whatever the I/O type; with fp32 I/O every output
  is bitwise that of the I/O-typed entry point.  A bf16 column sum is the
  fp32 one rounded to bf16, except where the fp32 value is exactly halfway
  between two bf16 values (there the fp64 sum decides).
- A bf16 column sum is rounded once from the fp64 sum: a column whose exact
  sum is 1 + 2^-8 + 2^-30 (just above the midpoint of 1 and 1 + 2^-7) gives
  1 + 2^-7, where rounding through fp32 first would land on the midpoint and
  tie to 1.
- A sequence split into shares whose fp32 column sums are added in share
  order (what a sequence-parallel group does across devices) matches the
  whole sequence's oracle sums to the fp32 bound, and the shares' dx rows are
  bitwise the whole call's.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_adaln_amd as adaln
import oracle
import workloads
from gpu_helpers import TOL, assert_rel_floored, bits, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _upload(pd):
    p = pd.problem
    return (to_dev(pd.x, p.dtype), to_dev(pd.dy, p.dtype), to_dev(pd.shift, p.dtype),
            to_dev(pd.scale, p.dtype), torch.from_numpy(pd.offsets).cuda())


def _fwd_bwd(pd, x, dy, shift, scale, off, f32sums):
    p = pd.problem
    if p.dense:
        B, N, D = p.B, p.N, p.D
        y, mean, rstd = adaln.adaln_fwd(x.view(B, N, D), shift, scale, p.eps)
        fn = adaln.adaln_bwd_f32sums if f32sums else adaln.adaln_bwd
        dx, ds, dh = fn(dy.view(B, N, D), x.view(B, N, D), scale, mean, rstd)
    else:
        y, mean, rstd = adaln.adaln_fwd_varlen(x, shift, scale, off, p.eps)
        fn = adaln.adaln_bwd_varlen_f32sums if f32sums else adaln.adaln_bwd_varlen
        dx, ds, dh = fn(dy, x, scale, mean, rstd, off)
    torch.cuda.synchronize()
    return dx, ds, dh


def _oracle_sums(pd):
    p = pd.problem
    x = oracle.decode(pd.x, p.dtype)
    dy = oracle.decode(pd.dy, p.dtype)
    scale = oracle.decode(pd.scale, p.dtype)
    _, ds, dh = oracle.adaln_bwd(dy, x, scale, p.eps, pd.offsets)
    return ds, dh


def _check_bf16_is_f32_rounded(io, f32, what):
    """io (bf16) is f32 rounded to nearest-even bf16, except at exact bf16
    midpoints of f32, where either neighbour is a correct rounding of the
    fp64 sum behind both."""
    u = f32.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)
    got = io.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    want = f32.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    mid = (u & 0xFFFF) == 0x8000
    assert np.array_equal(got[~mid], want[~mid]), f"{what}: bf16 sum is not the fp32 sum rounded"
    lo = u[mid] >> 16
    assert np.all((got[mid] == lo) | (got[mid] == lo + 1)), f"{what}: bf16 sum at a midpoint off both neighbours"
    return int(mid.sum())


CASES = [
    ("bf16", 1152, [300] * 3, True),                 # vector row pass, several row slots per workgroup
    ("bf16", 5120, [1000], True),                    # video row width
    ("bf16", 3072, [5, 0, 300, 1, 129, 64], False),  # packed, an empty and a one-row sample
    ("bf16", 3072, [7] * 20, False),                 # packed, more samples than the narrow finish takes
    ("bf16", 98, [40, 40], True),                    # general row pass, per-column finish
    ("f32", 128, [256], True),                       # tiny workload's shape
    ("f32", 1152, [33, 0, 200], False),
]


@pytest.mark.parametrize("dtype,D,lengths,dense", CASES)
def test_f32sums_match_oracle_and_io_entry(dtype, D, lengths, dense):
    pd = workloads.make_problem_data(workloads.custom_problem(dtype, D, lengths, dense=dense), seed=11)
    say(f"[f32sums] {dtype} D={D} lengths={lengths[:6]} dense={dense}")
    ins = _upload(pd)
    dx_io, ds_io, dh_io = _fwd_bwd(pd, *ins, f32sums=False)
    dx_32, ds_32, dh_32 = _fwd_bwd(pd, *ins, f32sums=True)
    assert ds_32.dtype == torch.float32 and dh_32.dtype == torch.float32
    assert bits(dx_32) == bits(dx_io), "dx differs between the two entry points"
    ds_ref, dh_ref = _oracle_sums(pd)
    rel = TOL["f32"]["rel"]
    e_s = assert_rel_floored(to_host64(ds_32), ds_ref, rel, "dscale (fp32 sums)")
    e_h = assert_rel_floored(to_host64(dh_32), dh_ref, rel, "dshift (fp32 sums)")
    if dtype == "f32":
        assert bits(ds_32) == bits(ds_io) and bits(dh_32) == bits(dh_io)
        mids = 0
    else:
        mids = _check_bf16_is_f32_rounded(ds_io, ds_32, "dscale") + _check_bf16_is_f32_rounded(dh_io, dh_32, "dshift")
    say(f"  rel dscale {e_s:.2e} dshift {e_h:.2e}; fp32 sums on a bf16 midpoint: {mids}")


# Sample 0 has 12 rows.  Tiles hold at least 4 rows, so its rows split into
# three tiles, and rows 0, 5 and 10 fall into different ones whether a tile
# takes a contiguous run of rows or every third row: each tile's fp32 partial
# of column C holds one of the three values exactly, and only the fp64 finish
# adds them.
C, C_NEG = 7, 9
SUM_EXACT = 1.0 + 2.0 ** -8 + 2.0 ** -30
BF16_ONCE = 1.0 + 2.0 ** -7        # nearest bf16 to SUM_EXACT (it lies above the midpoint 1 + 2^-8)
F32_ONCE = 1.0 + 2.0 ** -8         # nearest fp32 to SUM_EXACT (2^-30 is below half an fp32 ulp at 1)


@pytest.mark.parametrize("D,dense,extra_samples", [(128, True, 0), (128, False, 19), (98, True, 0)])
def test_bf16_column_sums_rounded_once(D, dense, extra_samples):
    lengths = [12] * (1 + extra_samples) if dense else [12] + [5] * extra_samples
    pd = workloads.make_problem_data(workloads.custom_problem("bf16", D, lengths, dense=dense), seed=12)
    dy = np.zeros((pd.problem.R, D), dtype=np.float32)
    for row, v in ((0, 1.0), (5, 2.0 ** -8), (10, 2.0 ** -30)):
        dy[row, C] = v
        dy[row, C_NEG] = -v
    pd.dy = (dy.view(np.uint32) >> 16).astype(np.uint16)      # all exact in bf16
    say(f"[rounding] D={D} dense={dense} samples={len(lengths)}")
    ins = _upload(pd)
    _, _, dh_io = _fwd_bwd(pd, *ins, f32sums=False)
    _, _, dh_32 = _fwd_bwd(pd, *ins, f32sums=True)
    got = to_host64(dh_io)
    assert got[0, C] == BF16_ONCE and got[0, C_NEG] == -BF16_ONCE, (got[0, C], got[0, C_NEG])
    got32 = to_host64(dh_32)
    assert got32[0, C] == F32_ONCE and got32[0, C_NEG] == -F32_ONCE, (got32[0, C], got32[0, C_NEG])
    rest = np.ones(got.shape, dtype=bool)
    rest[0, [C, C_NEG]] = False
    assert not got[rest].any() and not got32[rest].any()


@pytest.mark.parametrize("dtype,D,N,shares", [("bf16", 1152, 4000, 4), ("bf16", 5120, 2400, 4), ("f32", 1152, 999, 3)])
def test_sequence_shares_add_up(dtype, D, N, shares):
    B = 2
    pd = workloads.make_problem_data(workloads.custom_problem(dtype, D, [N] * B, dense=True), seed=13)
    say(f"[shares] {dtype} B={B} N={N} D={D} shares={shares}")
    x, dy, shift, scale, _ = _upload(pd)
    x, dy = x.view(B, N, D), dy.view(B, N, D)
    _, mean, rstd = adaln.adaln_fwd(x, shift, scale, pd.problem.eps)
    dx_w, ds_w, dh_w = adaln.adaln_bwd_f32sums(dy, x, scale, mean, rstd)
    cuts = [N * k // shares for k in range(shares + 1)]
    ds_sp = np.zeros((B, D))
    dh_sp = np.zeros((B, D))
    dx_parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        part = lambda t: t[:, lo:hi].contiguous()
        dx_k, ds_k, dh_k = adaln.adaln_bwd_f32sums(part(dy), part(x), scale, part(mean), part(rstd))
        ds_sp += to_host64(ds_k)                  # added in share order
        dh_sp += to_host64(dh_k)
        dx_parts.append(dx_k)
    torch.cuda.synchronize()
    assert bits(torch.cat(dx_parts, dim=1)) == bits(dx_w), "a share's dx rows differ from the whole call's"
    ds_ref, dh_ref = _oracle_sums(pd)
    rel = TOL["f32"]["rel"]
    e_s = assert_rel_floored(ds_sp, ds_ref, rel, "dscale (shares added)")
    e_h = assert_rel_floored(dh_sp, dh_ref, rel, "dshift (shares added)")
    e_ws = assert_rel_floored(to_host64(ds_w), ds_ref, rel, "dscale (whole)")
    say(f"  shares added: rel dscale {e_s:.2e} dshift {e_h:.2e}; whole sequence dscale {e_ws:.2e}")
