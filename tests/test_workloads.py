"""Seeded input generators: encoding, reproducibility, shapes, bucket sizes."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import configs as wc


def test_bf16_encoding_matches_torch_rne():
    g = np.random.Generator(np.random.PCG64(7))
    f = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(10.0),
        # exact ties: low 16 bits = 0x8000, both parities of the kept lsb
        (np.arange(0, 4000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38], dtype=np.float32),
    ])
    f = f[np.isfinite(f) | np.isinf(f)]
    got = workloads.encode_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = workloads.encode_bf16_rne(np.array([np.nan], dtype=np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_draws_independent_of_thread_count(monkeypatch):
    p = workloads.custom_problem("bf16", 1024, [6000], dy_sigma=1e-2)   # > one chunk of draws
    monkeypatch.setattr(wc, "_threads", lambda: 1)
    a = workloads.make_problem_data(p, 17)
    monkeypatch.setattr(wc, "_threads", lambda: 7)
    b = workloads.make_problem_data(p, 17)
    for name in ("x", "shift", "scale", "dy"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = workloads.make_problem_data(p, 18)
    assert not np.array_equal(a.x, c.x)


@pytest.mark.parametrize("name", ["tiny_fp32", "dit_bf16", "mmdit_bf16"])
def test_config_shapes_and_distributions(name):
    for pd in workloads.make_config(name):
        p = pd.problem
        assert pd.x.shape == (p.R, p.D) and pd.dy.shape == (p.R, p.D)
        assert pd.shift.shape == (p.B, p.D) and pd.scale.shape == (p.B, p.D)
        assert pd.offsets[0] == 0 and pd.offsets[-1] == p.R and pd.offsets.dtype == np.int64
        want = np.float32 if p.dtype == "f32" else np.uint16
        assert pd.x.dtype == want
        sc = oracle.decode(pd.scale, p.dtype)
        assert abs(sc.std() - 0.1) < 0.02
        dy = oracle.decode(pd.dy, p.dtype)
        assert abs(dy.std() / p.dy_sigma - 1) < 0.05
        if p.outlier_frac:
            rows = pd.meta["outlier_rows"]
            assert rows.size == round(0.01 * p.R)
            x = oracle.decode(pd.x, p.dtype)
            assert np.abs(x[rows]).mean() > 10 * np.abs(np.delete(x, rows, axis=0)).mean()


def test_tiny_row_offsets():
    pd = workloads.make_config("tiny_fp32")[0]
    m = pd.x.astype(np.float64).mean(axis=1)
    assert 1.5 < m.std() < 2.5          # per-row offset ~N(0, 2) dominates the row means


def test_ragged_buckets_follow_the_page_rule():
    total = 0
    for S, count in workloads.RAGGED_BUCKETS:
        assert oracle.b_shape(S, 65536, 2 ** 30, 2) == count
        total += S * count
    lens = workloads.ragged_lengths()
    assert len(lens) == 277 and sum(lens) == total == 229368
    sh = workloads.ragged_lengths(shuffle_seed=3)
    assert sorted(sh) == sorted(lens) and sh != lens


def test_algorithmic_bytes_video():
    p = workloads.CONFIGS["video_bf16"][0]
    b = workloads.algorithmic_bytes(p)
    assert b["fwd"] == 387_243_680 and b["bwd"] == 580_789_920 and b["total"] == 968_033_600


def test_packed_workload_is_its_problems_back_to_back():
    """pack() lays several problems' samples out in order, rows concatenated,
    each sample keeping its modulation, with the same algorithmic bytes as the
    separate calls; the packed MMDiT workload is the two MMDiT streams."""
    a = workloads.make_problem_data(workloads.custom_problem("bf16", 64, [5, 5], outlier_frac=0.1), 1)
    b = workloads.make_problem_data(workloads.custom_problem("bf16", 64, [9, 9]), 2)
    pk = workloads.pack([a, b], "packed_test")
    p = pk.problem
    assert not p.dense and p.lengths == (5, 5, 9, 9) and p.R == 28 and p.B == 4
    assert list(pk.offsets) == [0, 5, 10, 19, 28]
    for k in ("x", "dy", "shift", "scale"):
        assert np.array_equal(getattr(pk, k), np.concatenate([getattr(a, k), getattr(b, k)])), k
    total = sum(workloads.algorithmic_bytes(q.problem)["total"] for q in (a, b))
    assert workloads.algorithmic_bytes(p)["total"] == total
    assert workloads.PACKED_CONFIGS["mmdit_packed_bf16"] == "mmdit_bf16"
    assert [q.lengths for q in workloads.CONFIGS["mmdit_bf16"]] == [(512, 512), (4096, 4096)]
    assert "mmdit_packed_bf16" in workloads.config_names()
