"""Benchmark of the fused AdaLN forward + backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config video_bf16]

A step is one forward and one backward call of the workload (every hot-path
kernel: forward, backward row pass, backward finish) over one resident batch
of seeded synthetic bf16 inputs.  The default workload is the video-DiT
AdaLN at one device's sequence share: B=1, N=18900, D=5120.

S copies of the inputs and outputs stay resident in HBM (S >= 4, enough that
about 1 GB of other traffic separates two touches of one copy; six for the
video workload).  Step k runs the forward on copy k % S and the backward on
copy (k + S/2) % S, the way a layer's backward runs long after its forward in
training: no kernel reads data another kernel touched within the last ~1 GB
of traffic, so the 256 MB Infinity Cache cannot serve it and the figures are
HBM figures.  The warm-up runs at least 100 ms by default (the chip needs
~20 ms under load to settle) unless --warmup fixes its step count.

Output: one JSON line.  `value` is the whole-job throughput in GB/s of
algorithmic bytes (the minimal traffic of the method, see
workloads.algorithmic_bytes) over the wall-clock time of the K timed steps,
bracketed by device synchronisation; nothing else runs on the stream in that
region (`gpu_ms_per_step` is the same region timed by two events on the
launch stream).  `roofline` covers the backward call, the dominant one:
algorithmic bytes per call / mean call duration from HIP events recorded on
the launch stream right after the timed region, one event pair around each
block of ten back-to-back calls (each timing event stalls the queue for a
few microseconds, which is why none sits inside the timed region and why a
pair does not bracket a single call); `per_call_us` gives the 10th, 50th and
90th percentiles of those block means for the forward and the backward.
`device` records the GPU's name, architecture, CU count and memory (a
partitioned device shows fewer CUs and a slice of the bandwidth).
`cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload's rows on one host core, and reports the GPU path's errors on the
rows it computed (y, dx, rstd against the oracle: `errors`).

`ceilings` measures what the device delivers for the operator's access
mixes with the library's streaming probes (include/adaln_probe.h), on
buffers of the workload's own [R, D] size, after the timed region: a copy
(one read, one write: the forward's mix) and two reads to one write (the
backward row pass's), each the best of a small sweep of launch shapes.
`step_gbs` is the rate a step would reach if its forward bytes moved at the
copy rate and its backward bytes at the two-to-one rate, and
`pct_of_copy_ceiling` is `value` against it.  Small tensors (DiT's 19 MB)
are dominated by launch and ramp costs, which the same sweep measures for
plain streaming as well.  `versions` records ROCm,
HIP and torch, and `device.compute_partition` the partition mode.

`--bwd twopass` runs the backward through adaln_bwd_twopass instead (dx
pass, then a separate D-tile column pass that reads dy and x again): the
same work with more traffic, to measure what the fusion saves.  `--bwd
f32sums` runs the fp32-column-sum entry points (the same kernels; the byte
count stays that of the I/O-typed sums, 2*B*D*s fewer bytes than written).

`--cost-sweep` does the shape benchmarking of the batch scheduler instead
(see cost_sweep) and prints its own JSON line.

`--clock-trace` runs the same schedule (priming, warm-up, K steps) with the
engine clock sampled beside it by the library's clock probe on a second
stream, and prints the clock over time and per step instead of a throughput
line (see clock_trace).

`--impl torch` runs the unfused chain an eager framework executes instead
(LayerNorm without affine, multiply by 1 + scale, add shift; backward by
autograd), on the same resident copies, for context.  Every line reports
`activation_bytes`: what the forward keeps alive for the backward beyond
the inputs (the fused path: mean and rstd, 8 bytes per row).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak, GB/s
METRIC = "AdaLN fwd+bwd achieved HBM GB/s (% of MI355X peak) and rows/s, bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: as many as take at least --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="minimum warm-up time when --warmup is not given")
    ap.add_argument("--config", default="video_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "adaln_bwd_video_bf16_traffic.txt"),
                    help="measured HBM bytes per backward call (from rocprofv3 counters), if present")
    ap.add_argument("--bwd", choices=("fused", "twopass", "f32sums"), default="fused",
                    help="backward entry point: the fused adaln_bwd; adaln_bwd_twopass (dx pass, then "
                         "a separate D-tile column pass that reads dy and x again; dense workloads only); "
                         "or adaln_bwd_f32sums / adaln_bwd_varlen_f32sums (fp32 column sums)")
    ap.add_argument("--impl", choices=("hip", "torch"), default="hip",
                    help="hip: this library's kernels; torch: the unfused eager-PyTorch chain (dense "
                         "workloads only), for comparison")
    ap.add_argument("--cost-sweep", action="store_true",
                    help="time a synthetic per-group step over (B, S), fit step = a + b*B*S^p with "
                         "adaln_cost_fit and compare equal-token and dual-constraint grouping")
    ap.add_argument("--clock-trace", action="store_true",
                    help="sample the engine clock beside the bench's schedule (diagnostic; prints its own line)")
    ap.add_argument("--clock-samples", type=int, default=20000,
                    help="most clock samples --clock-trace takes")
    ap.add_argument("--clock-per-step", type=int, default=4,
                    help="clock samples queued with each step for --clock-trace (keep their total "
                         "time near the step's)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (counter calibration)")
    return ap.parse_args()


def upload(pd):
    import numpy as np
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if pd.problem.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    return {"x": dev(pd.x), "dy": dev(pd.dy), "shift": dev(pd.shift), "scale": dev(pd.scale),
            "offsets": torch.from_numpy(pd.offsets).cuda()}


def eager_adaln(x, shift, scale, eps):
    """The unfused chain an eager framework runs for AdaLN on [B, N, D]:
    LayerNorm without affine, multiply by (1 + scale), add shift, the
    modulation broadcast over N.  Each step is its own kernel, and autograd
    keeps what each step's backward needs."""
    import torch.nn.functional as F

    ln = F.layer_norm(x, (x.shape[-1],), eps=eps)
    return ln * (1 + scale[:, None, :]) + shift[:, None, :]


def saved_activation_bytes(fn, *args):
    """Run fn(*args) and count the bytes of the distinct storages autograd
    saves for its backward, leaving out the storages of the arguments
    themselves (the caller holds those anyway).  Returns (output, bytes)."""
    import torch

    inputs = {a.untyped_storage().data_ptr() for a in args if torch.is_tensor(a)}
    seen = {}

    def pack(t):
        st = t.untyped_storage()
        if st.data_ptr() not in inputs:
            seen[st.data_ptr()] = st.nbytes()
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        out = fn(*args)
    return out, sum(seen.values())


def cpu_baseline(pd, seconds, gpu_rows=None):
    """fp64 oracle on successive 128-row blocks of the workload (wrapping
    around to the first row after the last) until about `seconds` of CPU
    time; rows are independent, and each block's column sums are taken over
    its own rows (the same per-row work as the full sums).

    gpu_rows(lo, hi) -> (y, dx, rstd) as float64 arrays, when given: the GPU
    path's outputs of those rows, compared with the oracle's for the blocks of
    the first pass (errors: max abs error of y and dx, max relative error of
    rstd)."""
    import numpy as np

    import oracle

    p = pd.problem
    rows_done, t_used = 0, 0.0
    block = 128
    start = 0
    err = {"y_max_abs": 0.0, "dx_max_abs": 0.0, "rstd_max_rel": 0.0, "rows": 0}
    while t_used < seconds:
        if start >= p.R:
            start = 0
        lo, hi = start, min(p.R, start + block)
        b = int(oracle.sample_of_rows(pd.offsets, np.array([lo]))[0])
        hi = min(hi, int(pd.offsets[b + 1]))
        x = oracle.decode(pd.x[lo:hi], p.dtype)
        dy = oracle.decode(pd.dy[lo:hi], p.dtype)
        sh = oracle.decode(pd.shift[b:b + 1], p.dtype)
        sc = oracle.decode(pd.scale[b:b + 1], p.dtype)
        off = np.array([0, hi - lo], dtype=np.int64)
        t0 = time.process_time()
        y_ref, _, rstd_ref = oracle.adaln_fwd(x, sh, sc, p.eps, off)
        dx_ref, _, _ = oracle.adaln_bwd(dy, x, sc, p.eps, off)
        t_used += time.process_time() - t0
        if gpu_rows is not None and rows_done < p.R:
            y, dx, rstd = gpu_rows(lo, hi)
            err["y_max_abs"] = max(err["y_max_abs"], float(np.abs(y - y_ref).max()))
            err["dx_max_abs"] = max(err["dx_max_abs"], float(np.abs(dx - dx_ref).max()))
            err["rstd_max_rel"] = max(err["rstd_max_rel"], float((np.abs(rstd - rstd_ref) / rstd_ref).max()))
            err["rows"] += hi - lo
        rows_done += hi - lo
        start = hi
    import workloads

    per_row = workloads.algorithmic_bytes(p)["total"] / p.R
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    out = {
        "value": round(rows_done * per_row / t_used / 1e9, 4),
        "unit": "GB/s",
        "rows_per_s": round(rows_done / t_used, 1),
        "cores": 1,
        "cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd over {rows_done} rows of {p.name} (D={p.D}, "
                  f"{rows_done / p.R:.2f} passes over its {p.R} rows), 128-row blocks, "
                  f"{t_used:.1f} s of CPU time on one core",
    }
    if gpu_rows is not None:
        out["errors"] = {k: (v if k == "rows" else float(f"{v:.3e}")) for k, v in err.items()}
        out["errors"]["what"] = ("GPU path vs fp64 oracle on the rows above (first pass): max |y - ref|, "
                                 "max |dx - ref|, max |rstd - ref| / ref")
    return out


PROBE_SHAPES = [(wg, u) for wg in (1, 2, 4, 8, 16) for u in (1, 2, 4, 8)]


def ceilings(adaln, torch, np, runner, nbytes_fwd, nbytes_bwd):
    """Streaming ceilings for the workload's [R, D] tensor size: the best
    copy (1 read : 1 write) and two-to-one (2 reads : 1 write) rates over the
    launch shapes in PROBE_SHAPES, timed like the operator's calls (blocks of
    back-to-back passes over rotating resident copies, one event pair per
    block), on the runner's own buffers (x, dy read; y, dx written)."""
    sets = runner.sets
    nb = (runner.p.R * runner.p.D * runner.p.esize) // 16 * 16
    if nb == 0:
        return None
    u8 = lambda t: t.view(torch.uint8).view(-1)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    res = {}
    for mode, k in (("copy", 2), ("two_to_one", 3)):
        best = None
        for wg, un in PROBE_SHAPES:
            times = []
            for rep in range(3):
                e0, e1 = ev(), ev()
                e0.record()
                for i in range(6):
                    s = sets[(rep * 6 + i) % len(sets)]
                    adaln.adaln_probe_stream(mode, u8(s["x"]), u8(s["dy"]), u8(s["y"] if mode == "copy" else s["dx"]),
                                             wg, un, nbytes=nb)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / 6)
            gbs = k * nb / (float(np.median(times)) * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, wg, un)
        res[mode] = {"gbs": round(best[0], 1), "wg_per_cu": best[1], "unroll": best[2]}
    step = (nbytes_fwd + nbytes_bwd) / (nbytes_fwd / res["copy"]["gbs"] + nbytes_bwd / res["two_to_one"]["gbs"])
    res["step_gbs"] = round(step, 1)
    return res


def versions(torch):
    rocm = "unknown"
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"rocm": rocm, "hip": getattr(torch.version, "hip", None), "torch": torch.__version__}


def compute_partition(cus):
    """The device's compute partition mode from sysfs when it is readable, else
    what the visible CU count implies (256 CUs: the whole chip, SPX)."""
    import glob

    for path in sorted(glob.glob("/sys/class/drm/card*/device/current_compute_partition")):
        try:
            with open(path) as f:
                mode = f.read().strip()
            if mode:
                return mode
        except OSError:
            continue
    return "SPX (inferred: 256 CUs visible)" if cus == 256 else f"unknown ({cus} CUs visible)"


class Runner:
    """Resident copies of one problem's inputs/outputs and its fwd/bwd calls.

    Step k runs the forward on copy k % S and the backward on copy
    (k + S/2) % S; S is large enough that about 1 GB of other traffic
    separates two touches of the same copy."""

    def __init__(self, pd, adaln, torch, bwd_impl="fused"):
        self.pd, self.p, self.adaln, self.torch = pd, pd.problem, adaln, torch
        p = self.p
        if bwd_impl == "twopass" and not p.dense:
            raise SystemExit(f"--bwd twopass takes dense workloads; {p.name} is packed")
        self.bwd_fn = {"twopass": adaln.adaln_bwd_twopass,
                       "f32sums": adaln.adaln_bwd_f32sums}.get(bwd_impl, adaln.adaln_bwd)
        self.bwd_varlen_fn = (adaln.adaln_bwd_varlen_f32sums if bwd_impl == "f32sums"
                              else adaln.adaln_bwd_varlen)
        tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
        sdt = torch.float32 if bwd_impl == "f32sums" else tdt      # dscale / dshift
        base = upload(pd)
        S = 4
        per_set = max(1, 4 * p.R * p.D * p.esize)
        while (S // 2 - 1) * per_set < (1 << 30) and S < 64:
            S += 2
        self.S = S
        self.sets = []
        for _ in range(S):
            self.sets.append({
                "x": base["x"].clone(), "dy": base["dy"].clone(), "shift": base["shift"],
                "scale": base["scale"], "offsets": base["offsets"],
                "y": torch.empty_like(base["x"]), "dx": torch.empty_like(base["x"]),
                "mean": torch.empty(p.R, dtype=torch.float32, device="cuda"),
                "rstd": torch.empty(p.R, dtype=torch.float32, device="cuda"),
                "dscale": torch.empty(p.B, p.D, dtype=sdt, device="cuda"),
                "dshift": torch.empty(p.B, p.D, dtype=sdt, device="cuda")})
        self.ws = torch.empty(max(16, adaln.adaln_bwd_workspace_size(p.B, p.R, p.D, tdt)),
                              dtype=torch.uint8, device="cuda")
        if p.dense:                         # the [B, N, D] / [B, N] views, made once
            for s in self.sets:
                for k in ("x", "dy", "y", "dx"):
                    s[k + "3"] = s[k].view(p.B, p.N, p.D)
                for k in ("mean", "rstd"):
                    s[k + "2"] = s[k].view(p.B, p.N)

    def fwd(self, s):
        p, a = self.p, self.adaln
        if p.dense:
            a.adaln_fwd(s["x3"], s["shift"], s["scale"], p.eps, y=s["y3"], mean=s["mean2"], rstd=s["rstd2"])
        else:
            a.adaln_fwd_varlen(s["x"], s["shift"], s["scale"], s["offsets"], p.eps, y=s["y"],
                               mean=s["mean"], rstd=s["rstd"])

    def bwd(self, s):
        p = self.p
        if p.dense:
            self.bwd_fn(s["dy3"], s["x3"], s["scale"], s["mean2"], s["rstd2"], workspace=self.ws,
                        dx=s["dx3"], dscale=s["dscale"], dshift=s["dshift"])
        else:
            self.bwd_varlen_fn(s["dy"], s["x"], s["scale"], s["mean"], s["rstd"], s["offsets"],
                               workspace=self.ws, dx=s["dx"], dscale=s["dscale"], dshift=s["dshift"])

    def prime(self):
        for s in self.sets:                 # every copy gets its statistics
            self.fwd(s)

    def step(self, k):
        self.fwd(self.sets[k % self.S])
        self.bwd(self.sets[(k + self.S // 2) % self.S])


class TorchRunner:
    """The unfused eager-PyTorch chain (eager_adaln) on resident copies laid
    out like Runner's (dense workloads only): the forward builds the autograd
    graph of its copy (replacing the previous one), the backward takes
    torch.autograd.grad of it with the copy's dy."""

    def __init__(self, pd, torch):
        self.pd, self.p, self.torch = pd, pd.problem, torch
        p = self.p
        if not p.dense:
            raise SystemExit(f"--impl torch takes dense workloads; {p.name} is packed")
        base = upload(pd)
        S = 4
        per_set = max(1, 4 * p.R * p.D * p.esize)
        while (S // 2 - 1) * per_set < (1 << 30) and S < 64:
            S += 2
        self.S = S
        base["shift"].requires_grad_(True)
        base["scale"].requires_grad_(True)
        self.sets = [{"x": base["x"].clone().view(p.B, p.N, p.D).requires_grad_(True),
                      "dy": base["dy"].clone().view(p.B, p.N, p.D), "shift": base["shift"],
                      "scale": base["scale"], "y": None} for _ in range(S)]

    def fwd(self, s):
        s["y"] = eager_adaln(s["x"], s["shift"], s["scale"], self.p.eps)

    def bwd(self, s):
        # the graph stays alive: a copy's backward may run again before its
        # next forward (the step order only fixes which copy each call uses)
        self.torch.autograd.grad(s["y"], (s["x"], s["scale"], s["shift"]), s["dy"], retain_graph=True)

    def prime(self):
        for s in self.sets:
            self.fwd(s)

    step = Runner.step

    def activation_bytes(self):
        s = self.sets[0]
        _, n = saved_activation_bytes(eager_adaln, s["x"], s["shift"], s["scale"], self.p.eps)
        return n


SWEEP_D = 3072            # AdaLN width of the synthetic step
SWEEP_HEAD = 64           # width of the attention-score product
SWEEP_M_MEM = 1 << 18     # tokens per group (the memory budget)


def cost_sweep(adaln, torch, np):
    """Shape benchmarking on one GPU: the single-GPU synthetic form of the
    cost-fitting system of the AdaptiveLoad summary (section 2.A).

    The timed per-group step is this library's AdaLN forward + backward on
    [B, S, SWEEP_D] bf16 plus an fp32 attention-score product
    [B, S, 64] x [B, 64, S] (the O(S^2) term of a DiT block), on every (B, S)
    of a grid with B*S <= SWEEP_M_MEM.  adaln_cost_fit fits
    step = a + b*B*S^p; M_comp is then the compute of one sequence of the
    corpus's longest length, S_max^p: no group may cost more than the one
    step no batching can shorten.
    A seeded mixed-length corpus is cut into groups twice with
    adaln_sched_plan, by equal tokens (M_comp unbounded) and by the dual
    constraint, and each group's step is timed: the coefficient of variation
    of those times is the load imbalance if each group went to its own GPU."""
    import json as _json

    ev = lambda: torch.cuda.Event(enable_timing=True)
    cache = {}

    def step_ms(B, S, reps=5):
        key = (int(B), int(S))
        if key in cache:
            return cache[key]
        g = torch.Generator(device="cuda").manual_seed(1234)
        x = torch.randn(B, S, SWEEP_D, device="cuda", generator=g).to(torch.bfloat16)
        dy = (1e-2 * torch.randn(B, S, SWEEP_D, device="cuda", generator=g)).to(torch.bfloat16)
        mod = (0.1 * torch.randn(2, B, SWEEP_D, device="cuda", generator=g)).to(torch.bfloat16)
        q = torch.randn(B, S, SWEEP_HEAD, device="cuda", generator=g)
        kt = torch.randn(B, SWEEP_HEAD, S, device="cuda", generator=g)        # contiguous, not a view
        ws = torch.empty(adaln.adaln_bwd_workspace_size(B, B * S, SWEEP_D, torch.bfloat16), dtype=torch.uint8,
                         device="cuda")

        def run():
            y, mean, rstd = adaln.adaln_fwd(x, mod[0], mod[1], 1e-6)
            torch.bmm(q, kt)
            adaln.adaln_bwd(dy, x, mod[1], mean, rstd, workspace=ws)

        for _ in range(2):
            run()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            run()
        b.record()
        torch.cuda.synchronize()
        cache[key] = a.elapsed_time(b) / reps
        del x, dy, q, kt, ws
        torch.cuda.empty_cache()
        return cache[key]

    shapes = [(B, S) for S in (256, 512, 1024, 2048, 4096, 8192, 16384, 32760) for B in (1, 2, 4, 8)
              if B * S <= SWEEP_M_MEM]
    Bv = np.array([b for b, _ in shapes], dtype=np.float64)
    Sv = np.array([s for _, s in shapes], dtype=np.float64)
    tv = np.array([step_ms(b, s) for b, s in shapes])
    a, b, p, rss = adaln.adaln_cost_fit(Bv, Sv, tv, 0.5, 3.0)
    r_tok = float(np.corrcoef(tv, Bv * Sv)[0, 1])
    r_sq = float(np.corrcoef(tv, Bv * Sv ** 2)[0, 1])
    pred = lambda B, S: a + b * B * S ** p

    rng = np.random.default_rng(7)
    lengths = rng.choice([256, 1024, 4096, 16384, 32760], size=1024, p=[0.5, 0.2, 0.15, 0.1, 0.05])
    m_comp = int(np.ceil(float(lengths.max()) ** p))
    policies = {}
    for name, mc in (("equal_tokens", np.iinfo(np.int64).max), ("dual_constraint", m_comp)):
        group_of, n_groups = adaln.adaln_sched_plan(lengths, SWEEP_M_MEM, mc, p)
        sizes = np.bincount(group_of, minlength=n_groups)
        glen = np.zeros(n_groups, dtype=np.int64)
        glen[group_of] = lengths
        times = np.array([step_ms(int(n), int(S)) for n, S in zip(sizes, glen)])
        model = np.array([pred(int(n), int(S)) for n, S in zip(sizes, glen)])
        policies[name] = {"groups": int(n_groups), "cv_measured": round(adaln.adaln_load_cv(times), 4),
                          "cv_model": round(adaln.adaln_load_cv(model), 4),
                          "max_over_mean": round(float(times.max() / times.mean()), 3),
                          "batch_by_length": {int(S): int(sizes[glen == S].max()) for S in np.unique(glen)}}
    out = {"cost_sweep": {
        "step": f"AdaLN fwd+bwd [B,S,{SWEEP_D}] bf16 + fp32 scores [B,S,{SWEEP_HEAD}]x[B,{SWEEP_HEAD},S]",
        "shapes": len(shapes), "fit_ms": {"a": round(a, 5), "b": b, "p": round(p, 4), "rss": rss},
        "corr_time_tokens": round(r_tok, 3), "corr_time_tokens_S2": round(r_sq, 3),
        "m_mem": SWEEP_M_MEM, "m_comp": m_comp, "corpus": "1024 samples, lengths 256/1024/4096/16384/32760 "
        "with probabilities 0.5/0.2/0.15/0.1/0.05 (seed 7)", "policies": policies,
        "timings_ms": {f"{b}x{s}": round(t, 4) for (b, s), t in zip(shapes, tv)}}}
    print(_json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path.  Under "
              "sequence sharding each GPU runs this same one-GPU workload on its share of the "
              "rows, and only the per-sample dscale/dshift partial sums would need a cross-GPU sum.",
              file=sys.stderr)
        sys.exit(2)

    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import numpy as np
    import torch

    import diffusion_transformer_adaln_amd as adaln
    import workloads

    torch.cuda.set_device(0)
    if args.cost_sweep:
        cost_sweep(adaln, torch, np)
        return
    pds = workloads.make_config(args.config)
    if args.impl == "torch":
        runners = [TorchRunner(pd, torch) for pd in pds]
        act = sum(r.activation_bytes() for r in runners)
        act_note = "eager chain: storages autograd saves beyond x, shift, scale"
    else:
        runners = [Runner(pd, adaln, torch, args.bwd) for pd in pds]
        act = sum(8 * r.p.R for r in runners)
        act_note = "fused: mean and rstd (fp32, 8 bytes per row)"
    nbytes = {k: sum(workloads.algorithmic_bytes(r.p)[k] for r in runners) for k in ("fwd", "bwd", "total")}
    rows = sum(r.p.R for r in runners)
    main_r = max(runners, key=lambda r: r.p.R * r.p.D)     # the roofline reports its backward
    if args.clock_trace:
        clock_trace(args, runners, adaln, torch, np)
        return

    for r in runners:
        r.prime()
    # Warm-up.  Under sustained load the chip takes ~20 ms to settle: the
    # video step runs 179-190 us for its first ~20 ms, then 172 us (measured in
    # 10-step batches on MI355X), so by default the warm-up lasts at least
    # --warmup-ms, in synchronised batches of 10 steps so that the host clock
    # follows the GPU.  An explicit --warmup W runs exactly W steps.
    warmup = 0
    if args.warmup is not None:
        for k in range(args.warmup):
            for r in runners:
                r.step(k)
        warmup = args.warmup
    else:
        t_w = None          # starts after the first batch, which absorbs one-time costs
        while t_w is None or warmup < 20 or time.perf_counter() - t_w < args.warmup_ms * 1e-3:
            for _ in range(10):
                for r in runners:
                    r.step(warmup)
                warmup += 1
            torch.cuda.synchronize()
            if t_w is None:
                t_w = time.perf_counter()
    torch.cuda.synchronize()

    # Timed region: K steps and nothing else on the stream.  A timing event
    # stalls the queue for several microseconds, so only two bracket the
    # region (a GPU-side check of the host clock).
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    region = (ev(), ev())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record()
    for k in range(K):
        for r in runners:
            r.step(k)
    region[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms_per_step = region[0].elapsed_time(region[1]) / K

    # Per-call durations for the roofline, right after, on the same resident
    # copies and on the launch stream: blocks of BLOCK back-to-back calls of
    # the main workload's backward (then forward), the copies rotating, one
    # event pair per block.  A timing event between two kernels adds its own
    # dispatch bubble (2-3 us here), so a pair around a single call reads
    # high; over a block of ten the bubble is spread thin, and the figure still
    # includes every launch gap of the calls themselves.
    BLOCK = 10

    def per_call_ms(call):
        pairs = []
        for b in range(max(1, K // BLOCK)):
            e0, e1 = ev(), ev()
            e0.record()
            for i in range(BLOCK):
                call(main_r.sets[(b * BLOCK + i) % main_r.S])
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in pairs]) / BLOCK

    bwd_ms = per_call_ms(main_r.bwd)
    fwd_ms = per_call_ms(main_r.fwd)
    ms_per_step = wall * 1e3 / K
    gbs = nbytes["total"] / (ms_per_step * 1e-3) / 1e9
    rows_per_s = rows / (ms_per_step * 1e-3)
    main_bytes = workloads.algorithmic_bytes(main_r.p)
    bwd_gbs = main_bytes["bwd"] / (bwd_ms.mean() * 1e-3) / 1e9
    fwd_gbs = main_bytes["fwd"] / (fwd_ms.mean() * 1e-3) / 1e9
    p = main_r.p
    pd = main_r.pd

    if args.copy_probe:                 # plain copy of known size, for counter calibration
        src = torch.empty(1 << 27, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    ceil = None
    if args.impl == "hip":
        ceil = ceilings(adaln, torch, np, main_r, nbytes["fwd"], nbytes["bwd"])

    traffic = read_traffic(args.traffic_file, args.config) if (args.bwd, args.impl) == ("fused", "hip") else None
    bwd_name = {"fused": "adaln_bwd", "twopass": "adaln_bwd_twopass", "f32sums": "adaln_bwd_f32sums"}[args.bwd]
    if not all(pd.problem.dense for pd in pds):      # packed samples go through the varlen entry points
        bwd_name = bwd_name.replace("adaln_bwd", "adaln_bwd_varlen")
    if args.impl == "torch":
        bwd_name = "eager PyTorch autograd backward"

    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": " + ".join(
                       f"{r.p.name}: AdaLN fwd+bwd, B={r.p.B}, N={r.p.N if r.p.dense else 'ragged'}, "
                       f"D={r.p.D}, {r.p.dtype} I/O, fp32 statistics" for r in runners),
                   "name": args.config, "B": sum(r.p.B for r in runners), "rows": rows,
                   "D": p.D, "impl": args.impl, "bwd": bwd_name, "parallelism": "single GPU"},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count,
                   "hbm_gib": round(props.total_memory / 2 ** 30, 1),
                   "compute_partition": compute_partition(props.multi_processor_count)},
        "versions": versions(torch),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(rows_per_s, 1),
        "fwd_us": round(float(fwd_ms.mean()) * 1e3, 2),
        "bwd_us": round(float(bwd_ms.mean()) * 1e3, 2),
        "per_call_us": {k: {f"p{q}": round(float(np.percentile(v, q)) * 1e3, 2) for q in (10, 50, 90)}
                        | {"blocks": int(v.size), "calls_per_block": BLOCK}
                        for k, v in (("fwd", fwd_ms), ("bwd", bwd_ms))},
        "fwd_gbs": round(fwd_gbs, 1),
        "algorithmic_bytes_per_step": nbytes["total"],
        "activation_bytes": {"saved": act, "what": act_note},
        "roofline": {"bound": "hbm", "kernel": f"{bwd_name} on {p.name} (all of its launches)",
                     "achieved": round(bwd_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(bwd_gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
    }
    if ceil is not None:
        ceil["pct_of_copy_ceiling"] = round(100 * gbs / ceil["step_gbs"], 2)
        out["ceilings"] = ceil
    if not args.no_cpu_baseline:
        gpu_rows = None
        if args.impl == "hip":
            s0 = main_r.sets[0]
            main_r.fwd(s0)
            main_r.bwd(s0)
            torch.cuda.synchronize()

            def host64(t):
                if t.dtype == torch.bfloat16:
                    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
                    return u.view(np.float32).astype(np.float64)
                return t.cpu().numpy().astype(np.float64)

            def gpu_rows(lo, hi):
                return host64(s0["y"][lo:hi]), host64(s0["dx"][lo:hi]), host64(s0["rstd"][lo:hi])
        out["cpu_baseline"] = cpu_baseline(pd, args.cpu_seconds, gpu_rows)
    print(json.dumps(out), flush=True)


CLOCK_ITERS = 4000        # fma chain of one clock sample


def clock_trace(args, runners, adaln, torch, np):
    """The bench's schedule -- priming, the warm-up (W steps, or batches of ten
    until --warmup-ms have passed), K steps -- with the engine clock sampled
    beside it.  A second stream runs single-wave clock probes back to back
    (each times a chain of dependent fmas in shader-clock cycles and in
    wall-clock ticks), and a timestamp on the launch stream before every step
    puts the steps on the same wall clock.  Prints one JSON line: clock
    samples over time, each step's duration, and the mean clock over the
    warm-up and over the K steps.  Diagnostic only: the probes hold one wave
    slot, and no throughput is reported from this run."""
    khz = adaln.adaln_probe_wall_clock_khz()
    if khz <= 0:
        raise SystemExit("the device does not report its wall-clock rate")
    n_probe = max(256, args.clock_samples)
    probe = torch.zeros(3 * n_probe, dtype=torch.int64, device="cuda")
    cap = 4 + (args.warmup if args.warmup is not None else 100000) + args.steps
    marks = torch.zeros(cap, dtype=torch.int64, device="cuda")
    phase = []                                   # phase of the step after each mark
    side = torch.cuda.Stream()
    fed = [0]

    def feed(n):
        # clock samples queued on the side stream as the schedule is queued,
        # so that they run beside it rather than all before it
        for _ in range(min(n, n_probe - fed[0])):
            adaln.adaln_probe_clock(probe, fed[0], CLOCK_ITERS, stream=side)
            fed[0] += 1

    def mark(what):
        adaln.adaln_probe_mark(marks, len(phase))
        phase.append(what)
        feed(args.clock_per_step)

    torch.cuda.synchronize()
    feed(64)                                     # the idle clock before the schedule
    mark("prime")
    for r in runners:
        r.prime()
    k = 0
    if args.warmup is not None:
        for k in range(args.warmup):
            mark("warmup")
            for r in runners:
                r.step(k)
    else:
        t_w = None
        while (t_w is None or k < 20 or time.perf_counter() - t_w < args.warmup_ms * 1e-3) and len(phase) + 12 + args.steps < cap:
            for _ in range(10):
                mark("warmup")
                for r in runners:
                    r.step(k)
                k += 1
            torch.cuda.synchronize()
            if t_w is None:
                t_w = time.perf_counter()
    for k in range(args.steps):
        mark("timed")
        for r in runners:
            r.step(k)
    mark("end")
    feed(64)                                     # and after it
    torch.cuda.synchronize()

    m = marks.cpu().numpy()[:len(phase)].astype(np.int64)
    pr = probe.cpu().numpy().reshape(-1, 3).astype(np.int64)
    out = {"clock_trace": {"config": args.config, "steps": args.steps, "wall_clock_khz": int(khz),
                           "probe_iters": CLOCK_ITERS, **clock_summary(pr, m, phase, khz, np)}}
    print(json.dumps(out), flush=True)


def clock_summary(pr, m, phase, khz, np):
    """Clock samples and step marks of --clock-trace, summarised.

    pr: [n, 3] int64 rows (wall clock at the sample's start, shader-clock
    cycles, wall-clock ticks; rows never written are all zero); m: the
    marks' wall-clock stamps, one per entry of `phase` ("prime", "warmup",
    "timed", ..., "end"), each stamped before the step it names; khz: the
    wall clock's rate.  Times are ms from the first mark; a step lasts from
    its mark to the next; the clock over a window is the mean of the samples
    that start in it."""
    t0 = m[0]
    ok = pr[:, 2] > 0
    t_s = (pr[ok, 0] - t0) * 1.0 / khz
    mhz = pr[ok, 1] / pr[ok, 2] * khz / 1e3
    ph = np.array(phase)
    t_mark = (m - t0) * 1.0 / khz
    step_us = np.diff(t_mark) * 1e3
    w_idx = np.where(ph[:-1] == "warmup")[0]
    t_idx = np.where(ph[:-1] == "timed")[0]
    t_start = t_mark[t_idx[0]] if len(t_idx) else t_mark[-1]
    w_start = t_mark[w_idx[0]] if len(w_idx) else t_start

    def mean_in(lo, hi):
        sel = (t_s >= lo) & (t_s < hi)
        if not sel.any():
            return {"mean": None, "min": None, "samples": 0}
        return {"mean": round(float(mhz[sel].mean()), 1), "min": round(float(mhz[sel].min()), 1),
                "samples": int(sel.sum())}

    keep = np.where((t_s >= -1.0) & (t_s <= t_mark[-1] + 1.0))[0]
    if len(keep) > 600:
        keep = keep[:: int(np.ceil(len(keep) / 600))]
    return {
        "warmup": int(len(w_idx)),
        "probe_us": round(float(np.median(pr[ok, 2])) / khz * 1e3, 2) if ok.any() else None,
        "idle_mhz": round(float(np.median(mhz[t_s < 0])), 1) if (t_s < 0).any() else None,
        "prime_ms": round(float(w_start), 3),
        "warmup_mhz": mean_in(w_start, t_start),
        "timed_mhz": mean_in(t_start, t_mark[-1]),
        "timed_start_ms": round(float(t_start), 3), "end_ms": round(float(t_mark[-1]), 3),
        "timed_step_us": [round(float(v), 1) for v in step_us[t_idx]],
        "warmup_step_us": [round(float(v), 1) for v in step_us[w_idx]][:50],
        "samples_ms_mhz": [[round(float(t_s[i]), 3), round(float(mhz[i]), 0)] for i in keep],
    }


def read_traffic(path, config):
    """HBM bytes per backward call from a committed counter summary, if it was
    taken on this workload and on the current kernel sources (else None)."""
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("workload") != config or fields.get("kernel_source_sha") != kernel_source_sha():
            return None
        return int(fields["bwd_hbm_bytes_per_call"])
    except (OSError, ValueError, KeyError):
        return None


# The sources the operator's kernels and launch configuration come from (the
# host-only scheduler, csrc/adaln_sched.cpp, does not change them).
OPERATOR_SOURCES = ("adaln_api.cpp", "adaln_internal.hpp", "adaln_kernels.hip", "adaln_plan.cpp")


# string literal | character literal | line comment | block comment
_CODE_TOKENS = re.compile(r"""
    "(?:\\.|[^"\\\n])*"
  | '(?:\\.|[^'\\\n])*'
  | //[^\n]*
  | /\*.*?\*/
""", re.S | re.X)


def _code_only(text):
    """C++ source without comments, blank lines and indentation (string and
    character literals kept), so that editing a comment leaves the hash alone."""
    text = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def kernel_source_sha():
    """sha256 prefix over the operator's sources, comments and layout removed."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_transformer_adaln_amd", "csrc")
    for name in OPERATOR_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
