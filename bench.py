"""Benchmark of the fused AdaLN forward + backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config video_bf16]

A step is one forward and one backward call of the workload (every hot-path
kernel: forward, backward row pass, backward finish) over one resident batch
of seeded synthetic bf16 inputs.  The default workload is the video-DiT
AdaLN at one device's sequence share: B=1, N=18900, D=5120.

Four copies of the inputs and outputs stay resident in HBM.  Step k runs the
forward on copy k % 4 and the backward on copy (k + 2) % 4, the way a
layer's backward runs long after its forward in training: no kernel reads
data another kernel touched within the last ~1 GB of traffic, so the 256 MB
Infinity Cache cannot serve it and the figures are HBM figures.

Output: one JSON line.  `value` is the whole-job throughput in GB/s of
algorithmic bytes (the minimal traffic of the method, see
workloads.algorithmic_bytes) over the wall-clock time of the K timed steps,
bracketed by device synchronisation.  `roofline` covers the backward call,
the dominant one: algorithmic bytes per call / mean call duration from HIP
events recorded on the launch stream inside the timed region.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload's rows on one host core.
"""

from __future__ import annotations

import argparse
import json
import os
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
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="video_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per backward call (from rocprofv3 counters), if present")
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


def cpu_baseline(pd, seconds):
    """fp64 oracle on successive 128-row blocks of the workload until about
    `seconds` of CPU time; rows are independent, and each block's column sums
    are taken over its own rows (the same per-row work as the full sums)."""
    import numpy as np

    import oracle

    p = pd.problem
    rows_done, t_used = 0, 0.0
    block = 128
    start = 0
    while t_used < seconds and start < p.R:
        lo, hi = start, min(p.R, start + block)
        b = int(oracle.sample_of_rows(pd.offsets, np.array([lo]))[0])
        hi = min(hi, int(pd.offsets[b + 1]))
        x = oracle.decode(pd.x[lo:hi], p.dtype)
        dy = oracle.decode(pd.dy[lo:hi], p.dtype)
        sh = oracle.decode(pd.shift[b:b + 1], p.dtype)
        sc = oracle.decode(pd.scale[b:b + 1], p.dtype)
        off = np.array([0, hi - lo], dtype=np.int64)
        t0 = time.process_time()
        oracle.adaln_fwd(x, sh, sc, p.eps, off)
        oracle.adaln_bwd(dy, x, sc, p.eps, off)
        t_used += time.process_time() - t0
        rows_done += hi - lo
        start = hi
    import workloads

    per_row = workloads.algorithmic_bytes(p)["total"] / p.R
    return {
        "value": round(rows_done * per_row / t_used / 1e9, 4),
        "unit": "GB/s",
        "rows_per_s": round(rows_done / t_used, 1),
        "cores": 1,
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd on the first {rows_done} rows of {p.name} "
                  f"(D={p.D}), 128-row blocks, {t_used:.1f} s of CPU time",
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(a rank's work is the one-GPU workload; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import numpy as np
    import torch

    import diffusion_transformer_adaln_amd as adaln
    import workloads

    problems = workloads.CONFIGS[args.config]
    if len(problems) != 1:
        sys.exit(f"{args.config} has {len(problems)} problems; bench lines use single-problem workloads")
    torch.cuda.set_device(0)
    pd = workloads.make_config(args.config)[0]
    p = pd.problem
    nbytes = workloads.algorithmic_bytes(p)
    tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float32

    base = upload(pd)
    S = 4
    per_set = 4 * p.R * p.D * p.esize
    while (S // 2 - 1) * per_set < (1 << 30):
        S += 2
    sets = []
    for _ in range(S):
        s = {"x": base["x"].clone(), "dy": base["dy"].clone(), "shift": base["shift"], "scale": base["scale"],
             "offsets": base["offsets"],
             "y": torch.empty_like(base["x"]), "dx": torch.empty_like(base["x"]),
             "mean": torch.empty(p.R, dtype=torch.float32, device="cuda"),
             "rstd": torch.empty(p.R, dtype=torch.float32, device="cuda"),
             "dscale": torch.empty(p.B, p.D, dtype=tdt, device="cuda"),
             "dshift": torch.empty(p.B, p.D, dtype=tdt, device="cuda")}
        sets.append(s)
    ws_bytes = adaln.adaln_bwd_workspace_size(p.B, p.R, p.D, tdt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    if p.dense:
        def fwd(s):
            adaln.adaln_fwd(s["x"].view(p.B, p.N, p.D), s["shift"], s["scale"], p.eps,
                            y=s["y"].view(p.B, p.N, p.D), mean=s["mean"].view(p.B, p.N),
                            rstd=s["rstd"].view(p.B, p.N))

        def bwd(s):
            adaln.adaln_bwd(s["dy"].view(p.B, p.N, p.D), s["x"].view(p.B, p.N, p.D), s["scale"],
                            s["mean"].view(p.B, p.N), s["rstd"].view(p.B, p.N), workspace=ws,
                            dx=s["dx"].view(p.B, p.N, p.D), dscale=s["dscale"], dshift=s["dshift"])
    else:
        def fwd(s):
            adaln.adaln_fwd_varlen(s["x"], s["shift"], s["scale"], s["offsets"], p.eps, y=s["y"],
                                   mean=s["mean"], rstd=s["rstd"])

        def bwd(s):
            adaln.adaln_bwd_varlen(s["dy"], s["x"], s["scale"], s["mean"], s["rstd"], s["offsets"],
                                   workspace=ws, dx=s["dx"], dscale=s["dscale"], dshift=s["dshift"])

    for s in sets:                     # every copy gets its statistics
        fwd(s)
    for k in range(args.warmup):
        fwd(sets[k % S])
        bwd(sets[(k + S // 2) % S])
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        e = ev[k]
        e[0].record()
        fwd(sets[k % S])
        e[1].record()
        bwd(sets[(k + S // 2) % S])
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    ms_per_step = wall * 1e3 / K
    gbs = nbytes["total"] / (ms_per_step * 1e-3) / 1e9
    rows_per_s = p.R / (ms_per_step * 1e-3)
    bwd_gbs = nbytes["bwd"] / (bwd_ms.mean() * 1e-3) / 1e9
    fwd_gbs = nbytes["fwd"] / (fwd_ms.mean() * 1e-3) / 1e9

    traffic = None
    try:
        with open(args.traffic_json) as f:
            t = json.load(f)
        if t.get("config") == args.config and t.get("kernel_source_sha") == kernel_source_sha():
            traffic = t["bwd_bytes_per_call"]
    except (OSError, ValueError, KeyError):
        traffic = None

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": f"{p.name}: AdaLN fwd+bwd, B={p.B}, N={p.N if p.dense else 'ragged'}, "
                               f"D={p.D}, R={p.R} rows, {p.dtype} I/O, fp32 statistics",
                   "B": p.B, "rows": p.R, "D": p.D, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(rows_per_s, 1),
        "fwd_us": round(float(fwd_ms.mean()) * 1e3, 2),
        "bwd_us": round(float(bwd_ms.mean()) * 1e3, 2),
        "fwd_gbs": round(fwd_gbs, 1),
        "algorithmic_bytes_per_step": nbytes["total"],
        "roofline": {"bound": "hbm", "kernel": "adaln_bwd (row pass + finish)",
                     "achieved": round(bwd_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(bwd_gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pd, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def kernel_source_sha():
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_transformer_adaln_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
