"""Host-side pieces of bench.py: the source hash that ties a committed
counter summary to the kernels it was taken on, and the reading of that
summary."""

import bench


def test_code_only_drops_comments_and_layout_but_keeps_literals():
    src = ('int a = 1;  // note\n'
           '/* block\n   comment */ const char* s = "x // y /* z */";\n'
           '\n'
           "    char c = '/'; b = a; /* x */ c = 2;\n"
           'const char* q = "a\\"b // c";\n')
    assert bench._code_only(src) == ('int a = 1;\n'
                                     'const char* s = "x // y /* z */";\n'
                                     "char c = '/'; b = a;   c = 2;\n"
                                     'const char* q = "a\\"b // c";')
    # a comment edit leaves the text alone; a code edit does not
    assert bench._code_only(src.replace("note", "other note")) == bench._code_only(src)
    assert bench._code_only(src.replace("c = 2", "c = 3")) != bench._code_only(src)


def test_traffic_is_read_only_for_its_workload_and_sources(tmp_path):
    sha = bench.kernel_source_sha()
    assert len(sha) == 16
    f = tmp_path / "traffic.txt"
    f.write_text(f"# bwd: 1\nworkload: video_bf16\nkernel_source_sha: {sha}\nbwd_hbm_bytes_per_call: 123\n")
    assert bench.read_traffic(str(f), "video_bf16") == 123
    assert bench.read_traffic(str(f), "dit_bf16") is None
    f.write_text(f"workload: video_bf16\nkernel_source_sha: {'0' * 16}\nbwd_hbm_bytes_per_call: 123\n")
    assert bench.read_traffic(str(f), "video_bf16") is None
    assert bench.read_traffic(str(tmp_path / "missing.txt"), "video_bf16") is None


def test_more_than_one_gpu_is_refused_with_a_reason():
    import subprocess
    import sys

    run = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert run.returncode != 0
    assert "exactly one GPU" in run.stdout + run.stderr


def test_clock_summary_splits_the_schedule_and_converts_cycles():
    """--clock-trace's summary on a synthetic trace: a 100 MHz wall clock,
    marks for priming, two warm-up steps and three timed steps, samples at
    2.4 GHz before the schedule, 2.0 GHz over the warm-up and 1.5 GHz over
    the timed steps, and rows never written (all zero) ignored."""
    import numpy as np

    import bench

    khz = 100_000                                  # ticks per ms
    m0 = 10_000_000
    stamps_ms = [0.0, 0.5, 0.7, 0.9, 1.1, 1.3, 1.5]  # prime, warm-up x2, timed x3, end
    phase = ["prime", "warmup", "warmup", "timed", "timed", "timed", "end"]
    m = np.array([m0 + int(t * khz) for t in stamps_ms], dtype=np.int64)

    def sample(t_ms, ghz, dur_ms=0.05):
        ticks = int(dur_ms * khz)
        return [m0 + int(t_ms * khz), int(ghz * 1e6 * dur_ms), ticks]   # cycles = GHz * 1e9 * s

    rows = [sample(-0.2, 2.4), sample(-0.1, 2.4), sample(0.55, 2.0), sample(0.8, 2.0),
            sample(0.95, 1.5), sample(1.2, 1.5), sample(1.4, 1.5), [0, 0, 0], [0, 0, 0]]
    pr = np.array(rows, dtype=np.int64)
    s = bench.clock_summary(pr, m, phase, khz, np)
    assert s["warmup"] == 2 and s["prime_ms"] == 0.5 and s["timed_start_ms"] == 0.9 and s["end_ms"] == 1.5
    assert s["idle_mhz"] == 2400.0
    assert s["warmup_mhz"] == {"mean": 2000.0, "min": 2000.0, "samples": 2}
    assert s["timed_mhz"] == {"mean": 1500.0, "min": 1500.0, "samples": 3}
    assert s["timed_step_us"] == [200.0, 200.0, 200.0] and s["warmup_step_us"] == [200.0, 200.0]
    assert s["probe_us"] == 50.0 and len(s["samples_ms_mhz"]) == 7
