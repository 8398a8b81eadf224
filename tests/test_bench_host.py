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
