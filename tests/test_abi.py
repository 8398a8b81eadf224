"""The C-ABI library loads, exports every entry point include/adaln.h,
include/adaln_sched.h and include/adaln_probe.h declare, and rejects bad arguments before touching a device (no kernels
are launched here, and no HIP call is reached on these paths)."""

import ctypes
import os
import re
import subprocess

import pytest

import diffusion_transformer_adaln_amd as adaln
from diffusion_transformer_adaln_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("adaln.h", "adaln_sched.h", "adaln_probe.h")]


def declared_functions():
    names = set()
    for path in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(adaln_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.fail("libadaln.so is not built: run __graft_entry__.build() first")
    return adaln.load_library()


def test_header_matches_binding_and_exports(lib):
    decl = declared_functions()
    assert decl == sorted(adaln.EXPORTED), decl
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (adaln_\w+)", out))
    assert set(decl) <= exported, set(decl) - exported
    for name in decl:
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.adaln_abi_version() == 3
    for code, name in adaln._lib.STATUS_NAMES.items():
        assert adaln.adaln_status_str(code) == name
    assert adaln.adaln_status_str(99) == "ADALN_ERR_UNKNOWN"


P = ctypes.c_void_p
FAKE = 1 << 20        # distinct fake device addresses: validation never dereferences


def fwd(lib, x=FAKE, sh=FAKE * 2, sc=FAKE * 3, eps=1e-6, B=1, N=4, D=8, dt=1, y=FAKE * 4, m=FAKE * 5,
        r=FAKE * 6):
    return lib.adaln_fwd(P(x), P(sh), P(sc), eps, B, N, D, dt, None, P(y), P(m), P(r))


def bwd(lib, dy=FAKE, x=FAKE * 2, sc=FAKE * 3, m=FAKE * 4, r=FAKE * 5, B=1, N=4, D=8, dt=1, ws=FAKE * 6,
        wsb=1 << 20, dx=FAKE * 7, ds=FAKE * 8, dh=FAKE * 9):
    return lib.adaln_bwd(P(dy), P(x), P(sc), P(m), P(r), B, N, D, dt, P(ws), wsb, None, P(dx), P(ds), P(dh))


def test_forward_validation_codes(lib):
    assert fwd(lib, dt=7) == 2                          # unsupported dtype
    assert fwd(lib, B=0) == 1                           # B < 1
    assert fwd(lib, N=-1) == 1
    assert fwd(lib, D=0) == 1
    assert fwd(lib, D=65537) == 3                       # above ADALN_MAX_D
    assert fwd(lib, N=1 << 62, D=1024) == 3             # byte count overflows int64
    assert fwd(lib, eps=float("nan")) == 1
    assert fwd(lib, eps=float("inf")) == 1
    assert fwd(lib, eps=-1.0) == 1
    assert fwd(lib, x=0) == 1                           # null input
    assert fwd(lib, sh=0) == 1
    assert fwd(lib, m=0) == 1
    assert fwd(lib, y=FAKE + 8) == 5                    # y overlaps x
    assert fwd(lib, m=FAKE * 4 + 16) == 5               # mean overlaps y
    assert fwd(lib, r=FAKE * 3) == 5                    # rstd overlaps scale
    assert fwd(lib, N=0, x=0, y=0, m=0, r=0) == 0       # empty batch: nothing to do, no device touched


def test_varlen_validation_codes(lib):
    f = lib.adaln_fwd_varlen
    assert f(P(FAKE), P(FAKE * 2), P(FAKE * 3), 1e-6, None, 2, 8, 8, 1, None, P(FAKE * 4), P(FAKE * 5),
             P(FAKE * 6)) == 1                          # null offsets
    assert f(P(FAKE), P(FAKE * 2), P(FAKE * 3), 1e-6, P(FAKE * 7), 0, 8, 8, 1, None, P(FAKE * 4),
             P(FAKE * 5), P(FAKE * 6)) == 1             # B < 1
    assert f(P(FAKE), P(FAKE * 2), P(FAKE * 3), 1e-6, P(FAKE * 7), 2, -1, 8, 1, None, P(FAKE * 4),
             P(FAKE * 5), P(FAKE * 6)) == 1             # negative rows
    assert f(P(FAKE), P(FAKE * 2), P(FAKE * 3), 1e-6, P(FAKE * 4 + 8), 2, 8, 8, 1, None, P(FAKE * 4),
             P(FAKE * 5), P(FAKE * 6)) == 5             # y overlaps offsets
    b = lib.adaln_bwd_varlen
    assert b(P(FAKE), P(FAKE * 2), P(FAKE * 3), P(FAKE * 4), P(FAKE * 5), None, 2, 8, 8, 1, P(FAKE * 6),
             1 << 20, None, P(FAKE * 7), P(FAKE * 8), P(FAKE * 9)) == 1


def test_backward_validation_codes(lib):
    assert bwd(lib, dt=3) == 2
    assert bwd(lib, B=0) == 1
    assert bwd(lib, D=70000) == 3
    assert bwd(lib, dy=0) == 1
    assert bwd(lib, ds=0) == 1
    assert bwd(lib, ws=0) == 1                          # no workspace
    assert bwd(lib, ws=FAKE * 6 + 4) == 1               # workspace not 16-byte aligned


def test_twopass_validation_codes(lib):
    def tp(dy=FAKE, dt=1, B=1, ws=FAKE * 6, ds=FAKE * 8):
        return lib.adaln_bwd_twopass(P(dy), P(FAKE * 2), P(FAKE * 3), P(FAKE * 4), P(FAKE * 5), B, 4, 8, dt,
                                     P(ws), 1 << 20, None, P(FAKE * 7), P(ds), P(FAKE * 9))
    assert tp(dt=3) == 2
    assert tp(B=0) == 1
    assert tp(dy=0) == 1
    assert tp(ds=0) == 1
    assert tp(ws=FAKE * 6 + 4) == 1


def test_workspace_query_rejects_bad_sizes(lib):
    assert lib.adaln_bwd_workspace_size(0, 10, 8, 1) == 0
    assert lib.adaln_bwd_workspace_size(1, -1, 8, 1) == 0
    assert lib.adaln_bwd_workspace_size(1, 10, 0, 1) == 0
    assert lib.adaln_bwd_workspace_size(1, 10, 8, 5) == 0


def test_headers_compile_as_c_and_link(tmp_path, lib):
    """A plain C11 program includes the headers, links libadaln.so and calls
    the host-only entry points: the ABI is usable from C without torch."""
    import shutil

    cc = shutil.which("gcc")
    if cc is None or not os.path.isfile("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs gcc and the HIP runtime headers")
    src = tmp_path / "consumer.c"
    src.write_text(r'''
#include <stdio.h>
#include "adaln.h"
#include "adaln_sched.h"
#include "adaln_probe.h"
int main(void) {
  if (adaln_abi_version() != ADALN_ABI_VERSION) return 1;
  if (adaln_status_str(ADALN_ERR_ALIASING) == NULL) return 2;
  /* the pages' bucket rule at M_mem = 65536, M_comp = 2^30, p = 2: S = 4096 -> 16 */
  if (adaln_sched_batch_size(4096, 65536, (int64_t)1 << 30, 2.0) != 16) return 3;
  {
    const double load[4] = {1.0, 1.0, 1.0, 1.0};
    if (adaln_load_cv(load, 4) != 0.0) return 4;
  }
  /* every entry point is a linkable symbol */
  {
    typedef void (*fn_t)(void);
    fn_t fns[] = {(fn_t)adaln_fwd, (fn_t)adaln_bwd, (fn_t)adaln_fwd_varlen, (fn_t)adaln_bwd_varlen,
                  (fn_t)adaln_bwd_twopass, (fn_t)adaln_bwd_workspace_size, (fn_t)adaln_sched_plan,
                  (fn_t)adaln_cost_fit, (fn_t)adaln_probe_stream, (fn_t)adaln_probe_clock,
                  (fn_t)adaln_probe_mark, (fn_t)adaln_probe_wall_clock_khz};
    for (size_t i = 0; i < sizeof fns / sizeof fns[0]; ++i) if (fns[i] == NULL) return 5;
  }
  puts("ok");
  return 0;
}
''')
    exe = str(tmp_path / "consumer")
    libdir = os.path.dirname(LIB_PATH)
    # strict ISO C for this library's headers; ROCm's own headers (hipStream_t) come in
    # as system headers, since they are not pedantic-clean C themselves
    build = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-pedantic-errors", "-D__HIP_PLATFORM_AMD__",
                            "-isystem", "/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), str(src), "-o", exe,
                            "-L" + libdir, "-ladaln", "-Wl,-rpath," + libdir],
                           capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout, run.stderr[-2000:])


def test_probe_rejects_bad_arguments(lib):
    """The ceiling probe validates before any device call: sizes not a multiple
    of 16, bad grid shapes, missing or misaligned buffers, unknown modes."""
    st = lambda mode=0, a=FAKE, b=FAKE * 2, out=FAKE * 3, n=4096, wg=1, u=4: lib.adaln_probe_stream(
        mode, P(a), P(b), P(out), n, wg, u, None)
    bad = 1                      # ADALN_ERR_INVALID_ARG
    assert st(n=100) == bad and st(n=-16) == bad
    assert st(wg=0) == bad and st(wg=17) == bad
    assert st(u=3) == bad and st(u=16) == bad
    assert st(mode=7) == bad and st(mode=-1) == bad
    assert st(a=0) == bad and st(out=0) == bad
    assert st(mode=1, b=0) == bad
    assert st(a=FAKE + 8) == bad


def test_clock_probe_rejects_bad_arguments(lib):
    """The clock and mark probes validate before launching: a missing or
    misaligned buffer, a slot outside [0, n_slots), a chain length outside
    1 .. ADALN_PROBE_MAX_CLOCK_ITERS."""
    bad = 1                      # ADALN_ERR_INVALID_ARG
    clk = lambda out=FAKE, n=4, slot=0, it=100: lib.adaln_probe_clock(P(out), n, slot, it, None)
    assert clk(out=0) == bad and clk(out=FAKE + 4) == bad
    assert clk(n=0) == bad and clk(slot=-1) == bad and clk(slot=4) == bad
    assert clk(it=0) == bad and clk(it=(1 << 20) + 1) == bad
    mark = lambda out=FAKE, n=4, slot=0: lib.adaln_probe_mark(P(out), n, slot, None)
    assert mark(out=0) == bad and mark(out=FAKE + 2) == bad
    assert mark(n=0) == bad and mark(slot=-1) == bad and mark(slot=4) == bad
