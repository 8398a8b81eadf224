"""The library from a plain C11 program, with no Python or torch in the
process (tests/c/adaln_c_check.c, built by __graft_entry__.build()): forward
and backward through the C ABI on the GPU, checked against properties any
correct result has (LayerNorm rows of mean 0 and mean square var/(var+eps),
dx rows summing to 0, dshift equal to the row sum of dy), the fp32-sum entry
point agreeing bit for bit with the I/O-typed one for fp32 I/O, repeatability,
and two documented error codes."""

import os
import subprocess

import pytest

from diffusion_transformer_adaln_amd.build import C_CHECK_BIN

pytestmark = pytest.mark.gpu


def test_c_consumer_on_gpu():
    if not os.path.exists(C_CHECK_BIN):
        pytest.fail(f"{C_CHECK_BIN} is not built: run __graft_entry__.build() first")
    print(f"[c-consumer] {C_CHECK_BIN}", flush=True)
    run = subprocess.run([C_CHECK_BIN], capture_output=True, text=True, timeout=120)
    out = run.stdout + run.stderr
    print(out, flush=True)
    assert run.returncode == 0, out[-2000:]
    assert out.startswith("OK") or "\nOK" in out, out[-2000:]
