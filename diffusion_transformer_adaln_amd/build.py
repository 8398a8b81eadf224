"""Build the HIP library ``libadaln.so`` in-tree for gfx950.

    python -m diffusion_transformer_adaln_amd.build

Compiles csrc/adaln_api.cpp (host: validation and dispatch),
csrc/adaln_plan.cpp (host: row layouts, backward tiling, workspace layout),
csrc/adaln_sched.cpp (host: batch scheduling and cost model),
csrc/adaln_kernels.hip (gfx950 kernels), csrc/adaln_noalloc.hip (the
backward entry point that allocates nothing) and csrc/adaln_probe.hip
(streaming ceiling probes, include/adaln_probe.h) with hipcc into one shared
library
next to this file.  Every call recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libadaln.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [os.path.join(CSRC, "adaln_api.cpp"), os.path.join(CSRC, "adaln_plan.cpp"),
           os.path.join(CSRC, "adaln_sched.cpp"), os.path.join(CSRC, "adaln_kernels.hip"),
           os.path.join(CSRC, "adaln_probe.hip"), os.path.join(CSRC, "adaln_noalloc.hip")]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False, out: str = LIB_PATH) -> str:
    """Compile the library; returns its path.  Raises on a failed build."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc_path(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that line is noise
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        try:
            os.unlink(tmp)
        except OSError:
            pass
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


# A torch-free C consumer of the ABI, run by a GPU test (tests/c/adaln_c_check.c).
C_CHECK_SRC = os.path.join(ROOT, "tests", "c", "adaln_c_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c", "adaln_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_check(verbose: bool = False) -> str:
    """Compile the C consumer against the built library (host code only, with
    the system C compiler); returns the executable's path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for tests/c/adaln_c_check.c")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           C_CHECK_SRC, "-o", C_CHECK_BIN,
           "-L" + HERE, "-ladaln", "-Wl,-rpath,$ORIGIN/../../diffusion_transformer_adaln_amd",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"C consumer build failed ({proc.returncode}):\n{proc.stdout}{proc.stderr}")
    return C_CHECK_BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_check(verbose="-v" in sys.argv))
