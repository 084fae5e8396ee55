"""Build the plain C caller of libsas (a test tool) with gcc:
C11, include/sas.h, linked with libsas.so and the HIP runtime, no C++."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sas_c_caller.c")
OUT = os.path.join(HERE, "sas_c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found")
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "gated_block_sparse_select_amd"), "-lsas",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gated_block_sparse_select_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C caller build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {OUT}")
    return OUT


def ensure_built() -> str:
    return OUT if os.path.exists(OUT) else build()


if __name__ == "__main__":
    build(verbose=True)
