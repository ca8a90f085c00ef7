"""Build of the HIP library ``lib/libtah.so`` for gfx950 (hipcc, in-tree)."""

from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIBDIR, "libtah.so")
SOURCES = ["tah_abi.hip", "tah_encode.hip", "tah_decode.hip", "tah_select.hip", "tah_naive.hip", "tah_hadamard.hip",
           "tah_greedy.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every fused multiply-add is written out (fmaf), none is
# formed by the compiler, so the fp32 operation order is the one in the source.
# Packed fp32 instructions are disabled.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


# Per-file flags (none at present).
FILE_FLAGS: dict = {}


def _compile(src: str, out: str, extra: list) -> None:
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")


def build(extra: list | None = None, jobs: int = 4) -> str:
    """Compile every source and link the shared library. Always recompiles."""
    extra = list(extra or [])
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
    tmp = LIB_PATH + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], capture_output=True,
                       text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
