"""Compile the HIP library for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCE = os.path.join(PKG, "csrc", "attn_fwd.hip")
SOURCES = (SOURCE, os.path.join(PKG, "csrc", "attn_bwd.hip"), os.path.join(PKG, "csrc", "gemm.hip"))
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libattn_fwd.so")
# Debug build of the forward alone: LDS filled with NaN before any copy
# lands (tests compare it bit for bit with the library).
POISON_LIBRARY = os.path.join(PKG, "libattn_fwd_lds_poison.so")
# Debug build of the forward alone: every key tile takes the online-softmax
# rescale branch (new maximum, O and l rescaled, probabilities formed again),
# which ordinary inputs reach rarely; tests compare it with the oracle.
RESCALE_LIBRARY = os.path.join(PKG, "libattn_fwd_force_rescale.so")
# Test library: the forward's layout functions run on one tile, returning
# every fragment (the layout tests check them against host matrices).
LAYOUT_SOURCE = os.path.join(PKG, "csrc", "layout_probe.hip")
LAYOUT_LIBRARY = os.path.join(PKG, "liblayout_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Build libattn_fwd.so, the two debug builds of the forward (LDS
    poison, forced rescale) and the layout-probe test library in the package
    directory, the compiles in parallel; returns the library's path."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(LIBRARY, list(SOURCES), []),
            (POISON_LIBRARY, [SOURCE], ["-DATTN_DEBUG_POISON_LDS"]),
            (RESCALE_LIBRARY, [SOURCE], ["-DATTN_DEBUG_FORCE_RESCALE"]),
            (LAYOUT_LIBRARY, [LAYOUT_SOURCE], [])]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_compile, out, srcs, extra, verbose) for out, srcs, extra in jobs]:
            f.result()
    return LIBRARY


def _compile(out: str, sources: list, extra: list, verbose: bool) -> None:
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-o", tmp, *sources]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)


if __name__ == "__main__":
    print(build(verbose=True))
