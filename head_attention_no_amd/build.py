"""Build libfa355.so (the HIP library) in-tree with hipcc for gfx950.

Run ``python -m head_attention_no_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa355.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


# The attention kernel instances: (FA355_ELEM, element name, head dim).
# mha_launch.hip is compiled once per pair; fa355.hip holds the C ABI and
# the top-K kernel.
ELEMS = ((0, "f32"), (1, "bf16"), (2, "f16"))
DIMS = (32, 64, 128, 256)
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature and says so.
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=(), jobs: int = 0) -> str:
    """Compile every unit to an object in a temporary folder (in parallel),
    then link libfa355.so."""
    import concurrent.futures
    import tempfile

    common = [HIPCC, *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC]
    jobs = jobs or max(1, min(os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="fa355_build_") as tmpdir:
        units = [(os.path.join(CSRC, "fa355.hip"), os.path.join(tmpdir, "fa355.o"), [])]
        for elem, name in ELEMS:
            for d in DIMS:
                units.append((os.path.join(CSRC, "mha_launch.hip"),
                              os.path.join(tmpdir, f"mha_{name}_d{d}.o"),
                              [f"-DFA355_ELEM={elem}", f"-DFA355_HEAD_DIM={d}"]))
        cmds = [[*common, *defs, "-c", src, "-o", obj] for src, obj, defs in units]
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([*common, *[obj for _, obj, _ in units], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
