"""Build libar.so (the HIP library behind include/ar.h) for gfx950 with hipcc.

Usage: ``python -m ring_allreduce_reduction_virtual_amd.build`` or
``build_library()``.  Writes ``libar.so`` next to this file.  The
translation units compile in parallel; the library is replaced atomically.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libar.so")

SOURCES = ("ar_api.hip", "ar_kernels.hip", "ar_tree_kernels.hip", "ar_persistent_kernels.hip", "ar_dbt_kernels.hip",
           "ar_noalloc.hip")

# -ffp-contract=off: no fused multiply-add, every add/mul rounds on its own.
# -fno-fast-math: IEEE semantics (NaN, signed zero, no reassociation).
# -packed-fp32-ops: keep the compiler from pairing float32 arithmetic into
#  packed instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libar.so")
    return path


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


PROBE_SOURCE = "ar_probe.hip"
PROBE_PATH = os.path.join(PKG_DIR, "libarprobe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile libarprobe.so, the HBM ceiling probes bench.py measures (not part of libar.so)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="ar_probe_") as tmp:
        tmp_lib = os.path.join(tmp, "libarprobe.so")
        out = _run([cc, *HIPCC_FLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp_lib])
        if verbose and out.strip():
            print(out)
        staged = PROBE_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.chmod(staged, 0o755)
        os.replace(staged, PROBE_PATH)
    return PROBE_PATH


def build_library(verbose: bool = False) -> str:
    """Compile and link libar.so (and the probe library beside it); return libar.so's path."""
    with ThreadPoolExecutor(1) as ex:
        probe = ex.submit(build_probe, verbose)
        path = _build_main(verbose)
        probe.result()
    return path


def _build_main(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[cc, *HIPCC_FLAGS, f"-I{INCLUDE}", "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(len(cmds)) as ex:
            outs = list(ex.map(_run, cmds))
        tmp_lib = os.path.join(tmp, "libar.so")
        outs.append(_run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]))
        if verbose:
            for o in outs:
                if o.strip():
                    print(o)
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.chmod(staged, 0o755)
        os.replace(staged, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
