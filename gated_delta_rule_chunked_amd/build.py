"""Build the HIP library ``libkda.so`` in-tree for gfx950.

    python -m gated_delta_rule_chunked_amd.build

Compiles every source under ``csrc/`` with hipcc (device code for gfx950 only)
and links one shared library next to this file.  Always rebuilds.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
ARCH = "gfx950"
SOURCES = ["kda_api.cpp", "kda_intra.hip", "kda_inter.hip", "kda_scan.hip", "kda_bwd.hip", "kda_bwd_scan.hip"]

# Packed fp32 VALU ops are disabled on purpose (see the design notes); the host
# pass prints a harmless "not a recognized feature" warning for it.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-ffp-contract=fast"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE, text=True)
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    try:
        print(build(verbose="-v" in sys.argv))
    except subprocess.CalledProcessError as e:  # show the compiler's own message
        sys.stderr.write(e.stderr or "")
        raise SystemExit(1)
