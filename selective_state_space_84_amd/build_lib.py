"""Build the gfx950 selective-scan library in-tree with hipcc.

``python -m selective_state_space_84_amd.build_lib`` (or ``build()``) compiles
``csrc/*.hip`` in parallel and links ``libssm_scan.so`` next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(REPO, "include")
LIB = os.path.join(HERE, "libssm_scan.so")
SOURCES = ["scan_mode0.hip", "scan_mode1.hip", "scan_mode2.hip", "scan_mode3.hip", "scan_mode4.hip", "scan_mode5.hip",
           "scan_mode6.hip", "scan_mode7.hip", "scan_aux.hip",
           "update_kernel.hip", "conv_kernels.hip", "scan_bwd.hip", "ssd_kernel.hip", "abi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of the generated code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="ssm_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                             if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and text.strip():
                print(text)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join("%s:\n%s" % f for f in failed))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
