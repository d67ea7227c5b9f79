"""Build libssm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m state_space_model_ssm_amd.build

Each ``csrc/*.hip`` file is compiled with hipcc into ``_build/`` and linked
into ``state_space_model_ssm_amd/libssm.so``.  Packed-FP32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile every source and link libssm.so. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "is not a recognized feature" not in l)
        if pr.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text, flush=True)
    if failed:
        for src, text in failed:
            print(f"--- {src}\n{text}", file=sys.stderr)
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(s) for s, _ in failed))
    tmp = LIB + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
