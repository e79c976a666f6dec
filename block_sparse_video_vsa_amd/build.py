"""Build step: compile the gfx950 HIP sources into the in-tree libvsa.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/vsa_pack.hip", "csrc/vsa_attn.hip", "csrc/vsa_layout.hip", "csrc/vsa_merge.hip", "csrc/vsa_route.hip",
           "csrc/vsa_api.hip"]
OUTPUT = os.path.join(HERE, "libvsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build_library(verbose: bool = False) -> str:
    """Compile libvsa.so for gfx950 (always rebuilds).  Returns its path."""
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    tmp = OUTPUT + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libvsa.so")
    if verbose:
        noise = ("not a recognized feature", "--hip-link")
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if not any(n in l for n in noise))
        if msg.strip():
            print(msg)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
