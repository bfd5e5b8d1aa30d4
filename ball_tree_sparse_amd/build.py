"""Build libbtsparse.so for gfx950 with hipcc (in-tree).

Usage: python -m ball_tree_sparse_amd.build   (or __graft_entry__.build()).
Every call recompiles all HIP units.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbtsparse.so")
SOURCES = ["api.hip", "ball_attn.hip", "ball_attn_bwd.hip", "permute.hip", "tree.hip", "bsa.hip",
           "bsa_bwd.hip", "pool.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast-honor-pragmas",
]
# the tree's split rule is defined on fp32 values rounded after every
# operation, so nothing in that unit may be contracted into an FMA
PER_FILE = {"tree.hip": ["-ffp-contract=off"],
            # MFMA results straight into VGPRs: the backward reads every
            # accumulator element back, so AGPR copies only cost VALU issue
            "ball_attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False, jobs: int = 5) -> str:
    tmp = tempfile.mkdtemp(prefix="btsparse_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            extra = PER_FILE.get(src, [])
            cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = False
        for cmd, p in procs:
            out, _ = p.communicate()
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                sys.stderr.write(out + "\n")
                failed = True
            elif verbose and out.strip():
                print(out)
        if failed:
            raise RuntimeError("hipcc failed")
        tmp_lib = os.path.join(tmp, "libbtsparse.so")
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        shutil.move(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
