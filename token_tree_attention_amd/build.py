"""Build libtreeverify.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m token_tree_attention_amd.build  (or call build()).
Each .hip source compiles to an object under _build/, then one shared
library is linked next to this file.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtreeverify.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["abi.hip", "tree_build.hip", "tree_attention.hip", "tree_accept.hip", "tree_commit.hip",
           "tree_stochastic.hip", "tree_mask.hip", "tree_ddtree.hip",
           "tree_merge.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-source extras.  The attention kernel never produces or consumes NaN
# (masked scores are -inf, the running max starts finite), so max() needs no
# NaN quieting of its operands.
EXTRA = {"tree_attention.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, jobs: int = 5) -> str:
    """Compile every source (always) and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(" ".join(cmd) + "\n" + out)
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
