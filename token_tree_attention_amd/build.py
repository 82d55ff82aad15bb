"""Build libtreeverify.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m token_tree_attention_amd.build  (or call build()).
Each .hip source compiles to an object under _build/, then one shared
library is linked next to this file.  --debug builds
libtreeverify_debug.so (device bounds checks, TTV_DEBUG); --host-sanitized
the ASan/UBSan build of the host code.
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


DEBUG_OUT = os.path.join(HERE, "libtreeverify_debug.so")


def build(verbose: bool = False, jobs: int = 5, debug: bool = False) -> str:
    """Compile every source (always) and link the library; returns its path.

    debug=True builds libtreeverify_debug.so instead: the same sources with
    TTV_DEBUG defined, whose kernels check the bounds of their data-dependent
    accesses (read back with ttv_debug_report)."""
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    os.makedirs(out_dir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *(["-DTTV_DEBUG"] if debug else []), *EXTRA.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
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
    target = DEBUG_OUT if debug else OUT
    tmp = target + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, target)
    return target


SANITIZED = os.path.join(BUILD, "san", "libtreeverify_san.so")
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")


def build_host_sanitized() -> str:
    """The library's host code with AddressSanitizer and UndefinedBehaviorSanitizer,
    for argument-checking tests on a machine without a GPU.

    Each source is compiled with the sanitizers on the host pass only (the
    device code is built as usual, uninstrumented) and linked with clang++
    against the shared sanitizer runtime.  Load it with that runtime
    preloaded (``sanitizer_runtime()``) and TTV_LIBRARY set to its path.
    """
    out_dir = os.path.dirname(SANITIZED)
    os.makedirs(out_dir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fvisibility=hidden", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append(" ".join(cmd) + "\n" + out)
    if failed:
        raise RuntimeError("sanitized host build failed:\n" + "\n\n".join(failed))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib")
    _run([CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", "-o", SANITIZED, *objs,
          "-L" + rocm_lib, "-Wl,-rpath," + rocm_lib, "-lamdhip64"])
    return SANITIZED


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime the sanitized library links."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    elif "--debug" in sys.argv:
        print(build(verbose="-v" in sys.argv, debug=True))
    else:
        print(build(verbose="-v" in sys.argv))
