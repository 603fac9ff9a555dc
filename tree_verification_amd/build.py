"""Builds libsdtree.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m tree_verification_amd.build [--verbose]

Every .hip source under csrc/ is compiled to an object and linked into
tree_verification_amd/libsdtree.so.  The top-k and expansion sources are
compiled with -ffp-contract=off because their float32 arithmetic order is part
of their result.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsdtree.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
PER_FILE = {"topk.hip": ["-ffp-contract=off"], "expand.hip": ["-ffp-contract=off"]}
SOURCES = ["sdtree.hip", "attn.hip", "accept.hip", "commit.hip", "topk.hip", "expand.hip", "build.hip"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    if verbose:
        for _, err in results:
            sys.stderr.write(err)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    # -z defs: every symbol must resolve (a kernel whose host stub was not
    # emitted shows up here rather than at load time)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
