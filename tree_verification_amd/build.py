"""Builds libsdtree.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m tree_verification_amd.build [--verbose] [--debug]

Every .hip source under csrc/ is compiled to an object and linked into
tree_verification_amd/libsdtree.so.  The top-k and expansion sources are
compiled with -ffp-contract=off because their float32 arithmetic order is part
of their result.  --debug builds libsdtree_debug.so instead: the same library
with the kernels' device-side consistency checks (SDTREE_DEBUG) compiled in.
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
DEBUG_LIB = os.path.join(HERE, "libsdtree_debug.so")
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


def _compile(src, verbose, debug=False):
    obj = os.path.join(BUILD, "debug" if debug else "", src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *(["-DSDTREE_DEBUG"] if debug else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj, r.stderr


def build(verbose=False, debug=False):
    os.makedirs(os.path.join(BUILD, "debug") if debug else BUILD, exist_ok=True)
    out = DEBUG_LIB if debug else LIB
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose, debug), SOURCES))
    if verbose:
        for _, err in results:
            sys.stderr.write(err)
    objs = [o for o, _ in results]
    tmp = out + ".tmp"
    # -z defs: every symbol must resolve (a kernel whose host stub was not
    # emitted shows up here rather than at load time)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, debug="--debug" in sys.argv))
