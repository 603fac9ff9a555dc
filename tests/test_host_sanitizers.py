"""The C ABI's host code (argument checks, launch planning, workspace sizing)
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the host
layer is recompiled with both sanitizers (device code unchanged, since
-fsanitize applies to the host pass only), linked with the release build's
other objects into a separate library, and driven by tests/native/abi_fuzz.c
(a seeded sweep of extreme shapes through every sizing call, and the argument
checks of every entry point).  Any sanitizer report fails the run."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tree_verification_amd")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_host_layer_under_asan_ubsan(tmp_path):
    from tree_verification_amd import build as b
    others = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in b.SOURCES if s != "sdtree.hip"]
    if not all(os.path.exists(o) for o in others) or not os.path.exists(CLANG):
        pytest.skip("release objects or clang missing: run `python -m tree_verification_amd.build`")
    obj = str(tmp_path / "sdtree_san.o")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(PKG, "csrc"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", *host_san, "-c", os.path.join(PKG, "csrc", "sdtree.hip"), "-o", obj])
    so = str(tmp_path / "libsdtree_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, obj, *others, "-o", so])
    exe = str(tmp_path / "abi_fuzz")
    _run([CLANG, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "native", "abi_fuzz.c"), so, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([exe], env=env, timeout=600)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.startswith("checked ")
