"""The C ABI on the CPU: the library loads, exports every function the header
declares, sizes workspaces, and rejects bad arguments on the host before any
HIP call (so these run without a GPU)."""
import ctypes

import pytest

from tree_verification_amd import _lib

L = None


def setup_module():
    global L
    L = _lib.lib()


def test_exports_every_declared_function():
    names = _lib.declared_functions()
    assert len(names) == 16
    for n in names:
        assert hasattr(L, n), n


def test_debug_library_exports_every_declared_function():
    """libsdtree_debug.so (the build with device-side consistency checks)
    loads and exports the same functions."""
    import os
    assert os.path.exists(_lib.DEBUG_LIB_PATH), "run `python -m tree_verification_amd.build --debug`"
    D = ctypes.CDLL(_lib.DEBUG_LIB_PATH)
    for n in _lib.declared_functions():
        assert hasattr(D, n), n
    s = _shape()
    assert D.sd_workspace_bytes(1, ctypes.byref(s), 0) == L.sd_workspace_bytes(1, ctypes.byref(s), 0)


def test_status_strings():
    for code in range(8):
        assert L.sd_status_str(code)
    assert L.sd_status_str(99) == b"unknown status"


def _shape(**kw):
    base = dict(B=16, T=64, Hq=32, Hkv=8, D=128, bs=16, max_blocks=260, num_blocks=4160,
                dtype=1, tree_stride=64, scale=0.0)
    base.update(kw)
    return _lib.SdShape(*[base[f] for f, _ in _lib.SdShape._fields_])


FAKE = ctypes.c_void_p(0x1000)


def _attn(shape, ws_bytes=1 << 40, sel=None, ksel=0, null_q=False):
    return L.sd_tree_verify_attn(ctypes.byref(shape), None if null_q else FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, sel, ksel, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=30), 2), (dict(T=0), 2), (dict(B=0), 2), (dict(tree_stride=5), 2),
    (dict(dtype=7), 3), (dict(D=96), 4), (dict(bs=12), 4), (dict(T=5000, tree_stride=5000), 4),
    (dict(scale=-1.0), 1), (dict(scale=float("inf")), 1),
])
def test_attention_rejects_bad_shapes(kw, code):
    assert _attn(_shape(**kw)) == code


def test_attention_rejects_null_small_ws_and_bad_ksel():
    s = _shape()
    assert _attn(s, null_q=True) == 1
    need = L.sd_workspace_bytes(1, ctypes.byref(s), 0)
    assert need > 0
    assert _attn(s, ws_bytes=need - 1) == 5
    assert _attn(s, sel=FAKE, ksel=0) == 1
    assert _attn(s, sel=FAKE, ksel=65537) == 4
    assert _attn(s, sel=None, ksel=3) == 1


def test_workspace_sizes():
    s = _shape()
    assert L.sd_workspace_bytes(1, ctypes.byref(s), 0) >= 256
    # float32: header + one precomputed ancestor word per node
    assert L.sd_workspace_bytes(1, ctypes.byref(_shape(dtype=0)), 0) >= 256 + 16 * 64 * 8
    assert L.sd_workspace_bytes(1, ctypes.byref(s), 65537) == 0
    assert L.sd_workspace_bytes(1, ctypes.byref(s), 256) > 0
    assert L.sd_workspace_bytes(3, ctypes.byref(s), 32) >= 16 * 260 * 8 * 128 * 4
    assert L.sd_workspace_bytes(3, ctypes.byref(s), 0) == 0
    # commit: status header plus one completion counter per sequence
    assert L.sd_workspace_bytes(4, ctypes.byref(s), 0) == 256 + 256
    a = _lib.SdAcceptShape(16, 64, 128256, 1, 64)
    # 16 workgroups per sequence: barrier state for each of the 16 sequences
    assert L.sd_workspace_bytes(2, ctypes.byref(a), 0) == 256 + 16 * 8192
    one = _lib.SdAcceptShape(1000000, 5, 8, 0, 5)
    assert L.sd_workspace_bytes(2, ctypes.byref(one), 0) == 256
    assert L.sd_workspace_bytes(9, ctypes.byref(s), 0) == 0
    assert L.sd_workspace_bytes(1, None, 0) == 0


def test_accept_rejects_bad_arguments():
    def call(shape, tau=0.8, unif=FAKE, ws=256):
        return L.sd_accept(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, unif, tau, FAKE, FAKE, FAKE,
                           FAKE, ws, None)
    ok = _lib.SdAcceptShape(2, 8, 100, 1, 8)
    assert call(_lib.SdAcceptShape(0, 8, 100, 1, 8)) == 2
    assert call(_lib.SdAcceptShape(2, 8, 100, 1, 3)) == 2
    assert call(_lib.SdAcceptShape(2, 8, 100, 5, 8)) == 3
    assert call(_lib.SdAcceptShape(2, 5000, 100, 1, 5000)) == 4
    assert call(ok, tau=-0.5) == 1
    assert call(ok, tau=float("nan")) == 1
    assert call(ok, unif=None) == 1
    assert call(ok, ws=100) == 5


def test_accept_commit_rejects_bad_arguments():
    def call(shape, kv, tau=0.8, kpages=FAKE, ws=256):
        return L.sd_accept_commit(ctypes.byref(shape), None if kv is None else ctypes.byref(kv), FAKE,
                                  FAKE, FAKE, FAKE, FAKE, tau, FAKE, FAKE, FAKE, kpages, FAKE, FAKE,
                                  FAKE, None, FAKE, ws, None)
    ok = _lib.SdAcceptShape(2, 8, 100, 1, 8)
    kv = _shape(B=2, T=8, Hq=8, tree_stride=8)
    assert call(ok, None) == 1                        # no cache shape
    assert call(ok, _shape(B=3, T=8, Hq=8, tree_stride=8)) == 2      # B differs
    assert call(ok, _shape(B=2, T=9, Hq=8, tree_stride=9)) == 2      # T differs
    assert call(ok, _shape(B=2, T=8, Hq=8, tree_stride=8, D=96)) == 4
    assert call(ok, kv, kpages=None) == 1
    assert call(_lib.SdAcceptShape(2, 8, 100, 5, 8), kv) == 3
    assert call(ok, kv, tau=-1.0) == 1
    assert call(ok, kv, ws=100) == 5


def test_accept_commit_noalloc_rejects_bad_arguments():
    """Host checks of the no-workspace variant, before any HIP call: the same
    as sd_accept_commit's, and a status word is required."""
    def call(shape, kv, tau=0.8, kpages=FAKE, status=FAKE):
        return L.sd_accept_commit_noalloc(ctypes.byref(shape), None if kv is None else ctypes.byref(kv),
                                          FAKE, FAKE, FAKE, FAKE, FAKE, tau, FAKE, FAKE, FAKE, kpages,
                                          FAKE, FAKE, FAKE, None, status, None)
    ok = _lib.SdAcceptShape(2, 8, 100, 1, 8)
    kv = _shape(B=2, T=8, Hq=8, tree_stride=8)
    assert call(ok, None) == 1
    assert call(ok, _shape(B=3, T=8, Hq=8, tree_stride=8)) == 2
    assert call(ok, _shape(B=2, T=8, Hq=8, tree_stride=8, D=96)) == 4
    assert call(ok, kv, kpages=None) == 1
    assert call(_lib.SdAcceptShape(2, 8, 100, 5, 8), kv) == 3
    assert call(ok, kv, tau=-1.0) == 1
    assert call(ok, kv, status=None) == 1


def test_tree_build_rejects_bad_arguments():
    """Host checks of sd_tree_build, before any HIP call."""
    def call(T=64, V=100, dt=0, tau=1.0, root=0, ws=1 << 30, draft=FAKE, parent=FAKE):
        s = _lib.SdBuildShape(T, V, dt)
        return L.sd_tree_build(ctypes.byref(s), draft, tau, root, parent, FAKE, FAKE, None, FAKE, ws, None)
    assert call(T=0) == 2
    assert call(V=0) == 2
    assert call(dt=7) == 3
    assert call(T=3842) == 4                      # T - 1 + 256 candidates would exceed 4096
    assert call(T=3000, V=2000000) == 4           # T * V >= 2^32
    assert call(tau=0.0) == 1
    assert call(tau=float("inf")) == 1
    assert call(root=100) == 1
    assert call(root=-1) == 1
    assert call(draft=None) == 1
    assert call(parent=None) == 1
    assert call(ws=1000) == 5
    need = L.sd_workspace_bytes(7, ctypes.byref(_lib.SdBuildShape(2048, 32000, 0)), 0)
    assert need > 2048 * (8 + 8 + 4)
    assert L.sd_workspace_bytes(7, ctypes.byref(_lib.SdBuildShape(5000, 100, 0)), 0) == 0


def test_block_sums_calls_reject_bad_arguments():
    s = _shape()
    big = 1 << 40
    assert L.sd_block_sums(ctypes.byref(_shape(Hq=7)), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == 2
    assert L.sd_block_sums(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, big, None) == 1
    assert L.sd_block_sums(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == 5
    assert L.sd_block_sums_append(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, big, None) == 1
    assert L.sd_block_sums_append(ctypes.byref(_shape(D=96)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                  None) == 4
    assert L.sd_topk_blocks_cached(ctypes.byref(s), FAKE, None, FAKE, FAKE, 4, FAKE, FAKE, big, None) == 1
    assert L.sd_topk_blocks_cached(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, big, None) == 1
    assert L.sd_topk_blocks_cached(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 10, None) == 5
    # shared selection: neither K nor sums, k < 1, workspace too small
    assert L.sd_topk_blocks_shared(ctypes.byref(s), FAKE, None, None, FAKE, FAKE, 4, FAKE, FAKE, big, None) == 1
    assert L.sd_topk_blocks_shared(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, 0, FAKE, FAKE, big, None) == 1
    assert L.sd_topk_blocks_shared(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 10, None) == 5
    assert L.sd_workspace_bytes(5, ctypes.byref(s), 0) > 0


def test_tree_expand_rejects_bad_arguments():
    def call(E=4, V=100, dt=1, tau=0.8, k=8, ws=1 << 20, out=FAKE):
        return L.sd_tree_expand(ctypes.byref(_lib.SdExpandShape(E, V, dt)), FAKE, FAKE, tau, k, out, FAKE,
                                FAKE, FAKE, ws, None)
    assert call(E=0) == 2
    assert call(dt=7) == 3
    assert call(k=0) == 1
    assert call(k=401) == 1                 # more than E * V
    assert call(E=100, V=100, k=5000) == 4  # more than 4096
    assert call(tau=0.0) == 1
    assert call(out=None) == 1
    assert call(ws=64) == 5
    assert L.sd_workspace_bytes(6, ctypes.byref(_lib.SdExpandShape(4, 100, 1)), 8) > 0
    assert L.sd_workspace_bytes(6, ctypes.byref(_lib.SdExpandShape(4, 100, 1)), 0) == 0


def test_commit_and_topk_reject_bad_arguments():
    s = _shape()
    assert L.sd_kv_commit(ctypes.byref(_shape(Hq=7)), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                          256, None) == 2
    assert L.sd_kv_commit(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 256, None) == 1
    assert L.sd_kv_commit(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 256, None) == 5
    assert L.sd_topk_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 40, None) == 1
    assert L.sd_topk_blocks(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 10, None) == 5
    assert L.sd_device_status(None, None, None) == 1
