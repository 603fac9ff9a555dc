"""sd_attn_timing_events: an attention call given kernel timing events gives
the same output as one without, records both events (a positive elapsed time,
for the single-kernel bf16 call, a split call whose merge kernel records the
stop event, and the float32 call whose ancestor-mask kernel records the start
event), and the setting is used by one call only."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from synth import make_inputs, small_variant
from tests.devutil import to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _rt():
    path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
    rt = ctypes.CDLL(path)
    rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    rt.hipEventQuery.argtypes = [ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return rt


@pytest.mark.parametrize("name,kw", [
    ("llama3_8b_tree64", dict(B=2, ctx_lo=150, ctx_hi=260)),
    ("longctx_paged_tree16", {}),
    ("tiny_chain", {}),
])
def test_timing_events(name, kw):
    print("timing events:", name, flush=True)
    sys.stdout.flush()
    torch.cuda.init()
    c = small_variant(name, **kw)
    x = make_inputs(c)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    ref = tva.tree_verify_attn(*args)
    torch.cuda.synchronize()
    rt = _rt()
    e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
    assert rt.hipEventCreateWithFlags(ctypes.byref(e0), 0) == 0
    assert rt.hipEventCreateWithFlags(ctypes.byref(e1), 0) == 0
    try:
        tva.attn_timing_events(e0.value, e1.value)
        out = tva.tree_verify_attn(*args)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
        ms = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(ms), e0, e1) == 0
        assert 0.0 < ms.value < 1000.0
        # the setting was consumed: a second call leaves the events as they are
        first = ms.value
        out2 = tva.tree_verify_attn(*args)
        torch.cuda.synchronize()
        assert rt.hipEventElapsedTime(ctypes.byref(ms), e0, e1) == 0
        assert ms.value == first
        assert torch.equal(out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
    finally:
        rt.hipEventDestroy(e0)
        rt.hipEventDestroy(e1)
    assert tva.device_status() == 0
