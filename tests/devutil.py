"""Moving seeded inputs to the GPU and comparing results with the oracle."""
import numpy as np
import torch


def dev_tensor(a, dtype_tag=None, device="cuda"):
    """numpy -> device tensor; uint16 arrays tagged 'bf16' become bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_device(x, device="cuda"):
    """All buffers of a synth.Inputs on the GPU (a dict of tensors)."""
    d = dict(q=dev_tensor(x.q), k=dev_tensor(x.k_pages), v=dev_tensor(x.v_pages),
             table=dev_tensor(x.block_table), ctx=dev_tensor(x.ctx_lens),
             parent=dev_tensor(x.tree_parent), token=dev_tensor(x.tree_token),
             logits=dev_tensor(x.target_logits), unif=dev_tensor(x.uniforms))
    d["draft"] = None if x.draft_probs is None else dev_tensor(x.draft_probs)
    return d


def check_attention(gpu, ref, dtype, where=""):
    """fp32: row-normwise relative 1e-5; bf16: 2e-2 absolute, elementwise."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), where
    if dtype == "f32":
        err = np.abs(gpu - ref).max(axis=-1)
        nrm = np.abs(ref).max(axis=-1)
        bad = err > 1e-5 * nrm
        assert not bad.any(), "%s: %d rows over 1e-5 rel, worst %.3g" % (
            where, bad.sum(), (err / np.maximum(nrm, 1e-300)).max())
    else:
        err = np.abs(gpu - ref)
        assert err.max() <= 2e-2, "%s: max abs err %.4g" % (where, err.max())


def compare_accept(gpu, ref, events):
    """gpu/ref = (path, path_len, bonus) numpy.  A sequence may differ only
    after a decision whose margin is within the tolerance: a test with
    |r/q - u| < 1e-6, or a sample with |CDF - u Z| < 1e-6 Z.  Returns the
    number of excused sequences."""
    gp, gl, gb = gpu
    rp, rl, rb = ref
    excused = 0
    for b in range(len(rl)):
        if gl[b] == rl[b] and np.array_equal(gp[b], rp[b]) and gb[b] == rb[b]:
            continue
        # first divergence along the walk
        L = min(gl[b], rl[b])
        j = 0
        while j < L and gp[b, j] == rp[b, j]:
            j += 1
        # the decision that ended (or branched) the common prefix happened at node rp[b, j-1]
        node = int(rp[b, j - 1])
        ok = False
        for ev in events[b]:
            if ev[1] != node:
                continue
            if ev[0] == "test":
                _, _, _, r, q, u, _ = ev
                if q > 0 and abs(r / q - u) < 1e-6:
                    ok = True
            elif ev[0] == "sample":
                _, _, x, c, thr = ev
                z = c[-1]
                lo = max(x - 1, 0)
                if abs(c[x] - thr) < 1e-6 * z or (x > 0 and abs(c[lo] - thr) < 1e-6 * z):
                    ok = True
        assert ok, "sequence %d: gpu %s/%d/%d vs oracle %s/%d/%d" % (
            b, gp[b, :gl[b]].tolist(), gl[b], gb[b], rp[b, :rl[b]].tolist(), rl[b], rb[b])
        excused += 1
    return excused
