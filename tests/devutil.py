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


def _near_tie(ev, x_gpu=None):
    """A decision whose margin is within the tolerance: a test with
    |r/q - u| < 1e-6, or a sample with |CDF - u Z| < 1e-6 Z at the CDF
    boundary between the oracle's token and the GPU's (x_gpu), or, when the
    GPU's token is not known, at either boundary of the oracle's token."""
    if ev[0] == "test":
        _, _, _, r, q, u, _ = ev
        return q > 0 and abs(r / q - u) < 1e-6
    if ev[0] == "sample":
        _, _, x, c, thr = ev
        z = c[-1]
        if x_gpu is not None:
            return 0 <= x_gpu < len(c) and abs(c[min(x, x_gpu)] - thr) < 1e-6 * z
        return abs(c[x] - thr) < 1e-6 * z or (x > 0 and abs(c[x - 1] - thr) < 1e-6 * z)
    return False


def decisive_events(gpu_row, gpu_len, ref_row, ref_len, events):
    """The oracle's events at the first decision where the two walks part.
    Both walks start at the root and agree up to node rp[j - 1]; there
      * both stopped (only the bonus differs): the sample drawn at that node;
      * one side moved to child c and the other to a later child or stopped,
        or both moved to different children: the test of the smaller child
        (one side accepted it, the other rejected it), or, for target
        sampling, the sample drawn at that node (which picked the child);
      * greedy walks have no decision that may be excused."""
    L = min(gpu_len, ref_len)
    j = 1
    while j < L and gpu_row[j] == ref_row[j]:
        j += 1
    node = int(ref_row[j - 1])
    at = [ev for ev in events if ev[1] == node]
    g = int(gpu_row[j]) if j < gpu_len else None
    r = int(ref_row[j]) if j < ref_len else None
    if g is None and r is None:
        return [ev for ev in at if ev[0] == "sample"]
    tests = [ev for ev in at if ev[0] == "test"]
    if tests:
        c = min(x for x in (g, r) if x is not None)
        return [ev for ev in tests if ev[2] == c]
    return [ev for ev in at if ev[0] == "sample"]


def compare_accept(gpu, ref, events):
    """gpu/ref = (path, path_len, bonus) numpy.  A sequence may differ only
    when the decision at which the two walks part (decisive_events) is a near
    tie: a test with |r/q - u| < 1e-6, or a sample with |CDF - u Z| < 1e-6 Z.
    Returns the number of excused sequences."""
    gp, gl, gb = gpu
    rp, rl, rb = ref
    excused = 0
    for b in range(len(rl)):
        if gl[b] == rl[b] and np.array_equal(gp[b], rp[b]) and gb[b] == rb[b]:
            continue
        dec = decisive_events(gp[b], int(gl[b]), rp[b], int(rl[b]), events[b])
        # the GPU's own token is known when both walks stopped at one node
        same_stop = gl[b] == rl[b] and np.array_equal(gp[b], rp[b])
        x_gpu = int(gb[b]) if same_stop else None
        ok = len(dec) > 0 and any(_near_tie(ev, x_gpu) for ev in dec)
        assert ok, "sequence %d: gpu %s/%d/%d vs oracle %s/%d/%d" % (
            b, gp[b, :gl[b]].tolist(), gl[b], gb[b], rp[b, :rl[b]].tolist(), rl[b], rb[b])
        excused += 1
    return excused
