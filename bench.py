"""Benchmark of the tree-verification pass on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--settle-ms 200]
                    [--workload llama3_8b_tree64]

One step is one verification pass over one batch: tree-masked attention
(sd_tree_verify_attn, which also builds the ancestor masks), then the
acceptance walk and the commit of the accepted paths in one launch
(sd_accept_commit, which gives the results of sd_accept then sd_kv_commit);
the sparse workload first selects blocks from kept block key sums
(sd_topk_blocks_cached; the sums are built once for the starting lengths,
and a step's commit writes only positions past them) and attends sparsely.
Each timed step gets its own copy of the starting context lengths, made
before the timed region, so every step does the same work and no restore
copy runs between steps (the untimed steps restore them instead).  The K/V
pages are held in several copies (--kv-copies, default 2) and consecutive
steps use different ones, so a step cannot find the previous step's K/V in
the 256 MB last-level cache.

Prints one JSON line: verified tree tokens/s (B * T per step) over the timed
steps, the attention call against the HBM or MFMA roofline (algorithmic
bytes or FLOPs per call / event-timed call duration), and the CPU oracle
timed on a bounded sample of the same workload.  The attention call of every
10th timed step (--event-every; more often when fewer than 200 steps are
timed, so that at least 20 calls are) is timed with HIP events that its
first kernel records at its start and its last kernel at its end
(sd_attn_timing_events, hipExtLaunchKernelGGL): the kernels' own device time,
without the idle gap of event markers recorded on the stream around the call.  Before the warmup steps, untimed
steps run for --settle-ms so the GPU has left its idle clocks.

`secondary` lists the other workloads, each with its attention call against
its roofline (the call inside 40 whole steps, timed by its own kernels'
events as above; the mean of back-to-back calls alternating between two K/V
copies is `attention_loop_us`), its whole step, and the selection call of
the sparse modes; the
2048-node tree also reports the MFMA FLOPs its kernel executes against the
algorithmic ones.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
METRIC = "verified tree tokens/s + achieved HBM GB/s (or MFMA %) of tree-verify, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="before the warmup steps, run untimed steps for this long so the "
                         "GPU leaves its idle clocks (a step is ~0.15 ms; without this the "
                         "first tens of milliseconds of steps run up to 10%% slower)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="time the attention call of every N-th timed step with HIP events that "
                         "its kernels record at their start and end")
    ap.add_argument("--kv-copies", type=int, default=2,
                    help="K/V page copies, used by consecutive steps in turn")
    ap.add_argument("--workload", default="llama3_8b_tree64")
    ap.add_argument("--selection", choices=["per_row", "shared", "dense"], default="per_row",
                    help="sparse workload: one block selection per query row (sd_topk_blocks_cached), "
                         "one per (sequence, KV group) (sd_topk_blocks_shared), or none (dense "
                         "attention over the whole context)")
    ap.add_argument("--shared-selection", action="store_true", help="the same as --selection shared")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads' measurements (attention against its roofline, "
                         "the whole step, the selection calls)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device-to-device 3 times (a plain copy "
                         "kernel of known size that scales the HBM byte counters)")
    ap.add_argument("--sweep", choices=["tree", "topk", "expand", "calib"],
                    help="no bench line: one JSON line per point of a sweep instead.  tree: the "
                         "attention of the 8B-like shape (B 16, 32/8 heads, ctx 4096) over tree "
                         "sizes T = 1 .. 4096, across the HBM / MFMA crossover; topk: the block "
                         "selection of the 4 x 64K workload over k, from K and from kept sums; "
                         "expand: one draft-tree expansion step (sd_tree_expand) over batch "
                         "sizes, vocabulary 32000, k 2048, with the oracle timed beside it; "
                         "calib: the drafter's recalibration pass (chain attention over a "
                         "32/8-head, D 64 cache of 16 x 4096, then the identity-path commit) "
                         "over chain lengths T = 1 .. 32")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no run: turn the counter_collection.csv files of a rocprofv3 "
                         "--pmc FETCH_SIZE pass and a --pmc WRITE_SIZE pass (both of a run "
                         "with --copy-calibration) into profiles/traffic_attn_<workload>.json")
    return ap.parse_args()


def ancestor_sizes(parent):
    """|anc*(i)| for every node (depth + 1)."""
    T = len(parent)
    depth = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        depth[i] = depth[parent[i]] + 1 if parent[i] >= 0 else 0
    return depth + 1


def attention_cost(cfg, x, sel=None):
    """Algorithmic bytes and FLOPs of one attention call.
    Bytes: every context K/V row read once (the selected blocks' rows when
    sparse, deduplicated per KV group), the tree slots' K/V, q and out.
    FLOPs: 4 * D per (query head, visible key) pair."""
    e = 4 if cfg.dtype == "f32" else 2
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    ctx = x.ctx_lens.astype(np.int64)
    pairs = 0
    kv_rows = 0
    for b in range(B):
        par = x.tree_parent[0] if x.tree_parent.shape[0] == 1 else x.tree_parent[b]
        anc = int(ancestor_sizes(par).sum())
        if sel is None:
            pairs += Hq * (T * int(ctx[b]) + anc)
            kv_rows += Hkv * (int(ctx[b]) + T)
        else:
            G = Hq // Hkv
            for g in range(Hkv):
                blocks = np.unique(sel[b, :, g * G:(g + 1) * G].ravel())
                blocks = blocks[blocks >= 0]
                valid = np.minimum(cfg.bs, ctx[b] - blocks * cfg.bs).sum()
                kv_rows += int(valid) + T
            for i in range(T):
                for h in range(Hq):
                    s = sel[b, i, h]
                    s = s[s >= 0]
                    pairs += int(np.minimum(cfg.bs, ctx[b] - s * cfg.bs).sum())
            pairs += Hq * anc
    bytes_ = kv_rows * D * e * 2 + 2 * B * T * Hq * D * e
    flops = 4 * D * pairs
    return bytes_, flops


def accept_cost(cfg, plen):
    """Algorithmic bytes of one acceptance call: every visited node's target
    logits row, and for rejection sampling its draft probability row (float32),
    read once.  The visited nodes of a sequence are its accepted path (the
    last one is where the walk stops); residual passes reread the row from the
    workgroups' registers, and the test scalars are a few bytes."""
    e_logit = 2 if cfg.logit_dtype == "bf16" else 4
    per_row = cfg.V * (e_logit + (4 if cfg.mode == "mss" else 0))
    return int(np.asarray(plen, dtype=np.int64).sum()) * per_row


def roofline_for(cfg, bytes_, flops, seconds):
    ai = flops / bytes_
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if cfg.dtype == "f32":
        ridge = FP32_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        achieved = bytes_ / seconds / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    peak = FP32_PEAK_TFLOPS if cfg.dtype == "f32" else BF16_PEAK_TFLOPS
    achieved = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4)}


def executed_mfma_flops_256x32(cfg, x):
    """MFMA FLOPs the bf16 kernel issues when it runs 256-row query tiles over
    32-key tiles (its plan for the 2048-node tree workload): every tile of a
    (sequence, KV head, 256-row tile) runs 256 x 32 x D multiply-adds for the
    scores and as many for P V, over all context tiles and those tree tiles
    that hold an ancestor of one of the tile's nodes (the others are
    skipped)."""
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    G = Hq // Hkv
    rows, nk = 256, 32
    per_tile = 4 * rows * nk * D
    total = 0
    for b in range(B):
        par = x.tree_parent[0] if x.tree_parent.shape[0] == 1 else x.tree_parent[b]
        ctx_tiles = (int(x.ctx_lens[b]) + nk - 1) // nk
        nodes_per_tile = rows // G
        for q0 in range(0, T * G, rows):
            touched = set()
            for i in range(q0 // G, min(T, q0 // G + nodes_per_tile)):
                n = i
                while n >= 0:
                    touched.add(n // nk)
                    n = int(par[n]) if n > 0 else -1
            total += Hkv * (ctx_tiles + len(touched)) * per_tile
    return total


def bound_attention(w, sel=None, kv=0):
    """A closure calling sd_tree_verify_attn through the C ABI with its
    arguments marshalled once (so back-to-back calls are not spaced out by
    host-side argument handling)."""
    import ctypes
    from tree_verification_amd import _lib
    k, v = w.kvs[kv]
    shape = _lib.make_shape(w.q, k, w.table, w.parent)
    k_sel = 0 if sel is None else sel.shape[-1]
    need = _lib.workspace_bytes(_lib.SD_CALL_ATTN, shape, k_sel)
    ws = _lib._WS.get(w.q.device, need, _lib.SD_CALL_ATTN)
    fn = _lib.lib().sd_tree_verify_attn
    args = (ctypes.byref(shape), _lib._ptr(w.q), _lib._ptr(k), _lib._ptr(v), _lib._ptr(w.table),
            _lib._ptr(w.ctx), _lib._ptr(w.parent), _lib._ptr(sel), k_sel, _lib._ptr(w.out),
            _lib._ptr(ws), ws.numel(), _lib._stream(w.q.device))
    keep = (shape, ws)

    def call():
        assert fn(*args) == 0, keep
    return call


def loop_us(torch, calls, n=40, rounds=3):
    """Median over `rounds` of the mean device time of n back-to-back calls
    (cycling through `calls`), two HIP events around each round."""
    ts = []
    for _ in range(rounds):
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for j in range(n):
            calls[j % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n * 1e3)
    return float(np.median(ts))


def _between(text, start, end):
    i = text.index(start)
    return text[i:text.index(end, i)]


def attn_source_hash():
    """sha256 over what decides the attention kernels and their launch: the
    attention source, the plan function and the argument structs."""
    csrc = os.path.join(ROOT, "tree_verification_amd", "csrc")
    h = hashlib.sha256()
    h.update(open(os.path.join(csrc, "attn.hip"), "rb").read())
    host = open(os.path.join(csrc, "sdtree.hip")).read()
    h.update(_between(host, "static AttnPlan plan_attn", "\n}\n").encode())
    common = open(os.path.join(csrc, "common.h")).read()
    h.update(_between(common, "struct AttnPlan {", "};").encode())
    h.update(_between(common, "struct AttnArgs {", "};").encode())
    return h.hexdigest()


def traffic_for(kernel_key, workload):
    """HBM bytes per attention call from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes, if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel_key, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != attn_source_hash():
        return None
    return rec.get("bytes_per_call")


def _counter_means(path, counter):
    """Mean counter value (KiB per dispatch) of every kernel in a rocprofv3
    counter_collection.csv, keyed by (kernel name, grid size)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = (r["Kernel_Name"], int(r["Grid_Size"]))
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _calibration_kib(path, counter):
    """Mean counter value of the calibration copies: the last three copy
    dispatches of the run (bench.py issues them after everything else; the
    K/V page copies made at set-up launch the same kernel with the same grid)."""
    import csv
    vals = [(int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    last = [v for _, v in sorted(vals)[-3:]]
    return sum(last) / len(last)


def write_traffic(workload, fetch_csv, write_csv, copy_mib):
    """HBM bytes per attention call: FETCH_SIZE and WRITE_SIZE of the attention
    kernels (KiB per dispatch), each scaled by the ratio of the known size of
    the calibration copy to what the same counter reads for it."""
    copy_bytes = copy_mib << 20
    out = {"workload": workload, "copy_bytes": copy_bytes,
           "source_sha256": attn_source_hash(), "counters": {}}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        means = _counter_means(path, counter)
        cal = _calibration_kib(path, counter)
        scale = copy_bytes / (cal * 1024.0)
        attn = {n: v for (n, _), v in means.items()
                if "attn_mfma_kernel" in n or "attn_combine_kernel" in n}
        kib = sum(attn.values())
        out["counters"][counter] = {"attention_kib_per_call": round(kib, 3),
                                    "copy_kib": round(cal, 3), "scale": round(scale, 5),
                                    "bytes_per_call": int(kib * 1024.0 * scale),
                                    "kernels": sorted(attn)}
        total += kib * 1024.0 * scale
    out["bytes_per_call"] = int(total)
    path = os.path.join(ROOT, "profiles", "traffic_attn_%s.json" % workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


class HipEvent:
    """A HIP event on torch's current stream, created with
    hipEventDisableSystemFence: recording it skips the system-scope fence
    (an L2 writeback) that a default event performs, which would otherwise be
    counted inside the interval it bounds."""
    _rt = None

    @classmethod
    def runtime(cls):
        if cls._rt is None:
            import ctypes
            path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
            rt = ctypes.CDLL(path)     # the runtime torch already loaded
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._rt = rt
        return cls._rt

    def __init__(self, flags=0x20000000):
        import ctypes
        self.h = ctypes.c_void_p()
        assert self.runtime().hipEventCreateWithFlags(ctypes.byref(self.h), flags) == 0

    def record(self):
        import torch
        assert self.runtime().hipEventRecord(self.h, torch.cuda.current_stream().cuda_stream) == 0

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        assert self.runtime().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) == 0
        return ms.value

    def __del__(self):
        if self._rt is not None and self.h:
            self._rt.hipEventDestroy(self.h)


class Workload:
    def __init__(self, name, kv_copies=1, shared=False):
        import torch
        import tree_verification_amd as tva
        from synth import CONFIGS, make_inputs
        self.tva = tva
        self.torch = torch
        self.cfg = cfg = CONFIGS[name]
        self.x = x = make_inputs(cfg)

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
            return torch.from_numpy(a).cuda()
        self.q, self.k, self.v = dev(x.q), dev(x.k_pages), dev(x.v_pages)
        self.kvs = [(self.k, self.v)] + [(self.k.clone(), self.v.clone()) for _ in range(kv_copies - 1)]
        self.n_steps = 0
        self.table, self.ctx = dev(x.block_table), dev(x.ctx_lens)
        self.ctx0 = self.ctx.clone()
        self.parent, self.token = dev(x.tree_parent), dev(x.tree_token)
        self.logits, self.unif = dev(x.target_logits), dev(x.uniforms)
        self.draft = dev(x.draft_probs) if cfg.mode == "mss" else None
        self.tau = 0.0 if cfg.mode == "greedy" else cfg.temperature
        self.out = torch.empty_like(self.q)
        B, T = cfg.B, cfg.T
        self.path = torch.empty((B, T), dtype=torch.int32, device="cuda")
        self.plen = torch.empty(B, dtype=torch.int32, device="cuda")
        self.bonus = torch.empty(B, dtype=torch.int32, device="cuda")
        self.sel = None
        self.sums = None
        self.shared = shared
        if cfg.topk:
            self.sel = torch.empty((B, T, cfg.Hq, cfg.topk), dtype=torch.int32, device="cuda")
            # kept block key sums for the starting lengths: a commit writes only
            # positions >= ctx, so they stay current for every step (and for
            # both K/V copies, which agree below ctx)
            self.sums = self.tva.block_sums(self.k, self.table, self.ctx)

    def set_selection(self, mode):
        """Sparse workload: 'dense' attends to the whole context, 'per_row'
        selects blocks per query row from the kept sums, 'shared' one
        selection per (sequence, KV group)."""
        import torch
        cfg = self.cfg
        if mode == "dense":
            self.sel = None
        else:
            if self.sel is None:
                self.sel = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.topk), dtype=torch.int32, device="cuda")
            self.shared = mode == "shared"
            self.select(self.ctx)
            self.torch.cuda.synchronize()

    def select(self, ctx):
        if self.sel is not None and self.shared:
            self.tva.topk_blocks_shared(self.q, self.k, self.table, ctx, self.cfg.topk, sums=self.sums,
                                        sel=self.sel)
        elif self.sel is not None:
            self.tva.topk_blocks_cached(self.q, self.sums, self.k, self.table, ctx, self.cfg.topk,
                                        sel=self.sel)

    def attention(self, ctx=None):
        self.tva.tree_verify_attn(self.q, self.k, self.v, self.table, self.ctx if ctx is None else ctx,
                                  self.parent, out=self.out, sel_blocks=self.sel)

    def step(self, ev=None, ctx=None):
        """One pass.  With `ctx` (a fresh copy of the context lengths, which
        the commit advances) nothing is restored afterwards; without it the
        step runs on the workload's own lengths and restores them."""
        tva = self.tva
        restore = ctx is None
        if restore:
            ctx = self.ctx
        self.k, self.v = self.kvs[self.n_steps % len(self.kvs)]
        self.n_steps += 1
        self.select(ctx)
        if ev is not None:
            # the attention kernels themselves record the two events
            tva.attn_timing_events(ev[0].h.value, ev[1].h.value)
        self.attention(ctx)
        # the acceptance walk and the commit of its paths, in one launch
        tva.accept_commit(self.logits, self.draft, self.parent, self.token, self.unif, self.tau,
                          self.k, self.v, self.table, ctx,
                          path=self.path, path_len=self.plen, bonus=self.bonus)
        if restore:
            ctx.copy_(self.ctx0)


def time_calls(w, reps=10):
    """Per-call device times (event-timed loops of each call alone)."""
    torch = w.torch
    tva = w.tva
    res = {}

    def loop(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    res["attention_us"] = loop(w.attention)
    res["accept_us"] = loop(lambda: tva.accept(w.logits, w.draft, w.parent, w.token, w.unif, w.tau,
                                               path=w.path, path_len=w.plen, bonus=w.bonus))

    def commit():
        tva.kv_commit(w.k, w.v, w.table, w.ctx, w.path, w.plen)
        w.ctx.copy_(w.ctx0)
    res["commit_plus_restore_us"] = loop(commit)

    def accept_commit():
        tva.accept_commit(w.logits, w.draft, w.parent, w.token, w.unif, w.tau, w.k, w.v, w.table, w.ctx,
                          path=w.path, path_len=w.plen, bonus=w.bonus)
        w.ctx.copy_(w.ctx0)
    res["accept_commit_plus_restore_us"] = loop(accept_commit)
    if w.sel is not None:
        res["topk_cached_us"] = loop(lambda: tva.topk_blocks_cached(w.q, w.sums, w.k, w.table, w.ctx,
                                                                    w.cfg.topk, sel=w.sel))
        res["topk_from_k_us"] = loop(lambda: tva.topk_blocks(w.q, w.k, w.table, w.ctx, w.cfg.topk, sel=w.sel))
        res["topk_shared_cached_us"] = loop(lambda: tva.topk_blocks_shared(w.q, w.k, w.table, w.ctx, w.cfg.topk,
                                                                           sums=w.sums, sel=w.sel))
        # leave the selection the step uses in place
        if w.shared:
            tva.topk_blocks_shared(w.q, w.k, w.table, w.ctx, w.cfg.topk, sums=w.sums, sel=w.sel)
        else:
            tva.topk_blocks_cached(w.q, w.sums, w.k, w.table, w.ctx, w.cfg.topk, sel=w.sel)
        scratch = w.sums.clone()
        n_new = torch.full_like(w.ctx, 5)
        ctx_new = w.ctx + n_new
        res["block_sums_append_5_us"] = loop(lambda: tva.block_sums_append(w.k, w.table, ctx_new, n_new,
                                                                           scratch))

        def accept_commit_sums():
            # the acceptance, the commit and the sums' extension in one launch
            # (the scratch sums' values do not matter for the timing)
            tva.accept_commit(w.logits, w.draft, w.parent, w.token, w.unif, w.tau, w.k, w.v, w.table,
                              w.ctx, path=w.path, path_len=w.plen, bonus=w.bonus, sums=scratch)
            w.ctx.copy_(w.ctx0)
        res["accept_commit_sums_plus_restore_us"] = loop(accept_commit_sums)
    return {k: round(v, 1) for k, v in res.items()}


def step_loop_us(w, n=40):
    """Mean device time of n whole steps back to back (each on its own copy of
    the starting context lengths), two HIP events around the loop."""
    torch = w.torch
    for _ in range(4):
        w.step()
    ctxs = [w.ctx0.clone() for _ in range(n)]
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record()
    for j in range(n):
        w.step(None, ctxs[j])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def step_attention_us(w, n=40):
    """Mean duration of the attention call inside n whole steps (each on its
    own copy of the starting context lengths), timed with HIP events that
    the call's own kernels record at their start and end, after 200 ms of
    untimed steps."""
    torch = w.torch
    # untimed steps for 200 ms first: after the workload's set-up on the host
    # the GPU is back at its idle clocks
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        for _ in range(10):
            w.step()
        torch.cuda.synchronize()
    ctxs = [w.ctx0.clone() for _ in range(n)]
    evs = [(HipEvent(), HipEvent()) for _ in range(n)]
    torch.cuda.synchronize()
    for j in range(n):
        w.step(evs[j], ctxs[j])
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3


def measure_workload(w, label, n_calls=40):
    """One workload's attention against its roofline (the call inside n_calls
    whole steps, timed by its own kernels' events, as the headline workload's
    is), the mean of back-to-back calls alternating between the K/V copies
    (`attention_loop_us`), its whole step, and, for the sparse modes, the
    selection call."""
    torch, cfg = w.torch, w.cfg
    sel = w.sel
    t_us = step_attention_us(w, n=n_calls)
    calls = [bound_attention(w, sel, kv) for kv in range(len(w.kvs))]
    loop = loop_us(torch, calls, n=n_calls)
    sel_np = None if sel is None else sel.cpu().numpy()
    bytes_, flops = attention_cost(cfg, w.x, sel_np)
    roof = roofline_for(cfg, bytes_, flops, t_us * 1e-6)
    e = {"workload": cfg.name, "call": label, "attention_us": round(t_us, 2),
         "timed_calls": n_calls, "attention_loop_us": round(loop, 2),
         "bytes_per_call": int(bytes_), "flops_per_call": int(flops),
         "roofline": roof, "verified_tree_tokens_per_s": round(cfg.B * cfg.T / (t_us * 1e-6), 1)}
    if sel is not None:
        f = (lambda: w.tva.topk_blocks_shared(w.q, w.k, w.table, w.ctx, cfg.topk, sums=w.sums, sel=w.sel)) \
            if w.shared else \
            (lambda: w.tva.topk_blocks_cached(w.q, w.sums, w.k, w.table, w.ctx, cfg.topk, sel=w.sel))
        e["selection_us"] = round(loop_us(torch, [f], n=20), 2)
    step_us = step_loop_us(w)
    e["step_us"] = round(step_us, 2)
    e["step_tree_tokens_per_s"] = round(cfg.B * cfg.T / (step_us * 1e-6), 1)
    e["mean_path_len"] = round(float(w.plen.cpu().numpy().mean()), 3)
    return e


def tree_build_on_gpu(w):
    """The 2048-node tree built on the GPU (sd_tree_build) from the drafter
    table the input generator uses: its time (median of 5 builds, each
    waiting once per round) and whether it equals the tree the step verifies."""
    from synth.inputs import _normals, _rng, S_DRAFT
    torch, cfg = w.torch, w.cfg
    d = _normals(_rng(cfg, S_DRAFT), (cfg.T, cfg.V), cfg.logit_sigma, "f32")
    dt = torch.from_numpy(d).cuda()
    root = int(w.x.tree_token[0, 0])
    ts = []
    for _ in range(6):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p, tk, _, rounds = w.tva.tree_build(dt, 1.0, root)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    same = bool(np.array_equal(p.cpu().numpy(), w.x.tree_parent[0]) and
                np.array_equal(tk.cpu().numpy(), w.x.tree_token[0]))
    return {"tree_build_us": round(float(np.median(ts[1:])) * 1e6, 1), "tree_build_rounds": rounds,
            "tree_build_equals_input_tree": same}


def secondary_workloads():
    """The other four workloads, each measured as measure_workload does; the
    sparse workload three ways (dense attention, per-row selection, shared
    selection), the 2048-node tree with its executed-to-algorithmic MFMA
    FLOP ratio."""
    out = []
    for name in ("specexec_70b_tree2048", "longctx_paged_tree16", "sparse_topk32_ctx64k", "tiny_chain"):
        w = Workload(name, kv_copies=2)
        if w.cfg.topk:
            for mode in ("dense", "per_row", "shared"):
                w.set_selection(mode)
                out.append(measure_workload(w, {"dense": "attention (dense)",
                                                "per_row": "sparse attention, selection per query row",
                                                "shared": "sparse attention, selection per KV group"}[mode]))
        else:
            e = measure_workload(w, "attention")
            if name == "specexec_70b_tree2048":
                ex = executed_mfma_flops_256x32(w.cfg, w.x)
                e["executed_mfma_flops_per_call"] = int(ex)
                e["executed_over_algorithmic_flops"] = round(ex / e["flops_per_call"], 4)
                e.update(tree_build_on_gpu(w))
            out.append(e)
        print(json.dumps({"secondary_done": name}), file=sys.stderr, flush=True)
        del w
        import torch
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, budget_s):
    """The oracle on a bounded sample of the same workload, scaled to a step."""
    import oracle
    cfg, x = w.cfg, w.x
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    rng = np.random.default_rng(7)
    # attention rows: calibrate on a few rows, then fill about 60% of the budget
    sel = None
    if cfg.topk:
        t0 = time.perf_counter()
        sel = oracle.topk_blocks(x.q[:1, :1], x.k_pages, x.block_table[:1], x.ctx_lens[:1], cfg.bs,
                                 cfg.topk, cfg.dtype)
        topk_one = time.perf_counter() - t0          # block means of one sequence + 1 node
    def rows_of(n):
        return [(int(rng.integers(cfg.B)), int(rng.integers(cfg.T)), int(rng.integers(cfg.Hq)))
                for _ in range(n)]
    t0 = time.perf_counter()
    oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens, x.tree_parent,
                           cfg.bs, cfg.dtype, rows=rows_of(4))
    per_row = (time.perf_counter() - t0) / 4
    n_rows = int(max(8, min(4096, 0.6 * budget_s / max(per_row, 1e-6))))
    rows = rows_of(n_rows)
    t0 = time.perf_counter()
    oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens, x.tree_parent,
                           cfg.bs, cfg.dtype, rows=rows)
    t_attn = (time.perf_counter() - t0) / n_rows * cfg.B * cfg.T * cfg.Hq
    n_seq = min(cfg.B, 2)
    t0 = time.perf_counter()
    path, plen, _ = oracle.accept(x.target_logits[:n_seq], cfg.logit_dtype,
                                  None if x.draft_probs is None else x.draft_probs[:n_seq],
                                  x.tree_parent[:n_seq] if x.tree_parent.shape[0] > 1 else x.tree_parent,
                                  x.tree_token[:n_seq] if x.tree_token.shape[0] > 1 else x.tree_token,
                                  x.uniforms[:n_seq], w.tau)
    t_acc = (time.perf_counter() - t0) / n_seq * cfg.B
    t0 = time.perf_counter()
    oracle.commit(x.k_pages, x.v_pages, x.block_table[:n_seq], x.ctx_lens[:n_seq], path, plen, cfg.bs)
    t_commit = (time.perf_counter() - t0) / n_seq * cfg.B
    t_step = t_attn + t_acc + t_commit
    sample = ("%d attention rows of %d, acceptance and commit of %d of %d sequences, scaled to one step"
              % (n_rows, cfg.B * cfg.T * cfg.Hq, n_seq, cfg.B))
    if cfg.topk:
        t_step += topk_one * cfg.B
        sample += "; block selection of one sequence scaled by B"
    return {"value": round(cfg.B * cfg.T / t_step, 3), "unit": "verified tree tokens/s",
            "cores": int(threads), "kind": "oracle", "sample": sample,
            "step_s_est": round(t_step, 3)}


def _median_us(torch, fn, reps=10, rounds=5):
    ts = []
    for _ in range(rounds):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps * 1e3)
    return float(np.median(ts))


def sweep(kind):
    """Timing sweeps (one JSON line per point), each point after a 200 ms settle
    of its own calls.  Inputs are the workloads' seeded synthetic recipes with
    one dimension varied (a small vocabulary: only attention or selection is
    timed)."""
    import dataclasses
    import torch
    import tree_verification_amd as tva
    from synth import CONFIGS, make_inputs
    from tests.devutil import to_device

    def settle(fn):
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()

    if kind == "tree":
        base = CONFIGS["llama3_8b_tree64"]
        for T in (1, 4, 16, 32, 64, 80, 128, 256, 512, 1024, 2048, 4096):
            c = dataclasses.replace(base, T=T, V=16, max_parent_depth=8)
            x = make_inputs(c)
            d = to_device(x)
            f = lambda: tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
            settle(f)
            t = _median_us(torch, f) * 1e-6
            bytes_, flops = attention_cost(c, x)
            line = {"sweep": "tree", "T": T, "M": T * c.Hq // c.Hkv, "attention_us": round(t * 1e6, 1),
                    "hbm_tb_s": round(bytes_ / t / 1e12, 3), "mfma_tflop_s": round(flops / t / 1e12, 1),
                    "roofline": roofline_for(c, bytes_, flops, t),
                    "verified_tree_tokens_per_s": round(c.B * T / t, 1)}
            print(json.dumps(line), flush=True)
            del d, x
    elif kind == "calib":
        # the drafter's recalibration pass: chain attention over its cache
        # (32/8 heads, D 64, 16 x 4096 context), then the identity-path commit
        base = dataclasses.replace(CONFIGS["llama3_8b_tree64"], Hq=32, Hkv=8, D=64, tree="chain",
                                   max_parent_depth=0, max_children=0, V=16)
        for T in (1, 2, 4, 8, 16, 32):
            c = dataclasses.replace(base, T=T)
            x = make_inputs(c)
            d = to_device(x)
            path = torch.arange(T, dtype=torch.int32, device="cuda").repeat(c.B, 1).contiguous()
            plen = torch.full((c.B,), T, dtype=torch.int32, device="cuda")
            ctx0 = d["ctx"].clone()
            f = lambda: tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])

            def g():
                tva.kv_commit(d["k"], d["v"], d["table"], d["ctx"], path, plen)
                d["ctx"].copy_(ctx0)
            settle(f)
            t = _median_us(torch, f) * 1e-6
            t_c = _median_us(torch, g)
            bytes_, flops = attention_cost(c, x)
            line = {"sweep": "calib", "T": T, "attention_us": round(t * 1e6, 1),
                    "commit_plus_restore_us": round(t_c, 1), "hbm_tb_s": round(bytes_ / t / 1e12, 3),
                    "attention_bytes": int(bytes_), "recalibrated_tokens_per_s": round(c.B * T / t, 1)}
            print(json.dumps(line), flush=True)
            del d, x
    elif kind == "expand":
        import oracle
        from synth.inputs import f32_to_bf16_bits
        V, k = 32000, 2048
        for E in (1, 8, 64, 256, 1024):
            rng = np.random.default_rng(E)
            l = f32_to_bf16_bits((rng.standard_normal((E, V)) * 3).astype(np.float32))
            cum = (-rng.random(E) * 5).astype(np.float32)
            dl = torch.from_numpy(l.view(np.int16)).cuda().view(torch.bfloat16)
            dc = torch.from_numpy(cum).cuda()
            kk = min(k, E * V)
            f = lambda: tva.tree_expand(dl, dc, 0.6, kk)
            settle(f)
            t = _median_us(torch, f)
            t0 = time.perf_counter()
            oracle.expand(l, "bf16", cum, 0.6, kk)
            t_cpu = time.perf_counter() - t0
            line = {"sweep": "expand", "E": E, "V": V, "k": kk, "expand_us": round(t, 1),
                    "logit_bytes": E * V * 2, "hbm_tb_s": round(E * V * 2 / t / 1e6, 3),
                    "oracle_cpu_ms": round(t_cpu * 1e3, 1)}
            print(json.dumps(line), flush=True)
    else:
        base = CONFIGS["sparse_topk32_ctx64k"]
        x = make_inputs(base)
        d = to_device(x)
        sums = tva.block_sums(d["k"], d["table"], d["ctx"])
        for k in (1, 8, 16, 32, 64, 128, 256):
            f_k = lambda: tva.topk_blocks(d["q"], d["k"], d["table"], d["ctx"], k)
            f_c = lambda: tva.topk_blocks_cached(d["q"], sums, d["k"], d["table"], d["ctx"], k)
            settle(f_c)
            t_k = _median_us(torch, f_k)
            t_c = _median_us(torch, f_c)
            sel = f_c()
            torch.cuda.synchronize()
            sel_np = sel.cpu().numpy()
            bytes_, flops = attention_cost(base, x, sel_np)
            f_a = lambda: tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"],
                                               sel_blocks=sel)
            try:
                t_a = _median_us(torch, f_a)
            except tva.SdError:
                t_a = None          # a selection the call does not support
            # one selection per (sequence, KV group)
            f_s = lambda: tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], k, sums=sums)
            t_s = _median_us(torch, f_s)
            sel_s = f_s()
            torch.cuda.synchronize()
            bytes_s, _ = attention_cost(base, x, sel_s.cpu().numpy())
            f_as = lambda: tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"],
                                                sel_blocks=sel_s)
            try:
                t_as = _median_us(torch, f_as)
            except tva.SdError:
                t_as = None
            line = {"sweep": "topk", "k": k, "topk_from_k_us": round(t_k, 1), "topk_cached_us": round(t_c, 1),
                    "sparse_attention_us": None if t_a is None else round(t_a, 1),
                    "selected_bytes": int(bytes_),
                    "sparse_attention_tb_s": None if t_a is None else round(bytes_ / t_a / 1e6, 3),
                    "topk_shared_us": round(t_s, 1),
                    "shared_sparse_attention_us": None if t_as is None else round(t_as, 1),
                    "shared_selected_bytes": int(bytes_s),
                    "shared_sparse_attention_tb_s": None if t_as is None else round(bytes_s / t_as / 1e6, 3)}
            print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.sweep:
        sweep(args.sweep)
        return
    if args.write_traffic:
        write_traffic(args.workload, args.write_traffic[0], args.write_traffic[1],
                      args.copy_calibration or 1024)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    selection = "shared" if args.shared_selection else args.selection
    w = Workload(args.workload, max(1, args.kv_copies), shared=selection == "shared")
    if w.cfg.topk and selection == "dense":
        w.set_selection("dense")
    cfg = w.cfg
    settle_steps = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(10):
            w.step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    # at least 20 bracketed calls (all of them for fewer than 20 steps)
    every = max(1, min(args.event_every, args.steps // 20))
    evs = {k: (HipEvent(), HipEvent()) for k in range(0, args.steps, every)}
    # each timed step gets its own copy of the context lengths (its commit
    # advances them), so no restore runs inside the timed region
    ctxs = [w.ctx0.clone() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        w.step(evs.get(k), ctxs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_s = float(np.mean([a.elapsed_time(b) for a, b in evs.values()])) * 1e-3
    step_s = (t1 - t0) / args.steps
    status = w.tva.device_status()
    assert status == 0, "device status bits set: %#x" % status
    plen = w.plen.cpu().numpy()

    sel_np = None if w.sel is None else w.sel.cpu().numpy()
    bytes_, flops = attention_cost(cfg, w.x, sel_np)
    roof = roofline_for(cfg, bytes_, flops, attn_s)
    # the committed counter figures are for the default selection of the workload
    roof["traffic"] = None if (w.shared or (cfg.topk and w.sel is None)) else traffic_for("attn", cfg.name)
    calls = time_calls(w)
    loop = [bound_attention(w, w.sel, kv) for kv in range(len(w.kvs))]
    calls["attention_loop_us"] = round(loop_us(torch, loop), 2)

    secondary = None
    if not args.no_secondary:
        secondary = [e for e in secondary_workloads() if e["workload"] != args.workload]

    # the acceptance call: its bytes (the path of the last timed step) over its
    # own per-call time
    acc_bytes = accept_cost(cfg, plen)
    acc_s = calls["accept_us"] * 1e-6
    accept = {"bytes_per_call": acc_bytes, "accept_us": calls["accept_us"],
              "achieved_gb_s": round(acc_bytes / acc_s / 1e9, 1),
              "frac_of_hbm_peak": round(acc_bytes / acc_s / 1e9 / 8000.0, 4),
              "bound": "latency (a sequential walk: one cross-workgroup exchange per node and per rejection)"}
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    value = cfg.B * cfg.T / step_s
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the workload, no datasets or weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "D": cfg.D, "ctx": [cfg.ctx_lo, cfg.ctx_hi], "block": cfg.bs, "V": cfg.V,
                   "accept": cfg.mode, "temperature": w.tau, "topk": cfg.topk or None,
                   "selection": (("none (dense attention)" if w.sel is None else
                                  "shared per KV group" if w.shared else "per query row")
                                 if cfg.topk else None),
                   "kv_copies": len(w.kvs)},
        "roofline": dict(roof, kernel="sd_tree_verify_attn (tree-masked attention kernel)",
                         attention_us=round(attn_s * 1e6, 2), timed_calls=len(evs),
                         bytes_per_call=int(bytes_),
                         flops_per_call=int(flops)),
        "verified_tree_tokens_per_s_attention": round(cfg.B * cfg.T / attn_s, 1),
        "cpu_baseline": cpu,
        "accept": accept,
        "accepted_tokens_per_s": round(float(plen.sum()) / step_s, 1),
        "mean_path_len": round(float(plen.mean()), 3),
        "calls_us": calls,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
