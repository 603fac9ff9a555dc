"""ctypes binding of libsdtree.so: argument marshalling only.

Every step of the verification pass runs in the library's HIP kernels; this
module turns torch tensors (device memory, the current HIP stream) into the
C ABI's plain pointers and sizes.  There is no CPU fallback: if the library
is not built, or a tensor is not on the GPU, calls raise.
"""
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdtree.so")
# the same library with the kernels' device-side consistency checks
DEBUG_LIB_PATH = os.path.join(_HERE, "libsdtree_debug.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "sdtree.h")

SD_F32, SD_BF16 = 0, 1
SD_CALL_ATTN, SD_CALL_ACCEPT, SD_CALL_TOPK, SD_CALL_COMMIT, SD_CALL_BLOCK_SUMS, SD_CALL_EXPAND, \
    SD_CALL_BUILD = 1, 2, 3, 4, 5, 6, 7
STATUS = {0: "SD_OK", 1: "SD_INVALID_ARG", 2: "SD_BAD_SHAPE", 3: "SD_BAD_DTYPE",
          4: "SD_UNSUPPORTED", 5: "SD_CAPACITY", 6: "SD_HIP_ERROR", 7: "SD_DEVICE_DATA_ERROR"}
ERR_BITS = {0x1: "parent", 0x2: "block", 0x4: "capacity", 0x8: "token", 0x10: "selection",
            0x20: "timeout", 0x40: "build", 0x80: "debug check"}


class SdShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("bs", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("tree_stride", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class SdAcceptShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("V", ctypes.c_int32),
                ("logit_dtype", ctypes.c_int32), ("tree_stride", ctypes.c_int32)]


class SdExpandShape(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("V", ctypes.c_int32), ("logit_dtype", ctypes.c_int32)]


class SdBuildShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("V", ctypes.c_int32), ("logit_dtype", ctypes.c_int32)]


class SdError(RuntimeError):
    def __init__(self, call, code):
        super().__init__("%s returned %s" % (call, STATUS.get(code, code)))
        self.code = code


_P = ctypes.c_void_p
_LIB = None
_LIB_FILE = LIB_PATH


def declared_functions():
    """Names of the functions include/sdtree.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(sd_\w+)\s*\(", text, re.M)))


def use_library(path):
    """Makes the binding call the library at `path` from now on (LIB_PATH by
    default; DEBUG_LIB_PATH is the build with device-side consistency checks).
    Returns the path it replaces."""
    global _LIB, _LIB_FILE
    prev = _LIB_FILE
    _LIB_FILE = path
    _LIB = None
    return prev


def lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_FILE):
        raise RuntimeError("%s is not built; run `python -m tree_verification_amd.build%s`"
                           % (os.path.basename(_LIB_FILE), " --debug" if _LIB_FILE == DEBUG_LIB_PATH else ""))
    L = ctypes.CDLL(_LIB_FILE)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    sig = {
        "sd_tree_verify_attn": [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P, _P, i32, _P, _P, sz, _P],
        "sd_accept": [ctypes.POINTER(SdAcceptShape), _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                      _P, sz, _P],
        "sd_kv_commit": [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
        "sd_accept_commit": [ctypes.POINTER(SdAcceptShape), ctypes.POINTER(SdShape), _P, _P, _P, _P, _P,
                             ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
        "sd_accept_commit_noalloc": [ctypes.POINTER(SdAcceptShape), ctypes.POINTER(SdShape), _P, _P, _P,
                                     _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "sd_topk_blocks": [ctypes.POINTER(SdShape), _P, _P, _P, _P, i32, _P, _P, sz, _P],
        "sd_topk_blocks_cached": [ctypes.POINTER(SdShape), _P, _P, _P, _P, i32, _P, _P, sz, _P],
        "sd_topk_blocks_shared": [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, i32, _P, _P, sz, _P],
        "sd_block_sums": [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, sz, _P],
        "sd_tree_expand": [ctypes.POINTER(SdExpandShape), _P, _P, ctypes.c_float, i32, _P, _P, _P, _P, sz,
                           _P],
        "sd_block_sums_append": [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P, sz, _P],
        "sd_tree_build": [ctypes.POINTER(SdBuildShape), _P, ctypes.c_float, i32, _P, _P, _P,
                          ctypes.POINTER(ctypes.c_int32), _P, sz, _P],
        "sd_device_status": [_P, _P, ctypes.POINTER(ctypes.c_uint32)],
        "sd_attn_timing_events": [_P, _P],
        "sd_workspace_bytes": [i32, _P, i32],
        "sd_status_str": [i32],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.sd_workspace_bytes.restype = ctypes.c_size_t
    L.sd_status_str.restype = ctypes.c_char_p
    _LIB = L
    return L


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(name, code):
    if code != 0:
        raise SdError(name, code)


_dtype_code = {torch.float32: SD_F32, torch.bfloat16: SD_BF16}


def make_shape(q, k_pages, block_table, tree_parent, scale=0.0):
    B, T, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_pages.shape
    if D2 != D:
        raise ValueError("head dim mismatch")
    stride = 0 if tree_parent.shape[0] == 1 else T
    return SdShape(B, T, Hq, Hkv, D, bs, block_table.shape[1], nb, _dtype_code[q.dtype], stride,
                   float(scale))


class Workspace:
    """Zero-filled device scratch buffers, one per (device, call kind), grown on
    demand.  Call kinds never share a buffer: the acceptance walk keeps barrier
    counters in its workspace that must read zero when a call starts."""

    def __init__(self):
        self._buf = {}

    @staticmethod
    def _index(device):
        dev = torch.device(device)
        return dev.index if dev.index is not None else torch.cuda.current_device()

    def get(self, device, nbytes, kind):
        key = (self._index(device), kind)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda:%d" % key[0])
            self._buf[key] = buf
        return buf

    def all(self, device):
        idx = self._index(device)
        return [b for (i, _), b in self._buf.items() if i == idx]


_WS = Workspace()


def workspace_bytes(call, shape, extra=0):
    return lib().sd_workspace_bytes(call, ctypes.byref(shape), extra)


def attn_timing_events(start_event, stop_event):
    """The next tree_verify_attn call on this thread records the two hipEvent_t
    handles (ints; 0 = none) at its first kernel's start and its last kernel's
    end."""
    _check("sd_attn_timing_events", lib().sd_attn_timing_events(start_event or None, stop_event or None))


def tree_verify_attn(q, k_pages, v_pages, block_table, ctx_lens, tree_parent, out=None,
                     sel_blocks=None, scale=0.0, ws=None):
    shape = make_shape(q, k_pages, block_table, tree_parent, scale)
    if out is None:
        out = torch.empty_like(q)
    k_sel = 0 if sel_blocks is None else sel_blocks.shape[-1]
    need = workspace_bytes(SD_CALL_ATTN, shape, k_sel)
    if need == 0:
        raise SdError("sd_workspace_bytes", 2)
    ws = _WS.get(q.device, need, SD_CALL_ATTN) if ws is None else ws
    _check("sd_tree_verify_attn", lib().sd_tree_verify_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
        _ptr(ctx_lens), _ptr(tree_parent), _ptr(sel_blocks), k_sel, _ptr(out), _ptr(ws),
        ws.numel(), _stream(q.device)))
    return out


def accept(target_logits, draft_probs, tree_parent, tree_token, uniforms, temperature,
           path=None, path_len=None, bonus=None, ws=None):
    B, T, V = target_logits.shape
    shape = SdAcceptShape(B, T, V, _dtype_code[target_logits.dtype],
                          0 if tree_parent.shape[0] == 1 else T)
    dev = target_logits.device
    if path is None:
        path = torch.empty((B, T), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    need = workspace_bytes(SD_CALL_ACCEPT, shape)
    ws = _WS.get(dev, need, SD_CALL_ACCEPT) if ws is None else ws
    _check("sd_accept", lib().sd_accept(
        ctypes.byref(shape), _ptr(target_logits), _ptr(draft_probs), _ptr(tree_parent),
        _ptr(tree_token), _ptr(uniforms), float(temperature), _ptr(path), _ptr(path_len),
        _ptr(bonus), _ptr(ws), ws.numel(), _stream(dev)))
    return path, path_len, bonus


def accept_commit(target_logits, draft_probs, tree_parent, tree_token, uniforms, temperature,
                  k_pages, v_pages, block_table, ctx_lens, path=None, path_len=None, bonus=None,
                  ws=None, sums=None):
    """accept(...) then kv_commit(...) of its paths, in one launch (sd_accept_commit);
    with `sums` (kept block key sums) also their extension over the committed
    positions."""
    B, T, V = target_logits.shape
    shape = SdAcceptShape(B, T, V, _dtype_code[target_logits.dtype],
                          0 if tree_parent.shape[0] == 1 else T)
    nb, Hkv, bs, D = k_pages.shape
    kv_shape = SdShape(B, T, Hkv, Hkv, D, bs, block_table.shape[1], nb, _dtype_code[k_pages.dtype],
                       T, 0.0)
    dev = target_logits.device
    if path is None:
        path = torch.empty((B, T), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    need = workspace_bytes(SD_CALL_ACCEPT, shape)
    ws = _WS.get(dev, need, SD_CALL_ACCEPT) if ws is None else ws
    _check("sd_accept_commit", lib().sd_accept_commit(
        ctypes.byref(shape), ctypes.byref(kv_shape), _ptr(target_logits), _ptr(draft_probs),
        _ptr(tree_parent), _ptr(tree_token), _ptr(uniforms), float(temperature), _ptr(path),
        _ptr(path_len), _ptr(bonus), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_lens),
        _ptr(sums), _ptr(ws), ws.numel(), _stream(dev)))
    return path, path_len, bonus


def accept_commit_noalloc(target_logits, draft_probs, tree_parent, tree_token, uniforms,
                          temperature, k_pages, v_pages, block_table, ctx_lens, status,
                          path=None, path_len=None, bonus=None, sums=None):
    """sd_accept_commit_noalloc: accept_commit(...) with no workspace; sticky
    error bits are OR-ed into `status` (an int32 device tensor of one element)."""
    B, T, V = target_logits.shape
    shape = SdAcceptShape(B, T, V, _dtype_code[target_logits.dtype],
                          0 if tree_parent.shape[0] == 1 else T)
    nb, Hkv, bs, D = k_pages.shape
    kv_shape = SdShape(B, T, Hkv, Hkv, D, bs, block_table.shape[1], nb, _dtype_code[k_pages.dtype],
                       T, 0.0)
    dev = target_logits.device
    if path is None:
        path = torch.empty((B, T), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    _check("sd_accept_commit_noalloc", lib().sd_accept_commit_noalloc(
        ctypes.byref(shape), ctypes.byref(kv_shape), _ptr(target_logits), _ptr(draft_probs),
        _ptr(tree_parent), _ptr(tree_token), _ptr(uniforms), float(temperature), _ptr(path),
        _ptr(path_len), _ptr(bonus), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_lens),
        _ptr(sums), _ptr(status), _stream(dev)))
    return path, path_len, bonus


def kv_commit(k_pages, v_pages, block_table, ctx_lens, path, path_len, ws=None, sums=None):
    B, T = path.shape
    nb, Hkv, bs, D = k_pages.shape
    shape = SdShape(B, T, Hkv, Hkv, D, bs, block_table.shape[1], nb, _dtype_code[k_pages.dtype],
                    T, 0.0)
    need = workspace_bytes(SD_CALL_COMMIT, shape)
    ws = _WS.get(k_pages.device, need, SD_CALL_COMMIT) if ws is None else ws
    _check("sd_kv_commit", lib().sd_kv_commit(
        ctypes.byref(shape), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_lens),
        _ptr(sums), _ptr(path), _ptr(path_len), _ptr(ws), ws.numel(), _stream(k_pages.device)))


def tree_expand(draft_logits, cum_logp, temperature, k, ws=None):
    """sd_tree_expand: the k best children (row, token, score), best first."""
    E, V = draft_logits.shape
    shape = SdExpandShape(E, V, _dtype_code[draft_logits.dtype])
    dev = draft_logits.device
    row = torch.empty(k, dtype=torch.int32, device=dev)
    tok = torch.empty(k, dtype=torch.int32, device=dev)
    score = torch.empty(k, dtype=torch.float32, device=dev)
    need = workspace_bytes(SD_CALL_EXPAND, shape, k)
    if need == 0:
        raise SdError("sd_workspace_bytes", 2)
    ws = _WS.get(dev, need, SD_CALL_EXPAND) if ws is None else ws
    _check("sd_tree_expand", lib().sd_tree_expand(
        ctypes.byref(shape), _ptr(draft_logits), _ptr(cum_logp), float(temperature), int(k), _ptr(row),
        _ptr(tok), _ptr(score), _ptr(ws), ws.numel(), _stream(dev)))
    return row, tok, score


def tree_build(draft_logits, temperature, root_token=0, ws=None):
    """sd_tree_build: the best-first draft tree of T = draft_logits.shape[0]
    nodes; returns (parent int32 [T], token int32 [T], cum_logp float64 [T],
    rounds)."""
    T, V = draft_logits.shape
    shape = SdBuildShape(T, V, _dtype_code[draft_logits.dtype])
    dev = draft_logits.device
    parent = torch.empty(T, dtype=torch.int32, device=dev)
    token = torch.empty(T, dtype=torch.int32, device=dev)
    cum = torch.empty(T, dtype=torch.float64, device=dev)
    need = workspace_bytes(SD_CALL_BUILD, shape)
    if need == 0:
        raise SdError("sd_workspace_bytes", 2)
    ws = _WS.get(dev, need, SD_CALL_BUILD) if ws is None else ws
    rounds = ctypes.c_int32(0)
    _check("sd_tree_build", lib().sd_tree_build(
        ctypes.byref(shape), _ptr(draft_logits), float(temperature), int(root_token), _ptr(parent),
        _ptr(token), _ptr(cum), ctypes.byref(rounds), _ptr(ws), ws.numel(), _stream(dev)))
    return parent, token, cum, rounds.value


def _sums_shape(k_pages, block_table, ctx_lens):
    nb, Hkv, bs, D = k_pages.shape
    return SdShape(len(ctx_lens), 1, Hkv, Hkv, D, bs, block_table.shape[1], nb, _dtype_code[k_pages.dtype],
                   0, 0.0)


def block_sums(k_pages, block_table, ctx_lens, sums=None, ws=None):
    """Kept block key sums, float32 [num_blocks, Hkv, D] (sd_block_sums); a new
    zero-filled tensor unless `sums` is given."""
    nb, Hkv, bs, D = k_pages.shape
    if sums is None:
        sums = torch.zeros((nb, Hkv, D), dtype=torch.float32, device=k_pages.device)
    shape = _sums_shape(k_pages, block_table, ctx_lens)
    need = workspace_bytes(SD_CALL_BLOCK_SUMS, shape)
    ws = _WS.get(k_pages.device, need, SD_CALL_BLOCK_SUMS) if ws is None else ws
    _check("sd_block_sums", lib().sd_block_sums(
        ctypes.byref(shape), _ptr(k_pages), _ptr(block_table), _ptr(ctx_lens), _ptr(sums), _ptr(ws),
        ws.numel(), _stream(k_pages.device)))
    return sums


def block_sums_append(k_pages, block_table, ctx_lens, n_new, sums, ws=None):
    """Extends kept block sums by the n_new[b] positions a commit appended
    (ctx_lens after the commit) (sd_block_sums_append)."""
    shape = _sums_shape(k_pages, block_table, ctx_lens)
    need = workspace_bytes(SD_CALL_BLOCK_SUMS, shape)
    ws = _WS.get(k_pages.device, need, SD_CALL_BLOCK_SUMS) if ws is None else ws
    _check("sd_block_sums_append", lib().sd_block_sums_append(
        ctypes.byref(shape), _ptr(k_pages), _ptr(block_table), _ptr(ctx_lens), _ptr(n_new), _ptr(sums),
        _ptr(ws), ws.numel(), _stream(k_pages.device)))
    return sums


def topk_blocks_cached(q, sums, k_pages_like, block_table, ctx_lens, k, sel=None, ws=None):
    """sd_topk_blocks_cached: the top-k selection with means from kept block
    sums.  `k_pages_like` supplies the cache's shape and dtype only (not read)."""
    B, T, Hq, D = q.shape
    parent_like = torch.empty((1, T))
    shape = make_shape(q, k_pages_like, block_table, parent_like)
    if sel is None:
        sel = torch.empty((B, T, Hq, k), dtype=torch.int32, device=q.device)
    need = workspace_bytes(SD_CALL_TOPK, shape, k)
    ws = _WS.get(q.device, need, SD_CALL_TOPK) if ws is None else ws
    _check("sd_topk_blocks_cached", lib().sd_topk_blocks_cached(
        ctypes.byref(shape), _ptr(q), _ptr(sums), _ptr(block_table), _ptr(ctx_lens), int(k),
        _ptr(sel), _ptr(ws), ws.numel(), _stream(q.device)))
    return sel


def topk_blocks_shared(q, k_pages, block_table, ctx_lens, k, sums=None, sel=None, ws=None):
    """sd_topk_blocks_shared: one selection per (sequence, KV group), written
    to all the group's rows; means from the kept `sums` when given (K is then
    not read), else from `k_pages`."""
    B, T, Hq, D = q.shape
    parent_like = torch.empty((1, T))
    shape = make_shape(q, k_pages, block_table, parent_like)
    if sel is None:
        sel = torch.empty((B, T, Hq, k), dtype=torch.int32, device=q.device)
    need = workspace_bytes(SD_CALL_TOPK, shape, k)
    ws = _WS.get(q.device, need, SD_CALL_TOPK) if ws is None else ws
    _check("sd_topk_blocks_shared", lib().sd_topk_blocks_shared(
        ctypes.byref(shape), _ptr(q), _ptr(k_pages), None if sums is None else _ptr(sums),
        _ptr(block_table), _ptr(ctx_lens), int(k), _ptr(sel), _ptr(ws), ws.numel(), _stream(q.device)))
    return sel


def topk_blocks(q, k_pages, block_table, ctx_lens, k, sel=None, ws=None):
    B, T, Hq, D = q.shape
    parent_like = torch.empty((1, T))
    shape = make_shape(q, k_pages, block_table, parent_like)
    if sel is None:
        sel = torch.empty((B, T, Hq, k), dtype=torch.int32, device=q.device)
    need = workspace_bytes(SD_CALL_TOPK, shape, k)
    ws = _WS.get(q.device, need, SD_CALL_TOPK) if ws is None else ws
    _check("sd_topk_blocks", lib().sd_topk_blocks(
        ctypes.byref(shape), _ptr(q), _ptr(k_pages), _ptr(block_table), _ptr(ctx_lens), int(k),
        _ptr(sel), _ptr(ws), ws.numel(), _stream(q.device)))
    return sel


def device_status(ws=None, device="cuda"):
    """Reads and clears the sticky device error bits of a workspace (default:
    every workspace this binding allocated on the device), OR-ed together."""
    bufs = _WS.all(device) if ws is None else [ws]
    out = 0
    for w in bufs:
        bits = ctypes.c_uint32(0)
        code = lib().sd_device_status(_ptr(w), _stream(w.device), ctypes.byref(bits))
        if code not in (0, 7):
            raise SdError("sd_device_status", code)
        out |= bits.value
    return out
