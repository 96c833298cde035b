"""ctypes binding of libkascade.so, the gfx950 library declared in include/kascade.h.

Argument marshalling only: tensors are passed as device pointers and shapes,
every step runs in the library's HIP kernels. There is no fallback; if the
library has not been built, loading fails with an error.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkascade.so")

F32, BF16 = 0, 1
OP_ANCHOR_DECODE, OP_REUSE_DECODE, OP_ANCHOR_PREFILL, OP_REUSE_PREFILL = 0, 1, 2, 3
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 8 << 20   # KASCADE_NOALLOC_SCRATCH_BYTES

EXPORTS = ("kascade_validate", "kascade_workspace_bytes", "kascade_status_string",
           "kascade_anchor_decode", "kascade_reuse_decode", "kascade_reuse_decode_noalloc",
           "kascade_anchor_prefill", "kascade_reuse_prefill", "kascade_timing_enable",
           "kascade_timing_collect")


class KascadeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("kv_len", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("q_tile", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("shared_index_set", ctypes.c_int32),
    ]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("total_ms", ctypes.c_double),
                ("launches", ctypes.c_int64)]


class Library:
    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m long_context_amd.build` "
                               "or __graft_entry__.build()")
        self.path = path
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.kascade_validate.argtypes = [P, ctypes.c_int]
        lib.kascade_validate.restype = ctypes.c_int
        lib.kascade_workspace_bytes.argtypes = [P, ctypes.c_int]
        lib.kascade_workspace_bytes.restype = sz
        lib.kascade_status_string.argtypes = [ctypes.c_int]
        lib.kascade_status_string.restype = ctypes.c_char_p
        anchor = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        reuse = [P, vp, vp, vp, vp, vp, vp, sz, vp]
        for name, args in (("kascade_anchor_decode", anchor), ("kascade_anchor_prefill", anchor),
                           ("kascade_reuse_decode", reuse), ("kascade_reuse_prefill", reuse)):
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.kascade_reuse_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.kascade_reuse_decode_noalloc.restype = ctypes.c_int
        lib.kascade_timing_enable.argtypes = [ctypes.c_int]
        lib.kascade_timing_enable.restype = ctypes.c_int
        lib.kascade_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
        lib.kascade_timing_collect.restype = ctypes.c_int
        self.lib = lib

    # -- per-kernel timing -----------------------------------------------------
    def timing_enable(self, on=True):
        return self.lib.kascade_timing_enable(1 if on else 0)

    def timing_collect(self, max_entries=64):
        """{kernel name: (total ms, launches)} since the last collect; waits for the events."""
        buf = (KernelTime * max_entries)()
        n = self.lib.kascade_timing_collect(buf, max_entries)
        if n < 0:
            raise KascadeError(ERR_HIP, "kascade_timing_collect failed")
        return {buf[i].name.decode(): (buf[i].total_ms, buf[i].launches) for i in range(n)}

    # -- host-only queries ------------------------------------------------------
    def validate(self, prob, op):
        return self.lib.kascade_validate(ctypes.byref(prob), op)

    def workspace_bytes(self, prob, op):
        return self.lib.kascade_workspace_bytes(ctypes.byref(prob), op)

    def status_string(self, status):
        return self.lib.kascade_status_string(status).decode()

    def check(self, status, what):
        if status != OK:
            raise KascadeError(status, f"{what}: {self.status_string(status)} ({status})")

    # -- raw entry points (integer device addresses, 0 = NULL) -------------------
    def anchor_decode_raw(self, prob, q, k, v, out, idx, lse, ws, ws_bytes, stream):
        return self.lib.kascade_anchor_decode(ctypes.byref(prob), q, k, v, out, idx, lse, ws,
                                              ws_bytes, stream)

    def reuse_decode_raw(self, prob, q, k, v, idx, out, ws, ws_bytes, stream):
        return self.lib.kascade_reuse_decode(ctypes.byref(prob), q, k, v, idx, out, ws, ws_bytes,
                                             stream)

    def reuse_decode_noalloc_raw(self, prob, q, k, v, idx, out, stream):
        return self.lib.kascade_reuse_decode_noalloc(ctypes.byref(prob), q, k, v, idx, out, stream)

    def anchor_prefill_raw(self, prob, q, k, v, out, idx, lse, ws, ws_bytes, stream):
        return self.lib.kascade_anchor_prefill(ctypes.byref(prob), q, k, v, out, idx, lse, ws,
                                               ws_bytes, stream)

    def reuse_prefill_raw(self, prob, q, k, v, idx, out, ws, ws_bytes, stream):
        return self.lib.kascade_reuse_prefill(ctypes.byref(prob), q, k, v, idx, out, ws, ws_bytes,
                                              stream)


_library = None


def library():
    global _library
    if _library is None:
        _library = Library()
    return _library


# ---- tensor-level wrappers ---------------------------------------------------

def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def problem(q, k, top_k, q_tile=128, scale=0.0, shared=False):
    """Problem descriptor from Q [B,Hq,L,d] and K [B,Hkv,N,d]; shared=True asks
    for one index set shared by all heads instead of one per KV head."""
    B, Hq, L, d = q.shape
    Bk, Hkv, N, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)}")
    return Problem(B, Hq, Hkv, d, L, N, int(top_k), int(q_tile), float(scale), _dtype_code(q),
                   int(bool(shared)))


def idx_shape(prob):
    """Shape of the index sets for a problem: [B, S, tiles, k], S = Hkv or 1 (shared)."""
    sets = 1 if prob.shared_index_set else prob.num_kv_heads
    tiles = 1 if prob.q_len == 1 else -(-prob.kv_len // max(prob.q_tile, 1))
    return (prob.batch, sets, tiles, prob.top_k)


def _check_idx(idx, prob, what):
    want = idx_shape(prob)
    if tuple(idx.shape) != want or idx.dtype != torch.int32:
        raise ValueError(f"{what}: idx must be int32 {list(want)}, got {idx.dtype} {list(idx.shape)}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace(prob, op, device):
    """A zero-filled workspace tensor of kascade_workspace_bytes() bytes (None
    if zero). Decode workspaces must start zeroed (their arrival counters);
    every call leaves them so."""
    n = library().workspace_bytes(prob, op)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel())


def anchor_decode(q, k, v, top_k, out=None, lse=None, idx=None, ws=None, scale=0.0, stream=None,
                  shared=False, dense_only=False):
    """Anchor decode; returns idx [B,S,1,k] int32, S = Hkv or 1 with shared=True
    (and fills out/lse if given). dense_only=True passes no index buffer: the
    call is plain dense attention into out/lse and returns None."""
    lib = library()
    prob = problem(q, k, top_k, 1, scale, shared)
    if dense_only:
        idx = None
    else:
        if idx is None:
            idx = torch.empty(idx_shape(prob), dtype=torch.int32, device=q.device)
        _check_idx(idx, prob, "anchor_decode")
    if ws is None:
        ws = workspace(prob, OP_ANCHOR_DECODE, q.device)
    wp, wb = _ws(ws)
    lib.check(lib.anchor_decode_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx), _ptr(lse),
                                    wp, wb, _stream(stream)), "kascade_anchor_decode")
    return idx


def reuse_decode(q, k, v, idx, out=None, ws=None, scale=0.0, stream=None, shared=False):
    """Reuse decode over idx [B,S,1,k] (S = Hkv, or 1 with shared=True); returns out [B,Hq,1,d]."""
    lib = library()
    prob = problem(q, k, idx.shape[-1], 1, scale, shared)
    _check_idx(idx, prob, "reuse_decode")
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(prob, OP_REUSE_DECODE, q.device)
    wp, wb = _ws(ws)
    lib.check(lib.reuse_decode_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out), wp, wb,
                                   _stream(stream)), "kascade_reuse_decode")
    return out


def reuse_decode_noalloc(q, k, v, idx, out=None, scale=0.0, stream=None, shared=False):
    """Reuse decode through the allocation-free entry point (library-held
    scratch, no workspace); returns out [B,Hq,1,d]."""
    lib = library()
    prob = problem(q, k, idx.shape[-1], 1, scale, shared)
    _check_idx(idx, prob, "reuse_decode_noalloc")
    if out is None:
        out = torch.empty_like(q)
    lib.check(lib.reuse_decode_noalloc_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
                                           _stream(stream)), "kascade_reuse_decode_noalloc")
    return out


def anchor_prefill(q, k, v, top_k, q_tile=128, out=None, lse=None, idx=None, ws=None, scale=0.0,
                   stream=None, shared=False, dense_only=False):
    """Anchor causal prefill; returns idx [B,S,ceil(N/T),k] int32, S = Hkv or 1 with shared=True.
    dense_only=True passes no index buffer: plain dense causal attention into
    out/lse, returns None."""
    lib = library()
    prob = problem(q, k, top_k, q_tile, scale, shared)
    if dense_only:
        idx = None
    else:
        if idx is None:
            idx = torch.empty(idx_shape(prob), dtype=torch.int32, device=q.device)
        _check_idx(idx, prob, "anchor_prefill")
    if ws is None:
        ws = workspace(prob, OP_ANCHOR_PREFILL, q.device)
    wp, wb = _ws(ws)
    lib.check(lib.anchor_prefill_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx), _ptr(lse),
                                     wp, wb, _stream(stream)), "kascade_anchor_prefill")
    return idx


def reuse_prefill(q, k, v, idx, q_tile=128, out=None, ws=None, scale=0.0, stream=None, shared=False):
    """Reuse causal prefill over idx [B,S,tiles,k] (S = Hkv, or 1 with shared=True);
    returns out [B,Hq,N,d]."""
    lib = library()
    prob = problem(q, k, idx.shape[-1], q_tile, scale, shared)
    _check_idx(idx, prob, "reuse_prefill")
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(prob, OP_REUSE_PREFILL, q.device)
    wp, wb = _ws(ws)
    lib.check(lib.reuse_prefill_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out), wp, wb,
                                    _stream(stream)), "kascade_reuse_prefill")
    return out


# ---- a stack of layers with an anchor schedule ------------------------------

def anchor_schedule(n_layers, anchors):
    """Role of each layer under an anchor list: ("dense", None) before the first
    anchor, ("anchor", l) for an anchor layer l, ("reuse", a) for a layer that
    reuses the indices of the nearest preceding anchor a (Kascade abstract on
    the opentrain.ai page, "Abstract"; the summary's interface line takes a
    top-k and a list of anchor layers, "Practical Implications")."""
    anchors = sorted(set(int(a) for a in anchors))
    if not anchors:
        raise ValueError("at least one anchor layer is needed")
    if anchors[0] < 0 or anchors[-1] >= n_layers:
        raise ValueError(f"anchor layers must lie in [0, {n_layers})")
    roles, last = [], None
    for l in range(n_layers):
        if l in anchors:
            last = l
            roles.append(("anchor", l))
        elif last is None:
            roles.append(("dense", None))
        else:
            roles.append(("reuse", last))
    return roles


def kascade_attention(qs, ks, vs, top_k, anchors, q_tile=128, outs=None, scale=0.0, stream=None,
                      shared=False):
    """Kascade attention over a stack of layers, one call per layer through the
    C ABI. qs, ks, vs: per-layer tensors, decode (Q [B,Hq,1,d]) or causal
    prefill (Q [B,Hq,N,d]), K/V [B,Hkv,N,d]. Layers before the first anchor
    attend densely (the anchor call without an index buffer: dense output
    only, no scores kept and no selection),
    an anchor layer outputs dense attention and saves its top-k indices, every
    other layer attends only to the saved indices of the nearest preceding
    anchor, with its own Q, K and V. shared=True runs the non-head-aware
    ablation (one index set for all heads). Returns (per-layer outputs,
    {anchor layer: idx})."""
    n_layers = len(qs)
    if not (len(ks) == len(vs) == n_layers):
        raise ValueError("qs, ks and vs must have one tensor per layer")
    roles = anchor_schedule(n_layers, anchors)
    decode = qs[0].shape[2] == 1
    n = ks[0].shape[2]
    if outs is None:
        outs = [torch.empty_like(q) for q in qs]
    saved, ws_anchor, ws_reuse = {}, None, None
    for l, (role, src) in enumerate(roles):
        q, k, v = qs[l], ks[l], vs[l]
        if role in ("dense", "anchor"):
            # Dense layers pass no index buffer: no scores are kept, nothing is selected.
            kk = min(top_k, n) if decode else top_k
            dense_only = role == "dense"
            if decode:
                if ws_anchor is None:
                    ws_anchor = workspace(problem(q, k, kk, 1, scale, shared), OP_ANCHOR_DECODE, q.device)
                idx = anchor_decode(q, k, v, kk, out=outs[l], ws=ws_anchor, scale=scale, stream=stream,
                                    shared=shared, dense_only=dense_only)
            else:
                if ws_anchor is None:
                    ws_anchor = workspace(problem(q, k, kk, q_tile, scale, shared), OP_ANCHOR_PREFILL,
                                          q.device)
                idx = anchor_prefill(q, k, v, kk, q_tile, out=outs[l], ws=ws_anchor, scale=scale,
                                     stream=stream, shared=shared, dense_only=dense_only)
            if role == "anchor":
                saved[l] = idx
        elif decode:
            if ws_reuse is None:
                ws_reuse = workspace(problem(q, k, top_k, 1, scale, shared), OP_REUSE_DECODE, q.device)
            reuse_decode(q, k, v, saved[src], out=outs[l], ws=ws_reuse, scale=scale, stream=stream,
                         shared=shared)
        else:
            reuse_prefill(q, k, v, saved[src], q_tile, out=outs[l], scale=scale, stream=stream,
                          shared=shared)
    return outs, saved
