"""Python access to the fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg. The GPU package never imports it.

The arithmetic lives in kascade_oracle.c; this module only marshals numpy
arrays into the C calls. Inputs are the stored tensors: float32 arrays, or
bfloat16 given as their raw uint16/int16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_c_int_p = ctypes.POINTER(ctypes.c_int32)
_c_dbl_p = ctypes.POINTER(ctypes.c_double)


class OracleProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int),
        ("num_q_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("q_len", ctypes.c_int),
        ("kv_len", ctypes.c_int),
        ("top_k", ctypes.c_int),
        ("q_tile", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("dtype", ctypes.c_int),
        ("shared_index_set", ctypes.c_int),
    ]


def _ptr(a, ctype=ctypes.c_void_p):
    return a.ctypes.data_as(ctype) if a is not None else None


def _as_input(x):
    """float32 array or bf16 bits (uint16/int16) -> (contiguous array, dtype code)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype in (np.uint16, np.int16):
        return x.view(np.uint16), 1
    raise TypeError(f"oracle inputs must be float32 or bf16 bits, got {x.dtype}")


def _check_sets(idx, p, shared):
    """The oracle reads idx as [B, S, tiles, k]; refuse a smaller array."""
    sets = 1 if shared else p.num_kv_heads
    tiles = 1 if p.q_len == 1 else -(-p.kv_len // p.q_tile)
    if idx.size != p.batch * sets * tiles * p.top_k:
        raise ValueError(f"idx holds {idx.size} entries, expected [B={p.batch}, S={sets}, tiles={tiles}, "
                         f"k={p.top_k}]")


def _units(units, width):
    if units is None:
        return None, 0
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, width))
    return u, u.shape[0]


class Oracle:
    """Thin wrapper over one build of the oracle library."""

    def __init__(self, libpath=None):
        if libpath is None:
            libpath = _build.LIBRARY
            if not os.path.exists(libpath):
                _build.build()
        self.libpath = libpath
        lib = ctypes.CDLL(libpath)
        P = ctypes.POINTER(OracleProblem)
        vp = ctypes.c_void_p
        lib.oracle_anchor_decode.argtypes = [P, vp, vp, _c_int_p, ctypes.c_int, _c_int_p, _c_dbl_p, ctypes.c_int]
        lib.oracle_anchor_prefill.argtypes = [P, vp, vp, _c_int_p, ctypes.c_int, _c_int_p, _c_dbl_p, ctypes.c_int]
        lib.oracle_reuse_decode.argtypes = [P, vp, vp, vp, _c_int_p, _c_int_p, ctypes.c_int, _c_dbl_p, ctypes.c_int]
        lib.oracle_reuse_prefill.argtypes = [P, vp, vp, vp, _c_int_p, _c_int_p, ctypes.c_int, _c_dbl_p, ctypes.c_int]
        lib.oracle_dense.argtypes = [P, vp, vp, vp, ctypes.c_int, _c_int_p, ctypes.c_int, _c_dbl_p, _c_dbl_p, ctypes.c_int]
        lib.oracle_threads.argtypes = [ctypes.c_int]
        for f in (lib.oracle_anchor_decode, lib.oracle_anchor_prefill, lib.oracle_reuse_decode,
                  lib.oracle_reuse_prefill, lib.oracle_dense, lib.oracle_threads):
            f.restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def problem(q, k, top_k=1, q_tile=128, scale=None, dtype=0, shared=False):
        B, Hq, L, d = q.shape
        _, Hkv, N, _ = k.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        return OracleProblem(B, Hq, Hkv, d, L, N, int(top_k), int(q_tile), float(scale), dtype,
                             int(bool(shared)))

    def _check(self, rc, name):
        if rc != 0:
            raise ValueError(f"{name} failed with status {rc}")

    def threads(self, nthreads=0):
        """Threads the oracle's parallel loops run with for `nthreads` (0 = default)."""
        return int(self.lib.oracle_threads(int(nthreads)))

    # -- anchor -------------------------------------------------------------
    def anchor_decode(self, q, k, top_k, units=None, scale=None, threads=0, want_pooled=True, shared=False):
        """q [B,Hq,1,d], k [B,Hkv,N,d] -> (idx [U,k], pooled [U,N] or None), U = units (b, set)
        or B*S, S = Hkv (one set per KV head) or 1 (shared=True: one set for all heads)."""
        q, dt = _as_input(q)
        k, dt2 = _as_input(k)
        assert dt == dt2
        p = self.problem(q, k, top_k, 1, scale, dt, shared)
        u, nu = _units(units, 2)
        n = nu if u is not None else p.batch * (1 if shared else p.num_kv_heads)
        idx = np.empty((n, top_k), np.int32)
        pooled = np.empty((n, p.kv_len), np.float64) if want_pooled else None
        rc = self.lib.oracle_anchor_decode(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(u, _c_int_p), nu,
                                           _ptr(idx, _c_int_p), _ptr(pooled, _c_dbl_p), threads)
        self._check(rc, "oracle_anchor_decode")
        return idx, pooled

    def anchor_prefill(self, q, k, top_k, q_tile, units=None, scale=None, threads=0, want_pooled=True,
                       shared=False):
        """q [B,Hq,N,d], k [B,Hkv,N,d] -> (idx [U,k], pooled [U,N]), U = units (b,set,t) or all
        B*S*tiles, S = Hkv or 1 (shared=True)."""
        q, dt = _as_input(q)
        k, dt2 = _as_input(k)
        assert dt == dt2
        p = self.problem(q, k, top_k, q_tile, scale, dt, shared)
        u, nu = _units(units, 3)
        tiles = -(-p.kv_len // q_tile)
        n = nu if u is not None else p.batch * (1 if shared else p.num_kv_heads) * tiles
        idx = np.empty((n, top_k), np.int32)
        pooled = np.empty((n, p.kv_len), np.float64) if want_pooled else None
        rc = self.lib.oracle_anchor_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(u, _c_int_p), nu,
                                            _ptr(idx, _c_int_p), _ptr(pooled, _c_dbl_p), threads)
        self._check(rc, "oracle_anchor_prefill")
        return idx, pooled

    # -- reuse --------------------------------------------------------------
    def reuse_decode(self, q, k, v, idx, units=None, scale=None, threads=0, shared=False):
        """idx [B,S,1,k] (S = Hkv, or 1 with shared=True) -> out [U,d], U = units (b,h) or B*Hq."""
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        p = self.problem(q, k, idx.shape[-1], 1, scale, dt, shared)
        _check_sets(idx, p, shared)
        u, nu = _units(units, 2)
        n = nu if u is not None else p.batch * p.num_q_heads
        out = np.empty((n, p.head_dim), np.float64)
        rc = self.lib.oracle_reuse_decode(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx, _c_int_p),
                                          _ptr(u, _c_int_p), nu, _ptr(out, _c_dbl_p), threads)
        self._check(rc, "oracle_reuse_decode")
        return out

    def reuse_prefill(self, q, k, v, idx, q_tile, units=None, scale=None, threads=0, shared=False):
        """idx [B,S,tiles,k] (S = Hkv, or 1 with shared=True) -> out [U,d], U = units (b,h,i) or B*Hq*N."""
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        p = self.problem(q, k, idx.shape[-1], q_tile, scale, dt, shared)
        _check_sets(idx, p, shared)
        u, nu = _units(units, 3)
        n = nu if u is not None else p.batch * p.num_q_heads * p.q_len
        out = np.empty((n, p.head_dim), np.float64)
        rc = self.lib.oracle_reuse_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx, _c_int_p),
                                           _ptr(u, _c_int_p), nu, _ptr(out, _c_dbl_p), threads)
        self._check(rc, "oracle_reuse_prefill")
        return out

    # -- dense --------------------------------------------------------------
    def dense(self, q, k, v, causal, units=None, scale=None, threads=0, want_out=True):
        """-> (out [U,d] or None, lse [U]), U = units (b,h,i) or B*Hq*q_len."""
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        if v is not None:
            v, _ = _as_input(v)
        p = self.problem(q, k, 1, 1, scale, dt)
        u, nu = _units(units, 3)
        n = nu if u is not None else p.batch * p.num_q_heads * p.q_len
        out = np.empty((n, p.head_dim), np.float64) if want_out else None
        lse = np.empty((n,), np.float64)
        rc = self.lib.oracle_dense(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v) if v is not None else None,
                                   int(bool(causal)), _ptr(u, _c_int_p), nu, _ptr(out, _c_dbl_p),
                                   _ptr(lse, _c_dbl_p), threads)
        self._check(rc, "oracle_dense")
        return out, lse


_default = None


def default():
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
