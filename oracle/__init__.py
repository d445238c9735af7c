"""TEST INFRASTRUCTURE ONLY -- numpy front end of the fp64 CPU oracle.

The oracle (``nsa_oracle.c``) is a plain, slow statement of the Native
Sparse Attention forward pass and of its MoBA special case.  It exists to
check the GPU library and nothing else: only the tests, the smoke check and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the GPU library and never imports it.

A problem is described by a plain dict with the keys

    batch, q_len, kv_len, n_groups, heads_per_group, d_qk, d_v,
    block, top_k, window, force_first, force_current,
    use_cmp, use_slc, use_win, gate_logits, dtype ('bf16' | 'f32'), scale

and optionally sel_block (selection block, a multiple of block; 0 or absent:
the same as block).

Tensors are numpy arrays: ``uint16`` bit patterns for bf16, ``float32``
otherwise, in the layouts listed in ``nsa_oracle.h``.  Every result the
oracle computes is returned in float64, except the pooled block summaries,
which it rounds to the storage type exactly as the method stores them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB = os.path.join(_HERE, "libnsa_oracle.so")


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("block", ctypes.c_int32), ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
        ("force_first", ctypes.c_int32), ("force_current", ctypes.c_int32),
        ("use_cmp", ctypes.c_int32), ("use_slc", ctypes.c_int32), ("use_win", ctypes.c_int32),
        ("gate_logits", ctypes.c_int32), ("is_bf16", ctypes.c_int32),
        ("sel_block", ctypes.c_int32), ("scale", ctypes.c_double),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        lib.oracle_pool.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p]
        lib.oracle_select.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, ctypes.c_int64, p, p, p]
        lib.oracle_attend.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, p, p, p,
                                      ctypes.c_int64, p, p, p]
        lib.oracle_selected_lse.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, ctypes.c_int64, p]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Number of OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_threads())


def _cfg(prob: dict) -> _Cfg:
    c = _Cfg()
    for name, _ in _Cfg._fields_:
        if name == "is_bf16":
            c.is_bf16 = 1 if prob["dtype"] == "bf16" else 0
        elif name == "scale":
            c.scale = float(prob.get("scale", 0.0) or 0.0)
        elif name == "sel_block":
            c.sel_block = int(prob.get("sel_block", 0) or 0)
        else:
            setattr(c, name, int(prob[name]))
    return c


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _stored(a: np.ndarray, prob: dict) -> np.ndarray:
    want = np.uint16 if prob["dtype"] == "bf16" else np.float32
    if a.dtype != want:
        raise TypeError(f"expected {want.__name__} storage, got {a.dtype}")
    return np.ascontiguousarray(a)


def _rows(prob: dict, rows) -> np.ndarray:
    if rows is None:
        rows = np.arange(prob["batch"] * prob["q_len"], dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def pool(prob: dict, k: np.ndarray, v: np.ndarray):
    """Block means kc [B,nb,G,d_qk], vc [B,nb,G,d_v] in the storage type."""
    k, v = _stored(k, prob), _stored(v, prob)
    nb = prob["kv_len"] // prob["block"]
    B, G = prob["batch"], prob["n_groups"]
    kc = np.zeros((B, nb, G, prob["d_qk"]), dtype=k.dtype)
    vc = np.zeros((B, nb, G, prob["d_v"]), dtype=v.dtype)
    c = _cfg(prob)
    _check(_load().oracle_pool(ctypes.byref(c), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc)), "pool")
    return kc, vc


def select(prob: dict, q, kc, vc=None, rows=None, want_imp=True, want_cmp=True):
    """Selection for the given flat rows (b*T + t).

    Returns (idx [R,G,top_k] int32, imp [R,G,nbs] float64 or None (one
    importance per selection block), o_cmp [R,H,d_v] float64 or None)."""
    q, kc = _stored(q, prob), _stored(kc, prob)
    if want_cmp:
        vc = _stored(vc, prob)
    rows = _rows(prob, rows)
    R, G = len(rows), prob["n_groups"]
    H = G * prob["heads_per_group"]
    nbs = prob["kv_len"] // (prob.get("sel_block", 0) or prob["block"])
    idx = np.zeros((R, G, prob["top_k"]), dtype=np.int32)
    imp = np.zeros((R, G, nbs), dtype=np.float64) if want_imp else None
    ocmp = np.zeros((R, H, prob["d_v"]), dtype=np.float64) if want_cmp else None
    c = _cfg(prob)
    _check(_load().oracle_select(ctypes.byref(c), _ptr(q), _ptr(kc), _ptr(vc) if want_cmp else None,
                                 _ptr(rows), len(rows), _ptr(idx), _ptr(imp), _ptr(ocmp)), "select")
    return idx, imp, ocmp


def attend(prob: dict, q, k, v, gates, idx, o_cmp=None, rows=None):
    """Selected + window branches on the GIVEN selection idx [R,G,top_k]
    and the gated sum.  Returns (out, o_slc, o_win), each [R,H,d_v] float64."""
    q, k, v = _stored(q, prob), _stored(k, prob), _stored(v, prob)
    if gates is not None:
        gates = _stored(gates, prob)
    rows = _rows(prob, rows)
    R, H = len(rows), prob["n_groups"] * prob["heads_per_group"]
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(R, prob["n_groups"], prob["top_k"])
    if o_cmp is not None:
        o_cmp = np.ascontiguousarray(o_cmp, dtype=np.float64)
    out = np.zeros((R, H, prob["d_v"]), dtype=np.float64)
    oslc = np.zeros_like(out)
    owin = np.zeros_like(out)
    c = _cfg(prob)
    _check(_load().oracle_attend(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(gates),
                                 _ptr(idx), _ptr(o_cmp), _ptr(rows), len(rows),
                                 _ptr(out), _ptr(oslc), _ptr(owin)), "attend")
    return out, oslc, owin


def selected_lse(prob: dict, q, k, idx, rows=None):
    """Natural log-sum-exp of the selected branch's scaled logits on the
    GIVEN selection idx [R,G,top_k] (the normaliser of that branch's
    softmax): [R,H] float64, -inf where the key set is empty."""
    q, k = _stored(q, prob), _stored(k, prob)
    rows = _rows(prob, rows)
    R, H = len(rows), prob["n_groups"] * prob["heads_per_group"]
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(R, prob["n_groups"], prob["top_k"])
    lse = np.zeros((R, H), dtype=np.float64)
    c = _cfg(prob)
    _check(_load().oracle_selected_lse(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(idx), _ptr(rows), len(rows),
                                       _ptr(lse)), "selected_lse")
    return lse


def forward(prob: dict, q, k, v, gates, rows=None, kc=None, vc=None):
    """The whole forward for the given rows: pool (unless kc/vc are given),
    select, attend.  Returns a dict of float64 results plus the selection."""
    if kc is None or vc is None:
        kc, vc = pool(prob, k, v)
    idx, imp, ocmp = select(prob, q, kc, vc, rows=rows)
    out, oslc, owin = attend(prob, q, k, v, gates, idx, ocmp if prob["use_cmp"] else None, rows=rows)
    return {"kc": kc, "vc": vc, "idx": idx, "imp": imp, "o_cmp": ocmp,
            "o_slc": oslc, "o_win": owin, "out": out}
