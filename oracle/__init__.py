"""fp64 CPU oracle for the MoBA prefill forward pass — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never links or calls it,
and the two share no code.

The arithmetic lives in ``moba_ref.c`` (plain loops, fp64, OpenMP over rows);
this module only builds it with gcc and marshals numpy arrays. The method it
follows is the one on the PaperTrace page "2.1.3 MoBA": block means and the
unscaled gate of section 1 eq. (3), the causal mask / forced own block / k
counting the own block of section 2 and 2.1, and the single softmax over the
candidate union of eqs. (4)-(6), with eqs. (7)-(8) as a second form.

Every function is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoba_ref.so")

MODE_UNION, MODE_TWO_BRANCH, MODE_NAIVE = 0, 1, 2
ROUTING_PER_HEAD, ROUTING_SHARED = 0, 1


class _Problem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("dtype", ctypes.c_int32),
        ("routing", ctypes.c_int32),
    ]


def build() -> str:
    """Compile ``libmoba_ref.so`` (gcc, -O2, OpenMP; no GPU code)."""
    src = os.path.join(_HERE, "moba_ref.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        lib.moba_ref_block_means.restype = ctypes.c_int
        lib.moba_ref_block_means.argtypes = [P, vp, vp]
        lib.moba_ref_rows.restype = ctypes.c_int
        lib.moba_ref_rows.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_int,
                                      vp, vp, vp, ctypes.c_int]
        lib.moba_ref_backward.restype = ctypes.c_int
        lib.moba_ref_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.moba_ref_causal_full.restype = ctypes.c_int
        lib.moba_ref_causal_full.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_int]
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0  # bf16 bit patterns
    if a.dtype == np.float32:
        return 1
    raise TypeError(f"oracle inputs must be uint16 (bf16 bits) or float32, got {a.dtype}")


def _problem(q, k, B, topk, scale, routing=ROUTING_PER_HEAD):
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return _Problem(N, Hq, Hkv, d, B, topk, float(scale), _dtype_code(q), int(routing))


def _c(a, dt=None):
    return np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))


def block_means(k: np.ndarray, B: int) -> np.ndarray:
    """Block keys, eq. (3): fp64 array [Hkv, n-1, d]."""
    k = _c(k)
    N, Hkv, d = k.shape
    n = -(-N // B)
    pr = _Problem(N, Hkv, Hkv, d, B, 1, 1.0, _dtype_code(k))
    out = np.zeros((Hkv, max(n - 1, 0), d), np.float64)
    if n > 1:
        rc = _load().moba_ref_block_means(ctypes.byref(pr), k.ctypes.data, out.ctypes.data)
        if rc:
            raise ValueError(f"moba_ref_block_means failed ({rc})")
    return out


def rows(q, k, v, B, topk, rows, heads, scale=None, forced_sel=None, mode=MODE_UNION,
         want_o=True, kbar=None, nthreads=0, routing=ROUTING_PER_HEAD):
    """Evaluate the method on (row, head) pairs.

    ``routing``: ROUTING_PER_HEAD ranks blocks with each head's own query;
    ROUTING_SHARED ranks them once per KV-head group by the group's summed
    gate score (PaperTrace "2.1.3 MoBA", section 5.5 on GQA routing).

    Returns ``(sel, o, gap)``: ``sel`` int32 [R, k] ascending and -1 padded;
    ``o`` fp64 [R, d] (None when ``want_o`` is False); ``gap`` fp64 [R, 2] with the
    selection margin between the last selected and the best unselected history
    score and the larger of their magnitudes (NaN where nothing was left out).
    """
    q, k = _c(q), _c(k)
    if _dtype_code(k) != _dtype_code(q):
        raise TypeError("q and k must share a dtype")
    if v is not None:
        v = _c(v)
    pr = _problem(q, k, B, topk, scale, routing)
    rws = _c(np.asarray(rows), np.int64)
    hds = _c(np.asarray(heads), np.int32)
    R = rws.shape[0]
    sel = np.empty((R, topk), np.int32)
    o = np.empty((R, q.shape[2]), np.float64) if want_o else None
    gap = np.empty((R, 2), np.float64)
    fs = None
    if forced_sel is not None:
        fs = _c(np.asarray(forced_sel), np.int32)
        assert fs.shape == (R, topk)
    kb = None
    if kbar is not None:
        kb = _c(kbar, np.float64)
    rc = _load().moba_ref_rows(
        ctypes.byref(pr), q.ctypes.data, k.ctypes.data, v.ctypes.data if v is not None else None,
        kb.ctypes.data if kb is not None else None, rws.ctypes.data, hds.ctypes.data, R,
        fs.ctypes.data if fs is not None else None, mode, sel.ctypes.data,
        o.ctypes.data if o is not None else None, gap.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"moba_ref_rows failed ({rc})")
    return sel, o, gap


def all_rows(N, Hq):
    """(rows, heads) enumerating every (row, head) pair, row-major."""
    r = np.repeat(np.arange(N, dtype=np.int64), Hq)
    h = np.tile(np.arange(Hq, dtype=np.int32), N)
    return r, h


def prefill(q, k, v, B, topk, scale=None, mode=MODE_UNION, nthreads=0, routing=ROUTING_PER_HEAD):
    """Full layer: (sel [N, Hq, k], o [N, Hq, d] fp64)."""
    N, Hq, d = q.shape
    r, h = all_rows(N, Hq)
    sel, o, _ = rows(q, k, v, B, topk, r, h, scale=scale, mode=mode, nthreads=nthreads,
                     routing=routing)
    return sel.reshape(N, Hq, topk), o.reshape(N, Hq, d)


def causal_full(q, k, v, rows, heads, scale=None, nthreads=0):
    """Causal full softmax attention (eq. (1) with a causal mask), fp64 [R, d]."""
    q, k, v = _c(q), _c(k), _c(v)
    pr = _problem(q, k, 1, 1, scale)
    rws = _c(np.asarray(rows), np.int64)
    hds = _c(np.asarray(heads), np.int32)
    o = np.empty((rws.shape[0], q.shape[2]), np.float64)
    rc = _load().moba_ref_causal_full(ctypes.byref(pr), q.ctypes.data, k.ctypes.data,
                                      v.ctypes.data, rws.ctypes.data, hds.ctypes.data,
                                      rws.shape[0], o.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"moba_ref_causal_full failed ({rc})")
    return o


def prefill_varlen(q, k, v, cu, B, topk, scale=None, mode=MODE_UNION, nthreads=0):
    """Packed sequences: rows [cu[i], cu[i+1]) form sequence i, which is cut
    into its own blocks from its first row; its block means, gate, top-k and
    attention see only its own rows (PaperTrace "2.1.3 MoBA", section 5.1:
    with packed documents the blocks, their summaries and the gate share the
    document boundaries). Each sequence is therefore evaluated on its own.

    Returns (sel [N, Hq, k] with block indices counted within each sequence,
    o [N, Hq, d] fp64).
    """
    N, Hq, d = q.shape
    sel = np.full((N, Hq, topk), -1, np.int32)
    o = np.zeros((N, Hq, d), np.float64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b > a:
            s_i, o_i = prefill(q[a:b], k[a:b], v[a:b], B, topk, scale=scale, mode=mode,
                               nthreads=nthreads)
            sel[a:b], o[a:b] = s_i, o_i
    return sel, o


def backward(q, k, v, dout, B, topk, scale=None, sel=None, routing=ROUTING_PER_HEAD):
    """Gradients (dq [N, Hq, d], dk, dv [N, Hkv, d], fp64) of sum(dout * O) with the
    block selection held fixed (no gradient through the hard top-k ranking):
    the softmax-attention gradient over each row's candidate set, eqs. (4)-(6).
    ``sel`` defaults to the oracle's own selection."""
    q, k, v = _c(q), _c(k), _c(v)
    N, Hq, d = q.shape
    if sel is None:
        r, h = all_rows(N, Hq)
        sel, _, _ = rows(q, k, None, B, topk, r, h, want_o=False, routing=routing)
    sel = _c(np.asarray(sel).reshape(N, Hq, topk), np.int32)
    dout = _c(np.asarray(dout, dtype=np.float64))
    pr = _problem(q, k, B, topk, scale, routing)
    dq = np.empty((N, Hq, d), np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(k.shape, np.float64)
    rc = _load().moba_ref_backward(ctypes.byref(pr), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                   dout.ctypes.data, sel.ctypes.data, dq.ctypes.data,
                                   dk.ctypes.data, dv.ctypes.data)
    if rc:
        raise ValueError(f"moba_ref_backward failed ({rc})")
    return dq, dk, dv
