"""Seeded synthetic MoBA workloads (inputs only, no attention arithmetic).

The five workloads mirror the shapes of the experiments on the pages:

* ``tiny2k`` tiny single-head layer (N=2048, B=256, k=3), fp32 masters;
* ``mha8k`` the scaling-law setting at 8K (N=8192, B=512, k=3, 16 heads) —
  MoBA paper summary (PaperTrace "2.1.3 MoBA", section 2.1, eq. (9));
* ``mha32k_needles`` the same block/top-k at 32K with long-range "needle" blocks;
* ``coarse32k`` the efficient-vs-naive comparison shape (32K, 1 head, B=2048, k=3) —
  MoonshotAI/MoBA README, implementation details;
* ``llama8b_1m`` the Llama-3.1-8B 1M-token layer (B=4096, k=12) with 32 query heads
  sharing 8 KV heads — agihunt summary, results section;
* ``llama8b_128k`` the same layer at 128K rows (a training-sized shape for the
  backward pass).

Values come from ``synth.c`` (SplitMix64 counters + Box-Muller); the C
library is built by :func:`build` and loaded with ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoba_synth.so")

SEED_BASE = 0x4D6F424100000000


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    Hq: int
    Hkv: int
    d: int
    B: int
    k: int
    dtype: str = "bf16"          # "bf16" or "f32"
    off_std: float = 0.5
    needle_blocks: int = 0
    needle_gain: float = 0.0
    needle_row_frac: float = 0.0
    seed: int = SEED_BASE

    @property
    def n(self) -> int:
        return -(-self.N // self.B)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Workloads shaped like the pages' experiments, named by what they are:
# a tiny single-head layer (2K rows), a 16-head layer at 8K and at 32K (the
# latter with planted needle blocks), a single-head coarse-block layer at 32K,
# and a Llama-3.1-8B-shaped GQA layer (32 query / 8 KV heads) at 1M rows.
CONFIGS = {
    "tiny2k": Workload("tiny2k", 2048, 1, 1, 128, 256, 3, dtype="f32", seed=SEED_BASE | 1),
    "mha8k": Workload("mha8k", 8192, 16, 16, 128, 512, 3, seed=SEED_BASE | 2),
    "mha32k_needles": Workload("mha32k_needles", 32768, 16, 16, 128, 512, 3, needle_blocks=8,
                               needle_gain=1.5, needle_row_frac=0.01, seed=SEED_BASE | 3),
    "coarse32k": Workload("coarse32k", 32768, 1, 1, 128, 2048, 3, seed=SEED_BASE | 4),
    "llama8b_1m": Workload("llama8b_1m", 1048576, 32, 8, 128, 4096, 12, seed=SEED_BASE | 5),
    # the same GQA layer at 128K rows: a training-sized shape for the backward pass
    "llama8b_128k": Workload("llama8b_128k", 131072, 32, 8, 128, 4096, 12, seed=SEED_BASE | 6),
}


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("off_std", ctypes.c_double),
        ("n_needle_blocks", ctypes.c_int32),
        ("needle_gain", ctypes.c_double),
        ("needle_row_frac", ctypes.c_double),
    ]


def build() -> str:
    """Compile ``libmoba_synth.so`` with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
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
        lib.synth_qkv.restype = ctypes.c_int
        lib.synth_qkv.argtypes = [ctypes.c_uint64, ctypes.POINTER(_Cfg), ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_sample_rows.restype = None
        lib.synth_sample_rows.argtypes = [ctypes.c_uint64, ctypes.POINTER(_Cfg), ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_needle_blocks.restype = ctypes.c_int
        lib.synth_needle_blocks.argtypes = [ctypes.c_uint64, ctypes.POINTER(_Cfg), ctypes.c_int,
                                            ctypes.c_void_p]
        lib.synth_needle_rows.restype = ctypes.c_int64
        lib.synth_needle_rows.argtypes = [ctypes.c_uint64, ctypes.POINTER(_Cfg), ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_int64]
        _lib = lib
    return _lib


def _cfg(w: Workload) -> _Cfg:
    return _Cfg(w.N, w.Hq, w.Hkv, w.d, w.B, w.off_std, w.needle_blocks, w.needle_gain,
                w.needle_row_frac)


def _np_dtype(dtype: str):
    if dtype == "bf16":
        return np.uint16
    if dtype == "f32":
        return np.float32
    raise ValueError(dtype)


def make_qkv(w: Workload, dtype: str | None = None, which: str = "qkv"):
    """Return (q, k, v) numpy arrays shaped [N, H, d].

    bf16 tensors come back as ``uint16`` bit patterns; fp32 as ``float32``.
    Tensors not named in ``which`` are returned as ``None``.
    """
    dtype = dtype or w.dtype
    lib = _load()
    npdt = _np_dtype(dtype)
    q = np.empty((w.N, w.Hq, w.d), npdt) if "q" in which else None
    k = np.empty((w.N, w.Hkv, w.d), npdt) if "k" in which else None
    v = np.empty((w.N, w.Hkv, w.d), npdt) if "v" in which else None
    cfg = _cfg(w)
    rc = lib.synth_qkv(w.seed, ctypes.byref(cfg), 0 if dtype == "bf16" else 1,
                       q.ctypes.data if q is not None else None,
                       k.ctypes.data if k is not None else None,
                       v.ctypes.data if v is not None else None)
    if rc != 0:
        raise MemoryError("synth_qkv failed")
    return q, k, v


def sample_rows(w: Workload, count: int = 4096):
    """Seeded (rows, heads) sample covering every block and both block edges."""
    lib = _load()
    rows = np.empty(count, np.int64)
    heads = np.empty(count, np.int32)
    cfg = _cfg(w)
    lib.synth_sample_rows(w.seed, ctypes.byref(cfg), count, rows.ctypes.data, heads.ctypes.data)
    return rows, heads


def needle_blocks(w: Workload, g: int):
    lib = _load()
    out = np.empty(max(1, w.needle_blocks), np.int32)
    cfg = _cfg(w)
    got = lib.synth_needle_blocks(w.seed, ctypes.byref(cfg), g, out.ctypes.data)
    return out[:got].copy()


def needle_rows(w: Workload, h: int):
    lib = _load()
    out = np.empty(w.N, np.int64)
    cfg = _cfg(w)
    got = lib.synth_needle_rows(w.seed, ctypes.byref(cfg), h, out.ctypes.data, w.N)
    return out[:got].copy()


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def random_qkv(N, Hq, Hkv, d, seed, dtype="f32", scale_k=1.0, integer=False):
    """Small unstructured inputs for edge-case tests (numpy Generator, seeded).

    With ``integer=True`` the values are small integers, which makes block
    means and gate scores exact and forces ties.
    """
    rng = np.random.default_rng(seed)
    if integer:
        q = rng.integers(-2, 3, size=(N, Hq, d)).astype(np.float32)
        k = rng.integers(-2, 3, size=(N, Hkv, d)).astype(np.float32) * scale_k
        v = rng.integers(-3, 4, size=(N, Hkv, d)).astype(np.float32)
    else:
        q = rng.standard_normal((N, Hq, d)).astype(np.float32)
        k = (rng.standard_normal((N, Hkv, d)) * scale_k).astype(np.float32)
        v = rng.standard_normal((N, Hkv, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (f32_to_bf16(x) for x in (q, k, v))
    return q, k, v


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns (round to nearest even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def packed_layer_lengths(w: Workload, nseq: int = 16) -> np.ndarray:
    """The packed batch of a workload's layer: ``nseq`` seeded log-uniform
    lengths between max(B, N/64) and 3N/16 rows, summing to N."""
    return packed_lengths(w.N, nseq, w.seed ^ 0x5EC, max(w.B, w.N // 64), w.N * 3 // 16)


def packed_lengths(total: int, nseq: int, seed: int, lo: int, hi: int) -> np.ndarray:
    """Seeded sequence lengths for a packed batch: log-uniform in [lo, hi],
    rescaled to sum to ``total`` (the last one absorbs the rounding)."""
    rng = np.random.default_rng(seed)
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=nseq))
    lens = np.maximum(1, np.floor(x / x.sum() * total)).astype(np.int64)
    lens[-1] += total - lens.sum()
    return lens
