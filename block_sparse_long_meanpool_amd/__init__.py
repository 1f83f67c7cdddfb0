"""MoBA prefill forward on MI355X (gfx950) — Python binding of ``libmoba.so``.

This module only marshals arguments: it checks tensor shapes, allocates the
output and workspace through torch, and calls the C ABI declared in
``include/moba.h`` on torch's current HIP stream. Every stage of the
computation runs in the library's HIP kernels; if the library is missing the
calls raise, there is no other implementation behind them.

The operation (PaperTrace "2.1.3 MoBA", eqs. (2)-(8)): block means of K are
the routing keys, each query scores the blocks before its own with an unscaled
dot product, keeps its own block plus the best ``topk - 1`` earlier blocks
(ties to the lower index), and attends with one softmax over those tokens,
causally inside its own block.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoba.so")

MOBA_OK = 0
MOBA_ERR_INVALID_ARGUMENT = 1
MOBA_ERR_UNSUPPORTED = 2
MOBA_ERR_WORKSPACE_TOO_SMALL = 3
MOBA_ERR_HIP = 4
MOBA_DTYPE_BF16 = 0
MOBA_DTYPE_F32 = 1
MOBA_ROUTING_PER_HEAD = 0
MOBA_ROUTING_SHARED = 1
# Stage events: [0] start, [1..4] after these four stages, then per attention
# pass i: [5 + 2i] after its history attention, [6 + 2i] after its own-block
# attention with the merge (``stage_events(prob)`` events in all).
STAGES = ("meanpool", "gate_topk", "bucket", "vpack", "attn_hist", "attn_self_merge")

# Every symbol include/moba.h declares.
EXPORTS = (
    "moba_workspace_size", "moba_select_workspace_size", "moba_prefill", "moba_stage_events",
    "moba_prefill_ex",
    "moba_select", "moba_varlen_workspace_size", "moba_varlen_select_workspace_size",
    "moba_prefill_varlen", "moba_select_varlen",
    "moba_routing_stats_workspace_size", "moba_routing_stats",
    "moba_chunk_workspace_size", "moba_prefill_chunk", "moba_select_chunk",
    "moba_cache_bytes", "moba_cache_append", "moba_cached_workspace_size", "moba_prefill_cached",
    "moba_prefill_train", "moba_backward_workspace_size", "moba_backward",
    "moba_prefill_train_varlen", "moba_backward_varlen_workspace_size", "moba_backward_varlen",
    "moba_dense_workspace_size", "moba_dense_causal", "moba_noalloc_max_workspace",
    "moba_prefill_noalloc", "moba_status_string",
    "moba_last_error",
    "moba_debug_meanpool", "moba_debug_bucket_capacity", "moba_debug_bucket", "moba_debug_copy",
    "moba_debug_read_peak", "moba_debug_mfma_peak",
)


class MobaProblem(ctypes.Structure):
    _fields_ = [
        ("seqlen", ctypes.c_int64),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("routing", ctypes.c_int32),
        ("kv_heads_per_pass", ctypes.c_int32),
    ]


class MobaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _LIB
        text = lib.moba_status_string(status).decode() if lib else str(status)
        detail = lib.moba_last_error().decode() if lib else ""
        super().__init__(f"{where}: {text} ({detail})")
        self.status = status


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoba.so and declare its signatures (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python __graft_entry__.py` "
                          "(or block_sparse_long_meanpool_amd/build.py)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(MobaProblem)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    sig = {
        "moba_workspace_size": (sz, [P]),
        "moba_select_workspace_size": (sz, [P]),
        "moba_prefill": (ctypes.c_int, [P, vp, vp, vp, vp, vp, sz, vp]),
        "moba_stage_events": (sz, [P]),
        "moba_prefill_ex": (ctypes.c_int, [P, vp, vp, vp, vp, vp, sz, vp, vp]),
        "moba_select": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "moba_varlen_workspace_size": (sz, [P, i64, vp]),
        "moba_varlen_select_workspace_size": (sz, [P, i64, vp]),
        "moba_prefill_varlen": (ctypes.c_int, [P, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_select_varlen": (ctypes.c_int, [P, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_prefill_train": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_backward_workspace_size": (sz, [P]),
        "moba_backward": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_prefill_train_varlen": (ctypes.c_int, [P, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                     vp]),
        "moba_backward_varlen_workspace_size": (sz, [P, i64, vp]),
        "moba_backward_varlen": (ctypes.c_int, [P, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, sz, vp]),
        "moba_chunk_workspace_size": (sz, [P, i64]),
        "moba_prefill_chunk": (ctypes.c_int, [P, i64, vp, vp, vp, vp, vp, sz, vp]),
        "moba_select_chunk": (ctypes.c_int, [P, i64, vp, vp, vp, vp, sz, vp]),
        "moba_cache_bytes": (sz, [P, i64]),
        "moba_cache_append": (ctypes.c_int, [P, i64, i64, vp, vp, vp, vp]),
        "moba_cached_workspace_size": (sz, [P, i64]),
        "moba_prefill_cached": (ctypes.c_int, [P, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_routing_stats_workspace_size": (sz, [P]),
        "moba_routing_stats": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moba_noalloc_max_workspace": (sz, []),
        "moba_prefill_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
        "moba_dense_workspace_size": (sz, [P]),
        "moba_dense_causal": (ctypes.c_int, [P, vp, vp, vp, vp, vp, sz, vp]),
        "moba_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moba_last_error": (ctypes.c_char_p, []),
        "moba_debug_meanpool": (ctypes.c_int, [P, vp, vp, vp, sz, vp]),
        "moba_debug_bucket_capacity": (sz, [P]),
        "moba_debug_bucket": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "moba_debug_copy": (ctypes.c_int, [vp, vp, sz, vp]),
        "moba_debug_read_peak": (ctypes.c_int, [vp, sz, ctypes.c_int32, vp, vp]),
        "moba_debug_mfma_peak": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOBA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MOBA_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def make_problem(N, Hq, Hkv, d, block_size, topk, scale=None, dtype=MOBA_DTYPE_BF16,
                 routing=MOBA_ROUTING_PER_HEAD, kv_heads_per_pass=0) -> MobaProblem:
    """``kv_heads_per_pass``: KV heads per attention pass (0 = the library's
    choice); the workspace holds the history partials of one pass."""
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    return MobaProblem(int(N), int(Hq), int(Hkv), int(d), int(block_size), int(topk),
                       float(scale), int(dtype), int(routing), int(kv_heads_per_pass))


def stage_events(prob: MobaProblem) -> int:
    """Number of stage events ``prefill`` records for ``prob`` (0 if invalid)."""
    return load_library().moba_stage_events(ctypes.byref(prob))


def _problem_from(q, k, block_size, topk, scale, routing=MOBA_ROUTING_PER_HEAD,
                  kv_heads_per_pass=0):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [N, Hq, d] and k, v [N, Hkv, d]")
    N, Hq, d = q.shape
    if k.shape[0] != N or k.shape[2] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} vs k {tuple(k.shape)}")
    if k.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    return make_problem(N, Hq, k.shape[1], d, block_size, topk, scale, _dtype_code(q), routing,
                        kv_heads_per_pass)


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ok(status, where):
    if status != MOBA_OK:
        raise MobaError(status, where)


def workspace_size(prob: MobaProblem) -> int:
    return load_library().moba_workspace_size(ctypes.byref(prob))


def select_workspace_size(prob: MobaProblem) -> int:
    return load_library().moba_select_workspace_size(ctypes.byref(prob))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def prefill(q, k, v, block_size, topk, scale=None, out=None, workspace=None, events=None,
            routing=MOBA_ROUTING_PER_HEAD, kv_heads_per_pass=0):
    """MoBA prefill: O [N, Hq, d] from q [N, Hq, d], k, v [N, Hkv, d] (bf16 or fp32).

    ``scale`` defaults to 1/sqrt(d). ``events`` may be a list of
    ``stage_events(prob)`` torch.cuda.Event (created with timing) recorded at
    the stage boundaries on the current stream. ``routing``:
    MOBA_ROUTING_PER_HEAD or MOBA_ROUTING_SHARED (one selection per KV-head
    group). ``kv_heads_per_pass``: KV heads per attention pass (0 = the
    library's choice); the output does not depend on it.
    """
    lib = load_library()
    _check_dev(q, k, v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    prob = _problem_from(q, k, block_size, topk, scale, routing, kv_heads_per_pass)
    if out is None:
        out = torch.empty_like(q)
    _check_dev(out)
    need = lib.moba_workspace_size(ctypes.byref(prob))
    if need == 0:
        _ok(lib.moba_prefill(ctypes.byref(prob), None, None, None, None, None, 0, None),
            "moba_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    ev_arr = None
    if events is not None:
        nev = lib.moba_stage_events(ctypes.byref(prob))
        if len(events) != nev:
            raise ValueError(f"need {nev} events")
        for e in events:
            if not e.cuda_event:  # torch creates the HIP event on first record
                e.record()
        ev_arr = (ctypes.c_void_p * nev)(*[e.cuda_event for e in events])
    st = lib.moba_prefill_ex(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                             _stream(q.device), ev_arr)
    _ok(st, "moba_prefill")
    return out


def prefill_noalloc(q, k, v, block_size, topk, scale=None, out=None,
                    routing=MOBA_ROUTING_PER_HEAD, kv_heads_per_pass=0):
    """``prefill`` through the allocation-free entry point: the library's own
    fixed device scratch (``moba_noalloc_max_workspace()`` bytes per GPU)
    serves as the workspace, so the call allocates nothing (``out`` may be
    given to avoid the output allocation too)."""
    lib = load_library()
    _check_dev(q, k, v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    prob = _problem_from(q, k, block_size, topk, scale, routing, kv_heads_per_pass)
    if out is None:
        out = torch.empty_like(q)
    _check_dev(out)
    st = lib.moba_prefill_noalloc(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), _stream(q.device))
    _ok(st, "moba_prefill_noalloc")
    return out


def select(q, k, block_size, topk, out=None, workspace=None, routing=MOBA_ROUTING_PER_HEAD):
    """Selected blocks per (row, head): int32 [N, Hq, topk], ascending, -1 padded."""
    lib = load_library()
    _check_dev(q, k)
    prob = _problem_from(q, k, block_size, topk, None, routing)
    N, Hq, _ = q.shape
    if out is None:
        out = torch.empty((N, Hq, topk), dtype=torch.int32, device=q.device)
    need = lib.moba_select_workspace_size(ctypes.byref(prob))
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib.moba_select(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), out.data_ptr(),
                         workspace.data_ptr(), workspace.numel(), _stream(q.device))
    _ok(st, "moba_select")
    return out


def _cu_pair(cu_seqlens, device):
    """Host ctypes copy and device int64 tensor of the sequence offsets."""
    if isinstance(cu_seqlens, torch.Tensor):
        host = cu_seqlens.detach().to("cpu", torch.int64).contiguous()
    else:
        host = torch.tensor([int(x) for x in cu_seqlens], dtype=torch.int64)
    if host.dim() != 1 or host.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with nseq + 1 >= 2 entries")
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda and \
            cu_seqlens.dtype == torch.int64 and cu_seqlens.is_contiguous():
        dev = cu_seqlens
    else:
        dev = host.to(device)
    arr = (ctypes.c_int64 * host.numel())(*host.tolist())
    return arr, dev, host.numel() - 1


def varlen_workspace_size(prob: MobaProblem, cu_seqlens) -> int:
    """Workspace bytes of moba_prefill_varlen for sequence offsets ``cu_seqlens`` (0 if invalid)."""
    host = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    arr = (ctypes.c_int64 * len(host))(*host)
    return load_library().moba_varlen_workspace_size(ctypes.byref(prob), len(host) - 1, arr)


def prefill_varlen(q, k, v, cu_seqlens, block_size, topk, scale=None, out=None, workspace=None,
                   routing=MOBA_ROUTING_PER_HEAD, kv_heads_per_pass=0):
    """MoBA prefill over packed sequences: rows [cu[i], cu[i+1]) of q, k, v form
    sequence i; blocks restart at each sequence and never cross one. Equals
    ``prefill`` applied to every sequence on its own."""
    lib = load_library()
    _check_dev(q, k, v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    prob = _problem_from(q, k, block_size, topk, scale, routing, kv_heads_per_pass)
    cu_host, cu_dev, nseq = _cu_pair(cu_seqlens, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_dev(out)
    need = lib.moba_varlen_workspace_size(ctypes.byref(prob), nseq, cu_host)
    if need == 0:
        _ok(lib.moba_prefill_varlen(ctypes.byref(prob), nseq, cu_host, None, None, None, None,
                                    None, None, 0, None), "moba_varlen_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib.moba_prefill_varlen(ctypes.byref(prob), nseq, cu_host, cu_dev.data_ptr(),
                                 q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream(q.device))
    _ok(st, "moba_prefill_varlen")
    return out


def select_varlen(q, k, cu_seqlens, block_size, topk, out=None, workspace=None):
    """Selected global block ids per (row, head) for packed sequences:
    int32 [N, Hq, topk], ascending, -1 padded."""
    lib = load_library()
    _check_dev(q, k)
    prob = _problem_from(q, k, block_size, topk, None)
    cu_host, cu_dev, nseq = _cu_pair(cu_seqlens, q.device)
    N, Hq, _ = q.shape
    if out is None:
        out = torch.empty((N, Hq, topk), dtype=torch.int32, device=q.device)
    need = lib.moba_varlen_select_workspace_size(ctypes.byref(prob), nseq, cu_host)
    if need == 0:
        _ok(lib.moba_select_varlen(ctypes.byref(prob), nseq, cu_host, None, None, None, None,
                                   None, 0, None), "moba_varlen_select_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib.moba_select_varlen(ctypes.byref(prob), nseq, cu_host, cu_dev.data_ptr(),
                                q.data_ptr(), k.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream(q.device))
    _ok(st, "moba_select_varlen")
    return out


def _chunk_problem(q, k, block_size, topk, scale, routing, kv_heads_per_pass=0):
    if q.dim() != 3 or k.dim() != 3 or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [C, Hq, d] and k, v [N, Hkv, d]")
    if k.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    N, Hkv, d = k.shape
    return make_problem(N, q.shape[1], Hkv, d, block_size, topk, scale, _dtype_code(q), routing,
                        kv_heads_per_pass)


def prefill_train(q, k, v, block_size, topk, scale=None, routing=MOBA_ROUTING_PER_HEAD,
                  workspace=None, kv_heads_per_pass=0):
    """Forward for training: (O [N, Hq, d], lse [N, Hq] fp32), lse being each
    row's log2-sum-exp of scale*log2(e)*q.k over its keys."""
    lib = load_library()
    _check_dev(q, k, v)
    prob = _problem_from(q, k, block_size, topk, scale, routing, kv_heads_per_pass)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    need = lib.moba_workspace_size(ctypes.byref(prob))
    if need == 0:
        _ok(lib.moba_prefill_train(ctypes.byref(prob), None, None, None, None, None, None, 0, None),
            "moba_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib.moba_prefill_train(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream(q.device))
    _ok(st, "moba_prefill_train")
    return out, lse


def backward(q, k, v, o, lse, dout, block_size, topk, scale=None, routing=MOBA_ROUTING_PER_HEAD):
    """Gradients (dq, dk, dv) of sum(dout * O) with the block selection held fixed."""
    lib = load_library()
    _check_dev(q, k, v, o, lse, dout)
    prob = _problem_from(q, k, block_size, topk, scale, routing)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = lib.moba_backward_workspace_size(ctypes.byref(prob))
    if need == 0:
        _ok(lib.moba_backward(ctypes.byref(prob), *([None] * 10), 0, None),
            "moba_backward_workspace_size")
    ws = alloc_workspace(need, q.device)
    st = lib.moba_backward(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                           dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                           _stream(q.device))
    _ok(st, "moba_backward")
    return dq, dk, dv


class DecodeCache:
    """Decode cache of one sequence (moba_cache_*): the block means of its full
    blocks and the packed V copy, kept current by ``append`` as rows arrive, so
    that ``prefill`` (a chunk or decode step) does not recompute them from the
    whole KV cache. k and v passed to both are the KV cache tensors
    [capacity, Hkv, d] of which the first ``rows`` are valid."""

    def __init__(self, capacity, num_q_heads, num_kv_heads, block_size, topk, scale=None,
                 dtype=MOBA_DTYPE_BF16, routing=MOBA_ROUTING_PER_HEAD, head_dim=128,
                 device="cuda"):
        lib = load_library()
        self.capacity = int(capacity)
        self.Hq, self.Hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.block_size, self.topk, self.scale = block_size, topk, scale
        self.dtype, self.routing = dtype, routing
        self.rows = 0
        prob = self._problem(1)
        nbytes = lib.moba_cache_bytes(ctypes.byref(prob), self.capacity)
        if nbytes == 0:
            raise MobaError(lib.moba_cache_append(ctypes.byref(prob), self.capacity, 0, None, None,
                                                  None, None), "moba_cache_bytes")
        self.buf = alloc_workspace(nbytes, device)

    def _problem(self, rows):
        return make_problem(rows, self.Hq, self.Hkv, self.d, self.block_size, self.topk,
                            self.scale, self.dtype, self.routing)

    def append(self, k, v, rows):
        """Rows [self.rows, rows) of k and v are new: update the cache."""
        lib = load_library()
        _check_dev(k, v)
        if k.shape[0] != self.capacity or v.shape != k.shape:
            raise ValueError("k and v must be the [capacity, Hkv, d] KV cache tensors")
        prob = self._problem(rows)
        st = lib.moba_cache_append(ctypes.byref(prob), self.capacity, self.rows, k.data_ptr(),
                                   v.data_ptr(), self.buf.data_ptr(), _stream(k.device))
        _ok(st, "moba_cache_append")
        self.rows = int(rows)

    def workspace_size(self, q_rows):
        """Workspace bytes of ``prefill`` for q_rows queries at the current length."""
        prob = self._problem(self.rows)
        return load_library().moba_cached_workspace_size(ctypes.byref(prob), int(q_rows))

    def prefill(self, q, k, v, out=None, workspace=None):
        """O for the queries q [C, Hq, d] of the last C of the first self.rows
        positions (as ``prefill_chunk`` over k[:rows], v[:rows])."""
        lib = load_library()
        _check_dev(q, k, v)
        prob = self._problem(self.rows)
        C = q.shape[0]
        if out is None:
            out = torch.empty_like(q)
        need = lib.moba_cached_workspace_size(ctypes.byref(prob), C)
        if need == 0:
            _ok(lib.moba_prefill_cached(ctypes.byref(prob), self.capacity, C, None, None, None,
                                        None, None, None, 0, None), "moba_cached_workspace_size")
        if workspace is None:
            workspace = alloc_workspace(need, q.device)
        st = lib.moba_prefill_cached(ctypes.byref(prob), self.capacity, C, q.data_ptr(),
                                     k.data_ptr(), v.data_ptr(), self.buf.data_ptr(),
                                     out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream(q.device))
        _ok(st, "moba_prefill_cached")
        return out


def prefill_train_varlen(q, k, v, cu_seqlens, block_size, topk, scale=None,
                         routing=MOBA_ROUTING_PER_HEAD):
    """``prefill_train`` over packed sequences (the layout of ``prefill_varlen``):
    (O [N, Hq, d], lse [N, Hq] fp32)."""
    lib = load_library()
    _check_dev(q, k, v)
    prob = _problem_from(q, k, block_size, topk, scale, routing)
    cu_host, cu_dev, nseq = _cu_pair(cu_seqlens, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    need = lib.moba_varlen_workspace_size(ctypes.byref(prob), nseq, cu_host)
    if need == 0:
        _ok(lib.moba_prefill_train_varlen(ctypes.byref(prob), nseq, cu_host, *([None] * 7), 0,
                                          None), "moba_varlen_workspace_size")
    ws = alloc_workspace(need, q.device)
    st = lib.moba_prefill_train_varlen(ctypes.byref(prob), nseq, cu_host, cu_dev.data_ptr(),
                                       q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), ws.data_ptr(), ws.numel(),
                                       _stream(q.device))
    _ok(st, "moba_prefill_train_varlen")
    return out, lse


def backward_varlen(q, k, v, o, lse, dout, cu_seqlens, block_size, topk, scale=None,
                    routing=MOBA_ROUTING_PER_HEAD):
    """``backward`` over packed sequences: (dq, dk, dv)."""
    lib = load_library()
    _check_dev(q, k, v, o, lse, dout)
    prob = _problem_from(q, k, block_size, topk, scale, routing)
    cu_host, cu_dev, nseq = _cu_pair(cu_seqlens, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = lib.moba_backward_varlen_workspace_size(ctypes.byref(prob), nseq, cu_host)
    if need == 0:
        _ok(lib.moba_backward_varlen(ctypes.byref(prob), nseq, cu_host, *([None] * 10), 0, None),
            "moba_backward_varlen_workspace_size")
    ws = alloc_workspace(need, q.device)
    st = lib.moba_backward_varlen(ctypes.byref(prob), nseq, cu_host, cu_dev.data_ptr(),
                                  q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device))
    _ok(st, "moba_backward_varlen")
    return dq, dk, dv


def chunk_workspace_size(prob: MobaProblem, q_rows: int) -> int:
    """Workspace bytes of moba_prefill_chunk / moba_select_chunk (0 if invalid)."""
    return load_library().moba_chunk_workspace_size(ctypes.byref(prob), int(q_rows))


def prefill_chunk(q, k, v, block_size, topk, scale=None, out=None, workspace=None,
                  routing=MOBA_ROUTING_PER_HEAD, kv_heads_per_pass=0):
    """Chunked prefill / decode: q [C, Hq, d] are the queries of the last C
    positions of a sequence whose keys and values k, v [N, Hkv, d] include
    them. Returns O [C, Hq, d], equal to those rows of ``prefill`` over the
    whole sequence (C = 1 is one decode step)."""
    lib = load_library()
    _check_dev(q, k, v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    prob = _chunk_problem(q, k, block_size, topk, scale, routing, kv_heads_per_pass)
    C = q.shape[0]
    if out is None:
        out = torch.empty_like(q)
    _check_dev(out)
    need = lib.moba_chunk_workspace_size(ctypes.byref(prob), C)
    if need == 0:
        _ok(lib.moba_prefill_chunk(ctypes.byref(prob), C, None, None, None, None, None, 0, None),
            "moba_chunk_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib.moba_prefill_chunk(ctypes.byref(prob), C, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream(q.device))
    _ok(st, "moba_prefill_chunk")
    return out


def select_chunk(q, k, block_size, topk, routing=MOBA_ROUTING_PER_HEAD):
    """Selections of the last C positions (q [C, Hq, d]): int32 [C, Hq, topk]."""
    lib = load_library()
    _check_dev(q, k)
    prob = _chunk_problem(q, k, block_size, topk, None, routing)
    C, Hq, _ = q.shape
    out = torch.empty((C, Hq, topk), dtype=torch.int32, device=q.device)
    need = lib.moba_chunk_workspace_size(ctypes.byref(prob), C)
    if need == 0:
        _ok(lib.moba_select_chunk(ctypes.byref(prob), C, None, None, None, None, 0, None),
            "moba_chunk_workspace_size")
    ws = alloc_workspace(need, q.device)
    st = lib.moba_select_chunk(ctypes.byref(prob), C, q.data_ptr(), k.data_ptr(), out.data_ptr(),
                               ws.data_ptr(), ws.numel(), _stream(q.device))
    _ok(st, "moba_select_chunk")
    return out


def routing_stats(q, k, block_size, topk, routing=MOBA_ROUTING_PER_HEAD):
    """Routing diagnostics from the exact gate: dict of device tensors
    ``sel`` int32 [N, Hq, topk], ``margin`` fp32 [N, Hq] (NaN where nothing is
    left out), ``counts`` int32 [Hkv, n] (history selections per block) and
    ``union_size`` int32 [N, Hkv] (distinct history blocks per head group)."""
    lib = load_library()
    _check_dev(q, k)
    prob = _problem_from(q, k, block_size, topk, None, routing)
    N, Hq, _ = q.shape
    Hkv = k.shape[1]
    n = -(-N // block_size)
    dev = q.device
    sel = torch.empty((N, Hq, topk), dtype=torch.int32, device=dev)
    margin = torch.empty((N, Hq), dtype=torch.float32, device=dev)
    counts = torch.empty((Hkv, n), dtype=torch.int32, device=dev)
    union = torch.empty((N, Hkv), dtype=torch.int32, device=dev)
    need = lib.moba_routing_stats_workspace_size(ctypes.byref(prob))
    ws = alloc_workspace(need, dev)
    st = lib.moba_routing_stats(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), sel.data_ptr(),
                                margin.data_ptr(), counts.data_ptr(), union.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream(dev))
    _ok(st, "moba_routing_stats")
    return {"sel": sel, "margin": margin, "counts": counts, "union_size": union}


def dense_causal(q, k, v, scale=None, out=None, workspace=None):
    """Dense causal softmax attention (the full-attention baseline)."""
    lib = load_library()
    _check_dev(q, k, v)
    prob = _problem_from(q, k, q.shape[0], 1, scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(lib.moba_dense_workspace_size(ctypes.byref(prob)), q.device)
    st = lib.moba_dense_causal(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                               _stream(q.device))
    _ok(st, "moba_dense_causal")
    return out


def debug_meanpool(k, block_size):
    """Block means of k for the blocks that can be history: fp64 [Hkv, n-1, d]."""
    lib = load_library()
    _check_dev(k)
    N, Hkv, d = k.shape
    prob = make_problem(N, Hkv, Hkv, d, block_size, 1, None, _dtype_code(k))
    n = -(-N // block_size)
    kbar = torch.empty((Hkv, max(n - 1, 0), d), dtype=torch.float64, device=k.device)
    ws = alloc_workspace(lib.moba_select_workspace_size(ctypes.byref(prob)), k.device)
    ptr = kbar.data_ptr() if kbar.numel() else ws.data_ptr()
    st = lib.moba_debug_meanpool(ctypes.byref(prob), k.data_ptr(), ptr, ws.data_ptr(), ws.numel(),
                                 _stream(k.device))
    _ok(st, "moba_debug_meanpool")
    return kbar


def debug_bucket(sel, num_kv_heads, block_size, head_dim=128, dtype=MOBA_DTYPE_BF16):
    """Per-(KV head, block) lists from a selection: (offsets int32, entries int32)."""
    lib = load_library()
    _check_dev(sel)
    N, Hq, topk = sel.shape
    prob = make_problem(N, Hq, num_kv_heads, head_dim, block_size, topk, None, dtype)
    n = -(-N // block_size)
    cap = lib.moba_debug_bucket_capacity(ctypes.byref(prob))
    offsets = torch.empty(num_kv_heads * max(n - 1, 0) + 1, dtype=torch.int32, device=sel.device)
    entries = torch.empty(max(cap, 4), dtype=torch.int32, device=sel.device)
    ws = alloc_workspace(lib.moba_workspace_size(ctypes.byref(prob)), sel.device)
    st = lib.moba_debug_bucket(ctypes.byref(prob), sel.data_ptr(), offsets.data_ptr(),
                               entries.data_ptr(), ws.data_ptr(), ws.numel(), _stream(sel.device))
    _ok(st, "moba_debug_bucket")
    return offsets, entries[:cap]


def debug_copy(src, dst):
    lib = load_library()
    _check_dev(src, dst)
    nbytes = src.numel() * src.element_size()
    st = lib.moba_debug_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src.device))
    _ok(st, "moba_debug_copy")
    return dst


def debug_read_peak(src, out):
    """Read-only HBM stream probe over all bytes of ``src``; ``out`` is an
    int32 device tensor of ``workgroups * 256`` values whose XOR equals the
    XOR of every 32-bit word of ``src``."""
    lib = load_library()
    _check_dev(src, out)
    if out.dtype != torch.int32 or out.numel() % 256:
        raise ValueError("out must be an int32 tensor of workgroups * 256 values")
    nbytes = src.numel() * src.element_size()
    st = lib.moba_debug_read_peak(src.data_ptr(), nbytes, out.numel() // 256, out.data_ptr(),
                                  _stream(src.device))
    _ok(st, "moba_debug_read_peak")
    return out


def debug_mfma_peak(out, iters):
    """Matrix-core issue-rate probe: ``out`` is a float32 device tensor of
    ``workgroups * 256`` values (one per lane); each comes back as exactly
    ``16 * iters``. FLOP per call = ``workgroups * 4 * iters * 4 * 32768``."""
    lib = load_library()
    _check_dev(out)
    if out.dtype != torch.float32 or out.numel() % 256 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of workgroups * 256 values")
    st = lib.moba_debug_mfma_peak(out.numel() // 256, int(iters), out.data_ptr(),
                                  _stream(out.device))
    _ok(st, "moba_debug_mfma_peak")
    return out
