"""CPU-only checks of the C ABI: the library loads, exports what include/moba.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import block_sparse_long_meanpool_amd as moba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "moba.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"MOBA_API[^;(]*?\b(moba_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_symbols() == sorted(moba.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = moba.load_library()
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = moba.load_library()
    assert lib.moba_status_string(0) == b"MOBA_OK"
    assert lib.moba_status_string(3) == b"MOBA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moba_status_string(99) == b"MOBA_ERR_UNKNOWN"


def _prob(**kw):
    base = dict(N=4096, Hq=8, Hkv=2, d=128, block_size=256, topk=3, scale=0.088, dtype=0, kvpp=0)
    base.update(kw)
    return moba.make_problem(base["N"], base["Hq"], base["Hkv"], base["d"], base["block_size"],
                             base["topk"], base["scale"], base["dtype"],
                             kv_heads_per_pass=base["kvpp"])


BAD = [
    (dict(N=0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(Hq=0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(Hq=6, Hkv=4), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(block_size=0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(topk=0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.inf), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.nan), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(d=0), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(d=64), moba.MOBA_ERR_UNSUPPORTED),
    (dict(topk=33), moba.MOBA_ERR_UNSUPPORTED),
    (dict(N=1 << 20, block_size=64), moba.MOBA_ERR_UNSUPPORTED),
    (dict(N=1 << 24, Hq=64, Hkv=64, block_size=4096, topk=3), moba.MOBA_ERR_UNSUPPORTED),
    (dict(Hq=128, Hkv=1), moba.MOBA_ERR_UNSUPPORTED),
    # bf16: the packed V^T rows of a KV head would pass 2^32 bytes of 32-bit
    # buffer offsets (N * Hq * topk is still below 2^31)
    (dict(N=20_000_000, Hq=8, Hkv=8, block_size=4096, topk=12), moba.MOBA_ERR_UNSUPPORTED),
    (dict(kvpp=-1), moba.MOBA_ERR_INVALID_ARGUMENT),
    (dict(kvpp=3), moba.MOBA_ERR_INVALID_ARGUMENT),  # more than the 2 KV heads
]

FAKE = 1 << 20  # a non-NULL, aligned address that is never dereferenced: every case fails first


@pytest.mark.parametrize("kw,code", BAD)
def test_invalid_problems_rejected_before_any_hip_call(kw, code):
    lib = moba.load_library()
    p = _prob(**kw)
    assert lib.moba_workspace_size(ctypes.byref(p)) == 0
    assert lib.moba_select_workspace_size(ctypes.byref(p)) == 0
    st = lib.moba_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code
    assert lib.moba_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == code
    if not ({"block_size", "topk"} & set(kw)) and "N" not in kw or kw.get("N") == 0:
        # the dense baseline ignores block_size and topk
        assert lib.moba_dense_causal(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == code
    assert lib.moba_last_error()


def test_null_problem():
    lib = moba.load_library()
    assert lib.moba_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert lib.moba_workspace_size(None) == 0


@pytest.mark.parametrize("which", range(4))
def test_null_and_misaligned_tensors(which):
    lib = moba.load_library()
    p = _prob()
    ws = lib.moba_workspace_size(ctypes.byref(p))
    for bad in (None, FAKE + 2):
        ptrs = [FAKE] * 4
        ptrs[which] = bad
        assert lib.moba_prefill(ctypes.byref(p), *ptrs, FAKE, ws, None) == 1


def test_workspace_checks():
    lib = moba.load_library()
    p = _prob()
    ws = lib.moba_workspace_size(ctypes.byref(p))
    assert ws > 0 and ws % 256 == 0
    assert lib.moba_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == 3
    assert lib.moba_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, ws, None) == 1
    assert lib.moba_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE + 16, ws, None) == 1
    sws = lib.moba_select_workspace_size(ctypes.byref(p))
    assert 0 < sws < ws
    assert lib.moba_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, sws - 1, None) == 3


def test_workspace_scales_with_history_slots():
    """The partial buffers dominate: (k-1) slots of d fp16 values (+ one fp32) per (row, head)."""
    lib = moba.load_library()
    a = lib.moba_workspace_size(ctypes.byref(_prob(topk=3)))
    b = lib.moba_workspace_size(ctypes.byref(_prob(topk=5)))
    per_slot = 4096 * 8 * (128 * 2 + 4)
    assert per_slot * 2 <= b - a <= per_slot * 2 + 4096 * 8 * 2 * 4 * 2 + 4096 * 64


def test_copy_rejects_bad_arguments():
    lib = moba.load_library()
    assert lib.moba_debug_copy(None, FAKE, 16, None) == 1
    assert lib.moba_debug_copy(FAKE, FAKE, 15, None) == 1


def test_read_probe_rejects_bad_arguments():
    lib = moba.load_library()
    assert lib.moba_debug_read_peak(None, 16, 1, FAKE, None) == 1
    assert lib.moba_debug_read_peak(FAKE, 16, 1, None, None) == 1
    assert lib.moba_debug_read_peak(FAKE, 15, 1, FAKE, None) == 1
    assert lib.moba_debug_read_peak(FAKE + 4, 16, 1, FAKE, None) == 1
    assert lib.moba_debug_read_peak(FAKE, 16, 0, FAKE, None) == 1
    assert lib.moba_debug_read_peak(FAKE, 16, (1 << 20) + 1, FAKE, None) == 1


def test_mfma_probe_rejects_bad_arguments():
    lib = moba.load_library()
    assert lib.moba_debug_mfma_peak(1, 1, None, None) == 1
    assert lib.moba_debug_mfma_peak(0, 1, FAKE, None) == 1
    assert lib.moba_debug_mfma_peak(1, 0, FAKE, None) == 1
    assert lib.moba_debug_mfma_peak((1 << 20) + 1, 1, FAKE, None) == 1
    assert lib.moba_debug_mfma_peak(1, (1 << 20) + 1, FAKE, None) == 1


def _cu(*xs):
    return (ctypes.c_int64 * len(xs))(*xs)


VARLEN_BAD = [
    # (nseq, cu values, seqlen, expected status)
    (2, (1, 100, 4096), 4096, moba.MOBA_ERR_INVALID_ARGUMENT),    # cu[0] != 0
    (2, (0, 3000, 2000), 2000, moba.MOBA_ERR_INVALID_ARGUMENT),   # decreasing
    (2, (0, 100, 4000), 4096, moba.MOBA_ERR_INVALID_ARGUMENT),    # cu[nseq] != seqlen
    (0, (0,), 4096, moba.MOBA_ERR_INVALID_ARGUMENT),              # no sequence
    # one long sequence past the history-block limit of the whole batch
    (2, (0, 1 << 20, (1 << 20) + 64), (1 << 20) + 64, moba.MOBA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("nseq,cu,N,code", VARLEN_BAD)
def test_varlen_rejects_bad_offsets_before_any_hip_call(nseq, cu, N, code):
    lib = moba.load_library()
    bs = 64 if code == moba.MOBA_ERR_UNSUPPORTED else 256
    p = _prob(N=N, block_size=bs)
    c = _cu(*cu)
    assert lib.moba_varlen_workspace_size(ctypes.byref(p), nseq, c) == 0
    assert lib.moba_varlen_select_workspace_size(ctypes.byref(p), nseq, c) == 0
    st = lib.moba_prefill_varlen(ctypes.byref(p), nseq, c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 40, None)
    assert st == code
    assert lib.moba_select_varlen(ctypes.byref(p), nseq, c, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                  None) == code


def test_varlen_null_offsets_and_pointers():
    lib = moba.load_library()
    p = _prob(N=1000)
    c = _cu(0, 300, 300, 1000)
    ws = lib.moba_varlen_workspace_size(ctypes.byref(p), 3, c)
    assert ws > 0 and ws % 256 == 0
    args = [FAKE] * 5  # cu_dev, q, k, v, o
    assert lib.moba_prefill_varlen(ctypes.byref(p), 3, None, *args, FAKE, ws, None) == 1
    for i in range(5):
        for bad in (None, FAKE + 4):
            a = list(args)
            a[i] = bad
            assert lib.moba_prefill_varlen(ctypes.byref(p), 3, c, *a, FAKE, ws, None) == 1
    assert lib.moba_prefill_varlen(ctypes.byref(p), 3, c, *args, FAKE, ws - 1, None) == 3


def test_varlen_one_sequence_sizes_match_plain():
    """One packed sequence is the plain problem: the same workspace."""
    lib = moba.load_library()
    p = _prob(N=5000)
    c = _cu(0, 5000)
    assert lib.moba_varlen_workspace_size(ctypes.byref(p), 1, c) == lib.moba_workspace_size(
        ctypes.byref(p))
    assert lib.moba_varlen_select_workspace_size(ctypes.byref(p), 1, c) == \
        lib.moba_select_workspace_size(ctypes.byref(p))


def test_varlen_blocks_restart_per_sequence():
    """Blocks restart at each sequence: two sequences of 300 rows with B=256 have
    4 blocks (two of them partial), one sequence of 600 rows has 3."""
    lib = moba.load_library()
    p1 = _prob(N=600, Hq=1, Hkv=1, block_size=256, topk=3)
    assert lib.moba_debug_bucket_capacity(ctypes.byref(p1)) == 256 * 1 + 88 * 2
    a = lib.moba_varlen_workspace_size(ctypes.byref(p1), 2, _cu(0, 300, 600))
    b = lib.moba_workspace_size(ctypes.byref(p1))
    assert a > 0 and b > 0 and a != b
    # empty sequences add no block
    assert lib.moba_varlen_workspace_size(ctypes.byref(p1), 4, _cu(0, 0, 300, 300, 600)) == a


def test_chunk_rejects_bad_row_counts():
    lib = moba.load_library()
    p = _prob(N=1000)
    for bad in (0, -1, 1001):
        assert lib.moba_chunk_workspace_size(ctypes.byref(p), bad) == 0
        assert lib.moba_prefill_chunk(ctypes.byref(p), bad, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                      None) == 1
    ws = lib.moba_chunk_workspace_size(ctypes.byref(p), 1000)
    assert ws == lib.moba_workspace_size(ctypes.byref(p))  # all rows: the plain problem
    small = lib.moba_chunk_workspace_size(ctypes.byref(p), 1)
    assert 0 < small < ws
    assert lib.moba_prefill_chunk(ctypes.byref(p), 1, FAKE, FAKE, FAKE, FAKE, FAKE, small - 1,
                                  None) == 3


def test_cache_sizes():
    lib = moba.load_library()
    p = _prob(N=1000, block_size=256)
    a = lib.moba_cache_bytes(ctypes.byref(p), 1000)
    b = lib.moba_cache_bytes(ctypes.byref(p), 5000)
    assert 0 < a < b
    assert lib.moba_cache_bytes(ctypes.byref(p), 0) == 0
    # fp64 means of ceil(cap/B) - 1 blocks + bf16 V^T of ceil(cap/B) padded blocks
    n = -(-5000 // 256)
    expect = 8 * 2 * (n - 1) * 128 + 2 * 2 * 128 * n * 256
    assert expect <= b <= expect + 2 * 256
    f32 = lib.moba_cache_bytes(ctypes.byref(_prob(N=1000, block_size=256, dtype=1)), 5000)
    assert f32 < b  # no packed V for fp32
    cw = lib.moba_cached_workspace_size(ctypes.byref(p), 1)
    assert 0 < cw < lib.moba_chunk_workspace_size(ctypes.byref(p), 1)


def test_cache_append_rejects_bad_arguments():
    lib = moba.load_library()
    p = _prob(N=1000)
    assert lib.moba_cache_append(ctypes.byref(p), 999, 0, FAKE, FAKE, FAKE, None) == 1  # capacity
    assert lib.moba_cache_append(ctypes.byref(p), 2000, 1001, FAKE, FAKE, FAKE, None) == 1
    assert lib.moba_cache_append(ctypes.byref(p), 2000, -1, FAKE, FAKE, FAKE, None) == 1
    for i in range(3):
        ptrs = [FAKE, FAKE, FAKE]
        ptrs[i] = None
        assert lib.moba_cache_append(ctypes.byref(p), 2000, 0, *ptrs, None) == 1
    assert lib.moba_cache_append(ctypes.byref(p), 2000, 0, FAKE, FAKE, FAKE + 16, None) == 1


def test_prefill_cached_rejects_bad_arguments():
    lib = moba.load_library()
    p = _prob(N=1000)
    ws = lib.moba_cached_workspace_size(ctypes.byref(p), 4)
    args = lambda cap, rows, cache, n: (ctypes.byref(p), cap, rows, FAKE, FAKE, FAKE, cache, FAKE,
                                        FAKE, n, None)
    assert lib.moba_prefill_cached(*args(999, 4, FAKE, ws)) == 1          # capacity < seqlen
    assert lib.moba_prefill_cached(*args(2000, 0, FAKE, ws)) == 1         # q_rows
    assert lib.moba_prefill_cached(*args(2000, 1001, FAKE, ws)) == 1
    assert lib.moba_prefill_cached(*args(2000, 4, None, ws)) == 1         # cache
    assert lib.moba_prefill_cached(*args(2000, 4, FAKE + 16, ws)) == 1    # misaligned cache
    assert lib.moba_prefill_cached(*args(2000, 4, FAKE, ws - 1)) == 3     # workspace


def test_varlen_training_rejects_bad_arguments():
    lib = moba.load_library()
    p = _prob(N=1000)
    cu = _cu(0, 400, 1000)
    assert lib.moba_backward_varlen_workspace_size(ctypes.byref(p), 2, cu) > 0
    assert lib.moba_backward_varlen_workspace_size(ctypes.byref(p), 2, _cu(0, 400, 999)) == 0
    ws = lib.moba_backward_varlen_workspace_size(ctypes.byref(p), 2, cu)
    # one packed sequence needs the same workspace as the plain backward
    assert lib.moba_backward_varlen_workspace_size(ctypes.byref(p), 1, _cu(0, 1000)) == \
        lib.moba_backward_workspace_size(ctypes.byref(p))
    f = [FAKE] * 9
    assert lib.moba_backward_varlen(ctypes.byref(p), 2, cu, None, *f, FAKE, ws, None) == 1
    assert lib.moba_backward_varlen(ctypes.byref(p), 2, _cu(0, 1001, 1000), FAKE, *f, FAKE, ws,
                                    None) == 1
    f2 = list(f)
    f2[6] = None  # dq
    assert lib.moba_backward_varlen(ctypes.byref(p), 2, cu, FAKE, *f2, FAKE, ws, None) == 1
    assert lib.moba_backward_varlen(ctypes.byref(p), 2, cu, FAKE, *f, FAKE, ws - 1, None) == 3
    assert lib.moba_prefill_train_varlen(ctypes.byref(p), 2, cu, None, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, 1 << 40, None) == 1
    assert lib.moba_prefill_train_varlen(ctypes.byref(p), 2, cu, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         None, FAKE, 1 << 40, None) == 1


def test_packed_v_extent_limit():
    """bf16 problems are accepted up to the 32-bit offset range of the packed
    V^T rows (ceil(N/B) * ceil(B/64) * 64 < 16,909,320) and refused past it;
    fp32 problems do not read the packed copy and keep the larger range."""
    lib = moba.load_library()
    ok = _prob(N=16_777_216, Hq=1, Hkv=1, block_size=4096, topk=2)
    assert lib.moba_workspace_size(ctypes.byref(ok)) > 0
    big = _prob(N=16_912_384, Hq=1, Hkv=1, block_size=4096, topk=2)
    assert lib.moba_workspace_size(ctypes.byref(big)) == 0
    assert lib.moba_prefill(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 2
    assert b"16,909,320" in lib.moba_last_error()
    big32 = _prob(N=16_912_384, Hq=1, Hkv=1, block_size=4096, topk=2, dtype=1)
    assert lib.moba_workspace_size(ctypes.byref(big32)) > 0
    # the decode cache's capacity is held to the same limit
    small = _prob(N=4096, Hq=1, Hkv=1, block_size=4096, topk=2)
    assert lib.moba_cache_bytes(ctypes.byref(small), 16_777_216) > 0
    assert lib.moba_cache_bytes(ctypes.byref(small), 16_912_384) == 0


def test_noalloc_refuses_problems_beyond_its_scratch():
    """The allocation-free entry point checks the workspace its problem needs
    against its fixed scratch array before any HIP call."""
    lib = moba.load_library()
    assert lib.moba_noalloc_max_workspace() == 512 << 20
    big = _prob(N=1 << 20, Hq=32, Hkv=8, block_size=4096, topk=12)
    assert lib.moba_workspace_size(ctypes.byref(big)) > lib.moba_noalloc_max_workspace()
    assert lib.moba_prefill_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None) == 2
    assert b"512 MiB" in lib.moba_last_error()
    bad = _prob(N=0)
    assert lib.moba_prefill_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moba_prefill_noalloc(ctypes.byref(_prob()), FAKE, None, FAKE, FAKE, None) == 1


def test_attention_passes_cap_the_workspace():
    """History partials are held for one attention pass (group of KV heads)
    at a time: on the 1M-token 32/8-head k = 12 layer the library's choice is
    one KV head per pass, eight passes, and the workspace stays under 20 GB
    where one pass over all heads needs over 94 GiB of partials."""
    lib = moba.load_library()
    layer = dict(N=1 << 20, Hq=32, Hkv=8, block_size=4096, topk=12)
    auto = _prob(**layer)
    one = _prob(kvpp=1, **layer)
    whole = _prob(kvpp=8, **layer)
    ws_auto = lib.moba_workspace_size(ctypes.byref(auto))
    assert ws_auto == lib.moba_workspace_size(ctypes.byref(one))
    assert 0 < ws_auto < 20e9
    assert lib.moba_workspace_size(ctypes.byref(whole)) > 94 * 2**30
    assert lib.moba_stage_events(ctypes.byref(auto)) == 5 + 2 * 8
    assert lib.moba_stage_events(ctypes.byref(whole)) == 7
    assert lib.moba_stage_events(ctypes.byref(_prob(kvpp=3, **layer))) == 5 + 2 * 3
    assert lib.moba_stage_events(ctypes.byref(_prob(kvpp=9, **layer))) == 0
    # small problems keep one pass; the partials shrink with the pass size
    assert lib.moba_stage_events(ctypes.byref(_prob())) == 7
    per_kv = 4096 * 4 * 2 * (128 * 2 + 4)  # rows x G x (k-1) slots x (fp16 d + fp32)
    full = lib.moba_workspace_size(ctypes.byref(_prob(kvpp=2)))
    half = lib.moba_workspace_size(ctypes.byref(_prob(kvpp=1)))
    assert full - half == per_kv


def test_value_range_limit_is_documented():
    """The bf16 path keeps normalised partial rows in fp16: the header states
    the resulting bound on |V| (the GPU suite checks values just below it)."""
    text = open(os.path.join(ROOT, "include", "moba.h")).read()
    assert "|V| must stay below 65504" in text
