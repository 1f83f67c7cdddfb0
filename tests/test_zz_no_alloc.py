"""The allocation-free prefill entry point against moba_prefill, through the
C ABI: same kernels, so the outputs must be bit-identical; two calls in a row
share the library's scratch array, the second on a smaller problem."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_long_meanpool_amd as moba
import oracle
from tests._gpu import DEV, compare_rows, to_dev, to_np
import synth

pytestmark = pytest.mark.gpu


def _noalloc(lib, q, k, v, B, topk, scale, out):
    p = moba.make_problem(q.shape[0], q.shape[1], k.shape[1], q.shape[2], B, topk, scale,
                          moba.MOBA_DTYPE_BF16 if q.dtype == torch.bfloat16 else moba.MOBA_DTYPE_F32)
    st = lib.moba_prefill_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), torch.cuda.current_stream(q.device).cuda_stream)
    assert st == moba.MOBA_OK, lib.moba_last_error()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_prefill_twice(dtype):
    lib = moba.load_library()
    assert lib.moba_noalloc_max_workspace() == 512 << 20
    cases = [(6000, 8, 2, 256, 4, 11), (1500, 4, 4, 128, 3, 12)]  # the second smaller
    for N, Hq, Hkv, B, topk, seed in cases:
        q, k, v = synth.random_qkv(N, Hq, Hkv, 128, seed, dtype=dtype)
        tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
        scale = 0.09
        # garbage in the output buffer: the call must overwrite all of it
        out = torch.full_like(tq, 7.0)
        _noalloc(lib, tq, tk, tv, B, topk, scale, out)
        ref = moba.prefill(tq, tk, tv, B, topk, scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"N={N}: allocation-free output differs from moba_prefill"
        # and against the oracle on a sample of rows
        rng = np.random.default_rng(seed)
        rows = rng.integers(0, N, size=256)
        heads = rng.integers(0, Hq, size=256).astype(np.int32)
        sel = moba.select(tq, tk, B, topk).cpu().numpy()
        compare_rows(q, k, v, B, topk, scale, rows, heads, sel[rows, heads],
                     to_np(out)[rows, heads], dtype, f"noalloc N={N}")


def test_noalloc_binding_and_limit():
    lib = moba.load_library()
    q, k, v = synth.random_qkv(700, 2, 1, 128, 5)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o1 = moba.prefill_noalloc(tq, tk, tv, 64, 3, 0.1)
    o2 = moba.prefill(tq, tk, tv, 64, 3, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    # a problem whose workspace exceeds the scratch array is refused
    p = moba.make_problem(1 << 20, 32, 8, 128, 4096, 12, 0.088, moba.MOBA_DTYPE_BF16)
    assert lib.moba_workspace_size(ctypes.byref(p)) > lib.moba_noalloc_max_workspace()
    st = lib.moba_prefill_noalloc(ctypes.byref(p), tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                                  o1.data_ptr(), None)
    assert st == moba.MOBA_ERR_UNSUPPORTED
