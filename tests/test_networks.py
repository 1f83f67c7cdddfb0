"""The gate's sorting networks, checked on the host.

gate_topk.hip sorts each chunk's 16 candidate keys (and a row's kept block
indices) with the compare-exchange list kOddEven16. By the 0-1 principle a
comparator network sorts every input if it sorts every input of zeros and
ones, so all 2^16 such inputs are run through the list as written in the
source.
"""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(__file__), "..", "block_sparse_long_meanpool_amd", "csrc",
                   "gate_topk.hip")


def _network():
    text = open(SRC).read()
    m = re.search(r"kOddEven16\[63\]\[2\]\s*=\s*\{(.*?)\};", text, re.S)
    assert m, "kOddEven16 not found"
    pairs = [(int(a), int(b)) for a, b in re.findall(r"\{\s*(\d+)\s*,\s*(\d+)\s*\}", m.group(1))]
    assert len(pairs) == 63
    return pairs


def test_odd_even_16_sorts_every_zero_one_input():
    pairs = _network()
    x = np.arange(1 << 16, dtype=np.uint32)
    a = ((x[:, None] >> np.arange(16, dtype=np.uint32)) & 1).astype(np.uint8)
    for i, j in pairs:
        assert 0 <= i < j < 16
        hi = np.maximum(a[:, i], a[:, j])
        lo = np.minimum(a[:, i], a[:, j])
        a[:, i], a[:, j] = hi, lo
    assert np.all(a[:, :-1] >= a[:, 1:])  # descending for push16
    # the ascending use (kept indices) is the same network with min and max swapped


def test_odd_even_16_on_random_keys_matches_sort():
    pairs = _network()
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2**32, size=(4096, 16), dtype=np.uint64)
    ref = -np.sort(-a.astype(np.int64), axis=1)
    for i, j in pairs:
        hi = np.maximum(a[:, i], a[:, j])
        lo = np.minimum(a[:, i], a[:, j])
        a[:, i], a[:, j] = hi, lo
    assert np.array_equal(a.astype(np.int64), ref)
