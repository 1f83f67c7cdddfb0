"""Pins for the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, a library routine (torch's fp64 CPU attention) for
the special cases that reduce to it, an exact brute-force enumeration, and
invariants of the definition. Citations name the PaperTrace page "2.1.3 MoBA"
(yayajjiang.github.io) unless stated otherwise.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa_rows(q, k, v, mask, scale):
    """torch fp64 CPU attention with an explicit boolean mask [Hq, N, N]."""
    N, Hq, d = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=torch.from_numpy(mask),
        scale=scale)
    return o.permute(1, 0, 2).numpy()


def _f32(x):
    return np.asarray(x, np.float32)


# ---------------------------------------------------------------- P1, P2 ---
def _worked_inputs(x=7.0, y=-3.0, a=-5.0, b=8.0):
    g = _load("worked_example.json")
    keys = [x if t is None else t for t in g["keys"]]
    vals = list(g["values"])
    vals[0], vals[1], vals[5] = a, b, y
    N = g["N"]
    q = _f32(np.full((N, 1, 1), g["q_row"]))
    return g, q, _f32(keys).reshape(N, 1, 1), _f32(vals).reshape(N, 1, 1)


def test_p1_worked_example_matches_printed_numbers():
    """Section 2 worked example: selection, weights and output as printed."""
    g, q, k, v = _worked_inputs()
    pr = g["printed"]
    sel, o, _ = oracle.rows(q, k, v, g["B"], g["k"], [g["row"]], [0], scale=g["scale"])
    assert list(sel[0]) == pr["selected_blocks"]
    tol = 0.5 * 10 ** -pr["printed_decimals"]
    assert abs(o[0, 0] - pr["output"]) <= tol
    # block scores as printed (means 1 and 3)
    kb = oracle.block_means(k, g["B"])
    assert list(kb[0, :2, 0]) == pr["block_scores"]
    # the printed weights: recover them from the oracle by one-hot values
    w = []
    for r in pr["candidate_rows"]:
        onehot = np.zeros_like(v)
        onehot[r] = 1.0
        w.append(oracle.rows(q, k, onehot, g["B"], g["k"], [g["row"]], [0], scale=1.0)[1][0, 0])
    assert np.allclose(w, pr["weights"], atol=tol, rtol=0)
    assert abs(sum(w) - 1.0) < 1e-15
    # closed form: common denominator 1 + e^-2 + e^-3 after subtracting the max logit 4
    den = 1 + math.exp(-2) + math.exp(-3)
    assert abs(o[0, 0] - (10 + 20 * math.exp(-2) + 30 * math.exp(-3)) / den) < 1e-12


@pytest.mark.parametrize("x,y,a,b", [(100.0, 5.0, 0.0, 0.0), (-50.0, 1e3, 77.0, -9.0)])
def test_p1_invariant_to_unseen_entries(x, y, a, b):
    """The future key/value of the own block and the unselected block never matter."""
    g, q, k, v = _worked_inputs(x, y, a, b)
    _, o, _ = oracle.rows(q, k, v, g["B"], g["k"], [g["row"]], [0], scale=1.0)
    assert abs(o[0, 0] - 11.982153) < 1e-6


def test_p2_naive_sum_differs():
    """Section 2: adding separately normalised branches is wrong (41.19 vs 11.98)."""
    g, q, k, v = _worked_inputs()
    _, o_naive, _ = oracle.rows(q, k, v, 2, 2, [4], [0], scale=1.0, mode=oracle.MODE_NAIVE)
    hist = (10 + 20 * math.exp(-2)) / (1 + math.exp(-2))
    assert abs(o_naive[0, 0] - (hist + 30.0)) < 1e-12
    assert abs(o_naive[0, 0] - 41.192029) < 1e-6
    _, o, _ = oracle.rows(q, k, v, 2, 2, [4], [0], scale=1.0)
    assert abs(o_naive[0, 0] - o[0, 0]) > 29


def test_p2_naive_differs_on_random_rows_with_history():
    q, k, v = synth.random_qkv(64, 2, 1, 8, seed=11)
    r, h = oracle.all_rows(64, 2)
    sel, o, _ = oracle.rows(q, k, v, 8, 3, r, h)
    _, on, _ = oracle.rows(q, k, v, 8, 3, r, h, mode=oracle.MODE_NAIVE)
    has_hist = r >= 8
    diff = np.abs(on - o).max(axis=1)
    assert np.all(diff[has_hist] > 1e-3)
    assert np.all(diff[~has_hist] < 1e-14)


# ---------------------------------------------------------------- P3, P5 ---
def _causal_mask(N, Hq):
    m = np.tril(np.ones((N, N), bool))
    return np.broadcast_to(m, (Hq, N, N)).copy()


@pytest.mark.parametrize("N,Hq,Hkv,d,B,k", [(40, 2, 1, 8, 8, 5), (33, 4, 2, 16, 4, 9),
                                              (24, 1, 1, 4, 32, 1), (50, 3, 3, 8, 7, 8)])
def test_p3_full_attention_when_k_covers_all_blocks(N, Hq, Hkv, d, B, k):
    """Section 4: when k covers every legal block, MoBA is causal full attention."""
    assert k * B >= N
    q, kk, v = synth.random_qkv(N, Hq, Hkv, d, seed=N * 7 + k)
    scale = 0.37
    sel, o = oracle.prefill(q, kk, v, B, k, scale=scale)
    ref = _sdpa_rows(q, kk, v, _causal_mask(N, Hq), scale)
    assert np.max(np.abs(o - ref)) < 1e-12
    r, h = oracle.all_rows(N, Hq)
    o2 = oracle.causal_full(q, kk, v, r, h, scale=scale).reshape(N, Hq, d)
    assert np.max(np.abs(o2 - ref)) < 1e-12


def test_p5_block_size_one_is_token_topk():
    """B = 1: each query keeps its own token and the k-1 best earlier tokens by q.k."""
    N, d, k = 14, 4, 4
    q, kk, v = synth.random_qkv(N, 1, 1, d, seed=5)
    sel, o = oracle.prefill(q, kk, v, 1, k, scale=1.0)
    for p in range(N):
        s = [float(np.dot(q[p, 0].astype(np.float64), kk[j, 0].astype(np.float64))) for j in range(p)]
        order = sorted(range(p), key=lambda j: (-s[j], j))[: k - 1]
        keep = sorted(order) + [p]
        assert list(sel[p, 0, : len(keep)]) == keep
        z = np.array([np.dot(q[p, 0].astype(np.float64), kk[j, 0].astype(np.float64)) for j in keep])
        w = np.exp(z - z.max())
        w /= w.sum()
        ref = (w[:, None] * v[keep, 0].astype(np.float64)).sum(0)
        assert np.max(np.abs(o[p, 0] - ref)) < 1e-13


def test_p5_k_one_is_block_diagonal_causal():
    """k = 1: only the own block, causally — block-diagonal causal attention."""
    N, Hq, Hkv, d, B = 45, 2, 1, 8, 6
    q, kk, v = synth.random_qkv(N, Hq, Hkv, d, seed=3)
    sel, o = oracle.prefill(q, kk, v, B, 1, scale=0.5)
    blk = np.arange(N) // B
    m = np.tril(np.ones((N, N), bool)) & (blk[:, None] == blk[None, :])
    ref = _sdpa_rows(q, kk, v, np.broadcast_to(m, (Hq, N, N)).copy(), 0.5)
    assert np.max(np.abs(o - ref)) < 1e-12
    assert np.all(sel[:, :, 0] == blk[:, None])


def test_p5_block_covers_sequence_is_causal_full():
    N, d = 30, 8
    q, kk, v = synth.random_qkv(N, 2, 2, d, seed=4)
    _, o = oracle.prefill(q, kk, v, 64, 3, scale=0.3)
    ref = _sdpa_rows(q, kk, v, _causal_mask(N, 2), 0.3)
    assert np.max(np.abs(o - ref)) < 1e-12


# ---------------------------------------------------------------------- P4 ---
def _brute(q, k, v, B, topk, scale, shared=False):
    """Exact enumeration: every candidate set, Fractions for the gate, loops for attention.
    shared: the gate query is the sum of the head group's queries."""
    N, Hq, d = q.shape
    G = Hq // k.shape[1]
    sel_all, o_all = [], []
    for p in range(N):
        for h in range(Hq):
            g = h // G
            c = p // B
            if shared:
                qf = [sum(Fraction(float(q[p, g * G + hh, t])) for hh in range(G)) for t in range(d)]
            else:
                qf = [Fraction(float(x)) for x in q[p, h]]
            scores = []
            for i in range(c):
                mean = [sum(Fraction(float(k[j, g, t])) for j in range(i * B, (i + 1) * B)) / B
                        for t in range(d)]
                scores.append(sum(a * b for a, b in zip(qf, mean)))
            m = min(topk - 1, c)
            best, best_sum = None, None
            for combo in itertools.combinations(range(c), m):
                ssum = sum((scores[i] for i in combo), Fraction(0))
                if best is None or ssum > best_sum or (ssum == best_sum and combo < best):
                    best, best_sum = combo, ssum
            keys = [j for i in best for j in range(i * B, (i + 1) * B)]
            keys += list(range(c * B, p + 1))
            z = []
            for j in keys:
                z.append(scale * sum(float(q[p, h, t]) * float(k[j, g, t]) for t in range(d)))
            mx = max(z)
            w = [math.exp(x - mx) for x in z]
            den = sum(w)
            o = [sum(w[i] * float(v[j, g, t]) for i, j in enumerate(keys)) / den for t in range(d)]
            sel_all.append(list(best) + [c] + [-1] * (topk - m - 1))
            o_all.append(o)
    return np.array(sel_all), np.array(o_all)


@pytest.mark.parametrize("case", range(10))
def test_p4_brute_force(case):
    rng = np.random.default_rng(100 + case)
    B = int(rng.integers(1, 5))
    N = int(rng.integers(2, 17 if B == 1 else 33))
    topk = int(rng.integers(1, 6))
    d = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    integer = case % 2 == 0  # integer keys force exact gate ties
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=case, integer=integer)
    scale = float(rng.uniform(0.2, 1.5))
    sel, o = oracle.prefill(q, k, v, B, topk, scale=scale)
    bsel, bo = _brute(q, k, v, B, topk, scale)
    assert np.array_equal(sel.reshape(-1, topk), bsel)
    assert np.max(np.abs(o.reshape(-1, d) - bo)) < 1e-12


# ------------------------------------------------------- GQA shared routing ---
@pytest.mark.parametrize("case", range(6))
def test_shared_routing_brute_force(case):
    """One ranking per head group by the summed gate score (enumerated exactly)."""
    rng = np.random.default_rng(700 + case)
    B = int(rng.integers(1, 4))
    N = int(rng.integers(4, 25))
    topk = int(rng.integers(2, 5))
    d = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(2, 4))
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=70 + case, integer=case % 2 == 0)
    scale = float(rng.uniform(0.2, 1.5))
    sel, o = oracle.prefill(q, k, v, B, topk, scale=scale, routing=oracle.ROUTING_SHARED)
    bsel, bo = _brute(q, k, v, B, topk, scale, shared=True)
    assert np.array_equal(sel.reshape(-1, topk), bsel)
    assert np.max(np.abs(o.reshape(-1, d) - bo)) < 1e-12
    G = Hq // Hkv
    for g in range(Hkv):  # every head of a group holds the same selection
        assert np.all(sel[:, g * G:(g + 1) * G] == sel[:, g * G:g * G + 1])


def test_shared_routing_reduces_to_per_head():
    """Groups of one head, or groups whose heads share one query, rank as per head."""
    q, k, v = synth.random_qkv(96, 3, 3, 16, seed=4)
    a = oracle.prefill(q, k, v, 8, 4)
    b = oracle.prefill(q, k, v, 8, 4, routing=oracle.ROUTING_SHARED)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q1, k1, v1 = synth.random_qkv(96, 4, 1, 16, seed=6)
    q1[:] = q1[:, :1]  # the four heads of the group carry the same query
    a = oracle.prefill(q1, k1, v1, 8, 4)
    b = oracle.prefill(q1, k1, v1, 8, 4, routing=oracle.ROUTING_SHARED)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------ packed (varlen) ---
def _brute_packed(q, k, v, cu, B, topk, scale):
    """Packed rows without slicing: each row's blocks are counted from its own
    sequence's first row, and only rows of that sequence are candidates."""
    N, Hq, d = q.shape
    G = Hq // k.shape[1]
    sel_all, o_all = [], []
    for p in range(N):
        s = max(i for i in range(len(cu) - 1) if cu[i] <= p < cu[i + 1])
        a = cu[s]
        c = (p - a) // B
        for h in range(Hq):
            g = h // G
            qf = [Fraction(float(x)) for x in q[p, h]]
            scores = []
            for i in range(c):
                rows_i = range(a + i * B, a + (i + 1) * B)
                mean = [sum(Fraction(float(k[j, g, t])) for j in rows_i) / B for t in range(d)]
                scores.append(sum(x * y for x, y in zip(qf, mean)))
            m = min(topk - 1, c)
            best, best_sum = None, None
            for combo in itertools.combinations(range(c), m):
                ssum = sum((scores[i] for i in combo), Fraction(0))
                if best is None or ssum > best_sum or (ssum == best_sum and combo < best):
                    best, best_sum = combo, ssum
            keys = [j for i in best for j in range(a + i * B, a + (i + 1) * B)]
            keys += list(range(a + c * B, p + 1))
            z = [scale * sum(float(q[p, h, t]) * float(k[j, g, t]) for t in range(d)) for j in keys]
            mx = max(z)
            w = [math.exp(x - mx) for x in z]
            den = sum(w)
            o_all.append([sum(w[i] * float(v[j, g, t]) for i, j in enumerate(keys)) / den
                          for t in range(d)])
            sel_all.append(list(best) + [c] + [-1] * (topk - m - 1))
    return np.array(sel_all), np.array(o_all)


@pytest.mark.parametrize("case", range(6))
def test_packed_brute_force(case):
    """Packed sequences (with empty and one-row ones) against the unsliced enumeration."""
    rng = np.random.default_rng(500 + case)
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(0, 12, size=int(rng.integers(1, 5)))]
    lens[0] = max(lens[0], 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = int(cu[-1])
    topk = int(rng.integers(1, 5))
    d = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=50 + case, integer=case % 2 == 0)
    scale = float(rng.uniform(0.2, 1.5))
    sel, o = oracle.prefill_varlen(q, k, v, cu, B, topk, scale=scale)
    bsel, bo = _brute_packed(q, k, v, [int(x) for x in cu], B, topk, scale)
    assert np.array_equal(sel.reshape(-1, topk), bsel)
    assert np.max(np.abs(o.reshape(-1, d) - bo)) < 1e-12


def test_packed_short_sequences_are_causal_attention():
    """Sequences no longer than B are one block each: plain causal attention
    inside each sequence (the independent causal_full routine on each slice)."""
    B, topk, d = 16, 3, 8
    cu = np.array([0, 5, 16, 16, 23, 39], np.int64)
    N = int(cu[-1])
    q, k, v = synth.random_qkv(N, 4, 2, d, seed=77)
    sel, o = oracle.prefill_varlen(q, k, v, cu, B, topk, scale=0.4)
    assert np.all(sel[:, :, 0] == 0) and np.all(sel[:, :, 1:] == -1)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        r, h = oracle.all_rows(b - a, 4)
        ref = oracle.causal_full(q[a:b], k[a:b], v[a:b], r, h, scale=0.4)
        assert np.max(np.abs(o[a:b].reshape(-1, d) - ref)) < 1e-12


def test_packed_sequences_do_not_leak():
    """Changing one sequence's tokens leaves every other sequence's output bit-identical."""
    B, topk, d = 4, 3, 8
    cu = np.array([0, 13, 30, 41], np.int64)
    q, k, v = synth.random_qkv(41, 2, 1, d, seed=5)
    sel, o = oracle.prefill_varlen(q, k, v, cu, B, topk)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    k2[13:30] *= -3.0
    v2[13:30] += 1.0
    q2[13:30] = q2[13:30][::-1]
    sel2, o2 = oracle.prefill_varlen(q2, k2, v2, cu, B, topk)
    for a, b in ((0, 13), (30, 41)):
        assert np.array_equal(sel[a:b], sel2[a:b])
        assert np.array_equal(o[a:b], o2[a:b])
    assert not np.array_equal(o[13:30], o2[13:30])


# ---------------------------------------------------------------------- P6 ---
def test_p6_zero_keys_tie_to_lowest_blocks():
    """K == 0: every score and logit ties; the lowest blocks win and O is a plain mean."""
    N, Hq, d, B, topk = 40, 2, 8, 4, 4
    q, _, v = synth.random_qkv(N, Hq, 1, d, seed=9)
    k = np.zeros((N, 1, d), np.float32)
    sel, o = oracle.prefill(q, k, v, B, topk)
    for p in range(N):
        c = p // B
        m = min(topk - 1, c)
        want = list(range(m)) + [c] + [-1] * (topk - m - 1)
        keys = list(range(m * B)) + list(range(c * B, p + 1))
        mean = v[keys, 0].astype(np.float64).mean(0)
        for h in range(Hq):
            assert list(sel[p, h]) == want
            assert np.max(np.abs(o[p, h] - mean)) < 1e-14


def test_p6_negative_zero_equals_positive_zero():
    N, d, B = 24, 4, 4
    q, _, v = synth.random_qkv(N, 1, 1, d, seed=2)
    k = np.zeros((N, 1, d), np.float32)
    k[: 2 * B] = -0.0  # blocks 0 and 1 hold -0.0, the rest +0.0
    sel, _ = oracle.prefill(q, k, v, B, 3)
    assert list(sel[N - 1, 0]) == [0, 1, 5]


# ---------------------------------------------------------------------- P7 ---
def test_p7_recency_gate_is_block_sliding_window():
    """Section 3: a gate that always prefers recent blocks yields a blocked window."""
    N, Hq, d, B, topk = 64, 2, 8, 8, 3
    rng = np.random.default_rng(7)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    k = rng.standard_normal((N, 1, d)) * 0.05
    k += (np.arange(N) // B)[:, None, None] * 2.0 * u[None, None, :]
    q = np.abs(rng.standard_normal((N, Hq, 1))) * u[None, None, :] + 0.0
    q, k = _f32(q), _f32(k)
    v = _f32(rng.standard_normal((N, 1, d)))
    sel, o = oracle.prefill(q, k, v, B, topk, scale=0.25)
    blk = np.arange(N) // B
    win = (blk[None, :] >= blk[:, None] - (topk - 1)) & (blk[None, :] <= blk[:, None])
    m = np.tril(np.ones((N, N), bool)) & win
    ref = _sdpa_rows(q, k, v, np.broadcast_to(m, (Hq, N, N)).copy(), 0.25)
    assert np.max(np.abs(o - ref)) < 1e-12
    for p in range(N):
        c = p // B
        hist = list(range(max(0, c - topk + 1), c))
        assert list(sel[p, 0, : len(hist) + 1]) == hist + [c]


# ---------------------------------------------------------------------- P8 ---
def test_p8_mean_dilution_routes_to_diffuse_block():
    """Section 5.2: one key scoring 8 in 256 averages to 0.03125 < 0.05."""
    g = _load("dilution.json")
    B = g["B"]
    N = 3 * B
    k = np.zeros((N, 1, 1), np.float32)
    k[0, 0, 0] = g["block_a"]["spike"]
    k[B: 2 * B, 0, 0] = g["block_b"]["all"]
    q = np.ones((N, 1, 1), np.float32)
    v = np.ones((N, 1, 1), np.float32)
    kb = oracle.block_means(k, B)
    assert kb[0, 0, 0] == g["printed"]["score_a"]
    assert abs(kb[0, 1, 0] - g["printed"]["score_b"]) < 1e-8
    sel, _, gap = oracle.rows(q, k, v, B, 2, [N - 1], [0])
    assert list(sel[0]) == [1, 2]
    assert gap[0, 0] > 0


# ---------------------------------------------------------------------- P9 ---
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p9_merge_identity(seed):
    """Eqs. (7)-(8) on the two branches equal the union softmax of eq. (4)."""
    q, k, v = synth.random_qkv(96, 4, 2, 16, seed=seed)
    r, h = oracle.all_rows(96, 4)
    _, o, _ = oracle.rows(q, k, v, 8, 4, r, h, scale=0.25)
    _, o2, _ = oracle.rows(q, k, v, 8, 4, r, h, scale=0.25, mode=oracle.MODE_TWO_BRANCH)
    assert np.max(np.abs(o - o2) / (np.abs(o) + 1e-300)) < 1e-11 or np.max(np.abs(o - o2)) < 1e-13


# --------------------------------------------------------------------- P10 ---
def test_p10_invariants():
    N, Hq, Hkv, d, B, topk = 80, 2, 1, 8, 8, 3
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=21)
    r, h = oracle.all_rows(N, Hq)
    sel, o, _ = oracle.rows(q, k, v, B, topk, r, h)
    # weights sum to one: V == 1 gives O == 1
    _, o1, _ = oracle.rows(q, k, np.ones_like(v), B, topk, r, h)
    assert np.max(np.abs(o1 - 1.0)) < 1e-14
    # O lies in the per-coordinate hull of V over the candidate set
    for i in range(len(r)):
        p, c = r[i], r[i] // B
        keys = [j for b in sel[i] if 0 <= b < c for j in range(b * B, (b + 1) * B)]
        keys += list(range(c * B, p + 1))
        vv = v[keys, 0].astype(np.float64)
        assert np.all(o[i] >= vv.min(0) - 1e-12) and np.all(o[i] <= vv.max(0) + 1e-12)
    # permuting tokens inside a history block changes nothing
    perm = np.arange(N)
    perm[8:16] = perm[8:16][::-1]
    _, op, _ = oracle.rows(q, k[perm], v[perm], B, topk, r, h)
    mask = r >= 16
    assert np.max(np.abs(op[mask] - o[mask])) < 1e-12
    # causality: rewriting every key/value after row p leaves row p alone
    p0 = 43
    k2, v2 = k.copy(), v.copy()
    k2[p0 + 1:] = 9.0
    v2[p0 + 1:] = -9.0
    _, o3, _ = oracle.rows(q, k2, v2, B, topk, r, h)
    early = r <= p0
    assert np.array_equal(o3[early], o[early])


def test_oracle_bf16_widening_is_exact():
    """bf16 inputs are widened exactly: same result as the float32 copy of the values."""
    q, k, v = synth.random_qkv(48, 2, 2, 8, seed=5, dtype="bf16")
    qf, kf, vf = (synth.bf16_to_f32(x) for x in (q, k, v))
    s1, o1 = oracle.prefill(q, k, v, 8, 3)
    s2, o2 = oracle.prefill(qf, kf, vf, 8, 3)
    assert np.array_equal(s1, s2) and np.array_equal(o1, o2)


def test_gap_reports_selection_margin():
    q, k, v = synth.random_qkv(64, 1, 1, 4, seed=8)
    r, h = oracle.all_rows(64, 1)
    sel, _, gap = oracle.rows(q, k, v, 4, 3, r, h, want_o=False)
    kb = oracle.block_means(k, 4)
    for i in range(64):
        c = r[i] // 4
        if c <= 2:
            assert np.isnan(gap[i, 0])
            continue
        s = kb[0, :c] @ q[r[i], 0].astype(np.float64)
        srt = np.sort(s)[::-1]
        assert abs(gap[i, 0] - (srt[1] - srt[2])) < 1e-12


# ------------------------------------------------------------------ backward ---
def _loss(q, k, v, dout, B, topk, scale, sel):
    """sum(dout * O) with the selection forced (the ranking held fixed)."""
    N, Hq, d = q.shape
    r, h = oracle.all_rows(N, Hq)
    _, o, _ = oracle.rows(q, k, v, B, topk, r, h, scale=scale, forced_sel=sel.reshape(-1, topk))
    return float(np.sum(dout.reshape(-1, d) * o))


@pytest.mark.parametrize("routing", [0, 1])
def test_backward_matches_finite_differences(routing):
    """Central differences of sum(dO * O) in fp64 (inputs perturbed by 2^-12,
    exactly representable) against the analytic gradients, on entries of Q, K
    and V in history blocks and in the own block."""
    N, Hq, Hkv, d, B, topk, scale = 37, 4, 2, 6, 4, 3, 0.6
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=41)
    rng = np.random.default_rng(3)
    dout = rng.standard_normal((N, Hq, d))
    r, h = oracle.all_rows(N, Hq)
    sel, _, _ = oracle.rows(q, k, None, B, topk, r, h, want_o=False, routing=routing)
    dq, dk, dv = oracle.backward(q, k, v, dout, B, topk, scale=scale, sel=sel)
    eps = 2.0 ** -12
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            a_p, a_m = arr.copy(), arr.copy()
            a_p[idx] += eps
            a_m[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = a_p, a_m
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], dout, B, topk, scale, sel) -
                  _loss(args_m["q"], args_m["k"], args_m["v"], dout, B, topk, scale, sel)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_backward_closed_forms():
    """Weights sum to one: the dV of a KV head sums to the dO of its query heads.
    Constant V: every output equals that vector, so dQ and dK vanish."""
    N, Hq, Hkv, d, B, topk = 40, 4, 2, 8, 5, 3
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=8)
    dout = np.random.default_rng(9).standard_normal((N, Hq, d))
    dq, dk, dv = oracle.backward(q, k, v, dout, B, topk, scale=0.5)
    G = Hq // Hkv
    for g in range(Hkv):
        assert np.allclose(dv[:, g].sum(0), dout[:, g * G:(g + 1) * G].sum((0, 1)), atol=1e-12)
    vc = np.broadcast_to(v[:1], v.shape).copy()
    dq, dk, _ = oracle.backward(q, k, vc, dout, B, topk, scale=0.5)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


# ------------------------------------------------------- forced selection ---
def _forced_history(row_sel, c, topk):
    """The history set a forced selection row stands for: entries that are
    earlier blocks of the row (0 <= b < c), first occurrence only, at most
    topk - 1 of them in the given order; -1 pads, the own block and future
    blocks are no history (PaperTrace "2.1.3 MoBA", section 2: the own block is
    always attended causally and never ranked; section 5 lists forcing the
    candidate set as a diagnostic)."""
    out = []
    for b in row_sel:
        b = int(b)
        if 0 <= b < c and b not in out and len(out) < topk - 1:
            out.append(b)
    return out


def _forced_mask(N, Hq, B, rows, heads, fsel, topk, own_whole=False):
    """Boolean attention mask [Hq, N, N] of the forced candidate sets (rows
    outside `rows` keep only themselves so every softmax row is defined)."""
    m = np.zeros((Hq, N, N), bool)
    m[:, np.arange(N), np.arange(N)] = True
    for r, h, fs in zip(rows, heads, fsel):
        c = int(r) // B
        m[h, r, :] = False
        for b in _forced_history(fs, c, topk):
            m[h, r, b * B:(b + 1) * B] = True
        hi = min(N, (c + 1) * B) if own_whole else int(r) + 1
        m[h, r, c * B:hi] = True
    return m


def _forced_cases(N, Hq, B, topk, seed):
    """(rows, heads, forced rows) exercising every rule of forced selection."""
    rng = np.random.default_rng(seed)
    rows, heads, fsel = [], [], []
    for r in range(N):
        c = r // B
        for h in range(Hq):
            kind = (r * Hq + h) % 6
            if kind == 0:    # a random subset of earlier blocks, reversed order
                hist = list(rng.permutation(c)[: topk - 1])[::-1] if c else []
                row = hist + [-1] * (topk - len(hist))
            elif kind == 1:  # one earlier block repeated, then -1
                b = int(rng.integers(0, c)) if c else -1
                row = [b] * min(3, topk) + [-1] * (topk - min(3, topk))
            elif kind == 2:  # the own block first, then earlier blocks
                row = [c] + list(range(min(c, topk - 1)))
                row = (row + [-1] * topk)[:topk]
            elif kind == 3:  # future blocks and -1 mixed with one earlier block
                row = [c + 1, -1, (c - 1) if c else -7, c + 5] + [-1] * topk
                row = row[:topk]
            elif kind == 4:  # every earlier block, more than topk - 1 of them
                row = (list(range(c))[::-1] + [-1] * topk)[:topk]
            else:            # nothing forced: own block only
                row = [-1] * topk
            rows.append(r)
            heads.append(h)
            fsel.append(row)
    return np.array(rows, np.int64), np.array(heads, np.int32), np.array(fsel, np.int32)


@pytest.mark.parametrize("N,Hq,Hkv,d,B,topk,seed", [(48, 2, 1, 8, 6, 4, 1), (40, 4, 2, 4, 5, 3, 2),
                                                     (64, 3, 3, 8, 8, 5, 3)])
def test_forced_selection_matches_masked_softmax(N, Hq, Hkv, d, B, topk, seed):
    """Forced mode attends exactly the forced history blocks plus the causal own
    block, against torch's fp64 attention with that mask built here."""
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=seed)
    scale = 0.41
    rows, heads, fsel = _forced_cases(N, Hq, B, topk, seed)
    sel, o, gap = oracle.rows(q, k, v, B, topk, rows, heads, scale=scale, forced_sel=fsel)
    ref = _sdpa_rows(q, k, v, _forced_mask(N, Hq, B, rows, heads, fsel, topk), scale)
    assert np.max(np.abs(o - ref[rows, heads])) < 1e-12
    # the returned selection is the forced history ascending, then the own block
    for i in range(len(rows)):
        c = int(rows[i]) // B
        hist = sorted(_forced_history(fsel[i], c, topk))
        assert list(sel[i]) == hist + [c] + [-1] * (topk - len(hist) - 1)
    assert np.all(np.isnan(gap))
    # the two-branch form (eqs. (7)-(8)) agrees under forcing too
    _, o2, _ = oracle.rows(q, k, v, B, topk, rows, heads, scale=scale, forced_sel=fsel,
                           mode=oracle.MODE_TWO_BRANCH)
    assert np.max(np.abs(o2 - o)) < 1e-12


def test_forced_selection_is_discriminating():
    """The forced-mode pin above fails for the plausible wrong forced paths: a
    path that ignores the forced rows (natural ranking), one that takes the own
    block whole instead of causally, and one that drops repeated entries'
    later distinct blocks would all be off by far more than its tolerance."""
    N, Hq, Hkv, d, B, topk = 48, 2, 1, 8, 6, 4
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=1)
    scale = 0.41
    rows, heads, fsel = _forced_cases(N, Hq, B, topk, 1)
    ref = _sdpa_rows(q, k, v, _forced_mask(N, Hq, B, rows, heads, fsel, topk), scale)[rows, heads]
    # (a) ignoring forced_sel: the natural selection differs on many rows
    nat_sel, o_nat, _ = oracle.rows(q, k, v, B, topk, rows, heads, scale=scale)
    differs = np.abs(o_nat - ref).max(axis=1) > 1e-3
    assert differs.sum() > len(rows) // 4
    # the forced lowest-scoring choices really are off the natural ranking
    low = []
    for i in range(len(rows)):
        c = int(rows[i]) // B
        if c > topk - 1:
            s = q[rows[i], heads[i]].astype(np.float64) @ oracle.block_means(k, B)[0, :c].T
            low.append(sorted(np.argsort(s, kind="stable")[: topk - 1].tolist()))
    assert len(low) > 0
    # (b) own block whole (future keys of the block leak in)
    whole = _sdpa_rows(q, k, v, _forced_mask(N, Hq, B, rows, heads, fsel, topk, own_whole=True),
                       scale)[rows, heads]
    not_last = (rows % B) != B - 1
    assert np.all(np.abs(whole - ref).max(axis=1)[not_last] > 1e-6)
    # (c) the own block listed inside forced_sel must not count as history
    #     (it would then be attended whole): rows of kind 2 carry it first
    kind2 = ((rows * Hq + heads) % 6 == 2) & not_last
    assert kind2.any()
    assert np.all(np.abs(whole - ref).max(axis=1)[kind2] > 1e-6)


def test_forced_selection_equal_to_natural_reproduces_it():
    """Forcing the oracle's own selection gives its own output bit for bit, and
    forcing the lowest-scoring blocks gives the masked softmax of those."""
    N, Hq, Hkv, d, B, topk = 72, 2, 2, 8, 8, 3
    q, k, v = synth.random_qkv(N, Hq, Hkv, d, seed=9)
    r, h = oracle.all_rows(N, Hq)
    sel, o, _ = oracle.rows(q, k, v, B, topk, r, h, scale=0.3)
    _, of, _ = oracle.rows(q, k, v, B, topk, r, h, scale=0.3, forced_sel=sel)
    assert np.array_equal(o, of)
    kb = oracle.block_means(k, B)
    worst = np.full((len(r), topk), -1, np.int32)
    for i in range(len(r)):
        c = int(r[i]) // B
        s = q[r[i], h[i]].astype(np.float64) @ kb[h[i] // (Hq // Hkv), :c].T
        worst[i, : min(c, topk - 1)] = np.argsort(s, kind="stable")[: topk - 1]
    sel_w, o_w, _ = oracle.rows(q, k, v, B, topk, r, h, scale=0.3, forced_sel=worst)
    ref = _sdpa_rows(q, k, v, _forced_mask(N, Hq, B, r, h, worst, topk), 0.3)[r, h]
    assert np.max(np.abs(o_w - ref)) < 1e-12
    has_choice = (r // B) > topk - 1
    assert np.all(np.any(sel_w[has_choice] != sel[has_choice], axis=1))
