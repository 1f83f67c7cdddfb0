"""GPU parity: every stage and the whole MoBA prefill, through the C ABI, against
the fp64 oracle on the same seeded inputs.

Bars: block selections bit-exact except rows whose gate margin is below 1e-5
relative (those are re-checked with the GPU's selection forced into the
oracle); O max-abs <= 1e-2 and mean-abs <= 1e-3 for bf16 (fp32 accumulation),
max-abs <= 1e-5 for fp32. Block means (fp64 sums of the inputs) must match
exactly.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_meanpool_amd as moba
import oracle
import synth
from tests._gpu import DEV, check_output, check_selection, compare_rows, to_dev, to_np

pytestmark = pytest.mark.gpu

_CACHE = {}


def inputs(name, dtype=None):
    """Seeded workload inputs, host (numpy) and device, cached per (config, dtype)."""
    w = synth.CONFIGS[name]
    dtype = dtype or w.dtype
    key = (name, dtype)
    if key not in _CACHE:
        q, k, v = synth.make_qkv(w, dtype)
        _CACHE[key] = (w, q, k, v, to_dev(q), to_dev(k), to_dev(v))
    return _CACHE[key]


def small(N, Hq, Hkv, B, topk, seed, dtype="bf16", integer=False, zero_k=False):
    q, k, v = synth.random_qkv(N, Hq, Hkv, 128, seed, dtype=dtype, integer=integer)
    if zero_k:
        k = np.zeros_like(k)
    return q, k, v, to_dev(q), to_dev(k), to_dev(v)


def all_rows(N, Hq):
    return oracle.all_rows(N, Hq)


# ------------------------------------------------------------------ stages ---
@pytest.mark.parametrize("name,dtype", [("tiny2k", "f32"), ("tiny2k", "bf16"), ("mha8k", None), ("coarse32k", None)])
def test_meanpool_exact(name, dtype):
    w, q, k, v, tq, tk, tv = inputs(name, dtype)
    got = moba.debug_meanpool(tk, w.B).cpu().numpy()
    ref = oracle.block_means(k, w.B)
    if k.dtype == np.uint16:
        assert np.array_equal(got, ref)
    else:
        assert np.allclose(got, ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("N,Hkv,B", [(1000, 3, 96), (300, 2, 1), (777, 1, 250), (64, 4, 128)])
def test_meanpool_irregular(N, Hkv, B):
    q, k, v, tq, tk, tv = small(N, Hkv, Hkv, B, 2, seed=N + B)
    got = moba.debug_meanpool(tk, B).cpu().numpy()
    assert np.array_equal(got, oracle.block_means(k, B))


@pytest.mark.parametrize("name,dtype", [("tiny2k", "f32"), ("tiny2k", "bf16"), ("mha8k", None), ("coarse32k", None),
                                        ("mha32k_needles", None)])
def test_select_all_rows(name, dtype):
    w, q, k, v, tq, tk, tv = inputs(name, dtype)
    sel = moba.select(tq, tk, w.B, w.k).cpu().numpy()
    rows, heads = all_rows(w.N, w.Hq)
    ref_sel, _, gap = oracle.rows(q, k, None, w.B, w.k, rows, heads, want_o=False)
    check_selection(sel.reshape(-1, w.k), ref_sel, gap, name,
                    ctx=(q, k, w.B, rows, heads, oracle.ROUTING_PER_HEAD))


def _bucket_reference(sel, Hkv, B):
    N, Hq, k = sel.shape
    G = Hq // Hkv
    n = -(-N // B)
    lists = [[[] for _ in range(n - 1)] for _ in range(Hkv)]
    for r in range(N):
        c = r // B
        for h in range(Hq):
            for s in range(k - 1):
                b = sel[r, h, s]
                if 0 <= b < c:
                    lists[h // G][b].append((r * Hq + h) * (k - 1) + s)
    offs, ents = [0], []
    for g in range(Hkv):
        for b in range(n - 1):
            ents += lists[g][b]
            offs.append(len(ents))
    return np.array(offs), np.array(ents)


@pytest.mark.parametrize("N,Hq,Hkv,B,topk", [(2048, 4, 2, 128, 4), (999, 6, 3, 64, 3),
                                             (512, 8, 1, 32, 5)])
def test_bucket_lists(N, Hq, Hkv, B, topk):
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=7)
    sel = moba.select(tq, tk, B, topk)
    offs, ents = moba.debug_bucket(sel, Hkv, B)
    ro, re_ = _bucket_reference(sel.cpu().numpy(), Hkv, B)
    assert np.array_equal(offs.cpu().numpy(), ro)
    assert np.array_equal(ents.cpu().numpy()[: len(re_)], re_)


# ---------------------------------------------------------------- prefill ---
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,dtype", [("tiny2k", "f32"), ("tiny2k", "bf16"), ("mha8k", None), ("coarse32k", None),
                                        ("mha32k_needles", None)])
def test_prefill_all_rows(name, dtype):
    w, q, k, v, tq, tk, tv = inputs(name, dtype)
    o = moba.prefill(tq, tk, tv, w.B, w.k, w.scale)
    sel = moba.select(tq, tk, w.B, w.k)
    rows, heads = all_rows(w.N, w.Hq)
    (mx, mean), tied = compare_rows(q, k, v, w.B, w.k, w.scale, rows, heads,
                                    sel.cpu().numpy().reshape(-1, w.k),
                                    to_np(o).reshape(-1, w.d), dtype or w.dtype, name)
    print(f"{name} {dtype or w.dtype}: max|dO| {mx:.2e} mean {mean:.2e} tie-excused rows {tied}")


def test_prefill_mha32k_needles_sampled():
    w, q, k, v, tq, tk, tv = inputs("mha32k_needles")
    o = moba.prefill(tq, tk, tv, w.B, w.k, w.scale)
    sel = moba.select(tq, tk, w.B, w.k).cpu().numpy()
    rows, heads = synth.sample_rows(w, 4096)
    (mx, mean), tied = compare_rows(q, k, v, w.B, w.k, w.scale, rows, heads, sel[rows, heads],
                                    to_np(o)[rows, heads], "bf16", "mha32k_needles")
    # needle rows pick needle blocks: long-range selection is exercised
    hits = 0
    for h in range(2):
        nb = set(synth.needle_blocks(w, h).tolist())
        for r in synth.needle_rows(w, h):
            c = r // w.B
            legal = {b for b in nb if b < c}
            if len(legal) >= w.k - 1:
                hits += set(sel[r, h, : w.k - 1].tolist()) <= legal
    assert hits > 0
    print(f"mha32k_needles: max|dO| {mx:.2e} mean {mean:.2e} tie-excused rows {tied} needle rows routed {hits}")


@pytest.mark.timeout(1200)
def test_prefill_llama8b_1m_sampled():
    w, q, k, v, tq, tk, tv = inputs("llama8b_1m")
    o = moba.prefill(tq, tk, tv, w.B, w.k, w.scale)
    sel = moba.select(tq, tk, w.B, w.k)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    o_np = o.cpu()
    rows, heads = synth.sample_rows(w, 4096)
    kbar = oracle.block_means(k, w.B)
    got_o = o_np[torch.from_numpy(rows), torch.from_numpy(heads.astype(np.int64))].float().numpy()
    (mx, mean), tied = compare_rows(q, k, v, w.B, w.k, w.scale, rows, heads, sel_np[rows, heads],
                                    got_o.astype(np.float64), "bf16", "llama8b_1m")
    # selections on a larger seeded sample (gate only)
    r2, h2 = synth.sample_rows(w.with_(seed=w.seed ^ 0xABCDEF), 1 << 20)
    ref_sel, _, gap = oracle.rows(q, k, None, w.B, w.k, r2, h2, want_o=False, kbar=kbar)
    check_selection(sel_np[r2, h2], ref_sel, gap, "llama8b_1m sel",
                    ctx=(q, k, w.B, r2, h2, oracle.ROUTING_PER_HEAD))
    # every row: the fast tier (with band records) against the exact tier alone
    exact = moba.routing_stats(tq, tk, w.B, w.k)["sel"]
    assert torch.equal(sel, exact)
    print(f"llama8b_1m: max|dO| {mx:.2e} mean {mean:.2e} tie-excused rows {tied}")


# ------------------------------------- the benchmarked legs at their shapes ---
def _seq_samples(L, B, Hq, count, seed):
    """(rows, heads) inside one sequence of L rows: its first and last row, then
    rows cycling over its blocks at the block's first row, its last row, then
    seeded offsets; heads seeded."""
    rng = np.random.default_rng(seed)
    n = -(-L // B)
    rows = [0, L - 1]
    r = 0
    while len(rows) < count:
        c = r % n
        lo, hi = c * B, min(L, (c + 1) * B) - 1
        rows.append(lo if r < n else hi if r < 2 * n else int(rng.integers(lo, hi + 1)))
        r += 1
    rows = np.array(rows[:count], np.int64)
    return rows, rng.integers(0, Hq, size=count).astype(np.int32)


@pytest.mark.timeout(1200)
def test_varlen_llama8b_1m_sampled():
    """The packed-batch leg exactly as benchmarked: 16 seeded sequences of the
    1M-row layer (B = 4096, k = 12, 32/8 heads); 256 (row, head) pairs per
    sequence, its first and last row among them, against the oracle run on
    that sequence alone."""
    w, q, k, v, tq, tk, tv = inputs("llama8b_1m")
    lens = synth.packed_layer_lengths(w)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o = moba.prefill_varlen(tq, tk, tv, cu, w.B, w.k, w.scale)
    sel = moba.select_varlen(tq, tk, cu, w.B, w.k)
    torch.cuda.synchronize()
    base = _seq_base(cu, w.B)
    worst, tied_all = 0.0, 0
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        rows, heads = _seq_samples(b - a, w.B, w.Hq, 256, seed=1000 + i)
        gi = torch.from_numpy(rows + a)
        hi = torch.from_numpy(heads.astype(np.int64))
        s_loc = sel[gi, hi].cpu().numpy().astype(np.int64)
        s_loc = np.where(s_loc >= 0, s_loc - base[i], -1).astype(np.int32)
        got_o = o[gi, hi].float().cpu().numpy().astype(np.float64)
        (mx, mean), tied = compare_rows(q[a:b], k[a:b], v[a:b], w.B, w.k, w.scale, rows, heads,
                                        s_loc, got_o, "bf16", f"packed seq {i} ({b - a} rows)")
        worst, tied_all = max(worst, mx), tied_all + tied
    print(f"llama8b_1m packed: max|dO| {worst:.2e} tie-excused rows {tied_all}")


@pytest.mark.timeout(1200)
def test_shared_routing_llama8b_1m_sampled():
    """The group-shared routing leg as benchmarked (the 1M-row layer, heads of
    a KV head share the ranking by their summed gate score): O on the 4096
    seeded (row, head) pairs, the selection on 2^20 more."""
    w, q, k, v, tq, tk, tv = inputs("llama8b_1m")
    shared = moba.MOBA_ROUTING_SHARED
    o = moba.prefill(tq, tk, tv, w.B, w.k, w.scale, routing=shared)
    sel = moba.select(tq, tk, w.B, w.k, routing=shared)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    del sel
    rows, heads = synth.sample_rows(w, 4096)
    got_o = o[torch.from_numpy(rows), torch.from_numpy(heads.astype(np.int64))]
    got_o = got_o.float().cpu().numpy().astype(np.float64)
    del o
    kbar = oracle.block_means(k, w.B)
    (mx, mean), tied = compare_rows(q, k, v, w.B, w.k, w.scale, rows, heads, sel_np[rows, heads],
                                    got_o, "bf16", "llama8b_1m shared",
                                    routing=oracle.ROUTING_SHARED)
    r2, h2 = synth.sample_rows(w.with_(seed=w.seed ^ 0x5A5A5A), 1 << 20)
    ref_sel, _, gap = oracle.rows(q, k, None, w.B, w.k, r2, h2, want_o=False, kbar=kbar,
                                  routing=oracle.ROUTING_SHARED)
    check_selection(sel_np[r2, h2], ref_sel, gap, "llama8b_1m shared sel",
                    ctx=(q, k, w.B, r2, h2, oracle.ROUTING_SHARED))
    print(f"llama8b_1m shared: max|dO| {mx:.2e} mean {mean:.2e} tie-excused rows {tied}")


@pytest.mark.timeout(1200)
def test_chunk_and_decode_llama8b_1m():
    """The chunk / decode leg as benchmarked, over the 1M-row layer as its KV
    cache: a decode step (the last row, every head) and a 16,384-row chunk
    (1024 seeded pairs), recomputing the block means, and the decode step on a
    decode cache, all against the oracle at those positions."""
    w, q, k, v, tq, tk, tv = inputs("llama8b_1m")
    kbar = oracle.block_means(k, w.B)
    for C in (1, 16384):
        qc = tq[w.N - C:].contiguous()
        oc = moba.prefill_chunk(qc, tk, tv, w.B, w.k, w.scale)
        sc = moba.select_chunk(qc, tk, w.B, w.k)
        torch.cuda.synchronize()
        if C == 1:
            loc = np.zeros(w.Hq, np.int64)
            heads = np.arange(w.Hq, dtype=np.int32)
        else:
            rng = np.random.default_rng(4)
            loc = np.concatenate([[0, C - 1], rng.integers(0, C, size=1022)]).astype(np.int64)
            heads = rng.integers(0, w.Hq, size=loc.size).astype(np.int32)
        li, hi = torch.from_numpy(loc), torch.from_numpy(heads.astype(np.int64))
        got_o = oc[li, hi].float().cpu().numpy().astype(np.float64)
        got_s = sc[li, hi].cpu().numpy()
        compare_rows(q, k, v, w.B, w.k, w.scale, loc + (w.N - C), heads, got_s, got_o, "bf16",
                     f"llama8b_1m chunk of {C}")
        if C == 1:
            o_step = oc
        del oc, sc
    cache = moba.DecodeCache(w.N, w.Hq, w.Hkv, w.B, w.k, w.scale, device=tq.device)
    cache.append(tk, tv, w.N - 1)
    cache.append(tk, tv, w.N)
    od = cache.prefill(tq[w.N - 1:].contiguous(), tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(od, o_step)
    del cache


# ------------------------------------------------------------- edge cases ---
EDGE = [
    # N, Hq, Hkv, B, topk, dtype
    (1000, 2, 1, 96, 3, "bf16"),     # B does not divide N, partial key tiles
    (700, 4, 2, 48, 4, "bf16"),      # B < 64: masked key tiles
    (200, 2, 2, 256, 3, "bf16"),     # N < B: one partial block
    (1, 2, 1, 64, 3, "bf16"),        # a single row
    (300, 2, 1, 1, 4, "bf16"),       # B = 1: token-level routing
    (2048, 8, 2, 128, 1, "bf16"),    # k = 1: own block only
    (2048, 8, 8, 128, 16, "bf16"),   # k >= n: causal full attention
    (1536, 8, 1, 128, 5, "bf16"),    # G = 8
    (1536, 12, 3, 128, 4, "bf16"),   # odd KV head count
    (1000, 2, 1, 96, 3, "f32"),
    (2048, 4, 2, 128, 16, "f32"),
    (300, 2, 1, 1, 4, "f32"),
    (16, 4, 2, 4, 3, "bf16"),        # 16 rows: the few-row path over a whole prefill
    (13, 2, 1, 3, 4, "f32"),
]


@pytest.mark.parametrize("N,Hq,Hkv,B,topk,dtype", EDGE)
def test_prefill_edge(N, Hq, Hkv, B, topk, dtype):
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N * 31 + topk, dtype=dtype)
    scale = 0.09
    o = moba.prefill(tq, tk, tv, B, topk, scale)
    sel = moba.select(tq, tk, B, topk)
    rows, heads = all_rows(N, Hq)
    compare_rows(q, k, v, B, topk, scale, rows, heads, sel.cpu().numpy().reshape(-1, topk),
                 to_np(o).reshape(-1, 128), dtype, f"edge {N},{Hq},{Hkv},{B},{topk}")


def test_zero_keys_ties_are_exact():
    """K == 0: every gate score ties; the lowest blocks must be chosen (no tie excuse)."""
    N, Hq, Hkv, B, topk = 1024, 4, 2, 64, 4
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=3, zero_k=True)
    sel = moba.select(tq, tk, B, topk).cpu().numpy().reshape(-1, topk)
    rows, heads = all_rows(N, Hq)
    ref_sel, ref_o, _ = oracle.rows(q, k, v, B, topk, rows, heads)
    assert np.array_equal(sel, ref_sel)
    o = moba.prefill(tq, tk, tv, B, topk)
    check_output(to_np(o).reshape(-1, 128), ref_o, "bf16", "zero K")


def test_integer_ties_are_exact():
    N, Hq, Hkv, B, topk = 640, 2, 1, 16, 5
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=5, integer=True)
    sel = moba.select(tq, tk, B, topk).cpu().numpy().reshape(-1, topk)
    rows, heads = all_rows(N, Hq)
    ref_sel, _, _ = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False)
    assert np.array_equal(sel, ref_sel)


@pytest.mark.parametrize("B", [128, 256, 512])
def test_softmax_overflow_rerun(B):
    """Spike keys past each block's first 32 keys score ~200 (log2 units) above
    the rest, beyond the 2^64 headroom of the fixed reference maximum and
    beyond fp32's range: the attention kernels must re-run those blocks from
    the true maxima (history and own block alike), else weights overflow to
    infinity. B = 128 runs the 32-query history engine (in-kernel re-run),
    B = 256 and 512 the 64-query one (tiles listed and recomputed by a second
    kernel); the own-block kernel re-runs its workgroups in place, at B = 512
    also those whose unmasked keys span several tiles."""
    N, Hq, Hkv, topk = 2048, 2, 1, 3
    q, k, v, _, _, _ = small(N, Hq, Hkv, B, topk, seed=41)
    u = np.random.default_rng(41).standard_normal(128)
    u /= np.linalg.norm(u)
    qf, kf = synth.bf16_to_f32(q), synth.bf16_to_f32(k)
    qf += (35.0 * u).astype(np.float32)  # every query leans along u
    spikes = [c * B + 40 + (7 * c) % 80 for c in range(N // B)]
    kf[spikes] += (45.0 * u).astype(np.float32)
    q, k = synth.f32_to_bf16(qf), synth.f32_to_bf16(kf)
    # O is then close to single V rows: V / 4 (exact) keeps |O| < 2, where
    # bf16's half-ulp stays below the 1e-2 bar
    v = synth.f32_to_bf16(synth.bf16_to_f32(v) * np.float32(0.25))
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    scale = 1.0 / np.sqrt(128.0)
    o = moba.prefill(tq, tk, tv, B, topk, scale)
    sel = moba.select(tq, tk, B, topk).cpu().numpy()
    assert bool(torch.isfinite(o.float()).all())
    rows, heads = all_rows(N, Hq)
    compare_rows(q, k, v, B, topk, scale, rows, heads, sel.reshape(-1, topk),
                 to_np(o).reshape(-1, 128), "bf16", "spike keys")


@pytest.mark.parametrize("B", [128, 256])
def test_values_near_the_fp16_partial_limit(B):
    """bf16 values up to 0.9 x 65504: the fp16 partial rows (history and the
    own-block staging, both convex combinations of V rows) stay finite and O
    matches the oracle at the usual bars relative to the value scale. Both
    history engines (B = 128: 32-query, B = 256: 64-query)."""
    N, Hq, Hkv, topk = 2048, 4, 2, 3
    q, k, v, _, _, _ = small(N, Hq, Hkv, B, topk, seed=77)
    big = np.float32(0.9 * 65504.0)
    vf = np.random.default_rng(77).uniform(-1.0, 1.0, size=v.shape).astype(np.float32) * big
    v = synth.f32_to_bf16(vf)
    assert float(np.abs(synth.bf16_to_f32(v)).max()) < 65504.0
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    scale = 0.09
    o = moba.prefill(tq, tk, tv, B, topk, scale)
    assert bool(torch.isfinite(o.float()).all())
    sel = moba.select(tq, tk, B, topk).cpu().numpy()
    rows, heads = all_rows(N, Hq)
    ref_sel, ref_o, gap = oracle.rows(q, k, v, B, topk, rows, heads, scale=scale)
    assert np.array_equal(sel.reshape(-1, topk), ref_sel)
    check_output(to_np(o).reshape(-1, 128) / float(big), ref_o / float(big), "bf16",
                 "values near the fp16 limit")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_baseline_and_full_coverage(dtype):
    """k covering every block equals causal full attention, and so does the dense kernel."""
    N, Hq, Hkv, B = 2304, 4, 2, 256
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, 9, seed=11, dtype=dtype)
    scale = 0.1
    od = moba.dense_causal(tq, tk, tv, scale)
    om = moba.prefill(tq, tk, tv, B, 9, scale)
    rows, heads = all_rows(N, Hq)
    ref = oracle.causal_full(q, k, v, rows, heads, scale=scale)
    check_output(to_np(od).reshape(-1, 128), ref, dtype, "dense")
    check_output(to_np(om).reshape(-1, 128), ref, dtype, "moba k>=n")


def test_deterministic():
    w, q, k, v, tq, tk, tv = inputs("mha8k")
    a = moba.prefill(tq, tk, tv, w.B, w.k, w.scale)
    b = moba.prefill(tq, tk, tv, w.B, w.k, w.scale)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_stage_events_and_copy():
    w, q, k, v, tq, tk, tv = inputs("mha8k")
    prob = moba.make_problem(w.N, w.Hq, w.Hkv, w.d, w.B, w.k, w.scale)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(moba.stage_events(prob))]
    moba.prefill(tq, tk, tv, w.B, w.k, w.scale, events=ev)
    torch.cuda.synchronize()
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    assert all(t >= 0 for t in times)
    src = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    dst = torch.empty_like(src)
    moba.debug_copy(src, dst)
    assert torch.equal(src, dst)


# ------------------------------------------------------- attention passes ---
PASSES = [
    # N, Hq, Hkv, B, topk, dtype, KV heads per pass
    (3000, 8, 4, 256, 4, "bf16", 1),  # 64-query history engine, four passes
    (3000, 8, 4, 256, 4, "bf16", 3),  # the last pass holds one KV head
    (2000, 6, 3, 96, 5, "bf16", 2),   # 32-query engine (B not a multiple of 256)
    (1500, 4, 2, 128, 3, "f32", 1),
]


@pytest.mark.parametrize("N,Hq,Hkv,B,topk,dtype,kvpp", PASSES)
def test_attention_passes(N, Hq, Hkv, B, topk, dtype, kvpp):
    """Attention in passes over groups of KV heads: the output equals the
    one-pass output bit for bit (each (row, head) is computed by the same
    tiles in the same order) and the oracle within the usual bars; every
    pass records its two stage events."""
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + 10 * kvpp, dtype=dtype)
    scale = 0.08
    code = moba.MOBA_DTYPE_BF16 if dtype == "bf16" else moba.MOBA_DTYPE_F32
    prob = moba.make_problem(N, Hq, Hkv, 128, B, topk, scale, code, kv_heads_per_pass=kvpp)
    passes = -(-Hkv // kvpp)
    assert moba.stage_events(prob) == 5 + 2 * passes
    whole = moba.make_problem(N, Hq, Hkv, 128, B, topk, scale, code, kv_heads_per_pass=Hkv)
    assert moba.workspace_size(prob) < moba.workspace_size(whole)
    one = moba.prefill(tq, tk, tv, B, topk, scale, kv_heads_per_pass=Hkv)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5 + 2 * passes)]
    got = moba.prefill(tq, tk, tv, B, topk, scale, events=ev, kv_heads_per_pass=kvpp)
    torch.cuda.synchronize()
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(len(ev) - 1))
    assert torch.equal(got, one)
    sel = moba.select(tq, tk, B, topk).cpu().numpy()
    rows, heads = all_rows(N, Hq)
    (mx, mean), tied = compare_rows(q, k, v, B, topk, scale, rows, heads,
                                    sel.reshape(-1, topk), to_np(got).reshape(-1, 128), dtype,
                                    f"passes {kvpp}")
    print(f"{passes} passes ({dtype}, B={B}): max|dO| {mx:.2e} mean {mean:.2e}")


def test_attention_passes_training_forward_and_shared_routing():
    """The training forward (O and the row log-sum-exps the backward reads)
    and group-shared routing in one KV head per pass equal their one-pass
    results bit for bit."""
    N, Hq, Hkv, B, topk = 3000, 8, 4, 256, 4
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=43)
    o1, l1 = moba.prefill_train(tq, tk, tv, B, topk, 0.09, kv_heads_per_pass=Hkv)
    o2, l2 = moba.prefill_train(tq, tk, tv, B, topk, 0.09, kv_heads_per_pass=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    a = moba.prefill(tq, tk, tv, B, topk, 0.09, routing=moba.MOBA_ROUTING_SHARED,
                     kv_heads_per_pass=Hkv)
    b = moba.prefill(tq, tk, tv, B, topk, 0.09, routing=moba.MOBA_ROUTING_SHARED,
                     kv_heads_per_pass=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_passes_varlen_chunk_noalloc():
    """Packed sequences, a chunk and the allocation-free entry point in one
    KV head per pass equal their one-pass results bit for bit."""
    lens = [1000, 1, 0, 2500, 333, 4113]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, Hq, Hkv, B, topk = int(cu[-1]), 8, 4, 256, 4
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=41)
    a = moba.prefill_varlen(tq, tk, tv, cu, B, topk, 0.09, kv_heads_per_pass=Hkv)
    b = moba.prefill_varlen(tq, tk, tv, cu, B, topk, 0.09, kv_heads_per_pass=1)
    assert torch.equal(a, b)
    C = 700
    a = moba.prefill_chunk(tq[-C:], tk, tv, B, topk, 0.09, kv_heads_per_pass=Hkv)
    b = moba.prefill_chunk(tq[-C:], tk, tv, B, topk, 0.09, kv_heads_per_pass=1)
    assert torch.equal(a, b)
    a = moba.prefill(tq, tk, tv, B, topk, 0.09, kv_heads_per_pass=Hkv)
    b = moba.prefill_noalloc(tq, tk, tv, B, topk, 0.09, kv_heads_per_pass=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------- packed (varlen) ---
def _seq_base(cu, B):
    nb = [-(-(int(cu[i + 1]) - int(cu[i])) // B) for i in range(len(cu) - 1)]
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


VARLEN = [
    # lengths, Hq, Hkv, B, topk, dtype
    ([1000, 1, 0, 2500, 333, 4113], 8, 2, 256, 4, "bf16"),
    ([64, 64, 640, 129, 1, 700], 4, 4, 64, 3, "bf16"),
    ([5, 17, 3000, 0, 2049], 6, 3, 100, 5, "bf16"),  # B not a multiple of 64
    ([1000, 1, 0, 2500, 333], 4, 2, 256, 4, "f32"),
    ([3, 0, 9, 4], 4, 2, 2, 3, "bf16"),  # 16 rows in all: the few-row path
]


@pytest.mark.parametrize("lens,Hq,Hkv,B,topk,dtype", VARLEN)
def test_varlen_matches_each_sequence_alone(lens, Hq, Hkv, B, topk, dtype):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = int(cu[-1])
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + 3 * topk, dtype=dtype)
    scale = 0.09
    o = moba.prefill_varlen(tq, tk, tv, cu, B, topk, scale)
    sel = moba.select_varlen(tq, tk, cu, B, topk).cpu().numpy()
    o = to_np(o)
    base = _seq_base(cu, B)
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        s_loc = sel[a:b].reshape(-1, topk).astype(np.int64)
        s_loc = np.where(s_loc >= 0, s_loc - base[i], -1).astype(np.int32)
        assert s_loc.min() >= -1 and s_loc.max() < base[i + 1] - base[i]
        rows, heads = all_rows(b - a, Hq)
        compare_rows(q[a:b], k[a:b], v[a:b], B, topk, scale, rows, heads, s_loc,
                     o[a:b].reshape(-1, 128), dtype, f"varlen seq {i} ({b - a} rows)")


def test_varlen_one_sequence_is_plain_prefill():
    q, k, v, tq, tk, tv = small(3000, 8, 2, 256, 4, seed=21)
    o1 = moba.prefill(tq, tk, tv, 256, 4, 0.09)
    o2 = moba.prefill_varlen(tq, tk, tv, [0, 3000], 256, 4, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_varlen_sequences_do_not_leak():
    """Rewriting one packed sequence leaves every other sequence's output bit-identical."""
    lens = [700, 1300, 900]
    cu = np.cumsum([0] + lens)
    q, k, v, tq, tk, tv = small(int(cu[-1]), 4, 2, 128, 3, seed=31)
    o1 = moba.prefill_varlen(tq, tk, tv, cu, 128, 3, 0.09).clone()
    tk2, tv2 = tk.clone(), tv.clone()
    tk2[700:2000] = -tk2[700:2000]
    tv2[700:2000] += 1.0
    o2 = moba.prefill_varlen(tq, tk2, tv2, cu, 128, 3, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1[:700], o2[:700]) and torch.equal(o1[2000:], o2[2000:])
    assert not torch.equal(o1[700:2000], o2[700:2000])


# ------------------------------------------------ GQA shared routing, stats ---
SHARED = [
    # N, Hq, Hkv, B, topk, dtype
    (3000, 8, 2, 128, 4, "bf16"),
    (2048, 12, 3, 96, 5, "bf16"),
    (1500, 4, 1, 64, 3, "f32"),
]


@pytest.mark.parametrize("N,Hq,Hkv,B,topk,dtype", SHARED)
def test_shared_routing_matches_oracle(N, Hq, Hkv, B, topk, dtype):
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + Hq, dtype=dtype)
    shared = moba.MOBA_ROUTING_SHARED
    o = moba.prefill(tq, tk, tv, B, topk, 0.09, routing=shared)
    sel = moba.select(tq, tk, B, topk, routing=shared).cpu().numpy()
    G = Hq // Hkv
    for g in range(Hkv):
        assert np.all(sel[:, g * G:(g + 1) * G] == sel[:, g * G:g * G + 1])
    rows, heads = all_rows(N, Hq)
    compare_rows(q, k, v, B, topk, 0.09, rows, heads, sel.reshape(-1, topk),
                 to_np(o).reshape(-1, 128), dtype, f"shared {N},{Hq},{Hkv},{B},{topk}",
                 routing=oracle.ROUTING_SHARED)


def test_varlen_with_shared_routing():
    lens = [900, 0, 1, 1700, 420]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, Hq, Hkv, B, topk = int(cu[-1]), 8, 2, 128, 4
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=91)
    o = to_np(moba.prefill_varlen(tq, tk, tv, cu, B, topk, 0.09,
                                  routing=moba.MOBA_ROUTING_SHARED))
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        ref_sel, ref_o = oracle.prefill(q[a:b], k[a:b], v[a:b], B, topk, scale=0.09,
                                        routing=oracle.ROUTING_SHARED)
        check_output(o[a:b].reshape(-1, 128), ref_o.reshape(-1, 128), "bf16", f"seq {i}")


def test_shared_fast_tier_equals_exact_tier():
    """bf16 group-shared routing with many rows runs the certified fast tier;
    its selection must equal the exact tier's on every row (both are exact),
    here with 255 candidate blocks per late row."""
    N, Hq, Hkv, B, topk = 16384, 8, 2, 64, 8
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=23)
    shared = moba.MOBA_ROUTING_SHARED
    fast = moba.select(tq, tk, B, topk, routing=shared).cpu().numpy()
    exact = moba.routing_stats(tq, tk, B, topk, routing=shared)["sel"].cpu().numpy()
    assert np.array_equal(fast, exact)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(N, 256, replace=False))
    heads = rng.integers(0, Hq, size=rows.size)
    ref_sel, _, gap = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False,
                                  routing=oracle.ROUTING_SHARED)
    check_selection(fast[rows, heads], ref_sel, gap, "shared fast tier",
                    ctx=(q, k, B, rows, heads, oracle.ROUTING_SHARED))


@pytest.mark.parametrize("topk,integer", [(3, False), (8, False), (12, False), (12, True),
                                           (16, False), (17, False)])
def test_fast_tier_equals_exact_tier(topk, integer):
    """Per-head routing: the fast tier with its exact tier for uncertified rows
    (re-scoring either the whole row or only the undecided band of the fast
    list) must select exactly what the exact tier selects when it ranks every
    row. List lengths 6, 14, 16 and 32; integer data gives many exact ties."""
    N, Hq, Hkv, B = 16384, 8, 2, 64
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=31 + topk, integer=integer)
    fast = moba.select(tq, tk, B, topk).cpu().numpy()
    exact = moba.routing_stats(tq, tk, B, topk)["sel"].cpu().numpy()
    assert np.array_equal(fast, exact)
    rng = np.random.default_rng(topk)
    rows = np.sort(rng.choice(N, 256, replace=False))
    heads = rng.integers(0, Hq, size=rows.size)
    ref_sel, _, gap = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False)
    check_selection(fast[rows, heads], ref_sel, gap, "fast tier",
                    ctx=(q, k, B, rows, heads, 0))


def test_fast_tier_at_the_history_block_limit():
    """8192 history blocks, the most the library takes: block indices need 13
    of the fast tier's key bits (so its truncation margin is widest and many
    rows go to the exact tier) and band records carry indices up to 8191."""
    N, Hq, Hkv, B, topk = 8193 * 16, 2, 1, 16, 12
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=77)
    fast = moba.select(tq, tk, B, topk).cpu().numpy()
    exact = moba.routing_stats(tq, tk, B, topk)["sel"].cpu().numpy()
    assert np.array_equal(fast, exact)
    rng = np.random.default_rng(77)
    rows = np.sort(np.concatenate([rng.choice(N - 64, 190, replace=False), np.arange(N - 64, N)]))
    heads = rng.integers(0, Hq, size=rows.size)
    ref_sel, _, gap = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False)
    check_selection(fast[rows, heads], ref_sel, gap, "fast tier, 8192 blocks",
                    ctx=(q, k, B, rows, heads, 0))


@pytest.mark.parametrize("kind", ["zero_k", "integer"])
def test_shared_routing_ties_are_exact(kind):
    """Exact ties in the group score (all-zero keys, or integer data) must go
    to the lower block, through the fast tier's refine path."""
    N, Hq, Hkv, B, topk = 1280, 4, 2, 32, 5
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=29, **{kind: True})
    sel = moba.select(tq, tk, B, topk, routing=moba.MOBA_ROUTING_SHARED).cpu().numpy()
    rows, heads = all_rows(N, Hq)
    ref_sel, _, _ = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False,
                                routing=oracle.ROUTING_SHARED)
    assert np.array_equal(sel.reshape(-1, topk), ref_sel)


@pytest.mark.parametrize("routing", [0, 1])
def test_routing_stats(routing):
    N, Hq, Hkv, B, topk = 2500, 8, 2, 100, 4
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=17)
    st = moba.routing_stats(tq, tk, B, topk, routing=routing)
    sel = st["sel"].cpu().numpy()
    margin = st["margin"].cpu().numpy().astype(np.float64)
    counts = st["counts"].cpu().numpy()
    union = st["union_size"].cpu().numpy()
    rows, heads = all_rows(N, Hq)
    ref_sel, _, gap = oracle.rows(q, k, None, B, topk, rows, heads, want_o=False, routing=routing)
    check_selection(sel.reshape(-1, topk), ref_sel, gap, "stats sel",
                    ctx=(q, k, B, rows, heads, routing))
    m, g = margin.reshape(-1), gap[:, 0]
    assert np.array_equal(np.isnan(m), np.isnan(g))
    ok = ~np.isnan(g)
    assert np.all(np.abs(m[ok] - g[ok]) <= 1e-6 * np.maximum(gap[ok, 1], 1e-30) + 1e-30)
    # counts and group unions from the selection itself
    n = -(-N // B)
    G = Hq // Hkv
    c_rows = np.arange(N) // B
    ref_counts = np.zeros((Hkv, n), np.int64)
    ref_union = np.zeros((N, Hkv), np.int64)
    for r in range(N):
        for g_ in range(Hkv):
            seen = set()
            for hh in range(G):
                for b in sel[r, g_ * G + hh, : topk - 1]:
                    if 0 <= b < c_rows[r]:
                        ref_counts[g_, b] += 1
                        seen.add(int(b))
            ref_union[r, g_] = len(seen)
    assert np.array_equal(counts, ref_counts)
    assert np.array_equal(union, ref_union)
    if routing == 1:
        assert np.all(union <= topk - 1)


# ------------------------------------------------- chunked prefill / decode ---
CHUNKS = [
    # N, Hq, Hkv, B, topk, C, dtype
    (3000, 8, 2, 128, 4, 1, "bf16"),      # one decode step
    (3000, 8, 2, 128, 4, 7, "bf16"),      # inside the last (partial) block
    (3000, 8, 2, 128, 4, 300, "bf16"),    # across blocks, partial first block
    (3000, 8, 2, 128, 4, 3000, "bf16"),   # the whole sequence
    (2048, 4, 4, 96, 5, 200, "bf16"),     # B not a multiple of 64
    (1500, 4, 2, 64, 3, 129, "f32"),
    (3000, 8, 2, 128, 4, 16, "bf16"),     # the largest chunk of the few-row (split-K) path
    (3000, 8, 2, 128, 4, 17, "bf16"),     # the smallest of the tiled path
    (1500, 4, 2, 64, 3, 5, "f32"),        # few-row path in fp32
    (5000, 4, 1, 1000, 3, 3, "bf16"),     # few rows, 4 splits of a block, partial last split
]


@pytest.mark.parametrize("N,Hq,Hkv,B,topk,C,dtype", CHUNKS)
def test_chunk_rows_match_full_prefill(N, Hq, Hkv, B, topk, C, dtype):
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + C, dtype=dtype)
    qc = tq[N - C:].contiguous()
    o = to_np(moba.prefill_chunk(qc, tk, tv, B, topk, 0.09))
    sel = moba.select_chunk(qc, tk, B, topk).cpu().numpy()
    rows, heads = all_rows(C, Hq)
    rows = rows + (N - C)  # positions in the sequence
    compare_rows(q, k, v, B, topk, 0.09, rows, heads, sel.reshape(-1, topk), o.reshape(-1, 128),
                 dtype, f"chunk {C} of {N}")
    full = to_np(moba.prefill(tq, tk, tv, B, topk, 0.09))[N - C:]
    assert np.max(np.abs(full - o)) <= (1e-2 if dtype == "bf16" else 1e-5)


def test_decode_steps():
    """Three decode steps on a growing cache, each checked against the oracle."""
    N0, Hq, Hkv, B, topk = 1535, 8, 2, 128, 4
    q, k, v, tq, tk, tv = small(N0 + 3, Hq, Hkv, B, topk, seed=123)
    for step in range(3):
        N = N0 + step + 1  # the cache holds the new row
        o = to_np(moba.prefill_chunk(tq[N - 1:N].contiguous(), tk[:N].contiguous(),
                                     tv[:N].contiguous(), B, topk, 0.09))
        sel = moba.select_chunk(tq[N - 1:N].contiguous(), tk[:N].contiguous(), B, topk)
        rows = np.full(Hq, N - 1, np.int64)
        heads = np.arange(Hq, dtype=np.int32)
        compare_rows(q[:N], k[:N], v[:N], B, topk, 0.09, rows, heads,
                     sel.cpu().numpy().reshape(-1, topk), o.reshape(-1, 128), "bf16",
                     f"decode step {step}")


CACHE = [
    # capacity, Hq, Hkv, B, topk, dtype, rows appended per step
    (2000, 4, 2, 256, 3, "bf16", [700, 1, 1, 1, 65, 1, 254, 258, 1, 255, 1]),
    (1500, 8, 2, 96, 4, "bf16", [1, 94, 1, 1, 200, 3, 500]),  # B not a multiple of 64
    (1200, 4, 1, 128, 3, "f32", [500, 1, 139, 1, 1]),
]


@pytest.mark.parametrize("cap,Hq,Hkv,B,topk,dtype,steps", CACHE)
def test_decode_cache_matches_recompute(cap, Hq, Hkv, B, topk, dtype, steps):
    """Appending rows to a decode cache and running the chunk on it gives the
    rows of moba_prefill_chunk over the same prefix (bit for bit in bf16: the
    cached means are exact fp64 sums, as are the recomputed ones); the last
    step is also checked against the oracle."""
    q, k, v, tq, tk, tv = small(cap, Hq, Hkv, B, topk, seed=cap + B, dtype=dtype)
    code = moba.MOBA_DTYPE_BF16 if dtype == "bf16" else moba.MOBA_DTYPE_F32
    cache = moba.DecodeCache(cap, Hq, Hkv, B, topk, 0.09, dtype=code, device=DEV)
    rows = 0
    for a in steps:
        rows += a
        cache.append(tk, tv, rows)
        C = min(a, 96)
        qc = tq[rows - C:rows].contiguous()
        got = cache.prefill(qc, tk, tv)
        ref = moba.prefill_chunk(qc, tk[:rows], tv[:rows], B, topk, 0.09)
        if dtype == "bf16":
            assert torch.equal(got, ref), f"rows {rows}"
        else:
            assert torch.allclose(got, ref, rtol=0, atol=1e-6), f"rows {rows}"
    sel = moba.select_chunk(qc, tk[:rows], B, topk).cpu().numpy()
    r, heads = all_rows(C, Hq)
    compare_rows(q[:rows], k[:rows], v[:rows], B, topk, 0.09, r + (rows - C), heads,
                 sel.reshape(-1, topk), to_np(got).reshape(-1, 128), dtype, f"cache {rows}")


# ------------------------------------------------------------------ backward ---
BWD = [
    # N, Hq, Hkv, B, topk, dtype, routing
    (700, 4, 2, 64, 3, "f32", 0),
    (700, 4, 2, 64, 3, "bf16", 0),
    (900, 6, 3, 96, 4, "bf16", 0),     # B not a multiple of 64, G = 2
    (600, 4, 1, 128, 1, "bf16", 0),    # own block only
    (800, 8, 2, 64, 4, "bf16", 1),     # group-shared routing
    (3072, 4, 1, 512, 3, "bf16", 0),   # G = 4, several query chunks and key tiles per block
    (2300, 4, 2, 200, 5, "bf16", 0),   # key tiles with ragged 32-key groups, partial last block
    (12, 2, 1, 4, 3, "bf16", 0),       # lse from the few-row forward path
    (12288, 4, 1, 4096, 12, "bf16", 0),  # the 1M-token layer's block shape (B = 4096, k = 12, G = 4)
]


def _grad_close(got, ref, dtype, what):
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-4 * scale, f"{what}: max err {err.max():.3e} vs |g| {scale:.3e}"
    else:
        assert err.max() <= 2e-2 * scale, f"{what}: max err {err.max():.3e} vs |g| {scale:.3e}"
        assert err.mean() <= 2e-3 * scale, f"{what}: mean err {err.mean():.3e} vs |g| {scale:.3e}"
    return float(err.max() / scale)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N,Hq,Hkv,B,topk,dtype,routing", BWD)
def test_backward_matches_oracle(N, Hq, Hkv, B, topk, dtype, routing):
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + 5 * topk, dtype=dtype)
    scale = 0.09
    o, lse = moba.prefill_train(tq, tk, tv, B, topk, scale, routing=routing)
    o_plain = moba.prefill(tq, tk, tv, B, topk, scale, routing=routing)
    assert torch.equal(o, o_plain)
    gen = torch.Generator(device="cpu").manual_seed(N)
    dout = torch.randn(tq.shape, generator=gen).to(tq.dtype).to(DEV)
    dq, dk, dv = moba.backward(tq, tk, tv, o, lse, dout, B, topk, scale, routing=routing)
    sel = moba.select(tq, tk, B, topk, routing=routing).cpu().numpy()
    rq, rk, rv = oracle.backward(q, k, v, to_np(dout), B, topk, scale=scale, sel=sel)
    worst = [_grad_close(to_np(dq), rq, dtype, "dq"), _grad_close(to_np(dk), rk, dtype, "dk"),
             _grad_close(to_np(dv), rv, dtype, "dv")]
    print(f"backward {N},{Hq},{Hkv},{B},{topk},{dtype},{routing}: max err / max|g| {worst}")


def test_backward_bf16_is_deterministic():
    """The bf16 backward sums dq from per-slot partials (no atomics), so two
    runs on the same inputs agree bit for bit."""
    N, Hq, Hkv, B, topk = 1500, 4, 2, 128, 4
    _, _, _, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=77, dtype="bf16")
    o, lse = moba.prefill_train(tq, tk, tv, B, topk, 0.09)
    gen = torch.Generator(device="cpu").manual_seed(3)
    dout = torch.randn(tq.shape, generator=gen).to(tq.dtype).to(DEV)
    a = moba.backward(tq, tk, tv, o, lse, dout, B, topk, 0.09)
    b = moba.backward(tq, tk, tv, o, lse, dout, B, topk, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


BWD_VARLEN = [
    # lengths, Hq, Hkv, B, topk, dtype
    ([700, 0, 1, 1300, 513], 4, 2, 128, 3, "bf16"),
    ([300, 900, 5], 4, 1, 96, 4, "bf16"),   # B not a multiple of 64
    ([400, 1, 600], 2, 2, 64, 3, "f32"),
]


@pytest.mark.parametrize("lens,Hq,Hkv,B,topk,dtype", BWD_VARLEN)
def test_backward_varlen_matches_each_sequence(lens, Hq, Hkv, B, topk, dtype):
    """Training on packed sequences: the packed forward (with row statistics)
    equals the packed inference forward, and the packed gradients equal the
    oracle's gradients of every sequence on its own."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = int(cu[-1])
    q, k, v, tq, tk, tv = small(N, Hq, Hkv, B, topk, seed=N + 11, dtype=dtype)
    scale = 0.09
    o, lse = moba.prefill_train_varlen(tq, tk, tv, cu, B, topk, scale)
    assert torch.equal(o, moba.prefill_varlen(tq, tk, tv, cu, B, topk, scale))
    gen = torch.Generator(device="cpu").manual_seed(N)
    dout = torch.randn(tq.shape, generator=gen).to(tq.dtype).to(DEV)
    dq, dk, dv = moba.backward_varlen(tq, tk, tv, o, lse, dout, cu, B, topk, scale)
    sel = moba.select_varlen(tq, tk, cu, B, topk).cpu().numpy()
    rq, rk, rv = np.zeros_like(to_np(dq)), np.zeros_like(to_np(dk)), np.zeros_like(to_np(dv))
    d_np = to_np(dout)
    base = 0  # first global block of the sequence
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            loc = sel[a:b].copy()
            loc[loc >= 0] -= base
            rq[a:b], rk[a:b], rv[a:b] = oracle.backward(q[a:b], k[a:b], v[a:b], d_np[a:b], B,
                                                        topk, scale=scale, sel=loc)
        base += -(-(b - a) // B)
    _grad_close(to_np(dq), rq, dtype, "dq")
    _grad_close(to_np(dk), rk, dtype, "dk")
    _grad_close(to_np(dv), rv, dtype, "dv")


def test_mfma_probe_runs_every_op():
    """The matrix-core probe's per-lane checksum is exactly 16 * iters when
    every one of its ops ran (operands 0.125, sums exact in fp32)."""
    for wgs, iters in ((3, 1), (512, 100), (1, 1 << 20)):
        out = torch.full((wgs * 256,), -1.0, dtype=torch.float32, device=DEV)
        moba.debug_mfma_peak(out, iters)
        torch.cuda.synchronize()
        assert bool((out == 16.0 * iters).all()), (wgs, iters)


def test_read_probe_sees_every_word():
    """The read probe's outputs XOR to the XOR of every 32-bit word of its
    input, for sizes that leave ragged last rounds and for more workgroups
    than rounds."""
    g = np.random.default_rng(7)
    for words, wgs in ((4, 1), (4 * 1024 * 3 + 8, 2), (4 * 1000, 64), (1 << 22, 37)):
        host = g.integers(-2**31, 2**31, size=words, dtype=np.int64).astype(np.int32)
        src = torch.from_numpy(host).to(DEV)
        out = torch.zeros(wgs * 256, dtype=torch.int32, device=DEV)
        moba.debug_read_peak(src, out)
        got = np.bitwise_xor.reduce(out.cpu().numpy())
        assert got == np.bitwise_xor.reduce(host), (words, wgs)
