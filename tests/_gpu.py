"""Helpers shared by the GPU tests: seeded inputs to device tensors and the
comparison rules against the fp64 oracle."""
import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")

# Tolerances (gate ties, bf16 and fp32 outputs) for the comparisons below.
TIE_REL = 1e-5
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
F32_MAX_ABS = 1e-5


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy bf16 bit patterns (uint16) or float32 -> device tensor of that dtype."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def excused(gap: np.ndarray) -> np.ndarray:
    """Rows whose selection margin is below the tie tolerance (relative)."""
    g, s = gap[:, 0], gap[:, 1]
    return np.isfinite(g) & (g < TIE_REL * s)


def _swaps_inside_tie_band(got_sel, ref_sel, gap, q, k, B, rows, heads, routing):
    """For rows whose selections differ: True where the GPU only swapped blocks
    inside the tie band, i.e. it kept as many history blocks, each block it
    added scores at least the oracle's last kept score minus the tolerance,
    and each block it dropped scores at most the best left-out score plus it
    (scores in fp64 from the oracle's block means)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    kbar = oracle.block_means(k, B)
    ok = np.zeros(len(rows), bool)
    for i in range(len(rows)):
        r, h = int(rows[i]), int(heads[i])
        c = r // B
        g = h // G
        qr = q[r].astype(np.float64) if q.dtype != np.uint16 else _bf16_bits_to_f64(q[r])
        qg = qr[g * G:(g + 1) * G].sum(axis=0) if routing == oracle.ROUTING_SHARED else qr[h]
        hg = {int(b) for b in got_sel[i] if 0 <= b < c}
        hr = {int(b) for b in ref_sel[i] if 0 <= b < c}
        if len(hg) != len(hr) or c not in set(int(b) for b in got_sel[i]):
            continue
        score = {b: float(qg @ kbar[g, b]) for b in hg | hr}
        s_last = min(score[b] for b in hr)
        s_next = s_last - gap[i, 0]
        tol = TIE_REL * gap[i, 1]
        ok[i] = (all(score[b] >= s_last - tol for b in hg - hr)
                 and all(score[b] <= s_next + tol for b in hr - hg))
    return ok


def _bf16_bits_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_selection(got_sel, ref_sel, gap, what="", ctx=None):
    """Selections equal except on tie-excused rows; returns the excused mismatching rows.

    ctx = (q, k, B, rows, heads, routing): on an excused row the GPU may only
    have swapped blocks whose scores lie inside the tie band (checked here);
    without ctx an excused row is accepted on its margin alone."""
    diff = np.any(got_sel != ref_sel, axis=1)
    ex = excused(gap)
    bad = diff & ~ex
    assert not bad.any(), (f"{what}: {bad.sum()} unexcused selection mismatches, e.g. rows "
                           f"{np.flatnonzero(bad)[:5]} got {got_sel[bad][:2]} want {ref_sel[bad][:2]}")
    tied = np.flatnonzero(diff & ex)
    if ctx is not None and tied.size:
        q, k, B, rows, heads, routing = ctx
        ok = _swaps_inside_tie_band(got_sel[tied], ref_sel[tied], gap[tied], q, k, B,
                                    np.asarray(rows)[tied], np.asarray(heads)[tied], routing)
        assert ok.all(), (f"{what}: {(~ok).sum()} excused rows swap blocks outside the tie band, "
                          f"e.g. rows {tied[~ok][:5]}")
    return tied


def check_output(got_o, ref_o, dtype, what=""):
    err = np.abs(got_o - ref_o)
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max |dO| {err.max():.3e} > {F32_MAX_ABS}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max |dO| {err.max():.3e} > {BF16_MAX_ABS}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean |dO| {err.mean():.3e} > {BF16_MEAN_ABS}"
    return float(err.max()), float(err.mean())


def compare_rows(q, k, v, B, topk, scale, rows, heads, got_sel, got_o, dtype, what="",
                 routing=oracle.ROUTING_PER_HEAD):
    """Oracle on (rows, heads); selection bit-exact up to ties, O within tolerance.

    Rows whose selection differs on a tie are re-evaluated by the oracle with
    the GPU's selection forced, and O is checked against that.
    """
    ref_sel, ref_o, gap = oracle.rows(q, k, v, B, topk, rows, heads, scale=scale, routing=routing)
    tied = check_selection(got_sel, ref_sel, gap, what, ctx=(q, k, B, rows, heads, routing))
    if tied.size:
        _, forced_o, _ = oracle.rows(q, k, v, B, topk, rows[tied], heads[tied], scale=scale,
                                     forced_sel=got_sel[tied], routing=routing)
        ref_o = ref_o.copy()
        ref_o[tied] = forced_o
    return check_output(got_o, ref_o, dtype, what), tied.size
