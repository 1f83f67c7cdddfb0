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


def check_selection(got_sel, ref_sel, gap, what=""):
    """Selections equal except on tie-excused rows; returns the excused mismatching rows."""
    diff = np.any(got_sel != ref_sel, axis=1)
    ex = excused(gap)
    bad = diff & ~ex
    assert not bad.any(), (f"{what}: {bad.sum()} unexcused selection mismatches, e.g. rows "
                           f"{np.flatnonzero(bad)[:5]} got {got_sel[bad][:2]} want {ref_sel[bad][:2]}")
    return np.flatnonzero(diff & ex)


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
    tied = check_selection(got_sel, ref_sel, gap, what)
    if tied.size:
        _, forced_o, _ = oracle.rows(q, k, v, B, topk, rows[tied], heads[tied], scale=scale,
                                     forced_sel=got_sel[tied], routing=routing)
        ref_o = ref_o.copy()
        ref_o[tied] = forced_o
    return check_output(got_o, ref_o, dtype, what), tied.size
