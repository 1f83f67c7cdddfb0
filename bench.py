#!/usr/bin/env python3
"""MoBA prefill benchmark on one MI355X.

One step = one ``moba_prefill`` call (all five stages: meanpool, gate + top-k,
bucketing, history attention, own-block attention + merge) over one layer of
synthetic input already resident in HBM. Default workload: the 1M-token
Llama-3.1-8B-shaped layer (N=1,048,576, 32 query heads over 8 KV heads,
d=128, B=4096, k=12, bf16).

Prints one JSON line with tokens/s, attended TFLOP/s against the bf16 MFMA
peak, per-stage times (hipEvents recorded on the library's stream), the
dominant kernel's roofline, the dense causal baseline on the same GPU and the
fp64 CPU oracle timed on a bounded row sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_long_meanpool_amd as moba  # noqa: E402
import synth  # noqa: E402

METRIC = "MoBA prefill tokens/s per layer + attended TFLOP/s (% of bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
STAGES = moba.STAGES


def pair_counts(w, lens=None):
    """Exact attended (query, key) pairs per head: own block causal + full history
    blocks, summed over the packed sequences ``lens`` (default: one of w.N rows)."""
    KH = w.k - 1
    own = hist = 0
    for L in (lens if lens is not None else [w.N]):
        for c in range(-(-int(L) // w.B)):
            rows = min(w.B, int(L) - c * w.B)
            own += rows * (rows + 1) // 2
            hist += rows * min(KH, c) * w.B
    return own, hist


def algorithmic_bytes(w):
    """Bytes a stage must move at minimum (per launch)."""
    nh = w.n - 1
    meanpool = w.N * w.Hkv * w.d * 2 + nh * w.Hkv * w.d * 8
    KH = w.k - 1
    entries = 0
    for c in range(w.n):
        rows = min(w.B, w.N - c * w.B)
        entries += rows * min(KH, c) * w.Hq
    bucket = 2 * w.N * w.Hq * w.k * 4 + 4 * entries + 4 * (w.Hkv * nh + 1)
    return meanpool, bucket, entries


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def read_traffic(kernel_tag):
    """HBM bytes per launch from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    src = fields.get("kernel_source_sha256")
    if src is None or "hbm_bytes_per_launch" not in fields:
        return None
    import hashlib
    cur = hashlib.sha256(open(os.path.join(ROOT, fields["kernel_source"]), "rb").read()).hexdigest()
    return float(fields["hbm_bytes_per_launch"]) if cur == src else None


def _best_ms(fn, reps=5):
    """Best of ``reps`` calls of ``fn`` timed by events on torch's current
    stream (the stream the binding launches on)."""
    fn()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best


def measured_peaks():
    """Measured denominators beside the published ones: the matrix-core
    issue-rate probe (four waves per workgroup, 2, 3 or 6 workgroups per
    compute unit, the best of the three), the read-only stream probe over
    2 GiB (4, 8 or 16 workgroups per compute unit, the best) and the plain
    copy kernel over 2 GiB (read + write bytes)."""
    best_tf, shape = 0.0, None
    for per_cu in (2, 3, 6):
        wgs = 256 * per_cu
        iters = 16384 * 512 // wgs
        out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        ms = _best_ms(lambda: moba.debug_mfma_peak(out, iters))
        if not bool((out == 16.0 * iters).all()):
            raise RuntimeError("matrix-core probe: checksum mismatch")
        tf = wgs * 4 * iters * 4 * 32768 / (ms / 1e3) / 1e12
        if tf > best_tf:
            best_tf, shape = tf, f"{wgs} workgroups x 4 waves x {iters} rounds of 4 ops"
        del out
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms = _best_ms(lambda: moba.debug_copy(src, dst))
    if not torch.equal(src, dst):
        raise RuntimeError("copy probe: wrong result")
    copy_gbps = 2 * nbytes / (ms / 1e3) / 1e9
    del dst
    best_rd, rd_shape = 0.0, None
    for per_cu in (4, 8, 16):
        out = torch.empty(256 * per_cu * 256, dtype=torch.int32, device="cuda")
        ms = _best_ms(lambda: moba.debug_read_peak(src, out))
        # src holds 2^29 words of 1: their XOR is 0
        if int(np.bitwise_xor.reduce(out.cpu().numpy())) != 0:
            raise RuntimeError("read probe: checksum mismatch")
        gbps = nbytes / (ms / 1e3) / 1e9
        if gbps > best_rd:
            best_rd, rd_shape = gbps, f"{256 * per_cu} workgroups x 256 threads"
        del out
    del src
    return {"mfma_bf16_tflops": best_tf, "mfma_probe": shape,
            "hbm_read_gbps": best_rd,
            "hbm_read_probe": f"2 GiB read once, 16-byte loads, four in flight per thread, "
                              f"{rd_shape}",
            "hbm_copy_gbps": copy_gbps,
            "hbm_copy_probe": "16-byte grid-stride copy of 2 GiB; bytes = read + write"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_sample(w, rows_wanted):
    """The seeded (row, head) pairs of the CPU leg: every block, both edges."""
    rows, heads = synth.sample_rows(w, 4096)
    pick = np.linspace(0, len(rows) - 1, min(rows_wanted, len(rows))).astype(np.int64)
    return rows[pick], heads[pick]


def cpu_baseline(w, q, k, v, rows_wanted, gpu=None):
    """The oracle timed on the host over a seeded sample of (row, head) pairs;
    with ``gpu = (sel, o)``, the timed steps' selection and output at those
    pairs (fetched after the timed region), the same evaluation also gives
    the parity figures of the bench line."""
    import oracle  # the fp64 oracle: this leg only
    rows, heads = cpu_sample(w, rows_wanted)
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    kbar = oracle.block_means(k, w.B)
    t1 = time.perf_counter()
    ref_sel, ref_o, gap = oracle.rows(q, k, v, w.B, w.k, rows, heads, scale=w.scale, kbar=kbar,
                                      nthreads=threads)
    t2 = time.perf_counter()
    tok_s = (len(rows) / w.Hq) / (t2 - t1)
    parity = None
    if gpu is not None:
        got_sel, got_o = gpu
        same = (got_sel == ref_sel).all(axis=1)
        d = np.abs(got_o - ref_o)[same]
        parity = {"pairs": int(len(rows)), "selection_equal_pairs": int(same.sum()),
                  "selection_differs_pairs": int((~same).sum()),
                  "max_abs_dO": float(d.max()) if d.size else None,
                  "mean_abs_dO": float(d.mean()) if d.size else None,
                  "bars": "bf16: max <= 1e-2, mean <= 1e-3 (the GPU tests' bars)",
                  "note": "fp64 oracle on the seeded sample (every block, both block edges), "
                          "against the last timed step's O; |dO| over the pairs whose selection "
                          "equals the oracle's"}
    return {
        "value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "cpu_model": _cpu_model(),
        "extrapolated_layer_hours": w.N / tok_s / 3600.0,
        "sample": (f"{len(rows)} seeded (row, head) pairs of the same layer spread over all blocks; "
                   f"value = pairs/{w.Hq} per second of the fp64 dense-masked row evaluation; the "
                   f"one-time fp64 block means took {t1 - t0:.2f} s and are not in the rate"),
    }, parity


def routing_summary(st, w):
    """Summaries of moba_routing_stats over the whole layer: the histogram of
    selection margins (last kept minus best left-out gate score, absolute,
    per (row, head)), rows inside the tie band, how much the heads of one
    group agree and how the selections spread over blocks."""
    margin = st["margin"].float()
    fin = margin[torch.isfinite(margin)]
    edges = [0.0, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2, 1e-1, 1.0, 10.0, float("inf")]
    hist = [int(((fin >= a) & (fin < b)).sum()) for a, b in zip(edges[:-1], edges[1:])]
    G = w.Hq // w.Hkv
    rows = torch.arange(w.N, device=margin.device)
    hist_sel = torch.clamp(rows // w.B, max=w.k - 1)  # history blocks per (row, head)
    union = st["union_size"].float()
    full = hist_sel.float().unsqueeze(1) * G  # union if the G heads chose disjoint sets
    has = hist_sel > 0
    overlap = (union[has] / full[has].clamp(min=1)).mean()
    counts = st["counts"].double()
    tot = counts.sum(dim=1, keepdim=True)
    n = counts.shape[1]
    # selections a block could receive: its later rows x heads of the group
    nh = n - 1
    per_block = counts[:, :nh]
    top = torch.sort(per_block.flatten(), descending=True).values
    return {
        "margin_histogram": {"edges": edges[:-1] + ["inf"], "counts": hist,
                             "nothing_left_out": int((~torch.isfinite(margin)).sum())},
        "median_selection_margin": float(fin.median()) if fin.numel() else None,
        "tie_band_pairs_1e-5_abs": int((fin < 1e-5).sum()),
        "group_union_over_disjoint": float(overlap),
        "group_union_note": f"distinct history blocks of a KV head's {G} query heads / "
                            f"({G} x their history count): 1/{G} = all heads agree, 1 = disjoint",
        "block_frequency": {
            "history_selections": int(tot.sum()),
            "max_over_mean": float(per_block.max() / per_block.mean()),
            "top_1pct_share": float(top[: max(1, top.numel() // 100)].sum() / top.sum()),
            "never_selected_blocks": int((per_block == 0).sum()),
            "block0_share": float(per_block[:, 0].sum() / per_block.sum()),
        },
    }


def small_configs():
    """Per-stage times of the smaller parity configurations (secondary rows:
    launch-bound, reported rather than targeted)."""
    rows = {}
    for name in ("tiny2k", "mha8k", "mha32k_needles", "coarse32k"):
        ws_ = synth.CONFIGS[name]
        dt = "bf16" if ws_.dtype == "bf16" else "f32"
        a, b, c = (to_dev(x) for x in synth.make_qkv(ws_, dt))
        pr = moba.make_problem(ws_.N, ws_.Hq, ws_.Hkv, ws_.d, ws_.B, ws_.k, ws_.scale,
                               moba.MOBA_DTYPE_BF16 if dt == "bf16" else moba.MOBA_DTYPE_F32)
        wsp = moba.alloc_workspace(moba.workspace_size(pr), a.device)
        o = torch.empty_like(a)
        nev = moba.stage_events(pr)
        passes = (nev - 5) // 2
        for _ in range(3):
            moba.prefill(a, b, c, ws_.B, ws_.k, ws_.scale, out=o, workspace=wsp)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(10)]
        for ev in evs:
            moba.prefill(a, b, c, ws_.B, ws_.k, ws_.scale, out=o, workspace=wsp, events=ev)
        torch.cuda.synchronize()
        span = {s: [(i, i + 1)] for i, s in enumerate(STAGES[:4])}
        span["attn_hist"] = [(4 + 2 * i, 5 + 2 * i) for i in range(passes)]
        span["attn_self_merge"] = [(5 + 2 * i, 6 + 2 * i) for i in range(passes)]
        st = {s: float(np.median([sum(ev[x].elapsed_time(ev[y]) for x, y in span[s])
                                  for ev in evs])) for s in STAGES}
        tot = float(np.median([ev[0].elapsed_time(ev[-1]) for ev in evs]))
        own, hist = pair_counts(ws_)
        rows[name] = {"workload": f"N={ws_.N} Hq={ws_.Hq} Hkv={ws_.Hkv} d={ws_.d} B={ws_.B} "
                                  f"topk={ws_.k} {dt}",
                      "ms": tot, "tokens_per_s": ws_.N / (tot / 1e3),
                      "attended_tflops": 4.0 * ws_.d * ws_.Hq * (own + hist) / (tot / 1e3) / 1e12,
                      "stage_ms": st, "timing": "median of 10 event-timed calls"}
        del a, b, c, o, wsp
    return rows


def backward_leg(name="mha32k_needles", reps=5):
    """Training leg: forward with row statistics, then the backward pass (each
    the mean of `reps` calls), on the 32K layer or on the 128K-row GQA layer."""
    wb = synth.CONFIGS[name]
    bq, bk, bv = (to_dev(a) for a in synth.make_qkv(wb, "bf16"))
    gen = torch.Generator(device="cpu").manual_seed(1)
    dout = torch.randn(bq.shape, generator=gen).to(torch.bfloat16).to(bq.device)
    o_b, lse_b = moba.prefill_train(bq, bk, bv, wb.B, wb.k, wb.scale)
    moba.backward(bq, bk, bv, o_b, lse_b, dout, wb.B, wb.k, wb.scale)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(reps):
        o_b, lse_b = moba.prefill_train(bq, bk, bv, wb.B, wb.k, wb.scale)
    e1.record()
    for _ in range(reps):
        moba.backward(bq, bk, bv, o_b, lse_b, dout, wb.B, wb.k, wb.scale)
    e2.record()
    torch.cuda.synchronize()
    fms, bms = e0.elapsed_time(e1) / reps, e1.elapsed_time(e2) / reps
    bown, bhist = pair_counts(wb)
    pairs = wb.Hq * (bown + bhist)
    backward = {"workload": f"{wb.name}: N={wb.N} Hq={wb.Hq} Hkv={wb.Hkv} d={wb.d} B={wb.B} "
                            f"topk={wb.k}, bf16",
                "forward_train_ms": fms, "backward_ms": bms,
                "backward_tflops": 10.0 * wb.d * pairs / (bms / 1e3) / 1e12,
                "note": f"mean of {reps} calls; matrix cores, bf16 operands, fp32 accumulation; "
                        "the backward call recomputes the selection and its buckets; "
                        "FLOP = 5 products of 2d per attended pair"}
    del bq, bk, bv, dout, o_b, lse_b
    return backward


def chunk_leg(w, tq, tk, tv, prob):
    """Chunked prefill and decode over the layer's KV cache: one decode step
    and a 16,384-row chunk recomputing the block means, and the decode step
    on a decode cache."""
    chunk = {}
    for C in (1, 16384):
        qc = tq[w.N - C:].contiguous()
        oc = torch.empty_like(qc)
        wsc = moba.alloc_workspace(moba.chunk_workspace_size(prob, C), tq.device)
        moba.prefill_chunk(qc, tk, tv, w.B, w.k, w.scale, out=oc, workspace=wsc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5 if C == 1 else 2
        e0.record()
        for _ in range(reps):
            moba.prefill_chunk(qc, tk, tv, w.B, w.k, w.scale, out=oc, workspace=wsc)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        chunk["decode_step" if C == 1 else f"chunk_{C}"] = {
            "query_rows": C, "cache_rows": w.N, "ms": cms, "tokens_per_s": C / (cms / 1e3)}
        if C == 1:
            o_recompute = oc.clone()
        del wsc, oc
    # the same decode step on a decode cache: append the new row (its block
    # means only when it completes a block; its V column), then the step
    cache = moba.DecodeCache(w.N, w.Hq, w.Hkv, w.B, w.k, w.scale, device=tq.device)
    cache.append(tk, tv, w.N - 1)
    qd = tq[w.N - 1:].contiguous()
    od = torch.empty_like(qd)
    cache.rows = w.N - 1
    cache.append(tk, tv, w.N)
    wsd = moba.alloc_workspace(cache.workspace_size(1), tq.device)

    def cached_step():
        cache.rows = w.N - 1
        cache.append(tk, tv, w.N)
        cache.prefill(qd, tk, tv, out=od, workspace=wsd)

    cached_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        cached_step()
    e1.record()
    torch.cuda.synchronize()
    cms = e0.elapsed_time(e1) / reps
    # algorithmic bytes of a decode step: K and V rows of every selected block
    # (k - 1 full history blocks and the own block up to the row) of every head
    pos = w.N - 1
    own = pos - (pos // w.B) * w.B + 1
    sel_keys = (min(w.k - 1, pos // w.B) * w.B + own) * w.Hq
    dec_bytes = sel_keys * 2 * w.d * 2
    chunk["decode_step_cached"] = {
        "query_rows": 1, "cache_rows": w.N, "ms": cms, "tokens_per_s": 1 / (cms / 1e3),
        "selected_kv_bytes": dec_bytes, "step_gbps": dec_bytes / (cms / 1e3) / 1e9,
        "matches_recompute": bool(torch.equal(od, o_recompute)),
        "note": "moba_cache_append of the new row + moba_prefill_cached"}
    del cache, wsd, od
    return chunk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama8b_1m", choices=sorted(synth.CONFIGS))
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-small", action="store_true",
                    help="skip the per-stage rows of the smaller parity configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed-batch leg (16 sequences, same total rows)")
    ap.add_argument("--no-chunk", action="store_true",
                    help="skip the decode-step and chunked-prefill legs over the same KV cache")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training leg (forward with statistics + backward) on the 32K layer")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the group-shared routing leg and the routing-statistics timing")
    ap.add_argument("--only", choices=["backward", "chunk"], default=None,
                    help="only run that leg (the training leg on the 32K layer, or the "
                         "chunk / decode leg on the 1M-row cache) and print its JSON object")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured matrix-core and HBM-stream denominators")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run the plain copy kernel over this many MiB (hardware-counter "
                         "calibration of FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MoBA prefill path here runs on a single "
              "MI355X (a split by KV-head group across GPUs is not built).",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        moba.debug_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        print(json.dumps({"copy_bytes": nbytes}), flush=True)
        return

    if args.only == "backward":
        print(json.dumps({"backward": backward_leg(),
                          "backward_llama8b_128k": backward_leg("llama8b_128k", reps=3)}),
              flush=True)
        return

    w = synth.CONFIGS[args.config]
    dtype = "bf16" if w.dtype == "bf16" else "f32"
    t0 = time.perf_counter()
    q, k, v = synth.make_qkv(w, dtype)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    gen_s = time.perf_counter() - t0
    out = torch.empty_like(tq)
    prob = moba.make_problem(w.N, w.Hq, w.Hkv, w.d, w.B, w.k, w.scale,
                             moba.MOBA_DTYPE_BF16 if dtype == "bf16" else moba.MOBA_DTYPE_F32)
    if args.only == "chunk":
        print(json.dumps({"chunked": chunk_leg(w, tq, tk, tv, prob)}), flush=True)
        return
    ws = moba.alloc_workspace(moba.workspace_size(prob), tq.device)
    print(f"[bench] {w.name}: inputs ready in {gen_s:.1f} s, workspace {ws.numel() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    def step(ev=None):
        moba.prefill(tq, tk, tv, w.B, w.k, w.scale, out=out, workspace=ws, events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = moba.stage_events(prob)
    passes = (nev - 5) // 2  # attention passes over groups of KV heads
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
           for _ in range(args.steps)]
    for ev in evs:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # the four stages before attention, then history attention and own-block
    # attention + merge, each summed over the attention passes
    spans = {s: [(i, i + 1)] for i, s in enumerate(STAGES[:4])}
    spans["attn_hist"] = [(4 + 2 * i, 5 + 2 * i) for i in range(passes)]
    spans["attn_self_merge"] = [(5 + 2 * i, 6 + 2 * i) for i in range(passes)]
    stage_ms = {s: float(np.mean([sum(ev[a].elapsed_time(ev[b]) for a, b in spans[s])
                                  for ev in evs])) for s in STAGES}
    event_ms = float(np.mean([ev[0].elapsed_time(ev[-1]) for ev in evs]))
    print(f"[bench] {args.steps} steps: {ms_per_step:.2f} ms/step, stages {stage_ms}",
          file=sys.stderr, flush=True)

    gpu_sample = None
    if not args.no_cpu_baseline:
        # the timed steps' output and selection at the CPU leg's pairs, read
        # back now (later legs reuse the output buffer)
        srows, sheads = cpu_sample(w, args.cpu_rows)
        ir, ih = torch.from_numpy(srows).to(tq.device), torch.from_numpy(sheads.astype(np.int64)).to(tq.device)
        got_o = out[ir, ih].double().cpu().numpy()
        selt = moba.select(tq, tk, w.B, w.k)
        got_sel = selt[ir, ih].cpu().numpy()
        del selt
        gpu_sample = (got_sel, got_o)

    own, hist = pair_counts(w)
    flop_total = 4.0 * w.d * w.Hq * (own + hist)
    flop_hist = 4.0 * w.d * w.Hq * hist
    tokens_s = w.N / (ms_per_step / 1e3)
    tflops = flop_total / (ms_per_step / 1e3) / 1e12
    hist_tflops = flop_hist / (stage_ms["attn_hist"] / 1e3) / 1e12
    mp_bytes, bk_bytes, entries = algorithmic_bytes(w)

    dense = None
    if not args.no_dense:
        od = torch.empty_like(tq)
        moba.dense_causal(tq, tk, tv, w.scale, out=od)  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moba.dense_causal(tq, tk, tv, w.scale, out=od)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        dense_flop = 4.0 * w.d * w.Hq * (w.N * (w.N + 1) // 2)
        dense = {"ms": dms, "tflops": dense_flop / (dms / 1e3) / 1e12,
                 "speedup_moba_vs_dense": dms / ms_per_step}
        del od

    varlen = None
    if not args.no_varlen and dtype == "bf16":
        lens = synth.packed_layer_lengths(w)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))
        cu_dev = cu.to(tq.device)
        del ws  # the packed leg gets its own workspace
        wsv = moba.alloc_workspace(moba.varlen_workspace_size(prob, cu), tq.device)
        moba.prefill_varlen(tq, tk, tv, cu_dev, w.B, w.k, w.scale, out=out, workspace=wsv)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(2):
            moba.prefill_varlen(tq, tk, tv, cu_dev, w.B, w.k, w.scale, out=out, workspace=wsv)
        e1.record()
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / 2
        vown, vhist = pair_counts(w, lens)
        varlen = {"workload": f"{len(lens)} packed sequences of {int(lens.min())}..{int(lens.max())} "
                              f"rows (seeded log-uniform), {w.N} rows in all, same layer shape",
                  "ms": vms, "tokens_per_s": w.N / (vms / 1e3),
                  "attended_tflops": 4.0 * w.d * w.Hq * (vown + vhist) / (vms / 1e3) / 1e12}
        del wsv

    chunk = None
    if not args.no_chunk and dtype == "bf16":
        chunk = chunk_leg(w, tq, tk, tv, prob)

    shared = None
    if not args.no_shared and dtype == "bf16":
        moba.prefill(tq, tk, tv, w.B, w.k, w.scale, out=out, routing=moba.MOBA_ROUTING_SHARED)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moba.prefill(tq, tk, tv, w.B, w.k, w.scale, out=out, routing=moba.MOBA_ROUTING_SHARED)
        e1.record()
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1)
        e0.record()
        st = moba.routing_stats(tq, tk, w.B, w.k, routing=moba.MOBA_ROUTING_PER_HEAD)
        e1.record()
        torch.cuda.synchronize()
        stats_ms = e0.elapsed_time(e1)
        shared = {"ms": sms, "tokens_per_s": w.N / (sms / 1e3),
                  "routing_stats_ms": stats_ms,
                  "routing_stats": routing_summary(st, w)}
        del st

    backward = backward_large = None
    if not args.no_backward and dtype == "bf16":
        backward = backward_leg()
        backward_large = backward_leg("llama8b_128k", reps=3)

    small = None if args.no_small else small_configs()

    peaks = None if args.no_peaks else measured_peaks()

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(w, q, k, v, args.cpu_rows, gpu_sample)

    rec = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, per-block key offsets std 0.5)",
        "config": {"workload": f"{w.name}: MoBA prefill layer N={w.N} Hq={w.Hq} Hkv={w.Hkv} "
                               f"d={w.d} B={w.B} topk={w.k}",
                   "seq_len": w.N, "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.d,
                   "block_size": w.B, "topk": w.k, "parallelism": "none (1 GPU)"},
        "attended_tflops": tflops,
        "attended_frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "stage_ms": stage_ms,
        "events_total_ms": event_ms,
        "meanpool_gbps": mp_bytes / (stage_ms["meanpool"] / 1e3) / 1e9,
        "meanpool_frac_of_hbm_peak": mp_bytes / (stage_ms["meanpool"] / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "bucket_gbps": bk_bytes / (stage_ms["bucket"] / 1e3) / 1e9,
        "bucket_frac_of_hbm_peak": bk_bytes / (stage_ms["bucket"] / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "measured_peaks": peaks,
        "meanpool_frac_of_measured_read": (mp_bytes / (stage_ms["meanpool"] / 1e3) / 1e9
                                           / peaks["hbm_read_gbps"]) if peaks else None,
        "bucket_frac_of_measured_copy": (bk_bytes / (stage_ms["bucket"] / 1e3) / 1e9
                                         / peaks["hbm_copy_gbps"]) if peaks else None,
        "routed_entries": entries,
        "attention_passes": passes,
        # per launch: 1/passes of the history FLOP over the mean per-pass
        # duration, which is the same ratio as the totals
        "roofline": {"bound": "mfma", "kernel": "attn_hist_q64_bf16",
                     "achieved": hist_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": hist_tflops / PEAK_BF16_TFLOPS,
                     "frac_of_measured_peak": (hist_tflops / peaks["mfma_bf16_tflops"]
                                               if peaks else None),
                     "traffic": read_traffic("attn_hist_llama8b_1m")},
        "dense_causal": dense,
        "varlen": varlen,
        "shared_routing": shared,
        "chunked": chunk,
        "backward": backward,
        "backward_llama8b_128k": backward_large,
        "small_configs": small,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
