"""Benchmark: 128K block-sparse prefill layer + 128K batched decode step on one MI355X.

One step = the whole hot path once:
  prefill (Llama-3.1-8B-shaped layer, 32 query / 8 KV heads, head_dim 128,
  131072 tokens, block 128, per-head budgets with mean 6.25%):
    pool Q and K -> block scores -> per-head top-k (sa_select_blocks)
    -> LPT-ordered persistent block-sparse flash attention (sa_sparse_attn_prefill)
  decode (16 sequences x 131072-token KV cache, 12 streaming + 20 retrieval heads):
    scores against the cached pooled keys -> top-k (sa_select_blocks)
    -> union-of-group split-KV attention + combine (sa_sparse_attn_decode)
The greedy longest-load-first schedule depends only on the budgets, so it is
computed once on the host before timing (it is offline in the method), as is
the pooled-key cache of the decode KV cache.

Prints one JSON line.  `value` is the prefill milliseconds per layer (the
headline of the metric); attended TFLOP/s, decode GB/s and their roofline
fractions are reported beside it.  `roofline` covers the dominant kernel (the
prefill attention), timed with HIP events on the stream it runs on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-workload", default="llama3.1-8b-prefill-128k")
    ap.add_argument("--decode-workload", default="llama3.1-8b-decode-128k-b16")
    ap.add_argument("--bins-per-cu", type=int, default=2)
    ap.add_argument("--queues", type=int, default=8,
                    help="partitions of the prefill work queue (8: one per XCD; 1: one queue)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "all"], default="all")
    ap.add_argument("--calibrate", action="store_true",
                    help="also time the offline budget calibration (block attention mass on the GPU, recovery "
                         "table and max-min shifting on the host) on the 32K prefill workload")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the decode step over the same cache held in 128-token pages")
    ap.add_argument("--tail", action="store_true",
                    help="also measure the schedules' idle tail on the 64K Qwen2.5-72B-shaped layer (the 128K "
                         "layer is always measured)")
    ap.add_argument("--no-tail", action="store_true", help="skip the idle-tail measurement")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the MFMA and HBM-read rates this GPU sustains")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB) so that a "
                         "counter run can scale its HBM byte counters")
    return ap.parse_args()


def timed(fn, stream, reps, scrub=None):
    """Median / mean milliseconds of fn() with events on `stream`.  With
    ``scrub`` (a tensor), it is overwritten before every repetition, outside
    the timed region, so the caches (L2 and the 256 MB MALL) hold none of the
    inputs when fn starts."""
    import torch
    ts = []
    for _ in range(reps):
        if scrub is not None:
            scrub.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2], sum(ts) / len(ts), ts


def graph_timed(fn, stream, reps):
    """Median milliseconds of fn() captured once in a HIP graph and replayed on
    `stream` (the same kernels, without the host's launch path between them)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    ms = timed(g.replay, stream, reps)[0]
    del g
    return ms


def pct(ts, q):
    """q-quantile of sorted samples (nearest rank)."""
    return ts[min(len(ts) - 1, max(0, int(round(q * (len(ts) - 1)))))]


PREFILL_KERNEL_SOURCES = ("sa_prefill.hip", "sa_prefill_common.hpp", "sa_device.hpp")


def prefill_kernel_hash() -> str:
    """sha256 over the source files of the prefill attention kernel, in order."""
    h = hashlib.sha256()
    for name in PREFILL_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "head_heterogeneous_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_peaks(dev, stream, reps=7):
    """The roofline denominators this GPU sustains, from the library's two
    probes, each checked before its rate is used: the bf16 MFMA rate (8
    independent 32x32x16 chains per wave; operands of ones, every accumulator
    ending at an exact value, and pseudo-random operands, checked against the
    fp64 value of the same products) and the HBM streaming-read rate over a 4 GiB buffer (far beyond L2
    and the 256 MB MALL; the XOR of the probe's outputs must match that of the
    buffer).  Best of a few launch shapes, median of `reps` launches each."""
    import numpy as np
    import torch
    from head_heterogeneous_block_amd import metrics as M
    from head_heterogeneous_block_amd import sparse_attn as SA
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}
    # about 10 ms per launch, as long as the attention kernel, so the rate is
    # the one the chip holds at the clock its power limit allows under a
    # sustained matrix load, not a short burst at the boost clock
    iters = 45056
    best = None
    for per_cu in (1, 2):
        n_wg = n_cu * per_cu
        sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
        fl = SA.sa_measure_mfma_peak(n_wg, iters, sink)  # warm
        ms = timed(lambda: SA.sa_measure_mfma_peak(n_wg, iters, sink), stream, reps)[0]
        if not bool((sink == 128.0 * iters).all()):
            raise RuntimeError("MFMA probe: wrong accumulator values")
        rate = fl / (ms * 1e-3) / 1e12
        if best is None or rate > best[0]:
            best = (rate, n_wg, ms)
    out["mfma_bf16_tflops"] = best[0]
    # 256 CUs x 4 SIMDs x 1024 flops per clock (one 32x32x16 MFMA per 32 clocks)
    out["mfma_implied_clock_ghz"] = best[0] * 1e12 / (n_cu * 4 * 1024) / 1e9
    out["mfma_probe"] = f"{best[1]} workgroups x 4 waves x 8 chains x {iters} v_mfma_f32_32x32x16_bf16, {best[2]:.3f} ms"
    # the same loop on pseudo-random bf16 operands: real data draws more power,
    # and the power limit holds a lower clock (the rate attention can reach)
    best = None
    for per_cu in (1, 2):
        n_wg = n_cu * per_cu
        sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
        fl = SA.sa_measure_mfma_peak(n_wg, iters, sink, operands=1)  # warm
        ms = timed(lambda: SA.sa_measure_mfma_peak(n_wg, iters, sink, operands=1), stream, reps)[0]
        want, scale = M.mfma_probe_random_sink(n_wg, iters)
        if not np.all(np.abs(sink.cpu().double().numpy() - want) <= (iters + 8) * 2.0**-23 * scale + 1e-6):
            raise RuntimeError("MFMA probe (random operands): wrong accumulator values")
        rate = fl / (ms * 1e-3) / 1e12
        if best is None or rate > best[0]:
            best = (rate, n_wg, ms)
    out["mfma_bf16_random_tflops"] = best[0]
    out["mfma_random_implied_clock_ghz"] = best[0] * 1e12 / (n_cu * 4 * 1024) / 1e9
    out["mfma_random_probe"] = (f"{best[1]} workgroups x 4 waves x 8 chains x {iters} v_mfma_f32_32x32x16_bf16 on "
                                f"pseudo-random bf16 operands, {best[2]:.3f} ms")
    nbytes = 4 << 30
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    x = buf
    while x.numel() > 1:  # XOR fold of the whole buffer on the GPU
        h = x.numel() // 2
        x = torch.bitwise_xor(x[:h], x[h:2 * h]) if x.numel() % 2 == 0 else torch.cat(
            [torch.bitwise_xor(x[:h], x[h:2 * h]), x[2 * h:]])
    want = int(x.item())
    del x
    best = None
    for per_cu in (4, 8, 16, 32):
        n_wg = n_cu * per_cu
        sink = torch.empty(n_wg * 256, dtype=torch.int32, device=dev)
        SA.sa_measure_hbm_read(buf, n_wg, sink)
        ms = timed(lambda: SA.sa_measure_hbm_read(buf, n_wg, sink), stream, reps)[0]
        y = sink
        while y.numel() > 1:
            h = y.numel() // 2
            y = torch.bitwise_xor(y[:h], y[h:2 * h])  # n_wg * 256 is a power of two times n_cu
            if y.numel() % 2:
                break
        got = 0
        for v in y.cpu().tolist():
            got ^= v
        if got != want:
            raise RuntimeError("HBM read probe: XOR of the outputs does not match the buffer")
        rate = nbytes / (ms * 1e-3) / 1e9
        if best is None or rate > best[0]:
            best = (rate, n_wg, ms)
    del buf
    torch.cuda.empty_cache()
    out["hbm_read_gbps"] = best[0]
    out["hbm_probe"] = f"4 GiB non-temporal 16-byte reads, {best[1]} workgroups x 256 threads, {best[2]:.3f} ms"
    return out


def traffic_from_profiles():
    """HBM bytes per launch of the prefill attention kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on other kernel code."""
    path = os.path.join(ROOT, "profiles", "prefill_attention_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = prefill_kernel_hash()
    if rec.get("kernel_source_sha256") != h:
        return None
    return rec.get("bytes_per_launch")


def tail_report(spec_name, dev, stream, n_bins, queues, inp=None):
    """How well each schedule fills the chip to the end of the prefill
    attention: launches that record every workgroup's start and end on the
    GPU's constant clock (three per schedule after two warm-up launches, the
    schedules interleaved; the median one is reported).  busy_w = end_w - start_w; span = last end
    - first start; tail idle = 1 - sum(busy) / (slots * span) with slots the
    workgroups the chip runs at once (2 per CU); makespan/mean = max(busy) /
    mean(busy), beside the value the schedule predicts from the block counts
    (the loads)."""
    import numpy as np
    import torch
    from head_heterogeneous_block_amd import sparse_attn as SA
    from head_heterogeneous_block_amd import workloads as W
    spec = W.BY_NAME[spec_name] if isinstance(spec_name, str) else spec_name
    if inp is None:
        inp = W.make_prefill(spec, W.seed_of(spec), device=dev)
    base = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=n_bins, queue=True, queues=queues,
                          queue_group="kv_tiers")
    base.select(inp.q, inp.k)
    o = torch.empty_like(inp.q)
    loads = base.counts.reshape(-1).astype(np.int64)
    lpt_pred = SA.sa_lpt_schedule(loads.tolist(), n_bins)[3]
    plans = {
        "queue_xcd_partitions": (base, float(lpt_pred.max() / lpt_pred.mean())),
        "queue_one": (SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=n_bins, queue=True, queues=1,
                                     queue_group="kv_tiers"), float(lpt_pred.max() / lpt_pred.mean())),
        "queue_flat": (SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=n_bins, queue=True,
                                      queue_group="flat"), float(lpt_pred.max() / lpt_pred.mean())),
        "lpt_bins": (SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=n_bins), None),
        "natural_grid": (SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=0), None),
    }
    out = {"workload": spec.name, "workgroups": n_bins, "slots": n_bins,
           "predicted_note": "queues: makespan/mean of the LPT schedule of the loads onto the workgroups (the "
                             "greedy rule the queue runs online); bins: that of the bins themselves"}
    # every schedule warmed up, then three timed launches each, interleaved
    # across the schedules (no order bias); the median launch is reported
    stamps = {}
    for name, (pl, pred) in plans.items():
        if pl is not base:
            pl.share_tables(base)
        stamps[name] = torch.zeros((pl.grid(), 2), dtype=torch.int64, device=dev)
        for _ in range(2):
            pl.attend(inp.q, inp.k, inp.v, o)
    runs = {name: [] for name in plans}
    for _ in range(3):
        for name, (pl, pred) in plans.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            pl.attend_timed(inp.q, inp.k, inp.v, o, stamps=stamps[name])
            b.record(stream)
            b.synchronize()
            runs[name].append((a.elapsed_time(b), stamps[name].cpu().numpy().astype(np.float64)))
    for name, (pl, pred) in plans.items():
        if name == "lpt_bins":
            pred = float(pl.bin_load.max() / pl.bin_load.mean())
        ms, t = sorted(runs[name], key=lambda r: r[0])[1]
        t0, t1 = t[:, 0].min(), t[:, 1].max()
        busy = t[:, 1] - t[:, 0]
        span = t1 - t0
        rec = {"ms": ms, "ms_runs": [round(r[0], 4) for r in runs[name]], "span_ticks": span,
               "ticks_per_ms": span / ms if ms > 0 else None,
               "busy_idle_tail": 1.0 - busy.sum() / (n_bins * span)}
        if name != "natural_grid":
            rec.update({"busy_ms_p10_p50_p90": [float(np.percentile(busy, q)) / (span / ms) for q in (10, 50, 90)],
                        "busy_spread": float((busy.max() - busy.min()) / busy.mean()),
                        "makespan_over_mean_measured": float(busy.max() / busy.mean()),
                        "makespan_over_mean_predicted": pred,
                        "last_start_to_end_ms": float((t1 - t[:, 0].max()) / (span / ms))})
        else:
            # one workgroup per tile: the chip-wide occupancy over the last tenth of the span
            late = t0 + 0.9 * span
            occ = np.clip(np.minimum(t[:, 1], t1) - np.maximum(t[:, 0], late), 0, None).sum() / (n_bins * 0.1 * span)
            rec.update({"tiles": int(t.shape[0]), "occupancy_last_tenth": float(occ)})
        out[name] = rec
    del plans, base, inp, stamps, runs
    torch.cuda.empty_cache()
    return out


def budget_fit_ablation(pspec, dev, stream, n_bins, queues, reps):
    """The prefill layer under the two other readings of the fixed-total
    budget shift (the inputs' Q, K, V unchanged): "clamp" bisects the common
    factor with every ratio clamped to the stated range, "span" stretches the
    drawn ratios onto the whole range (lowest head at its bottom, highest at its
    top) at the same mean.  Per reading: the ratio range, the attended flops,
    the default schedule's attention time, and the idle-tail report."""
    import numpy as np
    import torch
    from head_heterogeneous_block_amd import metrics as M
    from head_heterogeneous_block_amd import sparse_attn as SA
    from head_heterogeneous_block_amd import workloads as W
    out = {}
    # "span" stretches log-uniform draws; the bimodal and count budgets have no draw range to stretch
    for fit in ("clamp", "span") if pspec.budget_kind == "loguniform" else ("clamp",):
        spec = pspec.with_(budget_fit=fit)
        inp = W.make_prefill(spec, W.seed_of(pspec), device=dev)
        r = np.asarray(inp.budget["ratio_q16"], dtype=np.float64) / 65536.0
        plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=n_bins, queue=True, queues=queues)
        plan.select(inp.q, inp.k)
        o = torch.empty_like(inp.q)
        att = lambda: plan.attend(inp.q, inp.k, inp.v, o)  # noqa: E731
        att()
        ms = timed(att, stream, reps)[0]
        flops = M.prefill_flops(plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy(), spec.seq_len,
                                spec.block, spec.head_dim)
        loads = plan.counts.reshape(-1).astype(np.int64)
        del plan, o
        torch.cuda.empty_cache()
        out[fit] = {"ratio_min": float(r.min()), "ratio_max": float(r.max()), "ratio_mean": float(r.mean()),
                    "attended_flops": flops, "attention_ms": ms, "attended_tflops": flops / (ms * 1e-3) / 1e12,
                    "max_tile_blocks": int(loads.max()),
                    "tail": tail_report(spec, dev, stream, n_bins, queues, inp=inp)}
        del inp
        torch.cuda.empty_cache()
        print(f"[bench] budget fit {fit}: ratios {r.min():.4f}..{r.max():.4f}, attention {ms:.3f} ms",
              file=sys.stderr, flush=True)
    return out


def calibration_timing(dev, stream):
    """Offline budget calibration on the 32K Llama-shaped layer: the block
    attention mass (two dense causal Q K^T passes) on the GPU, then the
    recovery table and the max-min shift to a mean ratio of 1/8 on the host."""
    import numpy as np
    import torch
    from head_heterogeneous_block_amd import sparse_attn as SA
    from head_heterogeneous_block_amd import workloads as W
    spec = W.LLAMA_32K
    inp = W.make_prefill(spec, W.seed_of(spec), device=dev)
    d = SA.make_prefill_desc(inp.q, inp.k, inp.v, inp.q, 128)
    nb = spec.n_blocks
    mass = torch.empty((spec.batch, spec.n_q_heads, nb, nb), dtype=torch.float32, device=dev)
    run = lambda: SA.sa_block_attention_mass(d, inp.q, inp.k, mass)  # noqa: E731
    run()
    ms = timed(run, stream, 3)[0]
    flops = 2 * 2.0 * spec.n_q_heads * spec.head_dim * sum(min(128, spec.seq_len - 128 * m) * (128 * m + 64.5)
                                                           for m in range(nb))
    host = mass.cpu().numpy()
    H = spec.n_q_heads
    bud = {"min_blocks": [2] * H, "ratio_q16": [0] * H, "n_sink": [1] * H, "n_local": [1] * H}
    step = 1024
    t0 = time.perf_counter()
    rec = SA.sa_budget_recovery(host, bud, step)
    t1 = time.perf_counter()
    ratios = SA.sa_budget_shift(rec, step, H * 8192)
    t2 = time.perf_counter()
    rmin = float(min(rec[h, ratios[h] // step - 1] for h in range(H)))
    # the output-aware variant: each head's output deviation from dense
    # attention on a grid of 16 ratios (the path's own prefill at each ratio)
    dstep = 4096
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    dev_tab = SA.deviation_table(inp.q, inp.k, inp.v, bud | {"granularity": [128] * H}, spec.block, dstep)
    t4 = time.perf_counter()
    # quality for the shift: 1 - deviation, as its running best along the grid
    # (a larger budget can swap one block for another and move the output a
    # little more; the shift is defined on tables that do not decrease)
    dshift = SA.sa_budget_shift(np.maximum.accumulate(1.0 - dev_tab, axis=1), dstep, H * 8192)
    return {"workload": spec.name, "mass_ms": ms, "mass_qk_tflops": flops / (ms * 1e-3) / 1e12,
            "recovery_table_host_ms": (t1 - t0) * 1e3, "shift_host_ms": (t2 - t1) * 1e3, "step_q16": step,
            "mean_ratio": 0.125, "lowest_recovery_equal_split": float(rec[:, 8192 // step - 1].min()),
            "lowest_recovery_shifted": rmin,
            "ratio_range": [int(np.min(ratios)), int(np.max(ratios))],
            "deviation_table_ms": (t4 - t3) * 1e3, "deviation_step_q16": dstep,
            "deviation_at_mean_ratio": [float(dev_tab[:, 8192 // dstep - 1].min()),
                                        float(dev_tab[:, 8192 // dstep - 1].max())],
            "deviation_shift_ratio_range": [int(np.min(dshift)), int(np.max(dshift))]}


def cpu_baseline_prefill(inp, block_idx, block_cnt, tiles_per_head=96, select_heads=(0, 4, 8, 12, 16, 20, 24, 28)):
    """The fp64 oracle on a bounded sample of the prefill workload, scaled to ms
    per layer: selection (pool, score, top-k over every query block) for a few
    query heads, scaled by the head count; attention for evenly spaced tiles of
    every query head, scaled by attended pairs."""
    import numpy as np
    import oracle as O
    from head_heterogeneous_block_amd import metrics as M
    from head_heterogeneous_block_amd import workloads as W
    spec = inp.spec
    G = spec.group
    t_sel = 0.0
    for h in select_heads:
        q = W.to_numpy(inp.q[:, [h]])
        k = W.to_numpy(inp.k[:, [h // G]])
        bud = {k2: np.asarray(v2)[[h]] for k2, v2 in inp.budget.items()}
        t0 = time.perf_counter()
        O.select_blocks_prefill(q, k, bud, spec.block)
        t_sel += time.perf_counter() - t0
    nb = spec.n_blocks
    ms = np.unique(np.linspace(0, nb - 1, tiles_per_head).astype(int))
    t_att = 0.0
    mask = np.zeros_like(block_cnt)
    for h in range(spec.n_q_heads):
        q = W.to_numpy(inp.q[:, [h]])
        k = W.to_numpy(inp.k[:, [h // G]])
        v = W.to_numpy(inp.v[:, [h // G]])
        t0 = time.perf_counter()
        O.attention_prefill_gather(q, k, v, block_idx[:, [h]], block_cnt[:, [h]], spec.block,
                                   tiles=[(0, 0, int(m)) for m in ms])
        t_att += time.perf_counter() - t0
        mask[0, h, ms] = block_cnt[0, h, ms]
    pairs_sample = M.prefill_pairs(block_idx, mask, spec.seq_len, spec.block)
    pairs_all = M.prefill_pairs(block_idx, block_cnt, spec.seq_len, spec.block)
    total_s = t_sel * spec.n_q_heads / len(select_heads) + t_att * pairs_all / pairs_sample
    desc = (f"selection of query heads {list(select_heads)} (all {nb} query blocks each) scaled by "
            f"{spec.n_q_heads}/{len(select_heads)}; attention of {len(ms)} evenly spaced query blocks of each of "
            f"the {spec.n_q_heads} heads ({pairs_sample / pairs_all:.2%} of attended pairs) scaled by attended pairs")
    return total_s * 1e3, t_sel + t_att, desc


def cpu_baseline_decode(inp, block_idx, block_cnt):
    """The oracle decode step for one sequence, scaled by the batch size."""
    import oracle as O
    from head_heterogeneous_block_amd import workloads as W
    q = W.to_numpy(inp.q[[0]])
    k = W.to_numpy(inp.k[[0]])
    v = W.to_numpy(inp.v[[0]])
    t0 = time.perf_counter()
    O.decode_select(q, k, inp.budget)
    O.decode_attention(q, k, v, block_idx[[0]], block_cnt[[0]], inp.budget["granularity"])
    dt = time.perf_counter() - t0
    return dt * inp.spec.batch * 1e3, dt


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the block-sparse path is a "
              "single-GPU path with no multi-GPU leg", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from head_heterogeneous_block_amd import metrics as M
    from head_heterogeneous_block_amd import sparse_attn as SA
    from head_heterogeneous_block_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] calibration copy: 1 GiB read + 1 GiB written (torch.neg)", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- prefill
    pspec = W.BY_NAME[args.prefill_workload]
    t0 = time.time()
    pin = W.make_prefill(pspec, W.seed_of(pspec), device=dev)
    torch.cuda.synchronize()
    print(f"[bench] prefill inputs {pspec.name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    n_bins = n_cu * args.bins_per_cu
    t0 = time.perf_counter()
    # work queue: n_bins persistent workgroups take the tiles in the order the
    # library picks for the size (SA_QUEUE_AUTO): beyond 256 query blocks per
    # head, load tiers, heaviest tier first, grouped by (sequence, KV head)
    # inside a tier and cut into one partition per XCD; up to 256, plain
    # longest first on one queue
    plan = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                          queues=args.queues)
    default_order = ("load tiers, %d XCD partitions" % (len(plan.queue_offsets) - 1) if plan.queue_offsets is not None
                     else "one queue (the library's choice for this size)")
    lpt_ms = (time.perf_counter() - t0) * 1e3
    o = torch.empty_like(pin.q)
    sel = lambda: plan.select(pin.q, pin.k)  # noqa: E731
    att = lambda: plan.attend(pin.q, pin.k, pin.v, o)  # noqa: E731

    # ---------------------------------------------------------------- decode
    dspec = W.BY_NAME[args.decode_workload]
    if args.only in ("decode", "all"):
        t0 = time.time()
        din = W.make_decode(dspec, W.seed_of(dspec), device=dev)
        dplan = SA.DecodePlan(din.q, din.k, din.v, din.budget)
        dplan.pool(din.k)
        do = torch.empty_like(din.q)
        torch.cuda.synchronize()
        print(f"[bench] decode inputs {dspec.name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        dsel = lambda: dplan.select(din.q, din.k)  # noqa: E731
        datt = lambda: dplan.attend(din.q, din.k, din.v, do)  # noqa: E731

    def step():
        if args.only in ("prefill", "all"):
            sel()
            att()
        if args.only in ("decode", "all"):
            dsel()
            datt()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing: barrier (single rank) + synchronize on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} timed steps, {wall_ms:.3f} ms/step", file=sys.stderr, flush=True)

    reps = max(args.steps, 5)
    res = {}
    scrub = torch.empty(512 << 18, dtype=torch.float32, device=dev)  # 512 MiB, twice the MALL
    if args.only in ("prefill", "all"):
        sel_med, _, sel_ts = timed(sel, stream, reps)
        res["sel_ms"] = sel_med
        res["sel_p10_p90_ms"] = [pct(sel_ts, 0.1), pct(sel_ts, 0.9)]
        att_med, att_mean, att_ts = timed(att, stream, reps)
        res["att_ms"] = att_med
        res["att_mean_ms"] = att_mean
        res["att_p10_p90_ms"] = [pct(att_ts, 0.1), pct(att_ts, 0.9)]
        res["att_scrub_ms"] = timed(att, stream, reps, scrub)[0]
        res["layer_graph_ms"] = graph_timed(lambda: (sel(), att()), stream, reps)
    if args.only in ("decode", "all"):
        res["dsel_ms"] = timed(dsel, stream, reps)[0]
        res["datt_ms"] = timed(datt, stream, reps)[0]
        dmed, _, dts = timed(lambda: (dsel(), datt()), stream, reps)
        res["dstep_ms"] = dmed
        res["dstep_p10_p90_ms"] = [pct(dts, 0.1), pct(dts, 0.9)]
        res["dstep_scrub_ms"] = timed(lambda: (dsel(), datt()), stream, reps, scrub)[0]
        res["dstep_graph_ms"] = graph_timed(lambda: (dsel(), datt()), stream, reps)
        if not args.no_paged:
            # the same decode step over the cache scattered into per-KV-head
            # pools of 128-token pages (the pools are built once, untimed)
            pk = W.make_paged(din.k, din.v, 128, W.seed_of(dspec))
            pplan = SA.PagedDecodePlan(din.q, pk.k_pages, pk.v_pages, pk.table, dspec.kv_len, din.budget)
            pplan.pool(pk.k_pages)
            po = torch.empty_like(din.q)
            pstep = lambda: (pplan.select(din.q, pk.k_pages), pplan.attend(din.q, pk.k_pages, pk.v_pages, po))  # noqa: E731
            pstep()
            do_ref = torch.empty_like(din.q)
            dplan.select(din.q, din.k)
            dplan.attend(din.q, din.k, din.v, do_ref)
            torch.cuda.synchronize()
            res["paged_same"] = bool(torch.equal(po, do_ref))
            res["paged_step_ms"] = timed(pstep, stream, reps)[0]
            del pk, pplan
            torch.cuda.empty_cache()

    flops = None
    if args.only in ("prefill", "all"):  # the block table is filled only when the prefill ran
        bidx = plan.block_idx.cpu().numpy()
        bcnt = plan.block_cnt.cpu().numpy()
        flops = M.prefill_flops(bidx, bcnt, pspec.seq_len, pspec.block, pspec.head_dim)
    dbytes = {"total": 0}
    if args.only in ("decode", "all"):
        dbidx = dplan.block_idx.cpu().numpy()
        dbcnt = dplan.block_cnt.cpu().numpy()
        nc = [-(-dspec.kv_len // int(g)) for g in din.budget["granularity"]]
        scoring = [int(dplan.counts[h]) > len(range(min(int(din.budget["n_sink"][h]), nc[h]))) +
                   min(int(din.budget["n_local"][h]), nc[h]) and int(dplan.counts[h]) < nc[h]
                   for h in range(dspec.n_q_heads)]
        dbytes = M.decode_bytes(dbidx, dbcnt, din.budget["granularity"], dspec.n_q_heads, dspec.n_kv_heads,
                                dspec.kv_len, dspec.head_dim, 2, scoring)

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks(dev, stream)
        print(f"[bench] measured peaks: {peaks}", file=sys.stderr, flush=True)

    prefill_ms = res.get("sel_ms", 0.0) + res.get("att_ms", 0.0)
    tflops = flops / (res["att_mean_ms"] * 1e-3) / 1e12 if "att_ms" in res else None
    traffic = traffic_from_profiles()
    pk_mfma = peaks["mfma_bf16_tflops"] if peaks else None
    pk_mfma_rnd = peaks["mfma_bf16_random_tflops"] if peaks else None
    roofline = {
        "bound": "mfma",
        "achieved": tflops,
        "peak": M.PEAK_BF16_FLOPS / 1e12,
        "unit": "TFLOP/s",
        "frac": tflops / (M.PEAK_BF16_FLOPS / 1e12) if tflops else None,
        "peak_measured": pk_mfma,
        "frac_measured": tflops / pk_mfma if tflops and pk_mfma else None,
        "peak_measured_random_operands": pk_mfma_rnd,
        "frac_measured_random_operands": tflops / pk_mfma_rnd if tflops and pk_mfma_rnd else None,
        "traffic": traffic,
        "kernel": "prefill_kernel (sa_sparse_attn_prefill)",
        "flops_per_launch": flops,
        "avg_launch_ms": res.get("att_mean_ms"),
    }
    dgbps = dbytes["total"] / (res["dstep_ms"] * 1e-3) / 1e9 if "dstep_ms" in res else None
    kv_gbps = dbytes["kv"] / (res["datt_ms"] * 1e-3) / 1e9 if "datt_ms" in res else None
    if args.only == "decode":
        # no prefill ran: the line's roofline is the decode step's (HBM-bound),
        # and there is no prefill time to report as the value
        pk_hbm = peaks["hbm_read_gbps"] if peaks and "hbm_read_gbps" in peaks else None
        roofline = {
            "bound": "hbm",
            "achieved": dgbps,
            "peak": M.PEAK_HBM_BYTES / 1e9,
            "unit": "GB/s",
            "frac": dgbps / (M.PEAK_HBM_BYTES / 1e9) if dgbps else None,
            "peak_measured": pk_hbm,
            "frac_measured": dgbps / pk_hbm if dgbps and pk_hbm else None,
            "traffic": None,
            "kernel": "decode step (sa_select_blocks + sa_sparse_attn_decode)",
            "bytes_per_step": dbytes["total"],
            "avg_step_ms": res.get("dstep_ms"),
        }

    ablation = {}
    if not args.no_ablation and args.only in ("prefill", "all"):
        nat = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=0)
        nat.share_tables(plan)
        ablation["natural_order_grid_ms"] = timed(lambda: nat.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        # persistent bins in natural (contiguous) order: tiles split evenly by count
        n_t = plan.counts.size
        offs = np.linspace(0, n_t, n_bins + 1).astype(np.int32)
        cont = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=0)
        cont.share_tables(plan)
        cont.bin_offsets = torch.from_numpy(offs).to(dev)
        cont.items_by_bin = torch.arange(n_t, dtype=torch.int32, device=dev)
        cont.n_bins = n_bins
        ablation["contiguous_bins_ms"] = timed(lambda: cont.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        ablation["default_order"] = default_order
        ablation["default_ms"] = res["att_ms"]
        if plan.queue_offsets is not None and args.queues == 8:
            ablation["queue_xcd_partitions_ms"] = res["att_ms"]
        else:
            xq = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                                queue_group="kv_tiers", queues=8)
            xq.share_tables(plan)
            ablation["queue_xcd_partitions_ms"] = timed(lambda: xq.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
            del xq
        grouped = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                                 queue_group="kv")
        grouped.share_tables(plan)
        ablation["queue_lpt_grouped_ms"] = timed(lambda: grouped.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        del grouped
        # one queue in load tiers
        other = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                               queue_group="kv_tiers", queues=1)
        other.share_tables(plan)
        ablation["queue_lpt_kv_tiers_ms"] = timed(lambda: other.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        del other
        # the queue grouped by query head (heaviest head first) instead of by KV head
        byhead = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                                queue_group="head")
        byhead.share_tables(plan)
        ablation["queue_lpt_by_query_head_ms"] = timed(lambda: byhead.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        del byhead
        # the same queue in plain longest-first order (no grouping by KV head)
        flat = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, queue=True,
                              queue_group="flat")
        flat.share_tables(plan)
        ablation["queue_lpt_flat_ms"] = timed(lambda: flat.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        # static LPT bins, each walked in item order
        lpt = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins)
        lpt.share_tables(plan)
        ablation["lpt_bins_ms"] = timed(lambda: lpt.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        asg = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, bin_order="lpt")
        asg.share_tables(plan)
        ablation["lpt_bins_assignment_order_ms"] = timed(lambda: asg.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        # two-level placement: chunks of (KV head, 64 query blocks) onto the 8 XCDs, then LPT inside each
        xcd = SA.PrefillPlan(pin.q, pin.k, pin.v, pin.budget, pspec.block, n_bins=n_bins, xcd_groups=8, xcd_chunk=64)
        xcd.share_tables(plan)
        ablation["lpt_xcd_two_level_ms"] = timed(lambda: xcd.attend(pin.q, pin.k, pin.v, o), stream, reps)[0]
        ablation["lpt_xcd_two_level_makespan_over_mean"] = float(xcd.bin_load.max() / xcd.bin_load.mean())
        loads = plan.counts.reshape(-1).astype(np.int64)
        cont_load = np.add.reduceat(loads, offs[:-1]) if n_t else loads
        ablation["lpt_makespan_over_mean"] = float(lpt.bin_load.max() / lpt.bin_load.mean())
        ablation["contiguous_makespan_over_mean"] = float(cont_load.max() / cont_load.mean())

    cpu = None
    cpu_dec = None
    if not args.no_cpu_baseline and args.only in ("prefill", "all"):
        # the host cores this process may run on; the BLAS pool (the oracle's
        # matrix products) is set to that many threads
        cores = len(os.sched_getaffinity(0))
        from threadpoolctl import threadpool_info, threadpool_limits
        with threadpool_limits(limits=cores):
            blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            cpu_ms, spent, desc = cpu_baseline_prefill(pin, bidx, bcnt)
        cpu = {"value": cpu_ms, "unit": "ms/layer", "cores": int(cores), "blas_threads": int(blas),
               "kind": "oracle", "sample": f"fp64 oracle on {pspec.name}: {desc}; {spent:.1f} s of CPU work"}
        print(f"[bench] cpu baseline (prefill) {spent:.1f} s", file=sys.stderr, flush=True)
        if args.only == "all":
            dms, dspent = cpu_baseline_decode(din, dbidx, dbcnt)
            cpu_dec = {"value": dms, "unit": "ms/step", "sample": f"sequence 0 of {dspec.batch}, scaled; "
                                                                   f"{dspent:.1f} s"}

    out = {
        "metric": "128K prefill ms/layer + attended TFLOP/s (%MFMA peak); decode KV GB/s (%HBM)",
        "value": prefill_ms if args.only in ("prefill", "all") else None,
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V with planted hot blocks)",
        "config": {"workload": f"prefill {pspec.name} (S={pspec.seq_len}, Hq={pspec.n_q_heads}, "
                               f"Hkv={pspec.n_kv_heads}, D={pspec.head_dim}, block={pspec.block}) + decode "
                               f"{dspec.name} (batch={dspec.batch}, L={dspec.kv_len})",
                   "global_batch": 1, "seq_len": pspec.seq_len, "parallelism": "single GPU",
                   "schedule": (f"work queue: {n_bins} workgroups, tiles in load tiers (quarter octave) heaviest first, grouped by (sequence, KV head) within a tier"
                                + (f"; cut into {len(plan.queue_offsets) - 1} partitions (one per XCD) of (load tier, sequence, KV head) runs placed by LPT, workgroup w starting on partition w mod {len(plan.queue_offsets) - 1} and moving on when it is empty"
                                   if plan.queue_offsets is not None else "")
                                if plan.queue_offsets is not None or pspec.n_blocks > 256 else
                                f"work queue: {n_bins} workgroups, one queue, tiles longest first (the library's order for up to 256 query blocks per head)")},
        "prefill": {"select_ms": res.get("sel_ms"), "select_p10_p90_ms": res.get("sel_p10_p90_ms"),
                    "attention_ms": res.get("att_ms"), "attention_p10_p90_ms": res.get("att_p10_p90_ms"),
                    "attention_ms_scrubbed": res.get("att_scrub_ms"),
                    "layer_ms_hip_graph": res.get("layer_graph_ms"),
                    "attended_tflops": tflops, "attended_flops": flops,
                    "mfma_frac": roofline["frac"], "schedule_host_ms": lpt_ms},
        "decode": {"select_ms": res.get("dsel_ms"), "attention_ms": res.get("datt_ms"),
                   "step_ms": res.get("dstep_ms"), "step_p10_p90_ms": res.get("dstep_p10_p90_ms"),
                   "step_ms_scrubbed": res.get("dstep_scrub_ms"),
                   "step_ms_hip_graph": res.get("dstep_graph_ms"),
                   "bytes": dbytes, "step_gbps": dgbps,
                   "hbm_frac": dgbps / (M.PEAK_HBM_BYTES / 1e9) if dgbps else None,
                   "hbm_frac_measured": dgbps / peaks["hbm_read_gbps"] if dgbps and peaks else None,
                   "kv_gbps_attention_kernel": kv_gbps},
        "decode_paged": None if "paged_step_ms" not in res else {
            "page_size": 128, "step_ms": res["paged_step_ms"],
            "step_gbps": dbytes["total"] / (res["paged_step_ms"] * 1e-3) / 1e9,
            "hbm_frac": dbytes["total"] / (res["paged_step_ms"] * 1e-3) / M.PEAK_HBM_BYTES,
            "same_output_as_contiguous": res["paged_same"]},
        "roofline": roofline,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "cpu_baseline_decode": cpu_dec,
        "ablation": ablation,
    }
    if args.calibrate:
        out["calibration"] = calibration_timing(dev, stream)
    if args.only in ("prefill", "all") and not args.no_tail:
        del plan
        torch.cuda.empty_cache()
        tails = [tail_report(pspec.name, dev, stream, n_bins, args.queues)]
        if args.tail:
            tails.append(tail_report("qwen2.5-72b-prefill-64k", dev, stream, n_bins, args.queues))
        out["tail"] = tails
    if args.only in ("prefill", "all") and not args.no_ablation:
        out["ablation"]["budget_fit"] = budget_fit_ablation(pspec, dev, stream, n_bins, args.queues, reps)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
