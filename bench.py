"""Benchmark: sparse MLA decode throughput on one MI355X.

Workload (the per-token shape the headline metric is quoted on): H=128
heads, table width / topk 2048 (128 SWA + 1920 compressed rows), BF16 q and
KV rows, 128k context at compress ratio 4 (32768 compressed rows per
request), per-head sinks, one token per request, decode batch T=512.  Inputs
are seeded synthetic tensors (sparse_mla_decode_gather_amd.workloads),
resident in HBM before timing starts.

A step is one sparse_mla_decode call (planner + split kernel [+ combine]).
Each launch is bracketed by HIP events on the stream it runs on, so the
average launch duration, gathered bytes and FLOPs give the roofline numbers.

Every timed region is preceded by the same step run back to back for about
200 ms of GPU time (--settle-ms), then the W warmup steps.  After an idle of
about 10 ms or more the board's power management runs the first few
launches at full clock, cuts the clock steeply a few milliseconds into the
burst and restores it over some tens of milliseconds of sustained load; a
short timed region right after the idle measures that transient rather
than the kernel's sustained rate.  The line also carries the rate of the
same W + K steps right after a 50 ms idle (``after_idle``), unsettled.

Besides the headline numbers the line carries: the pure-gather rate on the
same tables (sparse_mla_gather_only: compaction and row loads only, the
attainable gather bandwidth), the rate of the same call in the two-segment
form (sparse_mla_decode_segments with a 128-column SWA table and a
1920-column compressed table), the rate of the page-table form
(sparse_mla_decode_paged: the same 128 window rows plus 30 random pages of
64 consecutive compressed rows per token; same gathered bytes, page-local
rows), the combined-table builder (sparse_mla_build_indices) timed on the
same tables expressed as request-local positions and a 64-row block table
(it must rebuild them exactly), a cold-cache rate (a 1 GiB write between
launches evicts L2 and MALL), the per-T numbers for T in 1, 4, 8, 16, 64,
256 (the small T also as HIP-graph replays of 20 back-to-back launches),
the other configurations (tiny, batched with sinks, FP8, speculative
decode, and the long-context shape with packed 584-byte block-scaled FP8
rows) with their default plans and roofline fractions, and the roofline
fraction against peaks measured on the same device in the same run.

Prints ONE JSON line.  Options: --steps, --warmup, --gpus (1 only), --T,
--settle-ms, --no-cpu-baseline, --headline-only (the headline's settled
timed region alone, for profilers: its K launches are the headline kernel's
last K dispatches), --only-workload NAME.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA, published
ROW_BYTES = 1024                # one BF16 row of 512 elements
COUNTERS = os.path.join(ROOT, "profiles", "decode_long_context_T512_traffic.txt")
SETTLE_MS = 200.0               # back-to-back GPU time before each timed region


def active_slots_per_token(w):
    import torch
    K = w.K
    col = torch.arange(K, device=w.indices.device)[None, :]
    lens = w.topk_lens[:, None] if w.topk_lens is not None else K
    act = (col < lens) & (w.indices != -1)
    return act.sum(1).cpu()


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(COUNTERS):
        return None
    vals = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    from sparse_mla_decode_gather_amd.rocprof_summary import kernel_source_digest
    if vals.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(fn, steps, warmup, stream):
    """Run fn() warmup+steps times; HIP events around each timed launch on
    ``stream``.  Returns (total ms over the timed region, per-launch ms)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(
        enable_timing=True)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start.record(stream)
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return start.elapsed_time(end), per


def settle(fn, stream, ms):
    """Run fn() back to back for about ``ms`` of GPU time with no host wait
    in between, so that the timed region that follows sees the clock of
    sustained load rather than the power-management transient after an
    idle.  The launch count comes from the fastest of three timed launches
    after an untimed one (a process's first launch of a kernel also loads
    its code).  Returns the launches run."""
    import torch
    if ms <= 0:
        return 0
    fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    n = int(min(max(ms / max(best, 1e-3), 1.0), 20000))
    for _ in range(n):
        fn()
    return n + 4


def time_settled(fn, steps, warmup, stream, ms):
    """settle() then time_launches()."""
    settle(fn, stream, ms)
    return time_launches(fn, steps, warmup, stream)


def time_cold(fn, iters, stream):
    """Median per-launch ms of fn() with a 1 GiB device write before each
    launch (outside the timed window), so L2 and MALL start cold."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for i in range(iters):
        flush.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    times.sort()
    return times[len(times) // 2]


def time_graph(fn, launches=20, replays=5):
    """Per-launch ms of fn() captured `launches` times into one HIP graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (launches * replays)


def cpu_baseline(w, budget_s=10.0):
    """The oracle (NumPy fp64, as it stands) timed on a bounded sample of
    the same workload: whole passes over the batch's tokens, repeated until
    at least ``budget_s`` seconds of oracle work have run."""
    import numpy as np
    import torch
    import oracle
    from sparse_mla_decode_gather_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))

    # input marshalling (not timed): q and the rows the tokens name, on host
    tok = torch.arange(w.T)
    idx = w.indices.cpu().numpy().astype(np.int64)
    out_idx = idx.copy()
    pools = []
    for sl, pool in ((slice(0, 128), w.swa_pool), (slice(128, None), w.comp_pool)):
        part = idx[:, sl]
        ok = part >= 0
        uniq = np.unique(part[ok])
        pools.append(W.raw_bits(pool[torch.as_tensor(uniq, device=pool.device)]))
        rem = part.copy()
        rem[ok] = np.searchsorted(uniq, part[ok])
        out_idx[:, sl] = rem
    case = dict(q_bits=W.raw_bits(w.q), q_dtype=w.q_dtype, swa_bits=pools[0],
                comp_bits=pools[1], kv_dtype=w.kv_dtype,
                indices=out_idx.astype(np.int32),
                topk_lens=w.topk_lens.cpu().numpy(),
                sinks=w.sinks.cpu().numpy())
    done, secs, passes = 0, 0.0, 0
    while secs < budget_s:
        t0 = time.perf_counter()
        oracle.sparse_mla_decode(bmm1_scale=w.bmm1_scale,
                                 bmm2_scale=w.bmm2_scale,
                                 lse_scale=w.lse_scale, **case)
        secs += time.perf_counter() - t0
        done += w.T
        passes += 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(done / secs, 3), "unit": "tokens/s", "cores": cores,
            "cpu_model": model, "kind": "oracle",
            "sample": f"{passes} pass(es) over all {w.T} tokens of the same "
                      f"workload (NumPy float64 oracle, {secs:.1f} s)"}


def measured_peaks(stream):
    """Attainable peaks of this device, for the fractions against measured
    rather than published peaks: streaming HBM rates of library kernels
    (torch's sum and row sums over 4 GiB, one read pass each, and a 2 GiB
    copy counted as read + write) and dense BF16 GEMMs of 8192^3 on N(0,1)
    data (torch.matmul), each the best of several timed runs."""
    import torch
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    y = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
    rows = x.view(1 << 18, 4096)

    def best_ms(fn, n=8):
        best = float("inf")
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        return best
    rates = {
        "sum": x.numel() * 4 / (best_ms(lambda: x.sum()) * 1e-3) / 1e9,
        "row_sums": x.numel() * 4 / (best_ms(lambda: rows.sum(1)) * 1e-3) / 1e9,
        # a copy moves its bytes twice (read + write)
        "copy": 2 * y.numel() * 4 / (best_ms(lambda: y.copy_(x[: 1 << 29])) * 1e-3) / 1e9,
    }
    rd_gbps = max(rates.values())
    del x, y, rows
    g = torch.Generator(device="cuda").manual_seed(5)
    n = 8192
    A = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    B = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    for _ in range(3):
        A @ B
    best_mm = float("inf")
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        A @ B
        b.record(stream)
        torch.cuda.synchronize()
        best_mm = min(best_mm, a.elapsed_time(b))
    del A, B
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(rd_gbps, 1),
            "hbm_by_kernel_GBps": {k: round(v, 1) for k, v in rates.items()},
            "bf16_gemm_TFLOPs": round(2.0 * n ** 3 / (best_mm * 1e-3) / 1e12, 1),
            "how": "HBM: the best of torch's sum and row sums over 4 GiB fp32 and a "
                   "2 GiB copy (read + write bytes), 8 runs each; MFMA: best of 10 "
                   "bf16 8192^3 torch.matmul on N(0,1) data"}


MFMA_PEAK_BY_ROWS = {"bf16": MFMA_BF16_PEAK_TFLOPS, "fp8_e4m3fn": MFMA_BF16_PEAK_TFLOPS,
                     "packed_fp8_584": MFMA_BF16_PEAK_TFLOPS}
ROW_BYTES_BY_KV = {"bf16": 1024, "fp8_e4m3fn": 512, "packed_fp8_584": 584}


WORKLOAD_NAMES = ("tiny", "batched_sinks", "fp8", "spec_decode", "packed")


def other_workloads(stream, only=None, settle_ms=SETTLE_MS):
    """The other configurations with their default plans: per-launch time
    (HIP events around 30 back-to-back launches after settle(), and HIP-graph
    replays), gathered bytes and FLOPs of the active slots, and the fraction
    of the roofline max(bytes / HBM peak, FLOPs / MFMA peak).  FP8 rows are widened
    to BF16 and multiplied on BF16 MFMA, so BF16 is the MFMA peak."""
    import torch
    from sparse_mla_decode_gather_amd import lib, workloads as W
    res = {}
    for name, make in (("tiny", W.make_tiny), ("batched_sinks", W.make_batched_sinks),
                       ("fp8", W.make_fp8), ("spec_decode", W.make_spec_decode),
                       ("packed", lambda dev: W.make_packed(512, dev))):
        if only is not None and name != only:
            continue
        w = make("cuda")
        n = active_slots_per_token(w)
        rb = ROW_BYTES_BY_KV[w.kv_dtype]
        gathered = int(n.sum()) * rb
        flops = 4.0 * 512 * w.H * int(n.sum())
        out = torch.empty((w.T, w.H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
        plan = lib.plan_splits(w.T, w.H, w.K, lib.dtype_code(w.q),
                               lib.dtype_code(w.swa_pool))
        ws = lib.alloc_workspace(plan, w.T, w.H)

        def st(w=w, out=out, lse=lse, plan=plan, ws=ws):
            lib.decode_workload(w, out, lse, plan=plan, workspace=ws)
        _, per = time_settled(st, 30, 5, stream, settle_ms)
        avg = sum(per) / len(per)
        gms = time_graph(st)
        t_roof = max(gathered / (HBM_PEAK_GBPS * 1e9),
                     flops / (MFMA_PEAK_BY_ROWS[w.kv_dtype] * 1e12))
        res[name] = {"T": w.T, "H": w.H, "K": w.K, "q": w.q_dtype, "kv": w.kv_dtype,
                     "num_splits": plan.num_splits, "head_tiles": plan.head_tiles,
                     "gathered_bytes": gathered,
                     "launch_us": round(avg * 1e3, 2),
                     "graph_launch_us": round(gms * 1e3, 2),
                     "gathered_GBps": round(gathered / (gms * 1e-3) / 1e9, 1),
                     "tflops": round(flops / (gms * 1e-3) / 1e12, 1),
                     "bound": "hbm" if gathered / (HBM_PEAK_GBPS * 1e9) >=
                              flops / (MFMA_PEAK_BY_ROWS[w.kv_dtype] * 1e12) else "mfma",
                     "roofline_frac": round(t_roof / (gms * 1e-3), 4)}
        del w, out, lse, ws
        torch.cuda.empty_cache()
    return res


def side_measurements(w, step, plan, ws, out, lse, args, stream):
    """The headline's companions on the same tables: the pure-gather rate,
    the two-segment and page-table forms against the combined call, the
    combined-table builder and the cold-cache rate."""
    import torch
    from sparse_mla_decode_gather_amd import lib
    T = w.T

    def gather_step():
        lib.gather_only(w.q, w.swa_pool, w.comp_pool, w.indices,
                        topk_lens=w.topk_lens, plan=plan, stream=stream)
    _, gper = time_settled(gather_step, max(args.steps // 2, 5), 3, stream,
                           args.settle_ms)
    # the same tables in the two-segment form (128-column SWA table with its
    # length, 1920-column compressed table with its length)
    swa_tab, extra_tab = w.indices[:, :128], w.indices[:, 128:]
    swa_len = torch.clamp(w.topk_lens, max=128).int()
    extra_len = torch.clamp(w.topk_lens - 128, min=0).int()

    def seg_step():
        lib.decode_segments(w.q, w.swa_pool, w.comp_pool, swa_tab, extra_tab, out,
                            swa_topk_lens=swa_len, extra_topk_lens=extra_len,
                            out_lse=lse, seq_lens=w.seq_lens, sinks=w.sinks,
                            bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                            lse_scale=w.lse_scale, plan=plan, workspace=ws,
                            stream=stream)
    # alternate with the combined call so that both see the same clock
    settle(step, stream, args.settle_ms)
    sper, cper = [], []
    for _ in range(4):
        sper += time_launches(seg_step, 8, 2, stream)[1]
        cper += time_launches(step, 8, 2, stream)[1]
    # page-table form at the same size: the 128 window rows plus 30 pages of
    # 64 consecutive compressed rows per token (page IDs drawn without
    # repeats from the token's own 512-page compressed region)
    ps, npg = 64, (w.K - 128) // 64
    region = w.comp_pool.shape[0] // T // ps
    gen = torch.Generator().manual_seed(77)
    bt = torch.stack([torch.randperm(region, generator=gen)[:npg] + t * region
                      for t in range(T)]).int().cuda()
    tot = torch.full((T,), w.K, dtype=torch.int32, device="cuda")

    def paged_step():
        lib.decode_paged(w.q, w.swa_pool, w.comp_pool, swa_tab, bt, ps, out,
                         swa_topk_lens=swa_len, topk_lens=tot, out_lse=lse,
                         seq_lens=w.seq_lens, sinks=w.sinks,
                         bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                         lse_scale=w.lse_scale, plan=plan, workspace=ws,
                         stream=stream)
    settle(step, stream, args.settle_ms)
    pper, cper2 = [], []
    for _ in range(4):
        pper += time_launches(paged_step, 8, 2, stream)[1]
        cper2 += time_launches(step, 8, 2, stream)[1]
    # combined-table builder at the same shape: each request's compressed
    # rows expressed as positions in its own region, translated through a
    # block table of the region's 64-row pages, rebuild the same table
    region_rows = w.comp_pool.shape[0] // T
    req_base = (torch.arange(T, device="cuda", dtype=torch.int32) * region_rows)[:, None]
    comp_tab = w.indices[:, 128:]
    local_pos = torch.where(comp_tab >= 0, comp_tab - req_base, comp_tab).contiguous()
    bpr = region_rows // 64
    btab = (torch.arange(T * bpr, device="cuda", dtype=torch.int32).view(T, bpr)).contiguous()
    comp_lens = (w.topk_lens - 128).clamp(min=0).int()
    b_out = torch.empty_like(w.indices)
    b_lens = torch.empty_like(w.topk_lens)

    def build_step():
        lib.build_indices(swa_tab, local_pos, comp_local=True, comp_topk_lens=comp_lens,
                          block_tables=btab, page_size=64, out=b_out,
                          out_topk_lens=b_lens)
    # a few-microsecond kernel: timed as HIP-graph replays, so that the
    # Python argument marshalling between launches is not counted
    build_ms = time_graph(build_step, launches=20, replays=5)
    build_bytes = (2 * w.indices.numel() + btab.numel() + 2 * T) * 4
    build_ok = bool(torch.equal(b_out, w.indices) and torch.equal(b_lens, w.topk_lens))
    cold_ms = time_cold(step, 10, stream)
    gathered = int(active_slots_per_token(w).sum()) * ROW_BYTES
    return {
        "gather_only_GBps": round(gathered / (sum(gper) / len(gper) * 1e-3) / 1e9, 1),
        "gather_only_ms": sum(gper) / len(gper),
        "cold_cache_GBps": round(gathered / (cold_ms * 1e-3) / 1e9, 1),
        "two_segment_GBps": round(gathered / (sum(sper) / len(sper) * 1e-3) / 1e9, 1),
        "two_segment_vs_combined": round((sum(cper) / len(cper)) / (sum(sper) / len(sper)), 4),
        "paged_GBps": round(gathered / (sum(pper) / len(pper) * 1e-3) / 1e9, 1),
        "paged_vs_combined": round((sum(cper2) / len(cper2)) / (sum(pper) / len(pper)), 4),
        "build_indices": {"us": round(build_ms * 1e3, 2),
                          "GBps": round(build_bytes / (build_ms * 1e-3) / 1e9, 1),
                          "bytes": build_bytes,
                          "hbm_frac": round(build_bytes / (build_ms * 1e-3) / 1e9
                                            / HBM_PEAK_GBPS, 4),
                          "rebuilds_the_table": build_ok},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=512)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="GPU time of back-to-back launches of the same step "
                         "before each timed region's warmup (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline alone (settled; no after-idle run, "
                         "side measurements, T sweep, other configurations or "
                         "measured peaks): a short command to run under a "
                         "profiler; by default the line carries all of them")
    ap.add_argument("--only-workload", choices=WORKLOAD_NAMES,
                    help="time only this other configuration (as the default line "
                         "does) and print its record instead of the headline "
                         "line: a short command to run under a kernel tracer")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy three "
                         "times (known bytes) for counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the decode is measured on one GPU; --gpus {args.gpus} is "
              "not supported (tokens would shard across GPUs with no exchange, so "
              "the per-GPU rate is the one-GPU rate)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mla_decode_gather_amd import lib, workloads as W

    lib.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.only_workload:
        rec = other_workloads(stream, only=args.only_workload,
                              settle_ms=args.settle_ms)[args.only_workload]
        print(json.dumps({"workload": args.only_workload, **rec}), flush=True)
        return
    w = W.make_long_context(args.T, "cuda", seed=4000 + args.T)
    n_act = active_slots_per_token(w)
    T = w.T
    out = torch.empty((T, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    plan = lib.plan_splits(T, w.H, w.K)
    ws = lib.alloc_workspace(plan, T, w.H)

    def step():
        lib.decode(w.q, w.swa_pool, w.comp_pool, w.indices, out, out_lse=lse,
                   topk_lens=w.topk_lens, seq_lens=w.seq_lens, sinks=w.sinks,
                   bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                   lse_scale=w.lse_scale, plan=plan, workspace=ws, stream=stream)

    after_idle = None
    if not args.headline_only:
        # the same W + K steps right after an idle, not settled
        torch.cuda.synchronize()
        time.sleep(0.05)
        a_ms, a_per = time_launches(step, args.steps, args.warmup, stream)
        after_idle = (a_ms, sum(a_per) / len(a_per))
    total_ms, per = time_settled(step, args.steps, args.warmup, stream, args.settle_ms)
    if not args.headline_only:
        side = side_measurements(w, step, plan, ws, out, lse, args, stream)
    ms_step = total_ms / args.steps
    avg_launch_ms = sum(per) / len(per)
    gathered = int(n_act.sum()) * ROW_BYTES
    flops = 4.0 * 512 * w.H * int(n_act.sum())
    achieved_gbps = gathered / (avg_launch_ms * 1e-3) / 1e9
    achieved_tflops = flops / (avg_launch_ms * 1e-3) / 1e12
    hbm_frac = achieved_gbps / HBM_PEAK_GBPS
    mfma_frac = achieved_tflops / MFMA_BF16_PEAK_TFLOPS
    # roofline time = max(bytes / HBM peak, flops / MFMA peak)
    t_roof = max(gathered / (HBM_PEAK_GBPS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    bound = "hbm" if gathered / HBM_PEAK_GBPS >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e3) else "mfma"
    roofline = {
        "bound": bound,
        "achieved": round(achieved_gbps if bound == "hbm" else achieved_tflops, 1),
        "peak": HBM_PEAK_GBPS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
        "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
        "frac": round(t_roof / (avg_launch_ms * 1e-3), 4),
        "traffic": measured_traffic(),
        # achieved / frac divide by the average launch duration (HIP events
        # around each launch); the same on the whole timed region
        # (ms_per_step, which also holds the gaps between launches):
        "time_basis": "avg_launch_ms",
        "achieved_per_step": round((gathered / (ms_step * 1e-3) / 1e9) if bound == "hbm"
                                   else flops / (ms_step * 1e-3) / 1e12, 1),
        "frac_per_step": round(t_roof / (ms_step * 1e-3), 4),
    }
    result = {
        "metric": "decode tokens/s + gathered-KV GB/s, H=128 topk=2048 bf16; "
                  "% of roofline",
        "value": round(T * args.steps / (total_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"long-context decode batch: T={T} tokens (one per "
                               "request), H=128, topk=2048 (128 SWA + 1920 "
                               "compressed), BF16 q/KV, seq_len 131072, "
                               "compress ratio 4, sinks",
                   "T": T, "H": w.H, "K": w.K, "global_batch": T,
                   "parallelism": "single GPU"},
        "gathered_GBps": round(achieved_gbps, 1),
        "gathered_bytes_per_step": gathered,
        "tflops": round(achieved_tflops, 1),
        "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
        "avg_launch_ms": round(avg_launch_ms, 4),
        "settle": {"gpu_ms": args.settle_ms,
                   "what": "the same step back to back for about this much GPU "
                           "time before the W warmup steps of every timed region, "
                           "so that it sees the clock of sustained load and not "
                           "the power-management transient that follows an idle"},
        "plan": plan.as_dict(),
        "roofline": roofline,
    }
    if after_idle is not None:
        result["after_idle"] = {
            "idle_ms": 50, "ms_per_step": round(after_idle[0] / args.steps, 4),
            "avg_launch_ms": round(after_idle[1], 4),
            "gathered_GBps": round(gathered / (after_idle[1] * 1e-3) / 1e9, 1),
            "frac": round(t_roof / (after_idle[1] * 1e-3), 4),
            "what": "the same W warmup + K timed steps right after a 50 ms idle, "
                    "not settled"}
    if not args.headline_only:
        gms_gather = side.pop("gather_only_ms")
        result.update(side)
        result["decode_vs_gather_only"] = round(gms_gather / avg_launch_ms, 4)
        sweep = {}
        for t in (1, 4, 8, 16, 64, 256):
            if t > T:
                continue
            p = lib.plan_splits(t, w.H, w.K)
            wsp = lib.alloc_workspace(p, t, w.H)
            o2, l2 = out[:t], lse[:t]

            def st(t=t, p=p, wsp=wsp, o2=o2, l2=l2):
                lib.decode(w.q[:t], w.swa_pool, w.comp_pool, w.indices[:t], o2,
                           out_lse=l2, topk_lens=w.topk_lens[:t], sinks=w.sinks,
                           bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                           plan=p, workspace=wsp)   # current stream (graph capture)
            tot, pl = time_settled(st, 50, 5, stream, args.settle_ms)
            g = int(n_act[:t].sum()) * ROW_BYTES
            avg = sum(pl) / len(pl)
            sweep[str(t)] = {"tokens_per_s": round(t * 50 / (tot * 1e-3), 1),
                             "avg_launch_us": round(avg * 1e3, 2),
                             "gathered_GBps": round(g / (avg * 1e-3) / 1e9, 1),
                             "num_splits": p.num_splits, "head_tiles": p.head_tiles,
                             "roofline_frac": round(g / (HBM_PEAK_GBPS * 1e9) /
                                                    (avg * 1e-3), 4)}
            if t <= 16:
                gms = time_graph(st)
                sweep[str(t)]["graph_launch_us"] = round(gms * 1e3, 2)
                sweep[str(t)]["graph_gathered_GBps"] = round(g / (gms * 1e-3) / 1e9, 1)
        result["sweep"] = sweep
        result["workloads"] = other_workloads(stream, settle_ms=args.settle_ms)
        peaks = measured_peaks(stream)
        roofline["measured_peaks"] = peaks
        t_meas = max(gathered / (peaks["hbm_read_GBps"] * 1e9),
                     flops / (peaks["bf16_gemm_TFLOPs"] * 1e12))
        roofline["frac_vs_measured_peaks"] = round(t_meas / (avg_launch_ms * 1e-3), 4)
    if args.calibration_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = src.numel() * src.element_size()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
