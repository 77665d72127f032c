"""Benchmark: one routed block-sparse attention call on the H3-shaped
workload (B=1, H=56, T=9505 = 9216 video + 289 context tokens, D=128, bf16,
top-k ratio 0.1, self block forced, context tokens as exact sinks).

A step is one full call: sparse_attn_route (pool + route kernels) then
sparse_attn_fwd (video query rows) on the main stream, and dense_sink_fwd
(context rows, which need no routing) on a second stream forked at the start
of the step, launched after the routing kernels and joined at the step's
end, so the dense rows fill the GPU beside routing and the sparse rows.
The two halves write disjoint rows of ``out``.  ``--one-stream`` runs the
three calls back to back instead.  Inputs are resident in HBM
before the timed region.  Effective FLOPs count 4*128 per (query row, key)
pair scored exactly.

After the headline timing, a second pass runs the three calls back to back
on one stream with events between them: the per-stage times, the
attention-only rate and the sparse kernel's roofline come from that pass,
so each kernel is timed alone.

A third measurement (``fused_route``, skipped by ``--no-fused``) times the
call with the Top-K selection inside the attention kernel (pool, fused
sparse rows, dense rows, one stream) and reports whether its lists equal the
route kernel's.

A fourth measurement (``spark`` in the JSON line, skipped by ``--no-spark``)
times the Spark variant of the same call on the same inputs: global anchor,
virtual summaries, route, sparse rows with one virtual key per skipped video
block, dense rows, back to back on one stream with events between the
stages.  It does not change the headline numbers.

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU (a multi-GPU run would shard heads, see the design notes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBPS = 8000.0
METRIC = "ms/call and effective TFLOP/s (frac of bf16 peak), B1 H56 T9505 D128 top-k 0.1"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_pair_sparse_h3_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_05_amd", "csrc", "attn_pair.hip")
SPARSE_KERNEL = "attn_pair_kernel<false, false, false>"


def effective_flops_from_lists(cnt, idx, T, nvb, H, B):
    """4*D per exactly-scored (row, key) pair, from the GPU's own lists."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    keys_in_block = np.minimum(64, T - 64 * np.arange(-(-T // 64)))
    sparse_pairs = 0
    for b in range(B):
        for h in range(H):
            for i in range(nvb):
                sparse_pairs += 64 * int(keys_in_block[idx[b, h, i, :cnt[b, h, i]]].sum())
    dense_pairs = B * H * (T - 64 * nvb) * T
    return 4 * 128 * sparse_pairs, 4 * 128 * dense_pairs


# GPU time of untimed back-to-back steps before each measured loop, enough
# for the clock to reach its steady state under this load.
SETTLE_MS = 100.0


def fused_measure(sa, wl, q, k, v, kb, idx, cnt, out, dws, steps, sparse_flops):
    """Per-stage and whole-call times with the route inside the attention
    kernel (pool, fused sparse rows, dense rows; one stream), and whether its
    lists equal the route kernel's."""
    ss = wl.sink_start
    ws = sa.sparse_attn_pool(q, k, ss)
    _, (fidx, fcnt) = sa.sparse_attn_fwd_fused(q, k, v, ss, wl.topk_ratio, wl.local_radius, ws,
                                               key_bias=kb, out=out, return_route=True)
    torch.cuda.synchronize()
    same_lists = bool(torch.equal(fidx, idx) and torch.equal(fcnt, cnt))
    stream = torch.cuda.current_stream(q.device)
    stages = [
        ("pool", lambda: sa.sparse_attn_pool(q, k, ss, workspace=ws)),
        ("sparse_fwd_fused", lambda: sa.sparse_attn_fwd_fused(q, k, v, ss, wl.topk_ratio, wl.local_radius,
                                                              ws, key_bias=kb, out=out, check_bias=False)),
        ("dense_fwd", lambda: sa.dense_sink_fwd(q, k, v, ss, key_bias=kb, out=out, workspace=dws,
                                                check_bias=False)),
    ]
    for _ in range(3):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(stages))] for e in evs])
    call = np.array([e[0].elapsed_time(e[-1]) for e in evs])
    med = np.median(st, axis=0)
    names = [n for n, _ in stages]
    f_ms = float(st[:, names.index("sparse_fwd_fused")].mean())
    return {
        "path": "pool + sparse rows with the Top-K selected inside the attention kernel + dense rows, "
                "one stream",
        "ms_per_call_median": round(float(np.median(call)), 4),
        "stages_ms_median": {n: round(float(x), 4) for n, x in zip(names, med)},
        "lists_equal_route_kernel": same_lists,
        "sparse_fwd_fused_tflops": round(sparse_flops / (f_ms * 1e-3) / 1e12, 3),
    }


def spark_measure(sa, wl, q, k, v, kb, idx, cnt, ws, out, dws, steps, sparse_flops, dense_flops):
    """Per-stage and whole-call times of the Spark path (one stream)."""
    B, T, H, D = q.shape
    ss = wl.sink_start
    nb = -(-T // 64)
    nvb = ss // 64
    anchor = sa.spark_global_anchor(q, ss)
    aws = torch.empty(max(16, sa.sa_anchor_workspace_bytes(B, T, H, ss)), dtype=torch.uint8, device=q.device)
    ak, av, lm = sa.spark_reweight(anchor, k, v)
    stream = torch.cuda.current_stream(q.device)
    stages = [
        ("anchor", lambda: sa.spark_global_anchor(q, ss, out=anchor, workspace=aws)),
        ("reweight", lambda: sa.spark_reweight(anchor, k, v, ak=ak, av=av, lm=lm)),
        ("route", lambda: sa.sparse_attn_route(q, k, ss, wl.topk_ratio, wl.local_radius, block_idx=idx,
                                               block_cnt=cnt, workspace=ws)),
        ("sparse_fwd_spark", lambda: sa.sparse_attn_fwd_spark(q, k, v, ss, idx, cnt, (ak, av, lm),
                                                              key_bias=kb, out=out, check_bias=False)),
        ("dense_fwd", lambda: sa.dense_sink_fwd(q, k, v, ss, key_bias=kb, out=out, workspace=dws,
                                                check_bias=False)),
    ]
    for _ in range(3):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(stages))] for e in evs])
    call = np.array([e[0].elapsed_time(e[-1]) for e in evs])
    med = np.median(st, axis=0)
    mean = st.mean(axis=0)
    names = [n for n, _ in stages]
    # algorithmic HBM bytes of the summaries kernel: K and V read once, the
    # anchor read, ak / av / lm written
    rw_bytes = 2 * B * T * H * D * 2 + B * H * D * 2 + 2 * B * H * nb * D * 2 + B * H * nb * 4
    rw_ms = float(mean[names.index("reweight")])
    rw_gbps = rw_bytes / (rw_ms * 1e-3) / 1e9
    an_bytes = B * ss * H * D * 2
    an_gbps = an_bytes / (float(mean[names.index("anchor")]) * 1e-3) / 1e9
    # virtual (row, summary key) pairs: every sparse row times its skipped video blocks
    c = cnt.cpu().numpy()
    i_ = idx.cpu().numpy()
    exact_video = np.array([[[int((i_[b, h, r, :c[b, h, r]] < nvb).sum()) for r in range(i_.shape[2])]
                             for h in range(H)] for b in range(B)])
    virtual_pairs = int(64 * (nvb - exact_video).sum())
    sp_ms = float(mean[names.index("sparse_fwd_spark")])
    sp_flops = sparse_flops + 4 * D * virtual_pairs
    return {
        "path": "global anchor + virtual summaries + route + sparse rows with one virtual key per "
                "skipped video block + dense rows, one stream",
        "ms_per_call_median": round(float(np.median(call)), 4),
        "stages_ms_median": {n: round(float(x), 4) for n, x in zip(names, med)},
        "effective_gflop_exact": round((sparse_flops + dense_flops) / 1e9, 3),
        "virtual_pairs": virtual_pairs,
        "sparse_fwd_spark_tflops": round(sp_flops / (sp_ms * 1e-3) / 1e12, 3),
        "reweight_roofline": {"kernel": "reweight_kernel", "bound": "hbm", "achieved": round(rw_gbps, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(rw_gbps / HBM_PEAK_GBPS, 4),
                              "algorithmic_bytes_per_launch": rw_bytes, "launch_ms_mean": round(rw_ms, 4)},
        "anchor_gbps": round(an_gbps, 1),
    }


def traffic_for_current_kernel(workload_name):
    """HBM bytes per sparse-attention launch measured with rocprofv3 counters
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), if they
    were taken on the current kernel source and this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    src_hash = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if t.get("attn_src_sha256") != src_hash or not t.get("workload", "").startswith(workload_name + " "):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wl, heads):
    """Oracle (as written: NumPy, float64) on a bounded sample: the first
    `heads` heads of the same workload.  ``cores`` is the size of the BLAS
    thread pool its matrix products run on (the threads it used); the host's
    CPU count and torch's thread count are reported beside it."""
    import oracle.sparse_attention as ora
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    heads = min(heads, wl.q.shape[2])
    f = lambda t: t[:, :, :heads].float().contiguous().numpy()
    q, k, v = f(wl.q), f(wl.k), f(wl.v)
    t0 = time.perf_counter()
    _, _, rt = ora.routed_attention(q, k, v, wl.sink_start, wl.topk_ratio, wl.local_radius,
                                    key_bias=None if wl.key_bias is None else wl.key_bias.numpy())
    dt = time.perf_counter() - t0
    T = q.shape[1]
    flops = ora.effective_flops(T, heads, 1, rt.lists(), rt.nvb)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle routed_attention (pool+route+sparse+dense, float64 arithmetic, "
                      f"stricter than the fp32 the tolerances are stated for) on heads 0..{heads - 1} "
                      f"of the same workload ({flops / 1e9:.1f} effective GFLOP in {dt:.1f} s)",
            "blas_threads": int(threads), "os_cpu_count": os.cpu_count(),
            "torch_threads": torch.get_num_threads(), "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="h3", choices=["h3", "h3_bias", "mid", "long", "tiny", "h3_share"])
    ap.add_argument("--cpu-heads", type=int, default=56)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-spark", action="store_true",
                    help="skip the Spark approximate-branch measurement")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-route measurement")
    ap.add_argument("--one-stream", action="store_true",
                    help="run the dense rows after the sparse rows on one stream")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the routed attention "
              "path shards by head with no collective; run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        # an elementwise kernel (y = 1 * x over fp32) rather than copy_, which
        # may be served by a DMA engine that the shader counters do not see
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    import block_sparse_attention_05_amd as sa
    import workloads

    wl = workloads.NAMED[args.workload]()
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (wl.q, wl.k, wl.v))
    kb = None if wl.key_bias is None else wl.key_bias.to(dev)
    B, T, H, D = q.shape
    ss = wl.sink_start
    nvb = sa.sa_num_sparse_blocks(T, ss)
    max_sel = sa.sa_max_selected(T, ss, wl.topk_ratio, wl.local_radius)
    idx = torch.empty((B, H, nvb, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, nvb), dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, sa.sa_route_workspace_bytes(B, T, H, ss)), dtype=torch.uint8, device=dev)
    dws_n = sa.sa_dense_workspace_bytes(B, T, H, ss)
    dws = torch.empty(dws_n, dtype=torch.uint8, device=dev) if dws_n > 0 else None
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    side = stream if args.one_stream else torch.cuda.Stream(dev)   # default priority

    def route():
        sa.sparse_attn_route(q, k, ss, wl.topk_ratio, wl.local_radius, block_idx=idx, block_cnt=cnt,
                             workspace=ws)

    if kb is not None:
        sa.check_key_bias(kb, B, T, ss)   # once: the timed calls skip the host-synchronising check

    def sparse():
        sa.sparse_attn_fwd(q, k, v, ss, idx, cnt, key_bias=kb, out=out, check_bias=False)

    def dense():
        sa.dense_sink_fwd(q, k, v, ss, key_bias=kb, out=out, workspace=dws, check_bias=False)

    def step(sparse_ev=None):
        # sparse_ev: optional pair of events recorded on the main stream right
        # before and after the sparse launch
        if side is not stream:
            side.wait_stream(stream)
        route()
        if side is not stream:
            with torch.cuda.stream(side):   # queued behind the pool/route launches
                dense()
        if sparse_ev:
            sparse_ev[0].record(stream)
        sparse()
        if sparse_ev:
            sparse_ev[1].record(stream)
        if side is stream:
            dense()
        else:
            stream.wait_stream(side)

    # From a cold start, or after about a second without work, the first
    # 20-40 ms of back-to-back steps run up to a fifth slower than the steady
    # state while the GPU's clock comes up.  Every measured loop below
    # (diagnostics and headline alike) is therefore preceded by untimed steps
    # worth SETTLE_MS of GPU time; none of them is inside a timed region.
    def settle():
        done_ms, n = 0.0, 0
        while done_ms < SETTLE_MS:
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(20):
                step()
            a1.record(stream)
            torch.cuda.synchronize()
            done_ms += a0.elapsed_time(a1)
            n += 20
        return n

    step()
    torch.cuda.synchronize()
    sparse_flops, dense_flops = effective_flops_from_lists(cnt, idx, T, nvb, H, B)
    untimed = {"first_step": 1}

    untimed["settle_steps_1"] = settle()

    # per-call distribution of the same schedule: an event pair around every
    # call (the events sit on the main stream, which joins the side stream)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a0, a1 in cev:
        a0.record(stream)
        step()
        a1.record(stream)
    torch.cuda.synchronize()
    calls = np.array([a0.elapsed_time(a1) for a0, a1 in cev])
    untimed["per_call_steps"] = args.steps

    # per-stage timing: the three calls back to back on the main stream, with
    # events between them, so that each kernel is timed alone
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        route()
        evs[i][1].record(stream)
        sparse()
        evs[i][2].record(stream)
        dense()
        evs[i][3].record(stream)
    torch.cuda.synchronize()
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    med = np.median(st, axis=0)
    untimed["per_stage_steps"] = args.steps

    extra = {}
    if not args.no_fused:
        untimed["settle_steps_2"] = settle()
        extra["fused_route"] = fused_measure(sa, wl, q, k, v, kb, idx, cnt, out, dws, args.steps,
                                             sparse_flops)
        untimed["fused_route_passes"] = args.steps + 4
    if not args.no_spark:
        untimed["settle_steps_3"] = settle()
        extra["spark"] = spark_measure(sa, wl, q, k, v, kb, idx, cnt, ws, out, dws, args.steps,
                                       sparse_flops, dense_flops)
        untimed["spark_passes"] = args.steps + 3
    torch.cuda.synchronize()

    untimed["settle_steps_4"] = settle()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing: events only at the ends
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # the same back-to-back loop once more with an event between consecutive
    # steps (GPU time of each step in order, gaps between steps included),
    # events around every sparse launch (its duration as the timed steps run
    # it, the dense rows on the side stream overlapping part of it) and the
    # host's enqueue time per step
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    spev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    host_us = []
    torch.cuda.synchronize()
    sev[0].record(stream)
    for i in range(args.steps):
        h0 = time.perf_counter()
        step(spev[i])
        sev[i + 1].record(stream)
        host_us.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()
    seq_ms = [sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)]
    sparse_in_step = np.array([a0.elapsed_time(a1) for a0, a1 in spev])

    # bf16 MFMA peak from this device's CU count and peak clock:
    # 4 SIMDs x 1024 FLOP per clock per CU (one 32x32x16 MFMA per 32 clocks)
    cu, clk_khz = sa.sa_device_info(0)
    peak_dev = {"tflops": round(cu * clk_khz * 1e3 * 4096 / 1e12, 1), "cu": cu, "clock_mhz": clk_khz / 1e3}

    total_flops = sparse_flops + dense_flops
    tflops = total_flops / (ms * 1e-3) / 1e12
    # the sparse kernel's mean launch duration as the timed steps run it
    # (prices the roofline), and alone on one stream (the per-stage loop)
    sparse_ms = float(sparse_in_step.mean())
    sparse_alone_ms = float(st[:, 1].mean())
    achieved = sparse_flops / (sparse_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "D": D, "video_tokens": ss,
                   "sink_tokens": T - ss, "topk_ratio": wl.topk_ratio, "local_radius": wl.local_radius,
                   "key_bias": kb is not None, "inputs": "smooth-field+noise Q/K, N(0,1) V, seed 2"},
        "ms_per_call": round(ms, 4),
        "timed_after": {"loops": untimed, "settle_gpu_ms_each": SETTLE_MS, "warmup_steps": args.warmup,
                        "note": "untimed loops in run order: a first step, clock-settling steps, "
                                "per-call and per-stage timing, settling, the fused-route loop, "
                                "settling, the Spark loop, settling, then the warm-up steps and "
                                "the timed steps; the back-to-back list below is one more pass "
                                "right after them"},
        "back_to_back_steps_ms_in_order": [round(x, 4) for x in seq_ms],
        "host_enqueue_us_per_step_median_max": [round(float(np.median(host_us)), 1),
                                                round(float(np.max(host_us)), 1)],
        "ms_per_call_median_p10_p90": [round(float(np.median(calls)), 4),
                                       round(float(np.percentile(calls, 10)), 4),
                                       round(float(np.percentile(calls, 90)), 4)],
        "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "effective_gflop": round(total_flops / 1e9, 3),
        "stages_ms_median_one_stream": {"route": round(float(med[0]), 4), "sparse_fwd": round(float(med[1]), 4),
                             "dense_fwd": round(float(med[2]), 4)},
        "stages_ms_p10_p90_one_stream": {n: [round(float(np.percentile(st[:, j], 10)), 4),
                                  round(float(np.percentile(st[:, j], 90)), 4)]
                              for j, n in enumerate(("route", "sparse_fwd", "dense_fwd"))},
        "streams": 1 if side is stream else 2,
        "attention_only_tflops": round(total_flops / ((med[1] + med[2]) * 1e-3) / 1e12, 3),
        "attention_only_frac_of_bf16_peak": round(total_flops / ((med[1] + med[2]) * 1e-3) / 1e12
                                                  / BF16_PEAK_TFLOPS, 4),
        "peak_device_tflops": peak_dev,
        "roofline": {"kernel": SPARSE_KERNEL, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "algorithmic_gflop_per_launch": round(sparse_flops / 1e9, 3),
                     "launch_ms_mean": round(sparse_ms, 4),
                     "launch_ms_from": "events around each sparse launch in the back-to-back pass "
                                       "(same streams as the timed steps)",
                     "launch_ms_mean_alone_one_stream": round(sparse_alone_ms, 4),
                     "traffic": traffic_for_current_kernel(wl.name)},
    }
    res.update(extra)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_heads)
        cb.pop("seconds")
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
