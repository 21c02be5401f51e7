"""Benchmark of the Mixtral sparse-MoE feed-forward layer on one MI355X.

One step = one whole layer (router -> permute -> up+SwiGLU -> down ->
combine) through ``moe_ffn_forward`` on synthetic Mixtral-shaped inputs
(d=4096, f=14336, E=8, top-2, bf16 with fp32 accumulation) already resident
in HBM.  The headline is prefill: T=4096 tokens per layer, reported as
tokens/s over K timed steps (bracketed by device synchronisation), with the
median of per-step HIP-event times beside it.

Per-stage times come from ``moe_ffn_forward_timed``: the same launches,
with HIP events recorded on the layer's stream at each stage boundary, so
they describe the layer as it runs.  The shader clock during the prefill up
GEMM is read by that GEMM's clock-recording twin (shader cycles against the
constant 100 MHz reference counter, per workgroup).  A plain 1 GiB
device-to-device copy gives the measured HBM bandwidth.

Also in the line: the T=32 decode layer (us/layer, alternating two weight
sets), the tiny fp32 layer, the Zipf-skewed prefill layer, the softmax-over-
all-experts variant, the T-sweep and the 32-layer T=8192 stack (with the
end-to-end residual drift against the oracle's own pass of 256 tokens).  The
CPU baseline of each workload is the fp64 oracle on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at T=4096 + µs/layer at T=32; % of MFMA/HBM peak"
# Kernels the roofline entries describe (names as the profiler reports them).
UP_PREFILL_KERNEL = "moe::grouped_gemm_prefill_kernel<true, 1, false>"
UP_DECODE_KERNEL = "moe::decode_stream_kernel<true, false, 512, 2, 1, 3>"
REF_CLOCK_HZ = 100e6  # the reference counter the GEMM's clock twin reads


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-repeats", type=int, default=3)
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="untimed back-to-back layer calls before the warm-up steps of the T=4096 layers")
    p.add_argument("--stack-cpu-tokens", type=int, default=256,
                   help="sampled tokens the oracle carries through the 32 stacked layers")
    p.add_argument("--only", choices=["prefill", "skewed", "decode", "tiny", "sweep", "stack", "all"], default="all")
    p.add_argument("--sweep-steps", type=int, default=10)
    p.add_argument("--sweep-t", default=None,
                   help="comma-separated token counts to run in the T-sweep (default: the whole sweep)")
    p.add_argument("--stack-steps", type=int, default=20)
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return p.parse_args()


# --------------------------------------------------------------------------- GPU timing


def time_steps(fn, steps, warmup, torch, settle_ms=0.0):
    """Optionally `settle_ms` of back-to-back untimed calls (the shader clock
    takes some 20 steps of a 2 ms layer to settle from idle), then W untimed
    calls, then K calls bracketed by synchronisation; each call also between
    two HIP events on the current stream.  Returns the wall mean and the
    event median/min/max per call (ms)."""
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = [a.elapsed_time(b) for a, b in evs]
    return {"mean_ms": wall * 1e3, "median_ms": statistics.median(per), "min_ms": min(per), "max_ms": max(per)}


def stage_times(layer, steps, torch, moe, clock_rows=None):
    """Median per-stage times (ms) of the layer as it runs, from the events
    moe_ffn_forward_timed records between its launches.  ``clock_rows``: an
    int64 [steps, 4 * G] device tensor for the up GEMM's clock samples."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(steps)]
    for row in evs:  # creates the events before their handles are passed on
        for e in row:
            e.record()
    for _ in range(2):
        layer.timed(evs[0])
    torch.cuda.synchronize()
    for i in range(steps):
        layer.timed(evs[i], None if clock_rows is None else clock_rows[i])
    torch.cuda.synchronize()
    out = {}
    for j, name in enumerate(moe.STAGES):
        out[name] = statistics.median(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps))
    total = statistics.median(evs[i][0].elapsed_time(evs[i][7]) for i in range(steps))
    return out, total


def clock_summary(clk):
    """Shader clock of the up GEMM per workgroup: cycles over reference ticks."""
    import numpy as np

    c = clk.cpu().numpy().reshape(clk.shape[0], -1, 4).astype(np.float64)
    ok = (c[..., 3] > c[..., 2]) & (c[..., 1] > c[..., 0])
    mhz = (c[..., 1] - c[..., 0]) / (c[..., 3] - c[..., 2]) * REF_CLOCK_HZ / 1e6
    spans = [(row[:, 3].max() - row[:, 2].min()) / REF_CLOCK_HZ * 1e3 for row in c if (row[:, 3] > 0).all()]
    return {"mhz_median": float(np.median(mhz[ok])), "mhz_min": float(mhz[ok].min()), "mhz_max": float(mhz[ok].max()),
            "workgroups": int(c.shape[1]), "samples": int(ok.sum()),
            "gemm_ms_from_ref_counter": float(np.median(spans)) if spans else None}


def mfma_ceiling(torch, moe, target_ms=2.0):
    """The chip's bf16 MFMA ceiling under its power limit (moe_mfma_ceiling):
    the GEMM's MFMA pattern alone on random N(0,1) bf16 data, the clock it
    runs at and the rate it reaches."""
    import numpy as np

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    G = (n_cu // 8) * 8
    g = torch.Generator(device="cuda").manual_seed(77)
    ops = torch.randn(32768, generator=g, device="cuda").to(torch.bfloat16)
    clk = torch.zeros(4 * G, dtype=torch.int64, device="cuda")
    sink = torch.empty(G * 256, dtype=torch.float32, device="cuda")
    iters = 2000
    t_end = time.perf_counter() + 0.25  # the clock settles from idle, as for the layer
    while time.perf_counter() < t_end:
        moe.mfma_ceiling(ops, clk, sink, iters * 5)
        torch.cuda.synchronize()
    out = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.mfma_ceiling(ops, clk, sink, iters * 5)
        b.record()
        torch.cuda.synchronize()
        c = clk.cpu().numpy().reshape(G, 4).astype(np.float64)
        mhz = float(np.median((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * REF_CLOCK_HZ / 1e6))
        flops = G * 4 * 64 * iters * 5 * 16384.0
        out.append((flops / (a.elapsed_time(b) * 1e-3), mhz))
    med = sorted(out)[len(out) // 2]
    return {"tflops": med[0] / 1e12, "clock_mhz": med[1], "frac_of_peak": med[0] / 2.5e15,
            "runs_tflops": [round(r[0] / 1e12, 1) for r in out],
            "note": "median of 5 runs of 5.2 TFLOP each after 0.25 s of the same work"}


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of `nbytes`: (read + write) bytes / time."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t = time_steps(lambda: dst.copy_(src), reps, 3, torch)
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": 2 * nbytes / (t["median_ms"] * 1e-3) / 1e9, "bytes_copied": nbytes, "ms": t["median_ms"]}


def measured_traffic(workload, kernels):
    """HBM bytes per launch of `kernels` (a name or a tuple of names, summed)
    from the rocprofv3 FETCH_SIZE and WRITE_SIZE passes stored in
    data/traffic_<workload>.json, or None when none were taken or a kernel's
    source changed since they were."""
    from sparse_mixture_experts_kept_amd import rocprof_summary

    path = os.path.join(ROOT, "sparse_mixture_experts_kept_amd", "data", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        table = json.load(fh)["kernels"]
    total = 0.0
    for kernel in ((kernels,) if isinstance(kernels, str) else kernels):
        rec = table.get(kernel)
        current = rocprof_summary.source_hash(kernel)
        if rec is None or current is None or rec["source_sha256"] != current:
            return None
        total += rec["read_bytes"] + rec["write_bytes"]
    return total


# --------------------------------------------------------------------------- CPU oracle baselines


def _wide(t, torch):
    return t.detach().cpu().to(torch.float64).numpy()


def _blas_threads():
    import threadpoolctl

    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    return (blas[0]["num_threads"] if blas else 1), (blas[0].get("internal_api", "?") if blas else "?")


def cpu_layer(L, repeats, torch, label):
    """The fp64 oracle on every token of one layer (weights widened to fp64
    beforehand, not timed)."""
    from oracle import moe_oracle

    x = L["x"].cpu()
    T = x.shape[0]
    t0 = time.perf_counter()
    w = {k: [_wide(L[k][e], torch) for e in range(8)] for k in ("w1", "w3", "w2")}
    widen_s = time.perf_counter() - t0
    wg = L["w_gate"].cpu()
    bias = L.get("logit_bias")
    bias = None if bias is None else bias.cpu()
    t0 = time.perf_counter()
    for _ in range(repeats):
        moe_oracle.moe_ffn(x, wg, None, None, None, logit_bias=bias,
                           widen_expert=lambda e: (w["w1"][e], w["w3"][e], w["w2"][e]))
    dt = (time.perf_counter() - t0) / repeats
    threads, api = _blas_threads()
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"all {T} tokens of the {label} layer, fp64 NumPy, mean of {repeats} runs; {dt:.3f} s compute "
                      f"per run, weight widening to fp64 ({widen_s:.1f} s) excluded; "
                      f"{len(os.sched_getaffinity(0))} cores visible, BLAS {api} {threads} threads"}


def cpu_stack(stack, x0, n_tokens, torch, seed=57):
    """The oracle's own pass of `n_tokens` sampled tokens through every
    stacked layer (fp64 residual, RMSNorm, layers), timed without the weight
    widening; the GPU's residual after the last layer and its per-layer
    inputs u_l on the same tokens are compared with it.  A second pass with
    u_l and y_l rounded to bf16 where the GPU rounds them shows how far the
    stack alone carries such roundings."""
    import numpy as np

    from oracle import moe_oracle

    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(stack.T, size=n_tokens, replace=False))
    rows = torch.from_numpy(sample).cuda()
    stack.load_input(x0)
    cap = stack.forward(capture=tuple(range(stack.L)), rows=rows)
    torch.cuda.synchronize()
    resid_gpu = moe_oracle._f64(stack.resid.index_select(0, rows).cpu())
    u_gpu = [moe_oracle._f64(cap[l][0].cpu()) for l in range(stack.L)]
    del cap

    def bf16(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()

    prop = moe_oracle._f64(x0.index_select(0, rows).cpu())
    ctrl = prop.copy()
    compute_s = widen_s = 0.0
    u_drift = []
    for l, lw in enumerate(stack.weights):
        t0 = time.perf_counter()
        w = {k: [_wide(lw[k][e], torch) for e in range(8)] for k in ("w1", "w3", "w2")}
        wg = lw["w_gate"].cpu()
        widen_s += time.perf_counter() - t0

        def widen(e):
            return w["w1"][e], w["w3"][e], w["w2"][e]

        t0 = time.perf_counter()
        u = moe_oracle.rmsnorm(prop)
        prop = prop + moe_oracle.moe_ffn(u, wg, None, None, None, widen_expert=widen)["y"]
        compute_s += time.perf_counter() - t0
        u_drift.append(float(np.abs(u_gpu[l] - u).max() / np.abs(u).max()))
        uc = bf16(moe_oracle.rmsnorm(ctrl))
        ctrl = ctrl + bf16(moe_oracle.moe_ffn(uc, wg, None, None, None, widen_expert=widen)["y"])
        del w
    threads, api = _blas_threads()
    scale = np.abs(prop).max()
    return {
        "cpu_baseline": {"value": n_tokens / compute_s, "unit": "tokens/s (through all layers)", "cores": threads,
                         "kind": "oracle",
                         "sample": f"sampled: {n_tokens} of {stack.T} tokens (seeded) through all {stack.L} layers, "
                                   f"fp64 NumPy; {compute_s:.2f} s compute, weight widening ({widen_s:.1f} s) "
                                   f"excluded; BLAS {api} {threads} threads"},
        "residual_drift": {
            "tokens": n_tokens,
            "gpu_vs_oracle": float(np.abs(resid_gpu - prop).max() / scale),
            "oracle_bf16_rounded_vs_oracle": float(np.abs(ctrl - prop).max() / scale),
            "layer_input_drift": u_drift,
            "note": "max |x_L - x_L(oracle)| / max |x_L(oracle)| after the last layer; the control rounds u_l and "
                    "y_l to bf16 where the GPU rounds them, in an otherwise fp64 oracle pass"}}


# --------------------------------------------------------------------------- workloads


def prefill_section(L, args, torch, moe, A, label, want_clock):
    """Headline timing, stage times, clock and roofline of one T=4096 layer."""
    m = A.MIXTRAL
    d, f, E, k = m["d"], m["f"], m["E"], m["k"]
    T = L["dims"]["T"]
    layer = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], logit_bias=L.get("logit_bias"))
    t = time_steps(layer, args.steps, args.warmup, torch, settle_ms=args.settle_ms)
    counts = layer.counts.cpu().tolist()
    stages, stage_total = stage_times(layer, args.steps, torch, moe)
    out = {"t": t, "counts": counts, "stages": stages, "stage_total": stage_total}
    # the standalone permutation (moe_permute: per-group counts, then one wave
    # per 16-token group) on the layer's own routing, beside the layer's
    # permutation stage (which takes the group counts from the router): 20
    # calls on preallocated buffers captured into a HIP graph, so the replay
    # times the device work and its launch gaps, not Python
    ws = torch.empty((moe.permute_workspace_size(T),), dtype=torch.uint8, device="cuda")
    bufs = (torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
            torch.empty((T * k,), dtype=torch.int32, device="cuda"), torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    reps = 20
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.permute(layer.idx, workspace=ws, out=bufs)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            moe.permute(layer.idx, workspace=ws, out=bufs)
    tp = time_steps(graph.replay, args.steps, 3, torch)
    out["permute_standalone_ms"] = tp["median_ms"] / reps
    del graph
    if want_clock:
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        G = (n_cu // 8) * 8
        clk = torch.full((args.steps, 4 * G), -1, dtype=torch.int64, device="cuda")
        cstages, _ = stage_times(layer, args.steps, torch, moe, clock_rows=clk)
        out["clock"] = clock_summary(clk)
        out["clock"]["up_gemm_ms_clocked_twin"] = cstages["up_gemm"]
    out["rows"] = A.prefill_rows_issued(counts)
    out["gemm_rows"] = A.prefill_gemm_rows(counts)  # rows the up GEMM launch itself computes
    del layer
    _log(f"{label}: {t['mean_ms']:.3f} ms/layer (median {t['median_ms']:.3f}); stages "
         f"{json.dumps({k2: round(v, 4) for k2, v in stages.items()})} sum {stage_total:.3f}")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the layer is built and "
              "measured on a single MI355X (multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_mixture_experts_kept_amd import accounting as A
    from sparse_mixture_experts_kept_amd import inputs, moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 2, "copy_probe_bytes_written": dst.numel() * 2,
                          "launches": 3}))
        return
    moe.load_library()
    dev = "cuda"
    m = A.MIXTRAL
    d, f, E, k = m["d"], m["f"], m["E"], m["k"]
    cpu = not args.no_cpu_baseline
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "settle_ms": args.settle_ms,
              "settle_note": "before the W warm-up steps of each T=4096 layer, that layer runs back to back, untimed, "
                             "for settle_ms: from idle the shader clock needs about 20 steps to reach its steady "
                             "value, which is what a continuously running layer sees",
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded random Mixtral-shaped layer; no trained weights)"}
    result["copy_gbps"] = copy_bandwidth(torch)
    _log(f"copy: {result['copy_gbps']['gbps']:.0f} GB/s (1 GiB device-to-device, read + write)")
    result["mfma_ceiling"] = mfma_ceiling(torch, moe)
    _log(f"mfma ceiling: {result['mfma_ceiling']['tflops']:.0f} TFLOP/s at {result['mfma_ceiling']['clock_mhz']:.0f} MHz "
         "(the GEMM's MFMA pattern alone on random bf16)")

    if args.only in ("prefill", "all"):
        _log("prefill: generating T=4096 layer")
        L = inputs.make_workload("prefill", device=dev)
        T = L["dims"]["T"]
        P = prefill_section(L, args, torch, moe, A, "prefill", want_clock=True)
        t, stages = P["t"], P["stages"]
        sec = t["mean_ms"] * 1e-3
        flops = A.layer_flops(T, d, f, E, k)
        gemm_flops = P["gemm_rows"] * A.up_flops_per_slot(d, f)
        up_s = stages["up_gemm"] * 1e-3
        achieved = gemm_flops / up_s
        clock = P["clock"]
        clock_peak = A.PEAK_BF16_FLOPS * clock["mhz_median"] / 2400.0
        touched = sum(1 for c in P["counts"] if c > 0)
        result.update({
            "value": T / sec, "unit": "tokens/s", "ms_per_step": t["mean_ms"],
            "ms_per_step_median": t["median_ms"], "ms_per_step_min": t["min_ms"], "ms_per_step_max": t["max_ms"],
            "config": {"workload": "mixtral-moe-ffn-prefill", "T": T, "d": d, "f": f, "E": E, "k": k,
                       "routing": "near-uniform (router std 0.02)", "counts": P["counts"]},
            "layer_frac_of_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS,
            "stage_ms": stages, "stage_ms_sum": sum(stages.values()), "stage_ms_event_span": P["stage_total"],
            "moe_permute_ms": P["permute_standalone_ms"],
            "stage_ms_note": "medians over the timed steps of moe_ffn_forward_timed: the layer's own launches with "
                             "HIP events between stages on its stream",
            "clock_mhz": clock,
            "roofline": {"kernel": "up projection + SwiGLU, " + UP_PREFILL_KERNEL,
                         "bound": "mfma", "achieved": achieved / 1e12, "peak": A.PEAK_BF16_FLOPS / 1e12,
                         "unit": "TFLOP/s", "frac": achieved / A.PEAK_BF16_FLOPS,
                         "traffic": measured_traffic("prefill", UP_PREFILL_KERNEL),
                         "algorithmic_per_launch": gemm_flops, "rows_per_launch": P["gemm_rows"],
                         "launch_ms": stages["up_gemm"],
                         "clock_mhz": clock["mhz_median"],
                         "frac_of_clock_limited_peak": achieved / clock_peak,
                         "frac_of_measured_mfma_ceiling": achieved / (result["mfma_ceiling"]["tflops"] * 1e12),
                         "algorithmic_bytes_per_launch": A.up_bytes(T, d, f, k, touched)},
        })
        # the same layer with the softmax over all experts (pair not renormalised)
        layer_full = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], gating=moe.GATING_FULL)
        tf = time_steps(layer_full, args.steps, args.warmup, torch)
        result["prefill_full_gating"] = {"workload": "mixtral-moe-ffn-prefill, softmax over all experts",
                                         "T": T, "ms_per_layer": tf["mean_ms"], "ms_per_layer_median": tf["median_ms"],
                                         "tokens_per_s": T / (tf["mean_ms"] * 1e-3)}
        _log(f"prefill (full gating): {tf['mean_ms']:.3f} ms/layer")
        del layer_full
        if cpu:
            _log("cpu baseline: the fp64 oracle on every token of the prefill layer")
            result["cpu_baseline"] = cpu_layer(L, args.cpu_repeats, torch, "T=4096 prefill")
        del L
        torch.cuda.empty_cache()

    if args.only in ("skewed", "all"):
        _log("prefill_skewed: generating T=4096 layer with Zipf(1.2) slot shares")
        L = inputs.make_workload("prefill_skewed", device=dev)
        T = L["dims"]["T"]
        P = prefill_section(L, args, torch, moe, A, "prefill_skewed", want_clock=False)
        t = P["t"]
        counts = P["counts"]
        needed, gemm_rows, tail_rows = P["rows"]
        sk = {"workload": "mixtral-moe-ffn-prefill-zipf", "T": T, "ms_per_layer": t["mean_ms"],
              "ms_per_layer_median": t["median_ms"], "tokens_per_s": T / (t["mean_ms"] * 1e-3),
              "frac_of_bf16_peak": A.layer_flops(T, d, f, E, k) / (t["mean_ms"] * 1e-3) / A.PEAK_BF16_FLOPS,
              "stage_ms": P["stages"], "stage_ms_sum": sum(P["stages"].values()),
              "counts": counts, "slot_shares": [c / (T * k) for c in counts],
              "rows_needed": needed, "rows_issued_gemm": gemm_rows, "rows_issued_tails": tail_rows,
              "tile_padding_waste": (gemm_rows + tail_rows) / needed - 1.0}
        # capacity factor 1.0: each expert keeps at most T*k/E slots
        cap = T * k // E
        layer_cap = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], logit_bias=L["logit_bias"],
                            capacity=cap)
        tc = time_steps(layer_cap, args.steps, args.warmup, torch)
        kept = sum(min(c, cap) for c in counts)
        idx_l, _, logits_l = moe.router_topk(L["x"], L["w_gate"], L["logit_bias"], return_logits=True)
        loss = moe.load_balance_loss(logits_l, idx_l)
        tl = time_steps(lambda: moe.load_balance_loss(logits_l, idx_l), 20, 2, torch)
        sk["capacity_factor_1"] = {"capacity": cap, "ms_per_layer": tc["mean_ms"],
                                   "tokens_per_s": T / (tc["mean_ms"] * 1e-3), "slots_kept": kept,
                                   "slots_dropped": T * k - kept, "dropped_fraction": 1.0 - kept / (T * k)}
        sk["load_balance_loss"] = {"value": float(loss.cpu()[0]), "us_per_call": tl["median_ms"] * 1e3}
        _log(f"prefill_skewed with capacity {cap}: {tc['mean_ms']:.3f} ms/layer, {T * k - kept} of {T * k} "
             f"slots dropped; load-balance loss {float(loss.cpu()[0]):.4f}")
        del layer_cap
        if cpu:
            _log("cpu baseline: the fp64 oracle on every token of the skewed layer")
            sk["cpu_baseline"] = cpu_layer(L, max(1, args.cpu_repeats - 1), torch, "T=4096 Zipf-skewed prefill")
        result["prefill_skewed"] = sk
        del L
        torch.cuda.empty_cache()

    if args.only in ("decode", "all"):
        _log("decode: generating two T=32 layers")
        Ls = [inputs.make_workload("decode", device=dev, seed=s) for s in (2, 1002)]
        T = Ls[0]["dims"]["T"]
        layers = [moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"]) for L in Ls]
        flip = [0]

        def step():
            layers[flip[0]]()
            flip[0] ^= 1

        t = time_steps(step, args.decode_steps, 10, torch)
        sec = t["mean_ms"] * 1e-3
        counts = [lay.counts.cpu().tolist() for lay in layers]
        touched = min(sum(1 for c in cs if c > 0) for cs in counts)
        nbytes = A.decode_layer_bytes(T, d, f, E, k, touched)
        st0, _ = stage_times(layers[0], 50, torch, moe)
        st1, _ = stage_times(layers[1], 50, torch, moe)
        stages = {k2: (st0[k2] + st1[k2]) / 2 for k2 in st0}
        up_bytes = touched * 2 * d * f * 2
        _log(f"decode: {t['mean_ms'] * 1e3:.1f} us/layer; stages (ms) "
             f"{json.dumps({k2: round(v, 4) for k2, v in stages.items()})}")
        dec = {"workload": "mixtral-moe-ffn-decode", "T": T, "us_per_layer": t["mean_ms"] * 1e3,
               "us_per_layer_median": t["median_ms"] * 1e3, "tokens_per_s": T / sec,
               "experts_touched": touched, "layer_bytes": nbytes,
               "layer_frac_of_hbm_peak": nbytes / sec / A.PEAK_HBM_BYTES,
               "layer_frac_of_measured_copy": nbytes / sec / (result["copy_gbps"]["gbps"] * 1e9),
               "stage_ms": stages, "stage_ms_sum": sum(stages.values()),
               "roofline": {"kernel": "up projection + SwiGLU, " + UP_DECODE_KERNEL,
                            "bound": "hbm", "achieved": up_bytes / (stages["up_gemm"] * 1e-3) / 1e9,
                            "peak": A.PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                            "frac": up_bytes / (stages["up_gemm"] * 1e-3) / A.PEAK_HBM_BYTES,
                            "traffic": measured_traffic("decode", UP_DECODE_KERNEL),
                            "algorithmic_per_launch": up_bytes}}
        if cpu:
            _log("cpu baseline: the fp64 oracle on the decode layer")
            dec["cpu_baseline"] = cpu_layer(Ls[0], args.cpu_repeats, torch, "T=32 decode")
        result["decode"] = dec
        del layers, Ls
        torch.cuda.empty_cache()

    if args.only in ("tiny", "all"):
        L = inputs.make_workload("tiny_fp32", device=dev)
        lay = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"])
        t = time_steps(lay, 200, 20, torch)
        tiny = {"workload": "mixtral-moe-ffn-tiny-fp32", "T": 64, "d": 128, "f": 256,
                "us_per_layer": t["mean_ms"] * 1e3, "us_per_layer_median": t["median_ms"] * 1e3}
        if cpu:
            tiny["cpu_baseline"] = cpu_layer(L, 50, torch, "tiny fp32")
        result["tiny_fp32"] = tiny
        _log(f"tiny fp32: {t['median_ms'] * 1e3:.1f} us/layer")
        del lay, L

    if args.only in ("sweep", "all"):
        # T-sweep over both kernel families on one weight set (2.8 GB, far
        # beyond the 256 MB Infinity Cache, so every call streams from HBM).
        _log("sweep: generating a T=8192 layer")
        L = inputs.make_custom(8192, d, f, dtype="bf16", seed=6, device=dev)
        rows = []
        sweep_ts = (1, 4, 16, 32, 64, 96, 128, 192, 256, 512, 1024, 2048, 4096, 8192)
        if args.sweep_t:
            sweep_ts = tuple(int(v) for v in args.sweep_t.split(","))
            if any(t < 1 or t > 8192 for t in sweep_ts):
                raise SystemExit("--sweep-t: token counts from 1 to 8192")
        for T in sweep_ts:
            x = L["x"][:T].contiguous()
            row = {"T": T}
            for name, v in (("auto", moe.VARIANT_AUTO), ("decode", moe.VARIANT_DECODE),
                            ("prefill", moe.VARIANT_PREFILL)):
                lay = moe.FFN(x, L["w_gate"], L["w1"], L["w3"], L["w2"], variant=v)
                row[name + "_us"] = time_steps(lay, args.sweep_steps, 2, torch)["median_ms"] * 1e3
                del lay
            row["tokens_per_s"] = T / (row["auto_us"] * 1e-6)
            row["frac_of_bf16_peak"] = A.layer_flops(T, d, f, E, k) / (row["auto_us"] * 1e-6) / A.PEAK_BF16_FLOPS
            _log(f"sweep: {json.dumps({k2: round(v2, 3) if isinstance(v2, float) else v2 for k2, v2 in row.items()})}")
            rows.append(row)
        result["t_sweep"] = rows
        del L
        torch.cuda.empty_cache()

    if args.only in ("stack", "all"):
        from sparse_mixture_experts_kept_amd.stack import MoEStack

        w = inputs.WORKLOADS["stack"]
        _log(f"stack: generating {w['layers']} layers ({w['layers'] * A.expert_weight_bytes(d, f, E) / 1e9:.1f} GB)")
        stack = MoEStack(w["T"], w["d"], w["f"], w["layers"], seed=5)
        g = torch.Generator(device="cuda").manual_seed(5)
        x0 = torch.randn((w["T"], w["d"]), generator=g, device="cuda", dtype=torch.float32)

        def stack_step():
            stack.load_input(x0)
            stack.forward()

        t = time_steps(stack_step, args.stack_steps, 5, torch)
        hist = stack.hist.cpu().tolist()
        other = {}
        for mode in ("router", "none"):  # the combine as its own launch; also the router as its own launch
            stack.mode = mode
            other[mode] = time_steps(stack_step, max(2, args.stack_steps // 2), 2, torch)
        stack.mode = "combine"
        sec = t["mean_ms"] * 1e-3
        flops = w["layers"] * A.layer_flops(w["T"], d, f, E, k)
        _log(f"stack: {t['mean_ms']:.1f} ms per {w['layers']}-layer pass")
        st = {"workload": "mixtral-moe-ffn-stack", "T": w["T"], "layers": w["layers"],
              "ms_per_pass": t["mean_ms"], "ms_per_pass_median": t["median_ms"], "tokens_per_s": w["T"] / sec,
              "ms_per_layer": t["mean_ms"] / w["layers"], "frac_of_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS,
              "glue": "combine fused into the residual/RMSNorm/next-router glue (moe_ffn_forward_routed_residual)",
              "ms_per_pass_combine_unfused": other["router"]["mean_ms"],
              "ms_per_pass_unfused": other["none"]["mean_ms"],
              "ms_per_layer_saved_by_combine_fusion": (other["router"]["mean_ms"] - t["mean_ms"]) / w["layers"],
              "expert_weight_bytes_resident": w["layers"] * A.expert_weight_bytes(d, f, E),
              "routing_histograms": hist}
        if cpu:
            _log(f"stack: the oracle's own pass of {args.stack_cpu_tokens} sampled tokens through all layers")
            st.update(cpu_stack(stack, x0, args.stack_cpu_tokens, torch))
            _log(f"stack drift: {json.dumps(st['residual_drift']['gpu_vs_oracle'])}, control "
                 f"{json.dumps(st['residual_drift']['oracle_bf16_rounded_vs_oracle'])}")
        result["stack"] = st
        del stack
        torch.cuda.empty_cache()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
