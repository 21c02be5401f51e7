"""Benchmark of the Mixtral sparse-MoE feed-forward layer on one MI355X.

One step = one whole layer (router -> permute -> up+SwiGLU -> down ->
combine) through ``moe_ffn_forward`` on synthetic Mixtral-shaped inputs
(d=4096, f=14336, E=8, top-2, bf16 with fp32 accumulation) already resident
in HBM.  The headline is prefill: T=4096 tokens per layer, reported as
tokens/s.  The decode layer (T=32) is timed too and reported as us/layer in
the same JSON line, alternating between two independent weight sets.

Per-kernel times come from HIP events recorded on the stream the kernels run
on, around the staged calls (moe_expert_up etc.), in a second timed loop.
The CPU baseline is the fp64 oracle on a bounded sample of the same prefill
workload, on this host's cores.  The 32-layer stack (T=8192, 90 GB of expert
weights resident, RMSNorm + residual between layers) is reported as
end-to-end tokens/s with per-layer routing histograms.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at T=4096 + µs/layer at T=32; % of MFMA/HBM peak"
# Kernels the roofline entries describe (names as the profiler reports them).
# The prefill up projection is two launches: the GEMM over every full
# 256-row tile and the streaming kernel over the experts' short tails.
UP_PREFILL_KERNEL = ("moe::grouped_gemm_prefill_kernel<true, 1>", "moe::decode_stream_kernel<true, true, 256, 2, 2, 4>")
UP_DECODE_KERNEL = "moe::decode_stream_kernel<true, false, 512, 2, 1, 3>"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=4096, help="tokens of the prefill workload the oracle runs")
    p.add_argument("--cpu-repeats", type=int, default=3)
    p.add_argument("--only", choices=["prefill", "skewed", "decode", "sweep", "stack", "all"], default="all")
    p.add_argument("--sweep-steps", type=int, default=10)
    p.add_argument("--sweep-t", default=None,
                   help="comma-separated token counts to run in the T-sweep (default: the whole sweep)")
    p.add_argument("--stack-steps", type=int, default=3)
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return p.parse_args()


def time_layer(layer_fn, steps, warmup, torch):
    for _ in range(warmup):
        layer_fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer_fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def staged_timing(L, steps, torch, moe, variant):
    """Average per-stage kernel time (ms) with HIP events on the current stream."""
    x, wg, bias, w1, w3, w2 = L["x"], L["w_gate"], L.get("logit_bias"), L["w1"], L["w3"], L["w2"]
    T, d = x.shape
    idx, w = moe.router_topk(x, wg, bias)
    offs, sorted_slots, slot_rows = moe.permute(idx, d, w1.shape[1])
    h = moe.expert_up(x, offs, sorted_slots, w1, w3, variant=variant)
    y_rows = moe.expert_down(h, offs, w2, T, variant=variant)
    stages = ["router", "permute", "up", "down", "combine"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        e = ev[i]
        e[0].record()
        moe.router_topk(x, wg, bias)
        e[1].record()
        moe.permute(idx, d, w1.shape[1])
        e[2].record()
        moe.expert_up(x, offs, sorted_slots, w1, w3, variant=variant, h=h)
        e[3].record()
        moe.expert_down(h, offs, w2, T, variant=variant, y_rows=y_rows)
        e[4].record()
        moe.combine(y_rows, slot_rows, w, x.dtype)
        e[5].record()
    torch.cuda.synchronize()
    out = {}
    for j, name in enumerate(stages):
        out[name] = sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
    return out


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


def cpu_baseline(L, sample_tokens, repeats):
    """The fp64 oracle on `sample_tokens` tokens of the workload (weights
    widened to fp64 beforehand, not timed)."""
    import numpy as np
    import threadpoolctl

    from oracle import moe_oracle

    x = L["x"].cpu()
    T = x.shape[0]
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(T, size=min(sample_tokens, T), replace=False))
    t0 = time.perf_counter()
    w1 = [moe_oracle._f64(L["w1"][e].cpu()) for e in range(8)]
    w3 = [moe_oracle._f64(L["w3"][e].cpu()) for e in range(8)]
    w2 = [moe_oracle._f64(L["w2"][e].cpu()) for e in range(8)]
    widen_s = time.perf_counter() - t0
    xs = x[tok]
    wg = L["w_gate"].cpu()
    t0 = time.perf_counter()
    for _ in range(repeats):
        moe_oracle.moe_ffn(xs, wg, None, None, None, widen_expert=lambda e: (w1[e], w3[e], w2[e]))
    dt = (time.perf_counter() - t0) / repeats
    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    return {"value": len(tok) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(tok)} of {T} tokens of the prefill layer, fp64 NumPy, mean of {repeats} runs; "
                      f"{dt:.2f} s compute per run, weight widening to fp64 ({widen_s:.1f} s) excluded; "
                      f"{len(os.sched_getaffinity(0))} cores visible, BLAS "
                      f"{blas[0].get('internal_api', '?') if blas else '?'} {threads} threads"}


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
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded random Mixtral-shaped layer; no trained weights)"}

    if args.only in ("prefill", "all"):
        _log("prefill: generating T=4096 layer")
        L = inputs.make_workload("prefill", device=dev)
        T = L["dims"]["T"]
        layer = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"])
        sec = time_layer(layer, args.steps, args.warmup, torch)
        _log(f"prefill: {sec * 1e3:.3f} ms/layer")
        stages = staged_timing(L, args.steps, torch, moe, moe.VARIANT_AUTO)
        _log(f"prefill stages (ms): {json.dumps({k2: round(v, 4) for k2, v in stages.items()})}")
        flops = A.layer_flops(T, d, f, E, k)
        up_flops = T * k * A.up_flops_per_slot(d, f)
        up_s = stages["up"] * 1e-3
        result.update({
            "value": T / sec, "unit": "tokens/s", "ms_per_step": sec * 1e3,
            "config": {"workload": "mixtral-moe-ffn-prefill", "T": T, "d": d, "f": f, "E": E, "k": k,
                       "routing": "near-uniform (router std 0.02)", "counts": layer.counts.cpu().tolist()},
            "layer_frac_of_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS,
            "stage_ms": stages,
            "stage_ms_note": "each stage through its standalone entry point (the binding's output allocation and "
                             "launch gaps included; the permute stage is the general one-workgroup permutation, "
                             "which the layer replaces by the router's group counts and one wave per 16-token "
                             "group); the up stage is the roofline's GEMM + tail pair",
            "roofline": {"kernel": "up projection + SwiGLU: grouped_gemm_prefill_kernel<true, 1> + tail "
                                   "decode_stream_kernel<true, true, ...>",
                         "bound": "mfma", "achieved": up_flops / up_s / 1e12, "peak": A.PEAK_BF16_FLOPS / 1e12,
                         "unit": "TFLOP/s", "frac": up_flops / up_s / A.PEAK_BF16_FLOPS,
                         "traffic": measured_traffic("prefill", UP_PREFILL_KERNEL),
                         "algorithmic_per_launch": up_flops,
                         "algorithmic_bytes_per_launch": A.up_bytes(T, d, f, k, sum(1 for c in layer.counts.tolist() if c > 0))},
        })
        # the same layer with the softmax over all experts (pair not renormalised)
        layer_full = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], gating=moe.GATING_FULL)
        sec_full = time_layer(layer_full, args.steps, args.warmup, torch)
        result["prefill_full_gating"] = {"workload": "mixtral-moe-ffn-prefill, softmax over all experts",
                                         "T": T, "ms_per_layer": sec_full * 1e3, "tokens_per_s": T / sec_full}
        _log(f"prefill (full gating): {sec_full * 1e3:.3f} ms/layer")
        del layer_full
        if not args.no_cpu_baseline:
            _log("cpu baseline: running the fp64 oracle on a token sample")
            result["cpu_baseline"] = cpu_baseline(L, args.cpu_sample, args.cpu_repeats)
        del layer, L
        torch.cuda.empty_cache()

    if args.only in ("skewed", "all"):
        _log("prefill_skewed: generating T=4096 layer with Zipf(1.2) slot shares")
        L = inputs.make_workload("prefill_skewed", device=dev)
        T = L["dims"]["T"]
        layer = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], logit_bias=L["logit_bias"])
        sec = time_layer(layer, args.steps, args.warmup, torch)
        stages = staged_timing(L, args.steps, torch, moe, moe.VARIANT_AUTO)
        counts = layer.counts.cpu().tolist()
        needed, gemm_rows, tail_rows = A.prefill_rows_issued(counts)
        _log(f"prefill_skewed: {sec * 1e3:.3f} ms/layer, counts {counts}")
        result["prefill_skewed"] = {
            "workload": "mixtral-moe-ffn-prefill-zipf", "T": T, "ms_per_layer": sec * 1e3, "tokens_per_s": T / sec,
            "frac_of_bf16_peak": A.layer_flops(T, d, f, E, k) / sec / A.PEAK_BF16_FLOPS, "stage_ms": stages,
            "counts": counts, "slot_shares": [c / (T * k) for c in counts],
            "rows_needed": needed, "rows_issued_gemm": gemm_rows, "rows_issued_tails": tail_rows,
            "tile_padding_waste": (gemm_rows + tail_rows) / needed - 1.0}
        # capacity factor 1.0: each expert keeps at most T*k/E slots
        cap = T * k // E
        layer_cap = moe.FFN(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], logit_bias=L["logit_bias"],
                            capacity=cap)
        sec_cap = time_layer(layer_cap, args.steps, args.warmup, torch)
        kept = sum(min(c, cap) for c in counts)
        # the load-balancing loss on this layer's scores (one small launch)
        idx_l, _, logits_l = moe.router_topk(L["x"], L["w_gate"], L["logit_bias"], return_logits=True)
        loss = moe.load_balance_loss(logits_l, idx_l)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(20):
            moe.load_balance_loss(logits_l, idx_l)
        ev1.record()
        torch.cuda.synchronize()
        result["prefill_skewed"]["capacity_factor_1"] = {
            "capacity": cap, "ms_per_layer": sec_cap * 1e3, "tokens_per_s": T / sec_cap,
            "slots_kept": kept, "slots_dropped": T * k - kept, "dropped_fraction": 1.0 - kept / (T * k)}
        result["prefill_skewed"]["load_balance_loss"] = {"value": float(loss.cpu()[0]),
                                                          "us_per_call": ev0.elapsed_time(ev1) * 1e3 / 20}
        _log(f"prefill_skewed with capacity {cap}: {sec_cap * 1e3:.3f} ms/layer, "
             f"{T * k - kept} of {T * k} slots dropped; load-balance loss {float(loss.cpu()[0]):.4f}")
        del layer, layer_cap, L
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

        sec = time_layer(step, args.decode_steps, 10, torch)
        counts = [lay.counts.cpu().tolist() for lay in layers]
        touched = min(sum(1 for c in cs if c > 0) for cs in counts)
        nbytes = A.decode_layer_bytes(T, d, f, E, k, touched)
        st0 = staged_timing(Ls[0], 50, torch, moe, moe.VARIANT_AUTO)
        st1 = staged_timing(Ls[1], 50, torch, moe, moe.VARIANT_AUTO)
        stages = {k2: (st0[k2] + st1[k2]) / 2 for k2 in st0}
        up_bytes = touched * 2 * d * f * 2
        _log(f"decode: {sec * 1e6:.1f} us/layer; stages (ms) {json.dumps({k2: round(v, 4) for k2, v in stages.items()})}")
        dec = {"workload": "mixtral-moe-ffn-decode", "T": T, "us_per_layer": sec * 1e6, "tokens_per_s": T / sec,
               "experts_touched": touched, "layer_bytes": nbytes,
               "layer_frac_of_hbm_peak": nbytes / sec / A.PEAK_HBM_BYTES, "stage_ms": stages,
               "roofline": {"kernel": "decode_stream_kernel<UP> (up projection + SwiGLU)",
                            "bound": "hbm", "achieved": up_bytes / (stages["up"] * 1e-3) / 1e9,
                            "peak": A.PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                            "frac": up_bytes / (stages["up"] * 1e-3) / A.PEAK_HBM_BYTES,
                            "traffic": measured_traffic("decode", UP_DECODE_KERNEL),
                            "algorithmic_per_launch": up_bytes}}
        result["decode"] = dec
        if "value" not in result:
            result.update({"value": T / sec, "unit": "tokens/s", "ms_per_step": sec * 1e3,
                           "config": {"workload": "mixtral-moe-ffn-decode", "T": T, "d": d, "f": f, "E": E,
                                      "k": k}, "roofline": dec["roofline"]})

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
                row[name + "_us"] = time_layer(lay, args.sweep_steps, 2, torch) * 1e6
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

        sec = time_layer(stack_step, args.stack_steps, 1, torch)
        hist = stack.hist.cpu().tolist()
        stack.fused = False  # every layer routes its own input: the router as its own launch
        sec_unfused = time_layer(stack_step, args.stack_steps, 1, torch)
        stack.fused = True
        flops = w["layers"] * A.layer_flops(w["T"], d, f, E, k)
        _log(f"stack: {sec * 1e3:.1f} ms per {w['layers']}-layer pass")
        result["stack"] = {"workload": "mixtral-moe-ffn-stack", "T": w["T"], "layers": w["layers"],
                           "ms_per_pass": sec * 1e3, "tokens_per_s": w["T"] / sec,
                           "ms_per_layer": sec * 1e3 / w["layers"], "frac_of_bf16_peak": flops / sec / A.PEAK_BF16_FLOPS,
                           "ms_per_pass_router_unfused": sec_unfused * 1e3,
                           "expert_weight_bytes_resident": w["layers"] * A.expert_weight_bytes(d, f, E),
                           "routing_histograms": hist}
        del stack
        torch.cuda.empty_cache()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
