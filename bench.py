"""Throughput of the Hy3 MoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]

One step = one hy3moe_forward call (router, dispatch order, gate_up, down,
fp32 combine) over one batch of synthetic Hy3-shaped input already resident
in HBM.  The main line is the decode batch (T=64 tokens, d=4096, 192 experts,
top-8, d_ff=1536, bf16 experts); the prefill batch (T=8192) is reported in the
same JSON line under "prefill", and the skewed, FP8 (T=8192 and T=64) and
full-block (shared expert, route_norm, score bias; hy3moe_block_forward)
workloads under their own keys.  Per-kernel durations come from HIP events
recorded on the launch stream between the stages (the *_timed entry points).
Fractions of peak are against MI355X's published dense peaks (bf16 2.5
PFLOP/s, fp8 5.0 PFLOP/s, HBM 8 TB/s).

The cpu_baseline leg (skip with --no-cpu-baseline) runs the CPU oracle on the
host after the GPU work: its throughput on the whole decode batch (repeated
for at least 10 s) and on the whole prefill batch (expert weights copied to
the host and decoded to float64 before the timed region), and, per workload,
the GPU's routing against the oracle's on every token (near-tie tokens
flagged, chosen sets and slot orders that differ) under "routing_vs_oracle".

Prints one JSON line.  Only one GPU is used; --gpus N > 1 exits with a message.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from sparse_moe_layer_wave_amd import hy3moe, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
ROUTE_NORM_EPS = float(np.float32(1e-6))


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                 # creates the underlying hipEvent
    return evs


def algorithmic(c, n_touched):
    """Bytes and FLOPs a stage must move/compute, counting only touched
    experts' weights, each tensor once, and no padding.  With e4m3 experts the
    gate_up stage is the x quantiser (bf16 x in, e4m3 codes and row scales
    out) plus the gate_up product, whose h is the e4m3 activation with its row
    scale; weight scales are not counted."""
    T, d, E, k, F = c["T"], c["d"], c["E"], c["k"], c["F"]
    block = c.get("block", False)
    rows = T * k + (T if block else 0)              # the shared expert sees every token
    n_touched = n_touched + (1 if block else 0)
    fp8 = c.get("weights") in ("fp8", "fp8_block128")
    wb = 1 if fp8 else 2
    if fp8:
        gu_bytes = n_touched * 2 * F * d + T * d * 2 + rows * (F + 4)
        dn_bytes = n_touched * d * F + rows * (F + 4) + rows * d * 2
    else:
        gu_bytes = n_touched * 2 * F * d * wb + T * d * 2 + rows * F * 2
        dn_bytes = n_touched * d * F * wb + rows * F * 2 + rows * d * 2
    return {
        "gate_up": dict(bytes=gu_bytes, flops=2 * rows * d * 2 * F),
        "down": dict(bytes=dn_bytes, flops=2 * rows * F * d),
        "router": dict(bytes=E * d * 4 + T * d * 2 + rows * 8, flops=2 * T * d * E),
        # out: fp32, or bf16 out plus the bf16 residual read: 4 bytes per element either way
        "combine": dict(bytes=rows * d * 2 + T * k * 8 + T * d * 4, flops=2 * rows * d),
        "layer_flops": T * ((k + (1 if block else 0)) * 6 * d * F + 2 * d * E),
    }


def run_workload(cfg, steps, warmup):
    inp = inputs.make_inputs(cfg, device="cuda")
    c = inp["cfg"]
    T, d, E, k, F = c["T"], c["d"], c["E"], c["k"], c["F"]
    fp8 = c.get("weights") in ("fp8", "fp8_block128")
    block128 = c.get("weights") == "fp8_block128"
    block = c.get("block", False)
    if block:
        ws = torch.empty(hy3moe.block_workspace_size(T, d, E, k, F), dtype=torch.uint8, device="cuda")
    else:
        ws = hy3moe.alloc_workspace(T, d, E, k, F,
                                    hy3moe.WEIGHTS_FP8_E4M3 if fp8 else hy3moe.WEIGHTS_BF16)
    residual = c.get("residual", False)
    out = torch.empty((T, d), dtype=torch.bfloat16 if residual else torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def step(evs=None, return_routing=False):
        if residual:
            return hy3moe.block_forward_bf16(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                             inp["Ws_dn"], k, inp["scale"], residual=inp["residual"],
                                             norm_weight=inp["norm_w"], norm_eps=ROUTE_NORM_EPS,
                                             score_bias=inp["score_bias"], out=out, workspace=ws,
                                             stage_events=evs, return_routing=return_routing)
        if block:
            return hy3moe.block_forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                        inp["Ws_dn"], k, inp["scale"], norm_weight=inp["norm_w"],
                                        norm_eps=ROUTE_NORM_EPS, score_bias=inp["score_bias"], out=out,
                                        workspace=ws, stage_events=evs, return_routing=return_routing)
        if fp8:
            return hy3moe.forward_fp8(inp["x"], inp["W_gate"], inp["Wq_gu"], inp["s_gu"], inp["Wq_dn"],
                                      inp["s_dn"], k, inp["scale"], bias=inp["bias"], out=out,
                                      workspace=ws, stage_events=evs, return_routing=return_routing,
                                      block128=block128)
        return hy3moe.forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], k, inp["scale"],
                              bias=inp["bias"], out=out, workspace=ws, stage_events=evs,
                              return_routing=return_routing)

    for _ in range(warmup):
        step()
    _, idx_r, _ = step(return_routing=True)
    torch.cuda.synchronize()
    load = np.bincount(idx_r.cpu().numpy().reshape(-1), minlength=E)
    n_touched = int((load > 0).sum())
    evs = [_events(6) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
                for i, name in enumerate(hy3moe.STAGES)}
    # GPU time of each whole step (first to last stage event): median and spread
    step_gpu = np.array([evs[s][0].elapsed_time(evs[s][len(hy3moe.STAGES)]) for s in range(steps)])
    step_gpu_ms = {q: round(float(np.percentile(step_gpu, p)), 5) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    alg = algorithmic(c, n_touched)
    # what the routing check of the cpu_baseline leg needs: the GPU's routing
    # and the router's inputs, on the host
    routing = dict(name=c["name"], idx=idx_r.cpu().numpy(), x=inputs.bits(inp["x"]),
                   W_gate=inputs.bits(inp["W_gate"]), k=k, scale=inp["scale"],
                   bias=None if inp["bias"] is None else inputs.bits(inp["bias"]),
                   norm_w=inputs.bits(inp["norm_w"]) if block else None,
                   score_bias=inputs.bits(inp["score_bias"]) if block else None)
    res = dict(cfg=c, ms_per_step=elapsed / steps * 1e3, tokens_per_s=T * steps / elapsed, step_gpu_ms=step_gpu_ms,
               stage_ms=stage_ms, n_touched=n_touched, alg=alg,
               layer_tflops=alg["layer_flops"] * steps / elapsed / 1e12,
               hottest_over_mean=float(load.max() / load.mean()), routing=routing)
    del inp, ws, out
    torch.cuda.empty_cache()
    return res, idx


def roofline(res, kernel, bound):
    ms = res["stage_ms"][kernel]
    a = res["alg"][kernel]
    if bound == "hbm":
        achieved = a["bytes"] / (ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = a["flops"] / (ms * 1e-3) / 1e12
        fp8 = res["cfg"].get("weights") in ("fp8", "fp8_block128")
        peak, unit = (FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS), "TFLOP/s"
    fp8 = res["cfg"].get("weights") in ("fp8", "fp8_block128")
    label = kernel
    if fp8 and kernel == "gate_up":
        label = "gate_up stage (x quantiser, gate_up GEMM, h quantiser)"
    return {"bound": bound, "kernel": label, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic(kernel, res),
            "avg_kernel_ms": round(ms, 5)}


def traffic(kernel, res):
    """HBM bytes per launch of the stage's kernels (summed: the e4m3 gate_up
    stage is three) from the committed rocprofv3 counter summary, when it was
    taken on the current kernel sources; otherwise null."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{res['cfg']['name']}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in [rec["source"]] if isinstance(rec["source"], str) else rec["source"]:
        h.update(open(os.path.join(ROOT, "sparse_moe_layer_wave_amd", "csrc", src), "rb").read())
    if h.hexdigest()[:16] != rec.get("source_sha"):
        return None
    return rec.get("bytes_per_launch")


def _host_experts(t, experts):
    """Host float64 copies of the listed experts of a device weight tensor,
    keyed by expert (the oracle indexes them like the bit-pattern array)."""
    import oracle
    return {int(e): oracle.bf16_bits_to_f64(inputs.bits(t[int(e)])) for e in experts}


def _time_oracle(cfg, n_tokens, min_seconds=0.0):
    """oracle.forward on the first n_tokens of a bf16 workload, repeated until
    min_seconds have passed (at least once): the expert weights the batch
    touches are copied to the host and decoded to float64 first, outside the
    timed region; the timed region is the whole oracle forward (router,
    experts, combine).  Returns (tokens/s, seconds, experts, repeats)."""
    import oracle
    inp = inputs.make_inputs(cfg, device="cuda")
    c = inp["cfg"]
    x_bits = inputs.bits(inp["x"])[:n_tokens]
    W = inputs.bits(inp["W_gate"])
    b = None if inp["bias"] is None else inputs.bits(inp["bias"])
    touched = np.unique(oracle.route(x_bits, W, c["k"], inp["scale"], b).idx)
    gu, dn = _host_experts(inp["W_gu"], touched), _host_experts(inp["W_dn"], touched)
    del inp
    torch.cuda.empty_cache()
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < min_seconds:
        oracle.forward(x_bits, W, gu, dn, c["k"], inputs.ROUTER_SCALE, b)
        reps += 1
    el = time.perf_counter() - t0
    return n_tokens * reps / el, el, len(touched), reps


def _routing_vs_oracle(rt):
    """The GPU's routing of one workload against oracle.route on every token."""
    import oracle
    x = rt["x"]
    if rt["norm_w"] is not None:
        x = oracle.rms_norm_bf16(x, rt["norm_w"], ROUTE_NORM_EPS)
    r = oracle.route(x, rt["W_gate"], rt["k"], rt["scale"], rt["bias"], score_bias=rt["score_bias"])
    idx = rt["idx"].astype(np.int64)
    set_eq = np.all(np.sort(idx, axis=1) == np.sort(r.idx, axis=1), axis=1)
    slot_eq = np.all(idx == r.idx, axis=1)
    return {"tokens": int(idx.shape[0]), "near_tie": int(r.near_tie.sum()),
            "order_tie": int(r.order_tie.sum()), "set_diff": int((~set_eq).sum()),
            "slot_diff": int((~slot_eq).sum()),
            "set_diff_unflagged": int((~set_eq & ~r.near_tie).sum()),
            "slot_diff_unflagged": int((~slot_eq & ~r.order_tie).sum())}


def cpu_baseline_leg(routings):
    """The oracle on the host cores: the whole decode batch (repeated for at
    least 10 s) and the whole prefill batch; then the routing check of every
    workload."""
    from threadpoolctl import threadpool_info
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] + [1])
    vendor = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "unknown"
    dec, dec_s, dec_e, dec_n = _time_oracle("hy3_decode_T64", 64, min_seconds=10.0)
    pre, pre_s, pre_e, _ = _time_oracle("hy3_prefill_T8192", 8192)
    base = {"value": round(dec, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 64-token decode batch (hy3_decode_T64, {dec_e} experts) {dec_n} times, "
                      f"oracle.forward in NumPy float64 on {threads} BLAS threads ({vendor}), {dec_s:.1f} s; "
                      "expert weights copied to the host and decoded to float64 before the timed region",
            "host_cpus": len(os.sched_getaffinity(0)),
            "prefill": {"value": round(pre, 2), "unit": "tokens/s",
                        "sample": f"the whole 8192-token prefill batch (hy3_prefill_T8192, {pre_e} experts) once, "
                                  f"{pre_s:.1f} s, same method"}}
    checks = {rt["name"]: _routing_vs_oracle(rt) for rt in routings}
    return base, checks


def shares(steps, warmup):
    """The expert GEMMs at one GPU's share of a sharded layer (Hy3 dims, bf16).
    8-way expert parallelism gives each GPU 24 experts and, after the
    dispatch exchange, T*k/8 of the (token, slot) rows of a T-token batch: a
    24-expert layer with k = 8 over T/8 tokens has the same expert GEMMs
    (its router and combine are not the sharded ones).  d_ff parallelism gives
    each GPU all experts with d_ff/8 (192) or d_ff/4 (384) columns."""
    base = dict(inputs.CONFIGS["hy3_decode_T64"])
    cases = [("ep8_prefill_T8192", dict(base, T=1024, E=24, seed=11), "mfma"),
             ("ep8_decode_T64x8", dict(base, T=64, E=24, seed=12), "hbm"),
             ("tp8_decode_T64", dict(base, T=64, F=192, seed=13), "hbm"),
             ("tp4_decode_T64", dict(base, T=64, F=384, seed=14), "hbm")]
    out = {"shares": "expert GEMMs at one GPU's share (8 GPUs expert-parallel, or d_ff split 8 / 4 ways)"}
    for name, c, bound in cases:
        c["name"] = name
        res, _ = run_workload(c, steps, warmup)
        out[name] = {"T": c["T"], "E": c["E"], "d_ff": c["F"], "experts_touched": res["n_touched"],
                     "gemm_ms": round(res["stage_ms"]["gate_up"] + res["stage_ms"]["down"], 4),
                     "roofline": roofline(res, "gate_up", bound), "roofline_down": roofline(res, "down", bound)}
    return out


def _graph_ms(fn, reps):
    """Median time of fn's GPU work over reps replays of a HIP graph that
    captures it (launch overhead excluded)."""
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del graph
    return float(np.median(times))


def vendor_gemm(steps, warmup):
    """The T=8192 prefill expert GEMMs on the vendor GEMM library (torch.mm,
    which calls hipBLASLt / rocBLAS), beside this library's grouped kernels on
    the same workload: (a) one dense GEMM of all T*k rows against one expert's
    weights, the same FLOPs with every weight reused by every row; (b) one GEMM
    per expert on that expert's rows of the prefill routing, all launches
    captured in one HIP graph.  bf16 operands, fp32 accumulation, random data."""
    c = dict(inputs.CONFIGS["hy3_prefill_T8192"])
    res, _ = run_workload(c, steps, warmup)
    T, d, E, k, F = c["T"], c["d"], c["E"], c["k"], c["F"]
    counts = np.bincount(res["routing"]["idx"].reshape(-1), minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)])
    R = int(offs[-1])
    g = torch.Generator(device="cuda").manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, device="cuda", generator=g).to(torch.bfloat16)

    X, H = rnd(R, d), rnd(R, F)
    W_gu, W_dn = rnd(E, 2 * F, d), rnd(E, d, F)
    G, Y = torch.empty(R, 2 * F, dtype=torch.bfloat16, device="cuda"), torch.empty(R, d, dtype=torch.bfloat16, device="cuda")
    reps = max(steps, 10)
    sl = [(int(offs[e]), int(offs[e + 1])) for e in range(E) if counts[e] > 0]
    cases = {
        "dense_gate_up": (lambda: torch.mm(X, W_gu[0].t(), out=G), 2.0 * R * d * 2 * F),
        "per_expert_gate_up": (lambda: [torch.mm(X[a:b], W_gu[e].t(), out=G[a:b])
                                        for e, (a, b) in zip(np.nonzero(counts)[0], sl)], 2.0 * R * d * 2 * F),
        "dense_down": (lambda: torch.mm(H, W_dn[0].t(), out=Y), 2.0 * R * F * d),
        "per_expert_down": (lambda: [torch.mm(H[a:b], W_dn[e].t(), out=Y[a:b])
                                     for e, (a, b) in zip(np.nonzero(counts)[0], sl)], 2.0 * R * F * d),
    }
    out = {"vendor_gemm": "T=8192 prefill expert GEMMs: torch.mm (hipBLASLt / rocBLAS) against this library's "
                          "grouped kernels on the same routing", "rows": R, "experts": len(sl),
           "rows_per_expert": {"min": int(counts[counts > 0].min()), "mean": round(float(R / len(sl)), 1),
                               "max": int(counts.max())}}
    for name, (fn, flops) in cases.items():
        ms = _graph_ms(fn, reps)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1), "frac": round(flops / ms / 1e9 / 2500.0, 4)}
    for st in ("gate_up", "down"):
        rf = roofline(res, st, "mfma")
        out["grouped_" + st] = {"ms": rf["avg_kernel_ms"], "tflops": rf["achieved"], "frac": rf["frac"]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=8192 prefill line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the skewed T=65536, FP8 and full-block lines")
    ap.add_argument("--profile-workload", metavar="NAME",
                    help="run only the named workload (a profiler pass: one workload per run), "
                         "print its stage times and exit")
    ap.add_argument("--shares", action="store_true",
                    help="print one JSON line with the expert GEMMs at one GPU's share of an 8-way expert-parallel "
                         "or 8- / 4-way d_ff-parallel layer, and exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="print one JSON line comparing the T=8192 prefill expert GEMMs with torch.mm "
                         "(hipBLASLt / rocBLAS), dense and per expert, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 1 GiB device-to-device copy (outside every timed region), "
                         "a known byte count for scaling HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the layer is not sharded "
              "across GPUs", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()

    if args.shares:
        print(json.dumps(shares(args.steps, args.warmup)), flush=True)
        return
    if args.vendor_gemm:
        print(json.dumps(vendor_gemm(args.steps, args.warmup)), flush=True)
        return

    if args.profile_workload:
        if args.profile_workload not in inputs.CONFIGS:
            print(f"unknown workload {args.profile_workload!r}; one of {sorted(inputs.CONFIGS)}", file=sys.stderr)
            sys.exit(2)
        res, _ = run_workload(args.profile_workload, args.steps, args.warmup)
        print(json.dumps({"workload": args.profile_workload, "ms_per_step": round(res["ms_per_step"], 4),
                          "kernel_ms": {k: round(v, 5) for k, v in res["stage_ms"].items()},
                          "step_gpu_ms": res["step_gpu_ms"]}), flush=True)
        return

    dec, _ = run_workload("hy3_decode_T64", args.steps, args.warmup)
    routings = [dec.pop("routing")]
    line = {
        "metric": "MoE-layer tokens/s at T=64 & T=8192; % of HBM BW / % of MFMA peak",
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, Hy3 MoE layer shapes; random-init weights)",
        "config": {"workload": dec["cfg"]["name"], "T": 64, "d": 4096, "E": 192, "k": 8,
                   "d_ff": 1536, "experts_touched": dec["n_touched"]},
        "roofline": roofline(dec, "gate_up", "hbm"),
        "kernel_ms": {k: round(v, 5) for k, v in dec["stage_ms"].items()},
        "step_gpu_ms": dec["step_gpu_ms"],
        "layer_tflops": round(dec["layer_tflops"], 3),
    }
    if not args.no_prefill:
        pre, _ = run_workload("hy3_prefill_T8192", max(5, args.steps // 5), args.warmup)
        routings.append(pre.pop("routing"))
        line["prefill"] = {
            "workload": pre["cfg"]["name"], "tokens_per_s": round(pre["tokens_per_s"], 1),
            "ms_per_step": round(pre["ms_per_step"], 4),
            "layer_tflops": round(pre["layer_tflops"], 2),
            "layer_frac_of_bf16_peak": round(pre["layer_tflops"] / BF16_PEAK_TFLOPS, 4),
            "roofline": roofline(pre, "gate_up", "mfma"),
            "roofline_down": roofline(pre, "down", "mfma"),
            "kernel_ms": {k: round(v, 5) for k, v in pre["stage_ms"].items()},
            "step_gpu_ms": pre["step_gpu_ms"],
        }
    if not args.no_extra:
        for key, cfg, bound in (("skewed", "hy3_long_skewed_T65536", "mfma"), ("fp8", "hy3_fp8_T8192", "mfma"),
                                ("fp8_decode", "hy3_fp8_decode_T64", "hbm"),
                                ("block_decode", "hy3_block_decode_T64", "hbm"),
                                ("block_prefill", "hy3_block_prefill_T8192", "mfma"),
                                ("skewed_decode", "hy3_skewed_decode_T64", "hbm"),
                                ("fp8_block128_decode", "hy3_fp8_block128_decode_T64", "hbm"),
                                ("fp8_block128", "hy3_fp8_block128_T8192", "mfma"),
                                ("block_residual_prefill", "hy3_block_residual_T8192", "mfma")):
            n = args.steps if bound == "hbm" else max(3, args.steps // 10)
            res, _ = run_workload(cfg, n, min(args.warmup, 2))
            routings.append(res.pop("routing"))
            line[key] = {
                "workload": res["cfg"]["name"], "tokens_per_s": round(res["tokens_per_s"], 1),
                "ms_per_step": round(res["ms_per_step"], 4),
                "layer_tflops": round(res["layer_tflops"], 2),
                "hottest_over_mean": round(res["hottest_over_mean"], 2),
                "roofline": roofline(res, "gate_up", bound),
                "roofline_down": roofline(res, "down", bound),
                "kernel_ms": {k: round(v, 5) for k, v in res["stage_ms"].items()},
                "step_gpu_ms": res["step_gpu_ms"],
            }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["routing_vs_oracle"] = cpu_baseline_leg(routings)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
