"""Throughput of the Hy3 MoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]

One step = one hy3moe_forward call (router, dispatch order, gate_up, down,
fp32 combine) over one batch of synthetic Hy3-shaped input already resident
in HBM.  The main line is the decode batch (T=64 tokens, d=4096, 192 experts,
top-8, d_ff=1536, bf16 experts); the prefill batch (T=8192) is reported in the
same JSON line under "prefill", and the skewed, FP8 (T=8192 and T=64) and
full-block (shared expert, route_norm, score bias; hy3moe_block_forward)
workloads under their own keys.  Per-kernel durations come from HIP events recorded on the launch
stream between the stages (the *_timed entry points).

Under "prefill" / "at_measured_clock" the MFMA fractions are given once more
against the dense bf16 peak at the graphics clock amd-smi reports while the
prefill layer runs back to back (after the timed steps): MI355X lowers its
clock well below the 2.4 GHz of the published peak under sustained MFMA load.
"roofline" itself is always against the published peak.

Prints one JSON line.  Only one GPU is used; --gpus N > 1 exits with a message.
"""

import argparse
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from sparse_moe_layer_wave_amd import hy3moe, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
NOMINAL_SCLK_GHZ = 2.4         # graphics clock the dense peaks are quoted at


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                 # creates the underlying hipEvent
    return evs


def algorithmic(c, n_touched):
    """Bytes and FLOPs a kernel must move/compute, counting only touched
    experts' weights, each tensor once, and no padding."""
    T, d, E, k, F = c["T"], c["d"], c["E"], c["k"], c["F"]
    block = c.get("block", False)
    rows = T * k + (T if block else 0)              # the shared expert sees every token
    n_touched = n_touched + (1 if block else 0)
    wb = 1 if c.get("weights") in ("fp8", "fp8_block128") else 2     # weight scales not counted
    return {
        "gate_up": dict(bytes=n_touched * 2 * F * d * wb + T * d * 2 + rows * F * 2,
                        flops=2 * rows * d * 2 * F),
        "down": dict(bytes=n_touched * d * F * wb + rows * F * 2 + rows * d * 2,
                     flops=2 * rows * F * d),
        "router": dict(bytes=E * d * 4 + T * d * 2 + rows * 8, flops=2 * T * d * E),
        # out: fp32, or bf16 out plus the bf16 residual read: 4 bytes per element either way
        "combine": dict(bytes=rows * d * 2 + T * k * 8 + T * d * 4, flops=2 * rows * d),
        "layer_flops": T * ((k + (1 if block else 0)) * 6 * d * F + 2 * d * E),
    }


def _smi_gfx_clock_mhz():
    """Mean of the per-XCD graphics clocks amd-smi reports right now (MHz), or
    None when amd-smi is missing or prints no clock."""
    exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if exe is None:
        return None
    try:
        txt = subprocess.run([exe, "metric", "-c"], capture_output=True, text=True, timeout=15).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    mhz = [int(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", txt)]
    return sum(mhz) / len(mhz) if mhz else None


def clock_probe(step, seconds):
    """Graphics clock (GHz) while `step` runs back to back for about `seconds`
    (outside every timed region): amd-smi is sampled twice from a helper
    thread, after a third and two thirds of the time.  None if unavailable."""
    samples = []

    def sampler():
        for frac in (1 / 3, 2 / 3):
            time.sleep(seconds / 3)
            v = _smi_gfx_clock_mhz()
            if v is not None:
                samples.append(v)

    th = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    th.join()
    return round(sum(samples) / len(samples) / 1e3, 3) if samples else None


def run_workload(cfg, steps, warmup, clock_probe_s=0.0):
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
                                             norm_weight=inp["norm_w"], norm_eps=1e-6,
                                             score_bias=inp["score_bias"], out=out, workspace=ws,
                                             stage_events=evs, return_routing=return_routing)
        if block:
            return hy3moe.block_forward(inp["x"], inp["W_gate"], inp["W_gu"], inp["W_dn"], inp["Ws_gu"],
                                        inp["Ws_dn"], k, inp["scale"], norm_weight=inp["norm_w"],
                                        norm_eps=1e-6, score_bias=inp["score_bias"], out=out,
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
    res = dict(cfg=c, ms_per_step=elapsed / steps * 1e3, tokens_per_s=T * steps / elapsed, step_gpu_ms=step_gpu_ms,
               stage_ms=stage_ms, n_touched=n_touched, alg=alg,
               layer_tflops=alg["layer_flops"] * steps / elapsed / 1e12,
               hottest_over_mean=float(load.max() / load.mean()),
               sclk_ghz=clock_probe(step, clock_probe_s) if clock_probe_s > 0 else None)
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
    return {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic(kernel, res),
            "avg_kernel_ms": round(ms, 5)}


def traffic(kernel, res):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel source; otherwise null."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{res['cfg']['name']}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "sparse_moe_layer_wave_amd", "csrc", rec["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if sha != rec.get("source_sha"):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, max_seconds=25.0):
    """The oracle, as it stands, on the first tokens of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    class Lazy:                         # expert weights stay in HBM until the oracle needs one
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return inputs.bits(self.t[int(e)])

    inp = inputs.make_inputs(cfg, device="cuda")
    c = inp["cfg"]
    x_bits, W = inputs.bits(inp["x"]), inputs.bits(inp["W_gate"])
    b = None if inp["bias"] is None else inputs.bits(inp["bias"])
    gu, dn = Lazy(inp["W_gu"]), Lazy(inp["W_dn"])
    n = 0
    t0 = time.perf_counter()
    chunk = 4
    while n < c["T"] and time.perf_counter() - t0 < max_seconds:
        toks = np.arange(n, min(n + chunk, c["T"]))
        oracle.forward_tokens(toks, x_bits, W, gu, dn, c["k"], inputs.ROUTER_SCALE, b)
        n += len(toks)
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {c['T']} decode tokens, oracle.forward_tokens in chunks of "
                      f"{chunk} (NumPy float64, OpenBLAS), {el:.1f} s"}


def shares(steps, warmup):
    """The expert GEMMs at one GPU's share of a sharded layer (Hy3 dims, bf16).
    8-way expert parallelism gives each GPU 24 experts and, after the
    dispatch exchange, T*k/8 of the (token, slot) rows of a T-token batch: a
    24-expert layer with k = 8 over T/8 tokens has the same expert GEMMs
    (its router and combine are not the sharded ones).  d_ff parallelism gives
    each GPU all experts with d_ff/8 (192) or d_ff/4 (384) columns."""
    base = dict(inputs.CONFIGS[1])
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
    ap.add_argument("--clock-probe", type=float, default=2.5, metavar="SECONDS",
                    help="after the timed prefill steps, run them back to back this long while amd-smi "
                         "samples the graphics clock (0: skip)")
    ap.add_argument("--shares", action="store_true",
                    help="print one JSON line with the expert GEMMs at one GPU's share of an 8-way expert-parallel "
                         "or 8- / 4-way d_ff-parallel layer, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 1 GiB device-to-device copy (outside every timed region), "
                         "a known byte count for scaling HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the layer is not sharded "
              "across GPUs in this build", file=sys.stderr)
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

    if args.profile_workload:
        names = {c["name"]: i for i, c in inputs.CONFIGS.items()}
        if args.profile_workload not in names:
            print(f"unknown workload {args.profile_workload!r}; one of {sorted(names)}", file=sys.stderr)
            sys.exit(2)
        res, _ = run_workload(names[args.profile_workload], args.steps, args.warmup)
        print(json.dumps({"workload": args.profile_workload, "ms_per_step": round(res["ms_per_step"], 4),
                          "kernel_ms": {k: round(v, 5) for k, v in res["stage_ms"].items()},
                          "step_gpu_ms": res["step_gpu_ms"]}), flush=True)
        return

    dec, _ = run_workload(1, args.steps, args.warmup)
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
        pre, _ = run_workload(2, max(5, args.steps // 5), args.warmup, clock_probe_s=args.clock_probe)
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
        # the same fractions against the dense bf16 peak at the graphics clock
        # the GPU held while running this layer back to back (amd-smi)
        if pre["sclk_ghz"]:
            peak = BF16_PEAK_TFLOPS * pre["sclk_ghz"] / NOMINAL_SCLK_GHZ
            gu = line["prefill"]["roofline"]["achieved"]
            line["prefill"]["at_measured_clock"] = {
                "sclk_ghz": pre["sclk_ghz"], "bf16_peak_tflops": round(peak, 1),
                "gate_up_frac": round(gu / peak, 4),
                "down_frac": round(line["prefill"]["roofline_down"]["achieved"] / peak, 4),
                "layer_frac": round(pre["layer_tflops"] / peak, 4)}
        else:
            line["prefill"]["at_measured_clock"] = None
    if not args.no_extra:
        for key, cfg, bound in (("skewed", 3, "mfma"), ("fp8", 4, "mfma"), ("fp8_decode", 7, "hbm"),
                                ("block_decode", 5, "hbm"), ("block_prefill", 6, "mfma"),
                                ("skewed_decode", 8, "hbm"), ("fp8_block128_decode", 9, "hbm"),
                                ("fp8_block128", 10, "mfma"), ("block_residual_prefill", 11, "mfma")):
            n = args.steps if bound == "hbm" else max(3, args.steps // 10)
            res, _ = run_workload(cfg, n, min(args.warmup, 2))
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
        line["cpu_baseline"] = cpu_baseline(1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
