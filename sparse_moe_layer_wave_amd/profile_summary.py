"""Summarise rocprofv3 output of a bench.py run into a short text table.

    python -m sparse_moe_layer_wave_amd.profile_summary --trace T.csv \
        [--fetch F.csv --write W.csv] --command "..." --out profiles/NAME.md \
        [--traffic-json profiles/counters_gate_up_hy3_decode_T64.json --kernel "k_decode_gemm<0, 1, 1>" \
         [--grid-x 49152 --grid-y 24] --source gemm_decode.hip]

--trace is rocprofv3's kernel_trace.csv (--kernel-trace --output-format csv);
--fetch / --write are counter_collection.csv files of two --pmc runs
(FETCH_SIZE, WRITE_SIZE: KiB per dispatch).  The counters are scaled by what
they read for the run's first device copy (bench.py --copy-calibration copies
1 GiB before anything else), so "bytes" means bytes as a plain copy of known
size counts them.  The traffic JSON is what bench.py reports as
roofline.traffic while the kernels' source files are unchanged (sha256
prefix of their contents, in order).  --kernel and --source may repeat: a
stage of several kernels (the e4m3 gate_up stage: x quantiser, GEMM, h
quantiser) gets the sum of their per-call traffic.
"""

import argparse
import collections
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def _short(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("hy3::", "")


def _trace(path):
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]),
               int(r["Grid_Size_Z"]), int(r["Workgroup_Size_X"]))
        out[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def _counters(path, counter):
    per = collections.defaultdict(list)
    copies = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = _short(r["Kernel_Name"])
        v = float(r["Counter_Value"])
        per[(name, int(r["Grid_Size"]))].append(v)
        if "copy" in name.lower():
            copies.append((int(r["Dispatch_Id"]), v))
    # the calibration copy (bench.py --copy-calibration) is the run's first
    # copy dispatch; later copies (dtype conversions of the inputs) are not
    # of a known size
    scale = None
    if copies:
        _, v = min(copies)
        scale = COPY_BYTES / (v * 1024.0) if v > 0 else None
    return per, scale


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--command", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--kernel", action="append", help="kernel name for the traffic JSON (repeat: summed)")
    ap.add_argument("--grid-x", type=int, help="grid of that kernel's launch (default: any)")
    ap.add_argument("--grid-y", type=int)
    ap.add_argument("--source", action="append", help="source file (under csrc/) of those kernels (repeatable)")
    ap.add_argument("--workload", default="hy3_decode_T64")
    args = ap.parse_args()

    trace = _trace(args.trace)
    fetch = write = None
    fscale = wscale = None
    if args.fetch:
        fetch, fscale = _counters(args.fetch, "FETCH_SIZE")
    if args.write:
        write, wscale = _counters(args.write, "WRITE_SIZE")

    lines = ["# rocprofv3 summary", "", "Commands:", "", "```", args.command.strip(), "```", ""]
    if fscale:
        lines.append(f"Counter scale (1 GiB device copy): FETCH x{fscale:.3f}, WRITE x{wscale:.3f}")
        lines.append("")
    lines.append("| kernel | grid (threads) | block | calls | avg us | min us | fetch MB/call | write MB/call |")
    lines.append("|---|---|---|---|---|---|---|---|")
    rows = sorted(trace.items(), key=lambda kv: -sum(kv[1]))
    kernels = args.kernel or []
    part = {}
    for (name, gx, gy, gz, bx), durs in rows:
        if "hy3" not in name and "k_" not in name:
            continue
        fmb = wmb = ""
        gsize = gx * gy * gz
        if fetch is not None:
            fv = fetch.get((name, gsize))
            wv = write.get((name, gsize)) if write else None
            if fv and fscale:
                fmb = f"{sum(fv) / len(fv) * 1024 * fscale / 1e6:.1f}"
            if wv and wscale:
                wmb = f"{sum(wv) / len(wv) * 1024 * wscale / 1e6:.1f}"
            if (name in kernels and (len(kernels) > 1 or (args.grid_x in (None, gx) and args.grid_y in (None, gy)))
                    and fv and wv and fscale and wscale):
                part[name] = (sum(fv) / len(fv) * 1024 * fscale + sum(wv) / len(wv) * 1024 * wscale)
        lines.append(f"| {name} | ({gx},{gy},{gz}) | {bx} | {len(durs)} | "
                     f"{sum(durs) / len(durs) / 1e3:.1f} | {min(durs) / 1e3:.1f} | {fmb} | {wmb} |")
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if args.traffic_json and kernels and all(k in part for k in kernels):
        h = hashlib.sha256()
        for src in args.source:
            h.update(open(os.path.join(PKG, "csrc", src), "rb").read())
        one = lambda v: v[0] if len(v) == 1 else v
        rec = {"kernel": one(kernels), "workload": args.workload, "source": one(args.source),
               "source_sha": h.hexdigest()[:16],
               "bytes_per_launch": round(sum(part.values())),
               "how": "FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by a 1 GiB copy"}
        json.dump(rec, open(args.traffic_json, "w"), indent=1)
        print("traffic", rec)


if __name__ == "__main__":
    main()
