"""Per-kernel L1-to-L2 read latency from one rocprofv3 --pmc pass of bench.py.

    rocprofv3 --pmc TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCC_HIT_sum TCC_MISS_sum \\
        --output-format csv -d DIR -o run -- python3 bench.py --profile-workload NAME ...
    python -m sparse_moe_layer_wave_amd.l2_latency --pmc DIR/run_counter_collection.csv \\
        --command "..." --out profiles/NAME.md

For every kernel the table gives the median over its dispatches of the
L1 (TCP) to L2 (TCC) read requests (128-byte lines here), the mean latency
of those requests in cycles (summed latency / requests) and the L2 hit
fraction.  A kernel whose copy stream keeps a fixed number of lines in
flight per CU runs at that number x 128 bytes / latency per CU, which is
how the latency column bears on a kernel's time.
"""

import argparse
import collections
import csv

from .profile_summary import _short

COUNTERS = ("TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum")


def table(path):
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), r["Dispatch_Id"])
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    byk = collections.defaultdict(list)
    for (name, _), cs in per.items():
        byk[name].append(cs)
    rows = []
    for name, lst in byk.items():
        def med(f):
            v = sorted(f(c) for c in lst)
            return v[len(v) // 2]
        req = med(lambda c: c.get("TCP_TCC_READ_REQ_sum", 0.0))
        lat = med(lambda c: c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / max(c.get("TCP_TCC_READ_REQ_sum", 0.0), 1.0))
        hit = med(lambda c: c.get("TCC_HIT_sum", 0.0) / max(c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0), 1.0))
        rows.append((name, len(lst), req, lat, hit))
    rows.sort(key=lambda r: -r[2])
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--pmc", required=True, help="counter_collection.csv of a pass with %s" % " ".join(COUNTERS))
    ap.add_argument("--command", required=True, help="the command lines that produced the input")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    lines = ["# L1-to-L2 read latency per kernel", "", "Commands:", "", "```", a.command, "```", "",
             "| kernel | dispatches | L1-to-L2 read requests / call | mean latency (clk) | L2 hit fraction |",
             "|---|---|---|---|---|"]
    for name, n, req, lat, hit in table(a.pmc):
        if req < 1:
            continue
        lines.append(f"| {name} | {n} | {req / 1e6:.2f}M | {lat:.0f} | {hit:.3f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
