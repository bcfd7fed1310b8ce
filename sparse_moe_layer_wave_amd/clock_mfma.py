"""Per-kernel shader clock and MFMA busy fraction from one rocprofv3 --pmc pass.

    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES \\
        --output-format csv -d DIR -o run -- python3 bench.py --profile-workload NAME ...
    python -m sparse_moe_layer_wave_amd.clock_mfma --pmc DIR/run_counter_collection.csv \\
        --command "..." --out profiles/NAME.md

rocprofv3 sums every counter over its instances:
- GRBM_GUI_ACTIVE over the 8 XCDs (cycles of the graphics clock while busy), so
  the mean clock over a dispatch is GRBM_GUI_ACTIVE / 8 / its duration;
- SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs (256 CUs x 4), so the MFMA busy
  fraction is SQ_VALU_MFMA_BUSY_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8);
- SQ_BUSY_CU_CYCLES over the shader engines, each the sum over its SIMDs of
  busy quad-cycles, so the busy fraction is
  4 x SQ_BUSY_CU_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8).

The dense MFMA peak at the measured clock is the nominal peak (2.5 PFLOP/s
bf16 at 2.4 GHz) scaled by clock / 2.4 GHz.
"""

import argparse
import collections
import csv

from .profile_summary import _short

XCDS, SIMDS = 8, 1024
NOMINAL_GHZ = 2.4


def table(path):
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = {}
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), r["Dispatch_Id"])
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    byk = collections.defaultdict(list)
    for key, cs in per.items():
        gui = cs.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        if gui <= 0 or dur[key] <= 0:
            continue
        byk[key[0]].append((dur[key] / 1e3, gui / dur[key], cs.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * gui),
                            4.0 * cs.get("SQ_BUSY_CU_CYCLES", 0.0) / (SIMDS * gui)))
    rows = []
    for name, lst in byk.items():
        lst.sort()
        us, ghz, mfma, cu = lst[len(lst) // 2]          # the dispatch of median duration
        rows.append((name, len(lst), us, ghz, mfma, cu))
    rows.sort(key=lambda r: -r[2])
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--pmc", required=True,
                    help="counter_collection.csv of a pass with GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES")
    ap.add_argument("--command", required=True, help="the command lines that produced the input")
    ap.add_argument("--out", required=True)
    ap.add_argument("--min-us", type=float, default=20.0, help="omit kernels shorter than this")
    a = ap.parse_args()
    lines = ["# Shader clock and MFMA busy fraction per kernel", "", "Commands:", "", "```", a.command, "```", "",
             "Values of the dispatch with the median duration (under counter collection).", "",
             "| kernel | dispatches | duration (us) | mean clock (GHz) | MFMA busy | CU busy |",
             "|---|---|---|---|---|---|"]
    for name, n, us, ghz, mfma, cu in table(a.pmc):
        if us < a.min_us:
            continue
        lines.append(f"| {name} | {n} | {us:.1f} | {ghz:.2f} | {mfma:.3f} | {cu:.3f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
