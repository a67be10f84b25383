"""Summarize the grouped-GEMM profile of `bench.py --moe-only` (a rocprofv3
kernel trace plus TCC_HIT/TCC_MISS and FETCH_SIZE counter runs) as the
per-GEMM table of grouped_gemm_moe_layer.md.

Usage: python summarize_gemm_profile.py <profile dir with trace/, tcc/, fetch/>

--moe-only runs, per routing, three forward+backward layers and then each of
the six grouped GEMMs three times, always in the order FC1, FC2, FC2 dgrad,
FC2 wgrad, FC1 dgrad, FC1 wgrad; the GEMM dispatches are labelled from that
order.
"""
import collections
import csv
import statistics
import sys

ORDER = ["FC1 forward", "FC2 forward", "FC2 dgrad", "FC2 wgrad", "FC1 dgrad", "FC1 wgrad"]
MODE = {"FC1 forward": "NT bf16", "FC2 forward": "NT MXFP8", "FC2 dgrad": "NN MXFP8", "FC2 wgrad": "TN MXFP8",
        "FC1 dgrad": "NN MXFP8", "FC1 wgrad": "TN MXFP8"}
R, H, I = 65536, 2048, 768
FL = {"FC1 forward": 2 * R * 2 * I * H, "FC2 forward": 2 * R * H * I, "FC2 dgrad": 2 * R * H * I,
      "FC2 wgrad": 2 * R * H * I, "FC1 dgrad": 2 * R * 2 * I * H, "FC1 wgrad": 2 * R * 2 * I * H}
# algorithmic bytes (operands once, E8M0 scales, bf16 output once), as in the layer's scope table
BY = {"FC1 forward": 1275e6, "FC2 forward": 528e6, "FC2 dgrad": 447e6, "FC2 wgrad": 593e6, "FC1 dgrad": 787e6,
      "FC1 wgrad": 1048e6}
PEAK = {"NT bf16": 2500.0}
FETCH_SCALE = 2.0   # FETCH_SIZE calibration against a plain copy of known size


def labels(ids):
    per_routing = 6 * 3 + 6 * 3
    out = {}
    for k, d in enumerate(ids):
        j = k % per_routing
        out[d] = ORDER[j % 6] if j < 18 else ORDER[(j - 18) // 3]
    return out


def main(base):
    tr = [r for r in csv.DictReader(open(f"{base}/trace/moe_kernel_trace.csv")) if "gemm_kernel" in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    lab = labels([int(r["Dispatch_Id"]) for r in tr])
    dur = collections.defaultdict(list)
    for r in tr:
        dur[lab[int(r["Dispatch_Id"])]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(path, names):
        rows = [r for r in csv.DictReader(open(path)) if "gemm_kernel" in r["Kernel_Name"]]
        disp = sorted({int(r["Dispatch_Id"]) for r in rows})
        lb = labels(disp)
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in rows:
            if r["Counter_Name"] in names:
                acc[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        per = collections.defaultdict(list)
        for d, v in acc.items():
            per[lb[d]].append(v)
        return per

    tcc = counters(f"{base}/tcc/moe_counter_collection.csv", {"TCC_HIT_sum", "TCC_MISS_sum"})
    fet = counters(f"{base}/fetch/moe_counter_collection.csv", {"FETCH_SIZE"})
    print("| GEMM | mode | dispatches | median us | TFLOP/s | % of dense peak | algorithmic bytes | flop/B |"
          " roofline-attainable TFLOP/s | % of attainable | L2 hit rate | HBM read MB |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for g in ORDER:
        us = statistics.median(dur[g])
        tf = FL[g] / us / 1e6
        peak = PEAK.get(MODE[g], 5000.0)
        ai = FL[g] / BY[g]
        att = min(peak, ai * 8.0)   # flop/B x 8 TB/s, in TFLOP/s
        hits = statistics.median(v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"]) for v in tcc[g])
        mb = statistics.median(v["FETCH_SIZE"] for v in fet[g]) * 1024 * FETCH_SCALE / 1e6
        print(f"| {g} | {MODE[g]} | {len(dur[g])} | {us:.1f} | {tf:.0f} | {100 * tf / peak:.1f} | {BY[g] / 1e6:.0f} MB |"
              f" {ai:.0f} | {att:.0f} | {100 * tf / att:.1f} | {100 * hits:.1f} % | {mb:.0f} |")


if __name__ == "__main__":
    main(sys.argv[1])
