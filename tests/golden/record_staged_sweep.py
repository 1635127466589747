"""Record the measurements the tier gate's CPU test replays: from one JSON
line printed by `python bench.py` (default workload) on an MI355X, keep the
plain host-to-device copy curve, the copy curves through the ring, and per
context the measured staged step times and the HBM-resident per-layer decode
times.  These are measurements of this card, not values from the pages.

    python tests/golden/record_staged_sweep.py BENCH_JSON_FILE > tests/golden/staged_sweep_mi355x.json
"""
import json
import sys


def main(path):
    line = [x for x in open(path) if x.strip().startswith("{")][-1]
    tg = json.loads(line)["extra"]["tier_gate"]
    out = dict(source="bench.py default run (ctx128k) on one MI355X, extra.tier_gate",
               pcie_h2d_curve_MiB_GBps=tg["pcie_h2d_curve_MiB_GBps"],
               staged_copy_curve_MiB_GBps=tg["staged_copy_curve_MiB_GBps"],
               layers=16, num_kv_heads=4, window=1024, contexts=[])
    for row in tg["contexts"]:
        out["contexts"].append(dict(
            context=row["context"],
            resident_us_per_layer=dict(hybrid=row["resident_us_per_layer_hybrid"],
                                       exact=row["resident_us_per_layer_bf16"]),
            measured_ms={k: dict(hybrid=v["ms_hybrid"], exact=v["ms_bf16"]) for k, v in row.items()
                         if k.startswith("slots")}))
    json.dump(out, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main(sys.argv[1])
