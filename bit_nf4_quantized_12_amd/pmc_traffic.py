"""HBM traffic per launch of the roofline GEMM from two rocprofv3 counter runs.

Usage (after two runs of the same command, one per counter, on the GPU):

    rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -o run --output-format csv -- python3 bench.py \
        --steps 1 --warmup 0 --legs roofline,copycal --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE -d <write_dir> ... (same command)
    python -m bit_nf4_quantized_12_amd.pmc_traffic <fetch_dir> <write_dir> <out.json>

FETCH_SIZE / WRITE_SIZE (KiB per dispatch, summed over the L2 channels) are
calibrated with the `copycal` leg, one elementwise pass (bf16 negation) that
reads and writes exactly COPY_BYTES: factor = COPY_BYTES / counter bytes, per
direction. The result
records the sha256 of the GEMM source it was measured on; bench.py reports
the traffic only while that source is unchanged.
"""

import csv
import glob
import hashlib
import json
import os
import re
import sys

COPY_BYTES = 1 << 30
ROOFLINE_KERNEL = "gemm_kernel<512, 128, false, false, true, false>"
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")


def gemm_source_sha():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, counter value in bytes)}."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    out = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                d = (f, row["Dispatch_Id"])
                name, v = out.get(d, (row["Kernel_Name"], 0.0))
                out[d] = (name, v + float(row["Counter_Value"]) * 1024.0)
    return list(out.values())


def _mean(vals):
    return sum(vals) / len(vals) if vals else None


def summarize(fetch_dir, write_dir):
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _per_dispatch(d, counter)
        gemm = [v for n, v in rows if ROOFLINE_KERNEL in re.sub(r"\s+", " ", n)]
        copy = [v for n, v in rows if "neg_kernel" in n]
        if not gemm or not copy:
            raise SystemExit(f"{counter}: {len(gemm)} roofline launches, {len(copy)} copies found")
        # the calibration pass is a single dispatch moving COPY_BYTES each way
        res[counter] = {"gemm_bytes_per_launch": _mean(gemm), "gemm_launches": len(gemm),
                        "copy_counter_bytes": max(copy), "factor": COPY_BYTES / max(copy)}
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    traffic = f["gemm_bytes_per_launch"] * f["factor"] + w["gemm_bytes_per_launch"] * w["factor"]
    return {"kernel": ROOFLINE_KERNEL, "gemm_source_sha256": gemm_source_sha(),
            "traffic_bytes_per_launch": traffic, "fetch": f, "write": w,
            "copy_bytes": COPY_BYTES}


def main():
    if len(sys.argv) != 4:
        raise SystemExit(__doc__)
    out = summarize(sys.argv[1], sys.argv[2])
    with open(sys.argv[3], "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
