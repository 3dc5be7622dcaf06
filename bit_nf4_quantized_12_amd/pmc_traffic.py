"""HBM traffic per launch of a kernel from two rocprofv3 counter runs.

Usage (after two runs of the same command, one per counter, on the GPU):

    rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -o run --output-format csv -- python3 bench.py \
        --steps 1 --warmup 0 --legs roofline,copycal --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE -d <write_dir> ... (same command)
    python -m bit_nf4_quantized_12_amd.pmc_traffic <fetch_dir> <write_dir> <out.json> [kernel]

Per-shape tables of the same two runs (calibrated bytes per dispatch, one
row per kernel and grid size), and the matrix-core summary of a run with
SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE:

    python -m bit_nf4_quantized_12_amd.pmc_traffic table <fetch_dir> <write_dir> <kernel substring> ...
    python -m bit_nf4_quantized_12_amd.pmc_traffic mfma <run_dir> <kernel substring> ...

and the mean per dispatch of every counter of a run, per kernel and grid size:

    python -m bit_nf4_quantized_12_amd.pmc_traffic counters <run_dir> <kernel substring> ...

The kernel defaults to the benchmark step's input-gradient GEMM instance;
out.json for the roofline is profiles/roofline_gemm_traffic_<config>.json.

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
ROOFLINE_KERNEL = "gemm_kernel<512, 128, true, true, true, false>"
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")
PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def traffic_file(config):
    return os.path.join(PROFILES, f"roofline_gemm_traffic_{config}.json")


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


def _rows(run_dir):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                yield f, row


def _short(name):
    name = re.sub(r"^void ", "", name).replace("qlora::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def _by_shape(run_dir, kernels):
    """{(kernel, grid size): {counter: [per-dispatch value summed over instances]}}."""
    acc = {}
    for f, row in _rows(run_dir):
        name = re.sub(r"\s+", " ", row["Kernel_Name"])
        hit = [k for k in kernels if k in name]
        if not hit:
            continue
        key = (_short(name), int(row["Grid_Size"]))
        d = acc.setdefault(key, {}).setdefault(row["Counter_Name"], {})
        d[(f, row["Dispatch_Id"])] = d.get((f, row["Dispatch_Id"]), 0.0) + float(row["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def table(fetch_dir, write_dir, kernels):
    """Calibrated FETCH / WRITE bytes per dispatch, per kernel and grid size."""
    cal = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        copy = [v for n, v in _per_dispatch(d, counter) if "neg_kernel" in n]
        if not copy:
            raise SystemExit(f"{counter}: no calibration copy in {d}")
        cal[counter] = COPY_BYTES / max(copy)
    f = _by_shape(fetch_dir, kernels)
    w = _by_shape(write_dir, kernels)
    out = []
    for key in sorted(set(f) | set(w)):
        fv = f.get(key, {}).get("FETCH_SIZE", [])
        wv = w.get(key, {}).get("WRITE_SIZE", [])
        out.append({"kernel": key[0], "grid": key[1], "dispatches": len(fv),
                    "fetch_bytes": _mean(fv) * 1024.0 * cal["FETCH_SIZE"] if fv else None,
                    "write_bytes": _mean(wv) * 1024.0 * cal["WRITE_SIZE"] if wv else None})
    return {"factors": cal, "rows": out}


def mfma(run_dir, kernels):
    """Matrix-core busy fraction per kernel and grid size. GRBM_GUI_ACTIVE is
    summed over the 8 XCDs (rocprofv3 sums a counter over its instances) and
    SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs, so busy / (GUI / 8 * 1024)
    is the fraction of SIMD cycles with the matrix core busy; MOPS x 512 is
    the bf16 flops issued."""
    out = []
    for key, cs in sorted(_by_shape(run_dir, kernels).items()):
        busy = sum(cs.get("SQ_VALU_MFMA_BUSY_CYCLES", []))
        gui = sum(cs.get("GRBM_GUI_ACTIVE", []))
        mops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])
        out.append({"kernel": key[0], "grid": key[1], "dispatches": len(mops),
                    "mfma_busy_frac": busy / (gui / 8 * 1024) if gui else None,
                    "bf16_flops_per_dispatch": _mean(mops) * 512 if mops else None,
                    "gui_cycles_per_xcd_per_dispatch": gui / 8 / len(mops) if mops else None})
    return out


def counters(run_dir, kernels):
    """Mean per dispatch of every counter in a run, per kernel and grid size."""
    return [{"kernel": k[0], "grid": k[1], "dispatches": max(len(v) for v in cs.values()),
             "means": {c: _mean(v) for c, v in sorted(cs.items())}}
            for k, cs in sorted(_by_shape(run_dir, kernels).items())]


def _mean(vals):
    return sum(vals) / len(vals) if vals else None


def summarize(fetch_dir, write_dir, kernel=ROOFLINE_KERNEL):
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _per_dispatch(d, counter)
        gemm = [v for n, v in rows if kernel in re.sub(r"\s+", " ", n)]
        copy = [v for n, v in rows if "neg_kernel" in n]
        if not gemm or not copy:
            raise SystemExit(f"{counter}: {len(gemm)} roofline launches, {len(copy)} copies found")
        # the calibration pass is a single dispatch moving COPY_BYTES each way
        res[counter] = {"gemm_bytes_per_launch": _mean(gemm), "gemm_launches": len(gemm),
                        "copy_counter_bytes": max(copy), "factor": COPY_BYTES / max(copy)}
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    traffic = f["gemm_bytes_per_launch"] * f["factor"] + w["gemm_bytes_per_launch"] * w["factor"]
    return {"kernel": kernel, "gemm_source_sha256": gemm_source_sha(),
            "traffic_bytes_per_launch": traffic, "fetch": f, "write": w,
            "copy_bytes": COPY_BYTES}


def main():
    if len(sys.argv) >= 5 and sys.argv[1] == "table":
        print(json.dumps(table(sys.argv[2], sys.argv[3], sys.argv[4:]), indent=1))
        return
    if len(sys.argv) >= 4 and sys.argv[1] == "counters":
        print(json.dumps(counters(sys.argv[2], sys.argv[3:]), indent=1))
        return
    if len(sys.argv) >= 4 and sys.argv[1] == "mfma":
        print(json.dumps(mfma(sys.argv[2], sys.argv[3:]), indent=1))
        return
    if len(sys.argv) not in (4, 5):
        raise SystemExit(__doc__)
    out = summarize(sys.argv[1], sys.argv[2], *sys.argv[4:5])
    with open(sys.argv[3], "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
