"""HBM traffic and matrix-core activity per kernel launch from rocprofv3
counter runs.

Two runs of one benchmark workload under ``rocprofv3 --pmc`` (one with
FETCH_SIZE, one with WRITE_SIZE; both in KiB per dispatch) are reduced to the
average per launch of each GEMM kernel family.  Each counter is scaled by what
it reads for a plain device copy of known size (``bench.py --calib-copy``
copies 256 MiB), so the figures are bytes, whatever the counter's own unit or
coverage.  Optional runs add the matrix-core counters: one with
SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA work in units of 512 flops),
SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE, and one with the
derived MfmaUtil (percent of SIMD cycles with the MFMA unit busy).

    python -m moe_variable_size_amd.counters --workload config2 \\
        --fetch DIR --write DIR [--mfma DIR] [--util DIR] \\
        --out profiles/traffic_counters.json

DIR is the ``-d`` directory of a run made with ``--output-format csv``.  The
output file keeps one record per workload (others already in it are kept while
the kernel sources match).  The file carries the sha256 of the kernel sources;
``bench.py`` reports the traffic only while the sources still match.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("moe_variable_size_amd/csrc/mfma.hip", "moe_variable_size_amd/csrc/common.hpp",
                  "moe_variable_size_amd/csrc/api.hip")
COPY_BYTES = 256 << 20   # bench.py --calib-copy: 64 Mi float32 copied device to device

# forward-shaped kernels: mfma_fwd_kernel<BM, BN, WGM, WGN, MODE, Tout, F8, MX, COMB>
_FWD = re.compile(r"mfma_fwd_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), ([^,<>]+), (true|false), "
                  r"(true|false)(?:, (\d+))?>")
FWD_MODES = {0: "grouped_gemm", 1: "fused_fwd", 2: "gated_up", 3: "gated_down"}
# input-gradient kernels: mfma_dx_kernel<NW, GB, ROWS, COMB>; weight gradient:
# mfma_dw_kernel<Tout, NW, RM, SC, DYN>.  COMB 1 = the ranked combine
# ("_ranked" families); SC false = no routing weights ("_unweighted" for the
# plain dW); DYN (work queue or static deal) does not split a family.
_DX = re.compile(r"mfma_dx_kernel<(\d+), (true|false), (true|false)(?:, (\d+))?>")
_DW = re.compile(r"mfma_dw_kernel<[^,<>]+, (\d+), (\d+)(?:, (true|false))?(?:, (?:true|false))?>")


def source_digest() -> str:
    """sha256 over the kernel sources the counter figures belong to."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _family(name: str):
    """Kernel family of a demangled kernel name (None: not counted)."""
    if "copyBuffer" in name or "copy_kernel" in name or "CopyKernel" in name:
        return "copy"
    m = _FWD.search(name)
    if m:
        bm, mode = int(m.group(1)), int(m.group(5))
        f8, mx = m.group(7) == "true", m.group(8) == "true"
        fam = FWD_MODES.get(mode)
        if fam is None:
            return None
        if fam == "fused_fwd" and bm == 64:
            fam = "decode_fwd"
        fam = fam + "_mx" if mx else fam + "_fp8" if f8 else fam
        return fam + "_ranked" if m.group(9) == "1" else fam
    m = _DX.search(name)
    if m:
        gb, rows = m.group(2) == "true", m.group(3) == "true"
        fam = "gated_bwd_dh" if gb else "gated_bwd_dx" if rows else "bwd_dx"
        return fam + "_ranked" if m.group(4) == "1" else fam
    m = _DW.search(name)
    if m:
        fam = {0: "bwd_dw", 1: "gated_bwd_dw_down", 2: "gated_bwd_dw_gu"}.get(int(m.group(2)))
        return fam + "_unweighted" if fam == "bwd_dw" and m.group(3) == "false" else fam
    return None


def per_launch_kib(run_dir: str, counter: str) -> dict:
    """Average counter value per dispatch, per kernel family ("kib" is the
    counter's value, whatever its unit).  The calibration ("copy") family keeps
    only the copy dispatches with the largest grid: the 256 MiB calibration
    copy, not the small copies of results to the host."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per_dispatch = defaultdict(float)
    fam_of = {}
    copy_grid = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                fam = _family(row["Kernel_Name"])
                if fam is None:
                    continue
                key = (f, row["Dispatch_Id"])
                per_dispatch[key] += float(row["Counter_Value"])
                fam_of[key] = fam
                if fam == "copy":
                    copy_grid[key] = int(row["Grid_Size"])
    if copy_grid:
        big = max(copy_grid.values())
        for key, g in copy_grid.items():
            if g != big:
                del per_dispatch[key]
                del fam_of[key]
    sums, counts = defaultdict(float), defaultdict(int)
    for key, v in per_dispatch.items():
        sums[fam_of[key]] += v
        counts[fam_of[key]] += 1
    return {fam: {"kib": sums[fam] / counts[fam], "dispatches": counts[fam]} for fam in sums}


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")


def mfma_summary(mfma_dir, util_dir) -> dict:
    """Per kernel family: bf16 MFMA flops executed per launch (MOPS x 512),
    the raw busy-cycle counters and the derived MfmaUtil (percent)."""
    out = defaultdict(dict)
    if mfma_dir:
        for c in MFMA_COUNTERS:
            for fam, v in per_launch_kib(mfma_dir, c).items():
                if fam == "copy":
                    continue
                out[fam][c] = round(v["kib"], 1)
                if c == "SQ_INSTS_VALU_MFMA_MOPS_BF16":
                    out[fam]["mfma_bf16_flops"] = int(v["kib"] * 512)
    if util_dir:
        for fam, v in per_launch_kib(util_dir, "MfmaUtil").items():
            if fam != "copy":
                out[fam]["MfmaUtil_pct"] = round(v["kib"], 2)
    return dict(out)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True,
                    help="name of the benchmark line the runs profiled (config2, config3, ...)")
    ap.add_argument("--fetch", required=True, help="rocprofv3 -d directory of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="rocprofv3 -d directory of the WRITE_SIZE run")
    ap.add_argument("--mfma", help="rocprofv3 -d directory of the raw matrix-core counter run")
    ap.add_argument("--util", help="rocprofv3 -d directory of the MfmaUtil run")
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", action="append", default=[],
                    help="the profiling commands, recorded in the output")
    a = ap.parse_args(argv)
    fetch = per_launch_kib(a.fetch, "FETCH_SIZE")
    write = per_launch_kib(a.write, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no plain-copy dispatch found: run the bench with --calib-copy")
    f_scale = COPY_BYTES / (fetch["copy"]["kib"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"]["kib"] * 1024.0)
    kernels = {}
    for fam in sorted(set(fetch) & set(write)):
        if fam == "copy":
            continue
        fb = fetch[fam]["kib"] * 1024.0 * f_scale
        wb = write[fam]["kib"] * 1024.0 * w_scale
        kernels[fam] = {"fetch_kib_raw": round(fetch[fam]["kib"], 1),
                        "write_kib_raw": round(write[fam]["kib"], 1),
                        "fetch_bytes": int(fb), "write_bytes": int(wb),
                        "hbm_bytes_per_launch": int(fb + wb),
                        "dispatches": [fetch[fam]["dispatches"], write[fam]["dispatches"]]}
    for fam, m in mfma_summary(a.mfma, a.util).items():
        if fam in kernels:
            kernels[fam]["mfma"] = m
    wl = {"calibration": {"copy_bytes": COPY_BYTES,
                          "fetch_kib_raw": round(fetch["copy"]["kib"], 1),
                          "write_kib_raw": round(write["copy"]["kib"], 1),
                          "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
          "kernels": kernels, "commands": a.command}
    digest = source_digest()
    rec = {"source_sha256": digest, "workloads": {}}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            old = json.load(fh)
        if old.get("source_sha256") == digest:
            rec["workloads"] = old.get("workloads", {})
    rec["workloads"][a.workload] = wl
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(wl, indent=1))


if __name__ == "__main__":
    main()
