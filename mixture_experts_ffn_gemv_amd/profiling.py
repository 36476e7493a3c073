"""Turn rocprofv3 CSV output into the short text summaries kept with the
sources, and into the per-kernel HBM traffic record bench.py reports.

Traffic comes from two counter passes over the same command: FETCH_SIZE in
one, WRITE_SIZE in the other (KiB per dispatch).  Each pass first runs one
plain device copy of known size (bench.py --calib-copy-mb), and the ratio of
its known bytes to what the counter reports scales the kernels' readings.

Usage:
  python -m mixture_experts_ffn_gemv_amd.profiling traffic \
      --fetch DIR --write DIR --workload NAME --copy-mib 1024 \
      --kernel gemv_gateup=k_dec_gateup3 --kernel gemv_down_combine=k_dec_down3 \
      --out profiles/traffic.json
  python -m mixture_experts_ffn_gemv_amd.profiling stats --csv FILE
  python -m mixture_experts_ffn_gemv_amd.profiling counters --dir DIR
  python -m mixture_experts_ffn_gemv_amd.profiling parity --log FILE

parity: the GPU parity tests append one JSON line per compared case to the
file MOE_PARITY_LOG names; this prints them as a table (largest error
relative to its tolerance first).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(os.path.dirname(PKG), "profiles", "traffic.json")


# Source files each timed kernel is built from (device code and its launch).
KERNEL_SOURCES = {
    "gemv_gateup": ["common.h", "gemv.h", "route.h", "decode.h", "decode_u4.h", "moe_ffn.hip"],
    "gemv_down_combine": ["common.h", "gemv.h", "route.h", "decode.h", "moe_ffn.hip"],
    "gemv_down": ["common.h", "gemv.h", "route.h", "decode.h", "decode_u4.h", "moe_ffn.hip"],
    "router_route": ["common.h", "route.h", "decode.h", "moe_ffn.hip"],
    "router_gemv": ["common.h", "route.h", "moe_ffn.hip"],
    "gemm_gateup": ["common.h", "gemm.h", "gemm_big.h", "gemm_dma.h", "moe_ffn.hip"],
    "gemm_down": ["common.h", "gemm.h", "gemm_big.h", "gemm_dma.h", "moe_ffn.hip"],
    "wsum_backward": ["common.h", "backward.h", "moe_ffn.hip"],
    "glu_backward": ["common.h", "backward.h", "moe_ffn.hip"],
}


def kernel_source_sha(kernel: str = None) -> str:
    """sha256 over the named kernel's source files (every kernel source file
    when `kernel` is None), names and bytes, sorted."""
    if kernel is None:
        files = sorted(glob.glob(os.path.join(PKG, "csrc", "*")))
    else:
        files = sorted(os.path.join(PKG, "csrc", f) for f in KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes (read + write) per launch of `kernel` on `workload`, from the
    committed counter record, or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(workload, {}).get(kernel)
    if not k or kernel not in KERNEL_SOURCES or k.get("source_sha256") != kernel_source_sha(kernel):
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def _counter_csv(d: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {hits}")
    return hits[0]


def _per_kernel(path: str) -> dict:
    """kernel name -> list of counter values (one per dispatch)."""
    out: dict = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _find(agg: dict, key: str) -> list:
    vals = [v for name, vs in agg.items() if key in name for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {key!r}")
    return vals


def cmd_traffic(a) -> None:
    f = _per_kernel(_counter_csv(a.fetch))
    w = _per_kernel(_counter_csv(a.write))
    known_kib = a.copy_mib * 1024.0
    fetch_factor = known_kib / max(_find(f, "copyBuffer"))
    write_factor = known_kib / max(_find(w, "copyBuffer"))
    try:
        with open(a.out) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec.setdefault("kernels", {})
    cal = rec.setdefault("calibration", {})
    cal[a.workload] = {"copy_mib": a.copy_mib, "fetch_factor": fetch_factor,
                       "write_factor": write_factor}
    ks = rec["kernels"].setdefault(a.workload, {})
    for spec in a.kernel:
        label, key = spec.split("=", 1)
        fv, wv = _find(f, key), _find(w, key)
        ks[label] = {"symbol": key,
                     "source_sha256": kernel_source_sha(label) if label in KERNEL_SOURCES else None,
                     "fetch_kib": sum(fv) / len(fv), "write_kib": sum(wv) / len(wv),
                     "fetch_bytes": sum(fv) / len(fv) * 1024.0 * fetch_factor,
                     "write_bytes": sum(wv) / len(wv) * 1024.0 * write_factor}
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({a.workload: ks, "calibration": cal[a.workload]}, indent=1))


def cmd_stats(a) -> None:
    """Markdown table of the library's kernels from a --stats kernel CSV."""
    print("| kernel | calls | avg us | min us | max us | % of traced GPU time |")
    print("|---|---|---|---|---|---|")
    with open(a.csv) as fh:
        for r in csv.DictReader(fh):
            if "moe::" not in r["Name"]:
                continue
            name = r["Name"].replace("moe::", "").split("(")[0]
            print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.2f} |")


def cmd_counters(a) -> None:
    """Markdown table of per-dispatch averages of the counters of one
    --pmc pass, for the library's kernels (and the derived rates below)."""
    per: dict = {}
    with open(_counter_csv(a.dir)) as fh:
        for r in csv.DictReader(fh):
            if "moe::" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].replace("moe::", "").split("(")[0]
            per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    names = sorted({c for v in per.values() for c in v})
    print("| kernel | dispatches | " + " | ".join(names) + " |")
    print("|---|---|" + "---|" * len(names))
    avg = {}
    for k, v in per.items():
        avg[k] = {c: sum(x) / len(x) for c, x in v.items()}
        n = len(next(iter(v.values())))
        print(f"| `{k}` | {n} | " + " | ".join(f"{avg[k].get(c, float('nan')):.4g}"
                                                 for c in names) + " |")
    # derived: MFMA busy (per SIMD, over the GPU-active cycles of all SIMDs),
    # bf16 MFMA flops (512 per MOP), LDS bank-conflict cycles per active LDS cycle
    rows = []
    for k, c in avg.items():
        d = {}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
            d["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] * a.cus * 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            d["mfma_bf16_tflop"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e12
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
            d["lds_conflict_per_active"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
        if "SQ_INSTS_VALU" in c and "GRBM_GUI_ACTIVE" in c:
            # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
            d["valu_busy"] = c["SQ_INSTS_VALU"] * 4 / (c["GRBM_GUI_ACTIVE"] * a.cus * 4)
        if d:
            rows.append((k, d))
    if rows:
        print()
        print("| kernel | " + " | ".join(sorted({x for _, d in rows for x in d})) + " |")
        keys = sorted({x for _, d in rows for x in d})
        print("|---|" + "---|" * len(keys))
        for k, d in rows:
            print(f"| `{k}` | " + " | ".join(f"{d[x]:.4g}" if x in d else "" for x in keys) + " |")


def cmd_parity(a) -> None:
    """Markdown table of the per-case errors a GPU parity run logged."""
    rows = []
    with open(a.log) as fh:
        for line in fh:
            if line.strip():
                rows.append(json.loads(line))
    rows.sort(key=lambda r: -(r["out_err"] / r["tol"]))
    worst = rows[0]["out_err"] / rows[0]["tol"] if rows else float("nan")
    print(f"{len(rows)} comparisons, {len({r['case'] for r in rows})} cases; "
          f"largest error / tolerance {worst:.3g}")
    print()
    print("| case | T | tokens compared | max rel err | tolerance | err / tol | routing weight err |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        w = r.get("w_err")
        print(f"| {r['case']} | {r['T']} | {r['tokens']} | {r['out_err']:.3g} | {r['tol']:g} | "
              f"{r['out_err'] / r['tol']:.3g} | {'' if w is None else f'{w:.2g}'} |")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True, help="label=symbol substring")
    t.add_argument("--out", default=TRAFFIC_JSON)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--dir", required=True, help="output directory of one --pmc pass")
    c.add_argument("--cus", type=int, default=256, help="compute units of the GPU")
    q = sub.add_parser("parity")
    q.add_argument("--log", required=True, help="the MOE_PARITY_LOG file of a GPU test run")
    a = ap.parse_args()
    {"traffic": cmd_traffic, "stats": cmd_stats, "counters": cmd_counters,
     "parity": cmd_parity}[a.cmd](a)


if __name__ == "__main__":
    main()
