"""HBM traffic measurement support for the attention kernel.

    python -m online_softmax_03_amd.profiling copy [--mib 1024] [--reps 5]
        a plain device-to-device copy of a known size, run under
        `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` to calibrate the
        counters (bytes the copy must read and write per dispatch are known).

    python -m online_softmax_03_amd.profiling report --workload NAME \\
        --stats DIR --bench FILE [--traffic FILE] --command CMD \\
        [--pmc DIR --pmc-command CMD] --out FILE
        writes the markdown summary of a `rocprofv3 --kernel-trace --stats`
        run of bench.py: the attention kernel's launch statistics next to the
        bench line measured in the same process; with --pmc, also the SQ/GRBM
        counters of a separate `rocprofv3 --pmc` run (MFMA busy fraction,
        effective clock, VALU and LDS instructions per MFMA, bank conflicts).

    python -m online_softmax_03_amd.profiling tiles \\
        --run LABEL BENCH_JSON PMC_DIR FETCH_DIR WRITE_DIR ... \\
        --copy-fetch DIR --copy-write DIR --command CMD ... --out FILE
        writes the tile-choice table: for each run, the bench line's achieved
        TFLOP/s next to rocprofv3 SQ/GRBM counters of the same configuration
        (MFMA busy fraction, effective clock, VALU and LDS instructions per
        MFMA, LDS bank conflicts, HBM bytes and GB/s, registers, scratch).

    python -m online_softmax_03_amd.profiling summarize --workload NAME \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR [--out FILE]
        reads the rocprofv3 counter CSVs, scales the attention kernel's
        per-dispatch FETCH_SIZE and WRITE_SIZE by the copy kernel's
        measured/known ratio, and writes a JSON summary stamped with a hash of
        the kernel sources (bench.py reports the traffic only while the hash
        still matches).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")


# The sources that make up each profiled kernel: its device code, its
# instantiations and the host code that launches it.
KERNEL_SOURCES = {
    "attn_fwd_kernel": ["attn_common.h", "work_item.h", "attn_fwd_kernel.h", "attn_fwd_f32_kernel.h", "attn_merge.h",
                        "fa_table.h", "kern_d128_bf16.hip", "kern_d128_f16.hip", "kern_d64_bf16.hip",
                        "kern_d64_f16.hip", "kern_f32.hip", "kern_merge.hip", "fa_api.hip", "splitkv_launch.h",
                        "noalloc_api.hip"],
    "softmax": ["attn_common.h", "work_item.h", "softmax_kernel.h", "softmax_table.h", "kern_softmax.hip", "softmax_api.hip"],
    "attn_fwd_fp8": ["attn_common.h", "work_item.h", "attn_fwd_fp8_kernel.h", "fp8_table.h", "kern_fp8.hip", "fp8_api.hip"],
    "attn_bwd": ["attn_common.h", "work_item.h", "attn_bwd_kernel.h", "bwd_table.h", "kern_bwd_bf16.hip", "kern_bwd_f16.hip",
                 "bwd_api.hip"],
}


# Sources that no kernel's timing or traffic depends on (error texts).
HOST_ONLY_SOURCES = ["status.hip"]


def source_hash(kernel: str = "attn_fwd_kernel") -> str:
    """sha256 over the sources of one kernel (its identity for profiles)."""
    h = hashlib.sha256()
    files = [os.path.join(PKG, "csrc", f) for f in KERNEL_SOURCES[kernel]]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str, kernel: str = "attn_fwd_kernel") -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")


def current_traffic(workload: str, kernel: str = "attn_fwd_kernel", tile=None):
    """The measured traffic summary for `workload` if it was taken on the
    current kernel sources and on the same tile shape (`tile` = (B_r, B_c),
    or None where the kernel has one shape), else None."""
    path = traffic_file(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(_family(kernel)):
        return None
    if tile is not None and tuple(t.get("tile") or ()) != tuple(tile):
        return None
    return t


def _family(kernel: str) -> str:
    if kernel.startswith("softmax"):
        return "softmax"
    if kernel.startswith("attn_bwd"):
        return "attn_bwd"
    if kernel.startswith("attn_fwd_fp8"):
        return "attn_fwd_fp8"
    return "attn_fwd_kernel"


def _copy(mib: int, reps: int) -> None:
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def _counter_rows(d: str, counter: str, name_filter: str):
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                if name_filter not in row.get("Kernel_Name", ""):
                    continue
                vals.append(float(row["Counter_Value"]))
    return vals


def _summarize(a) -> None:
    fetch = _counter_rows(a.fetch, "FETCH_SIZE", a.kernel)
    write = _counter_rows(a.write, "WRITE_SIZE", a.kernel)
    cfetch = _counter_rows(a.copy_fetch, "FETCH_SIZE", a.copy_filter)
    cwrite = _counter_rows(a.copy_write, "WRITE_SIZE", a.copy_filter)
    if not (fetch and write and cfetch and cwrite):
        sys.exit("missing counter rows")
    known = a.copy_mib * 1024.0  # KiB read and written per copy dispatch
    # the copy dispatch that moves the full buffer is the largest one
    f_factor = known / max(cfetch)
    w_factor = known / max(cwrite)
    fetch_kib = sum(fetch) / len(fetch)
    write_kib = sum(write) / len(write)
    out = {
        "workload": a.workload,
        "kernel": a.kernel,
        "tile": [int(t) for t in a.tile.split(",")] if a.tile else None,
        "source_hash": source_hash(_family(a.kernel)),
        "dispatches": {"fetch": len(fetch), "write": len(write)},
        "fetch_kib_per_dispatch_raw": fetch_kib,
        "write_kib_per_dispatch_raw": write_kib,
        "copy_calibration": {"known_kib": known, "fetch_kib_raw": max(cfetch), "write_kib_raw": max(cwrite),
                             "fetch_factor": f_factor, "write_factor": w_factor},
        "hbm_bytes_per_launch": (fetch_kib * f_factor + write_kib * w_factor) * 1024.0,
        "hbm_read_bytes_per_launch": fetch_kib * f_factor * 1024.0,
        "hbm_write_bytes_per_launch": write_kib * w_factor * 1024.0,
        "commands": a.commands,
    }
    path = a.out or traffic_file(a.workload, a.kernel)
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out, indent=2))


def _report(a) -> None:
    stats = []
    for f in glob.glob(os.path.join(a.stats, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            stats.extend(csv.DictReader(fh))
    with open(a.bench) as fh:
        bench = json.loads([l for l in fh if l.startswith("{")][-1])
    lines = [f"# {a.kernel} on {a.workload} (MI355X)", "",
             "Produced by (from the repository root, on one MI355X):", "", "```"]
    lines += a.command
    lines += ["```", "", "## rocprofv3 kernel statistics", "",
              "| kernel | calls | average (ms) | min (ms) | max (ms) | share |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.1f}% |")
    rf = bench["roofline"]
    lines += ["", "## bench.py line of the same run", "", "```json", json.dumps(bench, indent=1), "```", "",
              f"bench.py's own HIP-event average over the timed launches: {rf['avg_launch_ms']:.4f} ms; "
              f"achieved {rf['achieved']} {rf['unit']} = {100 * rf['frac']:.1f}% of {rf['peak']} {rf['unit']}."]
    if a.traffic and os.path.exists(a.traffic):
        with open(a.traffic) as fh:
            t = json.load(fh)
        lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)", "",
                  f"- read {t['hbm_read_bytes_per_launch'] / 2**20:.1f} MiB, write "
                  f"{t['hbm_write_bytes_per_launch'] / 2**20:.1f} MiB per launch "
                  f"(raw KiB x copy-kernel factor: fetch {t['copy_calibration']['fetch_factor']:.3f}, "
                  f"write {t['copy_calibration']['write_factor']:.3f})",
                  f"- source hash of the kernel sources: `{t['source_hash']}`"]
    if a.pmc:
        avg_ms = {r["Name"]: float(r["AverageNs"]) / 1e6 for r in stats}
        kc = _kernel_counters(a.pmc)
        _counters_json(a, kc, avg_ms)
        lines += ["", "## Counters (rocprofv3 --pmc, one run)", "", "```"] + (a.pmc_command or []) + [
            "```", "",
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); clock = "
            "GRBM_GUI_ACTIVE / 8 / the kernel-trace average above.", "",
            "| kernel | MFMA busy | clock (GHz) | VALU / MFMA | LDS / MFMA | LDS bank conflicts |",
            "|---|---|---|---|---|---|"]
        for name in sorted(kc, key=lambda n: -kc[n].get("SQ_INSTS_MFMA", 0.0)):
            c = kc[name]
            if not c.get("SQ_INSTS_MFMA") or name not in avg_ms:
                continue
            xcd_cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
            lines.append(f"| `{name[:80]}` | {100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (xcd_cycles * N_SIMD):.1f}% | "
                         f"{xcd_cycles / (avg_ms[name] * 1e-3) / 1e9:.2f} | "
                         f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f} | "
                         f"{c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:.2f} | {c['SQ_LDS_BANK_CONFLICT']:.0f} |")
    if a.l2:
        l2 = _kernel_counters(a.l2)
        lines += ["", "## L2 (rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum, one run)", "", "```"] + (a.l2_command or []) + [
            "```", "", "| kernel | L2 hit | TCC_MISS x 128 B per launch (MiB) |", "|---|---|---|"]
        for name in sorted(l2, key=lambda n: -l2[n].get("TCC_MISS_sum", 0.0)):
            c = l2[name]
            if "TCC_HIT_sum" not in c or a.kernel not in name:
                continue
            hit = c["TCC_HIT_sum"] / max(1.0, c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
            lines.append(f"| `{name[:80]}` | {100 * hit:.1f}% | {c['TCC_MISS_sum'] * L2_LINE / 2**20:.1f} |")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters_file(workload: str, kernel: str = "attn_fwd_kernel") -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_counters.json")


def _counters_json(a, kc, avg_ms) -> None:
    """Writes the counter summary of the profiled kernel (the one with the
    most MFMA instructions): effective clock, MFMA busy fraction, instruction
    mix, and with --l2 the L2 hit rate; stamped with the source hash and tile
    so bench.py quotes it only for the same kernel and shape."""
    names = [n for n in kc if kc[n].get("SQ_INSTS_MFMA") and n in avg_ms]
    if not names:
        return
    name = max(names, key=lambda n: kc[n]["SQ_INSTS_MFMA"])
    c = kc[name]
    xcd_cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
    out = {
        "workload": a.workload, "kernel": a.kernel, "kernel_symbol": name,
        "tile": [int(t) for t in a.tile.split(",")] if a.tile else None,
        "source_hash": source_hash(_family(a.kernel)),
        "avg_launch_ms": avg_ms[name],
        "clock_ghz": xcd_cycles / (avg_ms[name] * 1e-3) / 1e9,
        "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * N_SIMD),
        "valu_per_mfma": c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"],
        "lds_per_mfma": c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"],
        "lds_bank_conflicts": c["SQ_LDS_BANK_CONFLICT"],
        "vgpr_count_rocprofv3": c.get("VGPR_Count"),
        "commands": (a.command or []) + (a.pmc_command or []) + (a.l2_command or []),
    }
    if a.l2:
        l2 = _kernel_counters(a.l2).get(name, {})
        if "TCC_HIT_sum" in l2:
            out["l2_hit"] = l2["TCC_HIT_sum"] / max(1.0, l2["TCC_HIT_sum"] + l2["TCC_MISS_sum"])
            out["tcc_miss_bytes_per_launch"] = l2["TCC_MISS_sum"] * L2_LINE
    with open(counters_file(a.workload, a.kernel), "w") as f:
        json.dump(out, f, indent=2)


def current_counters(workload: str, kernel: str = "attn_fwd_kernel", tile=None):
    """The committed counter summary for `workload` if it was taken on the
    current kernel sources and the same tile shape, else None."""
    path = counters_file(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(_family(kernel)):
        return None
    if tile is not None and tuple(t.get("tile") or ()) != tuple(tile):
        return None
    return t


# L2 (TCC) line size on MI355X, bytes
L2_LINE = 128

# MI355X: 8 XCDs (GRBM counters are summed over them), 256 CUs x 4 SIMDs.
N_XCD = 8
N_SIMD = 1024
TILE_COUNTERS = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                 "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"]


def _kernel_counters(d: str):
    """{kernel name: {counter: mean over dispatches, plus registers and
    scratch}} from a rocprofv3 counter-collection directory."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = per.setdefault(row["Kernel_Name"], {"_res": {}})
                k.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                k["_res"] = {"VGPR_Count": row.get("VGPR_Count"), "Accum_VGPR_Count": row.get("Accum_VGPR_Count"),
                             "SGPR_Count": row.get("SGPR_Count"), "Scratch_Size": row.get("Scratch_Size"),
                             "LDS_Block_Size": row.get("LDS_Block_Size")}
    out = {}
    for name, k in per.items():
        res = k.pop("_res")
        out[name] = {c: sum(v) / len(v) for c, v in k.items()}
        out[name].update(res)
    return out


def _tiles(a) -> None:
    cfetch = _counter_rows(a.copy_fetch, "FETCH_SIZE", "")
    cwrite = _counter_rows(a.copy_write, "WRITE_SIZE", "")
    known = a.copy_mib * 1024.0
    f_factor, w_factor = known / max(cfetch), known / max(cwrite)
    lines = ["# Tile choice: counters per configuration (MI355X)", "",
             "Produced by (from the repository root, on one MI355X), per configuration:", "", "```"]
    lines += a.command
    lines += ["```", "",
              "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); clock = "
              "GRBM_GUI_ACTIVE / 8 / the unprofiled launch time; HBM = (FETCH_SIZE x "
              f"{f_factor:.3f} + WRITE_SIZE x {w_factor:.3f}) per launch (factors from a plain 1 GiB copy) "
              "/ the unprofiled launch time. TFLOP/s and % of peak from the bench line of a separate, unprofiled "
              "run of the same configuration.", "",
              "| configuration | kernel | TFLOP/s | % of peak | MFMA busy | clock (GHz) | VALU / MFMA | LDS / MFMA "
              "| LDS bank conflicts | HBM read + write (MiB) | HBM GB/s | L2 hit | VGPRs allocated | scratch |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, bench_path, pmc, fetch_dir, write_dir, l2_dir in a.run:
        with open(bench_path) as fh:
            bench = json.loads([l for l in fh if l.startswith("{")][-1])
        rf = bench["roofline"]
        kc = _kernel_counters(pmc)
        name = max(kc, key=lambda n: kc[n].get("SQ_INSTS_MFMA", 0.0))
        c = kc[name]
        t = rf["avg_launch_ms"] * 1e-3
        xcd_cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * N_SIMD)
        clock = xcd_cycles / t / 1e9
        fk = _counter_rows(fetch_dir, "FETCH_SIZE", name)
        wk = _counter_rows(write_dir, "WRITE_SIZE", name)
        rd = sum(fk) / len(fk) * f_factor * 1024.0
        wr = sum(wk) / len(wk) * w_factor * 1024.0
        l2 = _kernel_counters(l2_dir).get(name, {})
        hit = (f"{100 * l2['TCC_HIT_sum'] / max(1.0, l2['TCC_HIT_sum'] + l2['TCC_MISS_sum']):.1f}%"
               if "TCC_HIT_sum" in l2 else "n/a")
        vg = int(float(c["VGPR_Count"])) * 2 if c.get("VGPR_Count") not in (None, "") else "n/a"
        lines.append(
            f"| {label} | `{name[:90]}` | {rf['achieved']:.1f} | {100 * rf['frac']:.1f}% | {100 * busy:.1f}% | "
            f"{clock:.2f} | {c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f} | "
            f"{c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:.2f} | {c['SQ_LDS_BANK_CONFLICT']:.0f} | "
            f"{rd / 2**20:.0f} + {wr / 2**20:.0f} | {(rd + wr) / t / 1e9:.0f} | {hit} | {vg} | "
            f"{c['Scratch_Size']} |")
    lines += ["", "The clock column divides the counted cycles by the unprofiled launch time, so it is an estimate "
              "of the clock the kernel ran at. VGPRs allocated = rocprofv3's VGPR_Count x 2: rocprofv3 "
              "multiplies the kernel descriptor's register granules by 4, but gfx950's unified register file "
              "allocates 8 registers per granule (e.g. the 128 x 32 tile at d = 128: 152 registers in 19 "
              "granules, which rocprofv3 prints as 76). Where LDS already limits the workgroups per CU, the "
              "compiler allocates more registers than the kernel uses. SQ_INSTS_VALU counts the MFMA "
              "instructions too, so VALU / MFMA includes 1 for the MFMA itself."]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--kernel", default="attn_fwd_kernel")
    s.add_argument("--tile", default=None, help="B_r,B_c of the profiled launch")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--copy-filter", default="")
    s.add_argument("--commands", nargs="*", default=[])
    s.add_argument("--out", default=None)
    r = sub.add_parser("report")
    r.add_argument("--workload", required=True)
    r.add_argument("--kernel", default="attn_fwd_kernel")
    r.add_argument("--stats", required=True)
    r.add_argument("--bench", required=True)
    r.add_argument("--traffic", default=None)
    r.add_argument("--command", nargs="*", default=[])
    r.add_argument("--pmc", default=None)
    r.add_argument("--pmc-command", nargs="*", default=[])
    r.add_argument("--l2", default=None, help="rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum output directory")
    r.add_argument("--l2-command", nargs="*", default=[])
    r.add_argument("--tile", default=None, help="B_r,B_c of the profiled launch")
    r.add_argument("--out", required=True)
    t = sub.add_parser("tiles")
    t.add_argument("--run", nargs=6, action="append",
                   metavar=("LABEL", "BENCH_JSON", "PMC_DIR", "FETCH_DIR", "WRITE_DIR", "L2_DIR"), required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--command", nargs="*", default=[])
    t.add_argument("--out", required=True)
    hs = sub.add_parser("hash")
    hs.add_argument("--kernel", default="attn_fwd_kernel")
    a = ap.parse_args()
    if a.cmd == "copy":
        _copy(a.mib, a.reps)
    elif a.cmd == "summarize":
        _summarize(a)
    elif a.cmd == "report":
        _report(a)
    elif a.cmd == "tiles":
        _tiles(a)
    else:
        print(source_hash(_family(a.kernel)))


if __name__ == "__main__":
    main()
