"""Turn rocprofv3 CSV output into the short text summaries kept beside the library.

    python -m gated_delta_rule_21_amd.profile_summary stats KERNEL_STATS_CSV --command "..." > out.md
    python -m gated_delta_rule_21_amd.profile_summary counters FETCH_CSV WRITE_CSV \\
        --kernel chunk_fwd_kernel --algorithmic-bytes N --command "..." > out.md

`stats` keeps the rows of a `--kernel-trace --stats` summary (kernel_stats.csv).
`counters` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs
(counter_collection.csv, values in KiB per dispatch).  It scales each counter by
what the same counter reads for the streaming calibration kernel (torch.neg over
1 GiB of fp32: 2^30 bytes read, 2^30 written), then reports HBM bytes per
launch of the named kernel.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAL_KERNEL = "neg_kernel"          # substring of torch's elementwise negation kernel
CAL_BYTES = 1 << 30


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name.replace("void ", "")[:110]


def kernel_source_digest() -> str:
    """sha256 (first 16 hex digits) of the chunk-forward sources, as bench.py computes it."""
    h = hashlib.sha256()
    for n in ("chunk_prep.hip", "chunk_state.hip", "chunk_fwd.hip", "chunk_common.h", "device_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_source_digest() -> str:
    h = hashlib.sha256()
    for n in ("decode_step.hip", "device_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def precond_source_digest() -> str:
    h = hashlib.sha256()
    for n in ("precond_scan.hip", "chunk_common.h", "device_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bwd_source_digest() -> str:
    h = hashlib.sha256()
    for n in ("chunk_bwd.hip", "bwd_common.h", "chunk_prep.hip", "chunk_common.h", "device_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats(path: str, command: str, top: int) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# rocprofv3 kernel-trace statistics", "", "command:", "", "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def per_dispatch(path: str, counter: str):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return vals


def pick(vals, sub: str):
    return [v for (d, n), v in vals.items() if sub in n]


def counters(fetch_csv: str, write_csv: str, kernels: str, algorithmic: float, command: str,
             digest: str) -> str:
    """`kernels`: name substrings separated by ';' (template names hold commas); the
    traffic of one call of the operation is the sum over them (each kernel runs once
    per call)."""
    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w = per_dispatch(write_csv, "WRITE_SIZE")
    cf, cw = pick(f, CAL_KERNEL), pick(w, CAL_KERNEL)
    if not (cf and cw):
        raise SystemExit("missing calibration dispatches")
    sf = CAL_BYTES / (1024 * statistics.median(cf))
    sw = CAL_BYTES / (1024 * statistics.median(cw))
    out = ["# HBM traffic counters", "", f"kernels: `{kernels}`", "", "commands (one counter per run):", "",
           "```", command, "```", "",
           "| quantity | value |", "|---|---|",
           f"| calibration FETCH_SIZE (KiB, median of {len(cf)}) | {statistics.median(cf):.1f} |",
           f"| calibration WRITE_SIZE (KiB, median of {len(cw)}) | {statistics.median(cw):.1f} |",
           f"| calibration bytes read / written | {CAL_BYTES} / {CAL_BYTES} |",
           f"| read scale (bytes per counted byte) | {sf:.4f} |",
           f"| write scale (bytes per counted byte) | {sw:.4f} |"]
    tot = 0.0
    for k in kernels.split(";"):
        kf, kw = pick(f, k), pick(w, k)
        if not (kf and kw):
            raise SystemExit(f"missing dispatches of {k}")
        fb = statistics.median(kf) * 1024 * sf
        wb = statistics.median(kw) * 1024 * sw
        tot += fb + wb
        out += [f"| `{k}` FETCH_SIZE / WRITE_SIZE (KiB, median of {len(kf)}) | "
                f"{statistics.median(kf):.1f} / {statistics.median(kw):.1f} |",
                f"| `{k}` HBM bytes read / written (scaled) | {fb:.4e} / {wb:.4e} |"]
    out += [f"| HBM bytes per call (all kernels) | {tot:.4e} |",
            f"| algorithmic bytes per call | {algorithmic:.4e} |",
            f"| traffic / algorithmic | {tot / algorithmic:.3f} |",
            "", f"hbm_bytes_per_launch: {tot:.6e}", f"kernel_source_sha256_16: {digest}", ""]
    return "\n".join(out)


def sq(paths, command: str, digest: str, title: str, useful_flops: float = 0.0) -> str:
    """Per-kernel means of SQ / GRBM counter passes (counter_collection.csv, one pass
    per file; the first dispatch of each kernel dropped as warm-up when there are
    more than two), per dispatch and per wave, with the MFMA-busy fraction of the
    kernel's time: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 (cycles per XCD)
    times 1024 SIMDs."""
    rows, meta = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"]).replace("gdr::", "")
            if CAL_KERNEL in k:
                continue
            rows.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                (int(r["Dispatch_Id"]), float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            meta[k] = (int(r["Grid_Size"]), int(r["Workgroup_Size"]), r["LDS_Block_Size"])
    out = [f"# {title}", "", "commands (one counter pass per run):", "", "```", command, "```", ""]
    busy_all = cyc_all = insts_all = 0.0
    for k, cs in rows.items():
        grid, wg, lds = meta[k]
        waves = grid // 64
        out += [f"## `{k}`", "", f"grid {grid} threads ({waves} waves), workgroup {wg}, LDS {lds} B", "",
                "| counter | per dispatch | per wave |", "|---|---|---|"]
        mean = {}
        dur = []
        for c, vals in sorted(cs.items()):
            vals = sorted(vals)[1:] if len(vals) > 2 else vals
            mean[c] = statistics.mean(v for _, v, _ in vals)
            dur += [t for _, _, t in vals]
            out.append(f"| {c} | {mean[c]:.5g} | {mean[c] / waves:.5g} |")
        out.append("")
        if "GRBM_GUI_ACTIVE" in mean:
            cyc = mean["GRBM_GUI_ACTIVE"] / 8
            out.append(f"- kernel time {statistics.mean(dur) / 1e3:.1f} us (profiled), {cyc:.4g} cycles per XCD, "
                       f"{cyc / statistics.mean(dur):.3f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                f = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024)
                busy_all += mean["SQ_VALU_MFMA_BUSY_CYCLES"]
                cyc_all += cyc
                out.append(f"- MFMA busy: {f:.4f} of the kernel's SIMD cycles")
            if "SQ_INSTS_MFMA" in mean:
                insts_all += mean["SQ_INSTS_MFMA"]
        if mean.get("SQ_LDS_IDX_ACTIVE", 0) > 0 and "SQ_LDS_BANK_CONFLICT" in mean:
            out.append(f"- LDS bank conflicts: {mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_LDS_IDX_ACTIVE']:.3f} of "
                       "LDS-active cycles")
        if "SQ_WAIT_ANY" in mean and mean.get("SQ_WAVE_CYCLES", 0) > 0:
            out.append(f"- waves waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES): {mean['SQ_WAIT_ANY'] / mean['SQ_WAVE_CYCLES']:.3f}"
                       f"; on LDS issue (SQ_WAIT_INST_LDS): {mean.get('SQ_WAIT_INST_LDS', 0) / mean['SQ_WAVE_CYCLES']:.3f}")
        out.append("")
    if cyc_all:
        out.append(f"All kernels of one call: MFMA busy {busy_all / (cyc_all * 1024):.4f} of their SIMD cycles.")
    if useful_flops and insts_all:
        issued = insts_all * 16384
        out.append(f"MFMA instructions per call {insts_all:.4g} (16x16x32 bf16, 16384 flop each): {issued:.4g} flop "
                   f"issued against {useful_flops:.4g} useful ({issued / useful_flops:.3f}x: zero-padded k = 16 steps, "
                   "full 16x16 tiles of triangular blocks).")
    out += ["", f"kernel_source_sha256_16: {digest}", ""]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--command", required=True)
    a.add_argument("--top", type=int, default=8)
    b = sub.add_parser("counters")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--kernel", required=True, help="name substring, or several separated by ';'")
    b.add_argument("--algorithmic-bytes", type=float, required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--digest", default="", help="source digest to record (default: the current sources')")
    c = sub.add_parser("sq")
    c.add_argument("csv", nargs="+")
    c.add_argument("--command", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--digest", default="")
    c.add_argument("--useful-flops", type=float, default=0.0)
    args = ap.parse_args(argv)
    if args.cmd == "sq":
        sys.stdout.write(sq(args.csv, args.command, args.digest or kernel_source_digest(), args.title,
                            args.useful_flops))
        return
    if args.cmd == "stats":
        sys.stdout.write(stats(args.csv, args.command, args.top))
    else:
        digest = args.digest or (decode_source_digest() if "decode" in args.kernel else
                  precond_source_digest() if "precond" in args.kernel else
                  bwd_source_digest() if "bwd" in args.kernel else kernel_source_digest())
        sys.stdout.write(counters(args.fetch_csv, args.write_csv, args.kernel, args.algorithmic_bytes,
                                  args.command, digest))


if __name__ == "__main__":
    main()
