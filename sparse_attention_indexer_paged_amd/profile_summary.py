"""Summarise rocprofv3 output into the short text files kept under profiles/.

  kernel stats:   python -m sparse_attention_indexer_paged_amd.profile_summary stats \\
                      --csv <..._kernel_stats.csv> --command "<rocprofv3 command>" --out <txt>
  HBM traffic:    python -m sparse_attention_indexer_paged_amd.profile_summary traffic \\
                      --fetch <fetch ..._counter_collection.csv> --write <write ..._counter_collection.csv> \\
                      --kernel paged_logits_kernel --copy-bytes 268435456 \\
                      [--sources logits.hip,score_mfma.h,sai_device.h,indexer_internal.h] \\
                      --command "<both rocprofv3 commands>" --out <txt>
  counters:       python -m sparse_attention_indexer_paged_amd.profile_summary counters \\
                      --csv <..._counter_collection.csv> --kernel prefill_logits_kernel \\
                      --command "<rocprofv3 command>" --out <txt>

FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  They are scaled by what the
same counters read for a plain device-to-device copy of --copy-bytes bytes
(the copy kernel reads and writes exactly that many bytes), and the traffic
line also records the hash of the logits kernel source it was taken on.
"""
import argparse
import csv
import hashlib
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))


def source_hash(files=("logits.hip", "sai_device.h")):
    """Hash of the kernel sources a counter summary was taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def logits_source_hash():
    return source_hash(("logits.hip", "sai_device.h"))


def _per_dispatch(path, counter):
    """kernel name -> list of per-dispatch counter values (summed over the
    counter's instances within a dispatch)."""
    disp = {}
    for row in csv.DictReader(open(path)):
        if row.get("Counter_Name") != counter:
            continue
        key = (row["Dispatch_Id"], row["Kernel_Name"])
        disp[key] = disp.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (_, name), v in disp.items():
        out.setdefault(name, []).append(v)
    return out


def _pick(d, needle):
    names = [n for n in d if needle in n]
    if not names:
        raise SystemExit(f"no kernel matching {needle!r}; have {sorted(d)[:8]}")
    return names[0], d[names[0]]


def traffic(args):
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE")
    write = _per_dispatch(args.write, "WRITE_SIZE")
    _, copy_f = _pick(fetch, args.copy_kernel)
    _, copy_w = _pick(write, args.copy_kernel)
    kib = args.copy_bytes / 1024.0
    f_fetch = kib / max(copy_f)
    f_write = kib / max(copy_w)
    name, kf = _pick(fetch, args.kernel)
    _, kw = _pick(write, args.kernel)
    fk = statistics.mean(kf) * f_fetch
    wk = statistics.mean(kw) * f_write
    lines = [
        f"# HBM traffic of {name} per dispatch (rocprofv3 PMC, KiB per dispatch, scaled)",
        f"commands: {args.command}",
        f"copy calibration: {args.copy_kernel} of {args.copy_bytes} bytes read "
        f"FETCH_SIZE {max(copy_f):.1f} KiB, WRITE_SIZE {max(copy_w):.1f} KiB -> factors "
        f"{f_fetch:.4f} / {f_write:.4f}",
        f"dispatches: {len(kf)} (fetch run), {len(kw)} (write run)",
        f"fetch_kib_per_dispatch_raw: {statistics.mean(kf):.1f}",
        f"write_kib_per_dispatch_raw: {statistics.mean(kw):.1f}",
        f"fetch_bytes_per_launch: {fk * 1024:.0f}",
        f"write_bytes_per_launch: {wk * 1024:.0f}",
        f"traffic_bytes_per_launch: {(fk + wk) * 1024:.0f}",
        f"kernel_source_hash: {source_hash(tuple(args.sources.split(',')))}",
    ]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(args):
    """Per-dispatch means of every counter collected for one kernel, with
    derived ratios when their counters are present: non-MFMA VALU
    instructions per MFMA (SQ_INSTS_VALU counts MFMAs too), the clock
    (GRBM_GUI_ACTIVE summed over the XCDs, over the dispatch duration), and
    the share of the SIMDs' cycles the MFMA pipe was busy."""
    disp = {}
    dur = {}
    name = None
    for row in csv.DictReader(open(args.csv)):
        if args.kernel not in row["Kernel_Name"]:
            continue
        name = row["Kernel_Name"]
        key = row["Dispatch_Id"]
        d = disp.setdefault(key, {})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        if row.get("Start_Timestamp") and row.get("End_Timestamp"):
            dur[key] = (float(row["End_Timestamp"]) - float(row["Start_Timestamp"])) * 1e-9
    if not disp:
        raise SystemExit(f"no dispatch of {args.kernel!r}")
    names = sorted({c for d in disp.values() for c in d})
    mean = {c: statistics.mean(d[c] for d in disp.values() if c in d) for c in names}
    lines = [f"# rocprofv3 counters of {name} (mean per dispatch over {len(disp)} dispatches)",
             f"command: {args.command}"]
    lines += [f"{c}: {mean[c]:.0f}" for c in names]
    if dur:
        lines.append(f"dispatch_duration_us (under the counter run): {statistics.mean(dur.values()) * 1e6:.1f}")
    if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean and mean["SQ_INSTS_MFMA"] > 0:
        lines.append(f"non_mfma_valu_per_mfma: {(mean['SQ_INSTS_VALU'] - mean['SQ_INSTS_MFMA']) / mean['SQ_INSTS_MFMA']:.2f}")
    if "GRBM_GUI_ACTIVE" in mean:
        cyc = mean["GRBM_GUI_ACTIVE"] / args.xcds
        lines.append(f"gpu_cycles_per_xcd: {cyc:.0f}")
        if dur:
            lines.append(f"clock_ghz: {cyc / statistics.mean(dur.values()) / 1e9:.2f}")
        simds = args.cus * 4
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            lines.append(f"mfma_busy_share: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / cyc:.3f}")
        if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean:
            valu = mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]
            lines.append(f"valu_issue_share (4 cycles per wave64 instruction): {valu * 4 / simds / cyc:.3f}")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# rocprofv3 kernel statistics", f"command: {args.command}",
             "name | calls | average_us | min_us | max_us | percent"]
    for r in rows:
        name = r["Name"] if len(r["Name"]) <= 200 else r["Name"][:200] + " ..."
        lines.append(f"{name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                     f"{float(r['Percentage']):.2f}")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", default="paged_logits_kernel")
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--copy-bytes", type=int, default=256 << 20)
    t.add_argument("--sources", default="logits.hip,score_mfma.h,sai_device.h,indexer_internal.h",
                   help="kernel sources (csrc/) whose hash the summary records")
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    args = ap.parse_args()
    {"traffic": traffic, "stats": stats, "counters": counters}[args.cmd](args)


if __name__ == "__main__":
    main()
