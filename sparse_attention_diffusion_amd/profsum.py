"""Summarise rocprofv3 CSV output for this library's kernels.

Two kinds of input, both written by rocprofv3 with ``--output-format csv``:

* a kernel trace (``--kernel-trace --stats``): per-kernel call counts and
  average durations;
* counter runs (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``) over a run of
  ``bench.py --traffic-probe``, which first copies 512 MiB with a plain copy
  kernel.  The counters read for that copy against its known size give the
  scale factors that turn the sparse kernel's counters into HBM bytes.

Usage:
  python -m sparse_attention_diffusion_amd.profsum --trace DIR [--fetch DIR --write DIR]
         --config cogvideox2b --command "..." --out profiles/
"""
import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "attn_bf16.hip")
COPY_BYTES = 512 << 20

SHORT = [("sparse_occ_kernel<64, false, false>", "sparse reshape R1 (d_pad 64)"),
         ("sparse_occ_kernel<64, true, false>", "sparse reshape R1, bf16 residual (d_pad 64)"),
         ("sparse_occ_kernel<64, false, true>", "sparse reshape R2 (d_pad 64)"),
         ("sparse_occ_kernel<64, true, true>", "sparse reshape R2, bf16 residual (d_pad 64)"),
         ("sparse_occ_kernel<80, false, false>", "sparse reshape R1 (d_pad 80)"),
         ("sparse_occ_kernel<80, true, false>", "sparse reshape R1, bf16 residual (d_pad 80)"),
         ("sparse_occ_kernel<80, false, true>", "sparse reshape R2 (d_pad 80)"),
         ("sparse_occ_kernel<80, true, true>", "sparse reshape R2, bf16 residual (d_pad 80)"),
         ("calib_kernel<64, 2, 2, true>", "calibration, bf16 residual (d_pad 64)"),
         ("calib_kernel<80, 2, 2, true>", "calibration, bf16 residual (d_pad 80)"),
         ("calib_kernel<64", "calibration (d_pad 64)"), ("calib_kernel<80", "calibration (d_pad 80)"),
         ("attn_f32_kernel", "float32 attention"),
         ("select_kernel", "selector: query pooling, scores, top-k"), ("pool_k_kernel", "selector: key pooling"),
         ("permute_kernel", "row reorder")]


def short_name(name):
    for key, label in SHORT:
        if key in name:
            return label
    return None


def source_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def trace_stats(d):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = []
    for r in rows:
        label = short_name(r["Name"])
        if label:
            out.append(dict(kernel=label, name=r["Name"][:120], calls=int(r["Calls"]),
                            avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                            max_us=float(r["MaxNs"]) / 1e3, total_ms=float(r["TotalDurationNs"]) / 1e6))
    return out


def counters(d, counter):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    copy = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        label = short_name(r["Kernel_Name"])
        if label:
            per.setdefault(label, []).append(float(r["Counter_Value"]))
    if not copy:
        raise RuntimeError("no copy probe dispatch in " + d)
    scale = COPY_BYTES / (max(copy) * 1024.0)  # counters are in KiB
    return scale, {k: sum(v) / len(v) * 1024.0 * scale for k, v in per.items()}, max(copy)


XCDS, CUS, SIMDS = 8, 256, 1024

# counter passes of the unit-utilisation summary (each fits one rocprofv3 --pmc run)
UNIT_PASSES = [
    "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES",
    "GRBM_GUI_ACTIVE TA_TA_BUSY_sum TD_TD_BUSY_sum TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum "
    "TCP_PENDING_STALL_CYCLES_sum",
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS",
    "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM SQ_INSTS_SMEM SQ_WAVES",
]


def unit_counters(dirs):
    """Mean per dispatch of every counter, per labelled kernel, with the GRBM
    cycle count of the same pass (counters of one pass are ratios of it)."""
    per = {}
    for d in dirs:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        acc = {}
        for r in rows:
            label = short_name(r["Kernel_Name"])
            if label:
                acc.setdefault(label, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for label, cs in acc.items():
            if "GRBM_GUI_ACTIVE" not in cs:
                raise RuntimeError(f"{d}: every pass needs GRBM_GUI_ACTIVE")
            grbm = sum(cs["GRBM_GUI_ACTIVE"]) / len(cs["GRBM_GUI_ACTIVE"])
            for name, v in cs.items():
                if name != "GRBM_GUI_ACTIVE":
                    per.setdefault(label, {})[name] = (sum(v) / len(v), grbm)
    return per


def unit_table(per):
    """Utilisation per kernel.  GRBM_GUI_ACTIVE is summed over the XCDs, so one
    XCD's cycles are GRBM / 8; SQ wave counters count 4-cycle units."""
    lines = ["| kernel | MFMA busy | VALU active | MFMA+VALU co-issue | TA busy | TD busy | L1 pending-stall | "
             "L1→L2 reads | mean latency (cycles) | reads in flight per CU |", "|---|---|---|---|---|---|---|---|---|---|"]
    for label in sorted(per):
        c = per[label]

        def frac(name, units, scale=1.0):
            if name not in c:
                return None
            v, grbm = c[name]
            return v * scale / (grbm / XCDS * units)
        req = c.get("TCP_TCC_READ_REQ_sum")
        lat = c.get("TCP_TCC_READ_REQ_LATENCY_sum")
        cells = [frac("SQ_VALU_MFMA_BUSY_CYCLES", SIMDS), frac("SQ_ACTIVE_INST_VALU", SIMDS, 4.0),
                 frac("SQ_VALU_MFMA_COEXEC_CYCLES", SIMDS), frac("TA_TA_BUSY_sum", CUS), frac("TD_TD_BUSY_sum", CUS),
                 frac("TCP_PENDING_STALL_CYCLES_sum", CUS)]
        txt = ["–" if x is None else f"{100 * x:.0f}%" for x in cells]
        txt.append("–" if req is None else f"{req[0] / 1e6:.1f} M")
        txt.append("–" if not (req and lat) else f"{lat[0] / req[0]:.0f}")
        txt.append("–" if lat is None else f"{lat[0] / (lat[1] / XCDS * CUS):.0f}")
        lines.append(f"| {label} | " + " | ".join(txt) + " |")
    # wave states (fractions of the waves' lifetime) and instructions per MFMA
    if not any("SQ_WAVE_CYCLES" in c or "SQ_INSTS_MFMA" in c for c in per.values()):
        return lines
    lines += ["", "| kernel | waiting on a counter (s_waitcnt) | ready, not issued | issuing | "
              "VALU per MFMA | LDS per MFMA | SALU per MFMA | VMEM per MFMA |", "|---|---|---|---|---|---|---|---|"]
    for label in sorted(per):
        c = per[label]
        wc = c.get("SQ_WAVE_CYCLES")
        mf = c.get("SQ_INSTS_MFMA")
        if wc is None and mf is None:
            continue
        st = [None if (wc is None or n not in c) else c[n][0] / wc[0]
              for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY")]
        mix = [None if (mf is None or not mf[0] or n not in c) else c[n][0] / mf[0]
               for n in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM")]
        txt = ["–" if x is None else f"{100 * x:.0f}%" for x in st] + ["–" if x is None else f"{x:.1f}" for x in mix]
        lines.append(f"| {label} | " + " | ".join(txt) + " |")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace")
    ap.add_argument("--units", nargs="+", help="counter directories of the UNIT_PASSES runs")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--config", default="cogvideox2b")
    ap.add_argument("--command", required=True, help="the command line that produced the trace")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)
    if args.units:
        lines = [f"# Unit utilisation per kernel (rocprofv3 --pmc): {args.config}", "", "Commands (one run per pass):",
                 ""] + ["    " + args.command.replace("COUNTERS", p) for p in UNIT_PASSES] + [
                 "", "Fractions are of the kernel's own active cycles (GRBM_GUI_ACTIVE per XCD) over all 1024 "
                 "SIMDs or 256 CUs.", ""] + unit_table(unit_counters(args.units)) + [
                 "", f"Kernel source sha256[:16] of attn_bf16.hip: {source_hash()}"]
        open(os.path.join(args.out, f"units_{args.config}.md"), "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if not args.trace:
        ap.error("--trace is required")
    stats = trace_stats(args.trace)
    lines = [f"# rocprofv3 kernel trace: {args.config}", "", "Command:", "", "    " + args.command, "",
             "| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for s in sorted(stats, key=lambda x: -x["total_ms"]):
        lines.append(f"| {s['kernel']} | {s['calls']} | {s['avg_us']:.2f} | {s['min_us']:.2f} | {s['max_us']:.2f} "
                     f"| {s['total_ms']:.3f} |")
    lines += ["", f"Kernel source sha256[:16] of attn_bf16.hip: {source_hash()}"]
    if args.fetch and args.write:
        fs, fetch, fraw = counters(args.fetch, "FETCH_SIZE")
        ws, write, wraw = counters(args.write, "WRITE_SIZE")
        lines += ["", "## HBM traffic per launch (rocprofv3 --pmc, scaled by a 512 MiB copy probe)", "",
                  "Command (one run per counter):", "", "    " + args.pmc_command, "",
                  f"Copy probe: FETCH_SIZE read {fraw:.0f} KiB and WRITE_SIZE {wraw:.0f} KiB for {COPY_BYTES >> 10} KiB "
                  f"moved; scale factors {fs:.3f} (fetch) and {ws:.3f} (write).", "",
                  "| kernel | fetch MB | write MB | total MB |", "|---|---|---|---|"]
        for k in sorted(set(fetch) | set(write)):
            f, w = fetch.get(k, 0.0), write.get(k, 0.0)
            lines.append(f"| {k} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} |")
        label = "sparse reshape R1 (d_pad 64)"
        if label in fetch and label in write:
            rec = dict(config=args.config, kernel=label, kernel_source_sha256_16=source_hash(),
                       fetch_bytes=fetch[label], write_bytes=write[label],
                       bytes_per_launch=fetch[label] + write[label], fetch_scale=fs, write_scale=ws,
                       command=args.pmc_command)
            json.dump(rec, open(os.path.join(args.out, f"sparse_attn_reshape_{args.config}_traffic.json"), "w"),
                      indent=1)
    open(os.path.join(args.out, f"kernels_{args.config}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
