"""Summaries of rocprofv3 CSV output for the profiles/ directory.

  stats   <kernel_stats.csv> <out.md> --command "..." [--trace <kernel_trace.csv>]
          per-kernel (or per kernel and grid) call count / total / average /
          min / max duration
  pmc     <counter_collection.csv>... --out <md> --command "..."
          per-kernel counter averages and derived utilisation ratios
  traffic <fetch counter_collection.csv> <write counter_collection.csv>
          --workload NAME --copy-mib M --out-json profiles/traffic.json
          --out-md profiles/<...>.md --command "..."
          HBM bytes per launch of each PSA kernel from FETCH_SIZE and
          WRITE_SIZE, scaled by what the same counters read for the
          calibration pass (dst = src * 1 over M MiB of float32: M MiB read,
          M MiB written).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import sys
from collections import defaultdict

PSA_SLOTS = (("psa_fwd_kernel", "fwd"), ("psa_bwd_pre_kernel", "bwd_pre"),
             ("psa_bwd_fused_kernel", "bwd_main"), ("psa_conv_dx_kernel", "conv_dx"),
             ("psa_conv_dx_pipe_kernel", "conv_dx_pipe"), ("psa_pad_rows_kernel", "pad_rows"),
             ("psa_conv_dw_reduce_kernel", "conv_dw_reduce"), ("psa_conv_dw_kernel", "conv_dw"),
             ("psa_conv_dw_pipe_kernel", "conv_dw_pipe"),
             ("psa_rows_copy_kernel", "rows_copy"))


def short_name(kernel: str) -> str:
    """Slot name plus dtype and the kernel's integer template arguments
    (head dims, then tile parameters), e.g. bwd_main<bf16,64,64,2,64,2,64>."""
    # rocprofv3 half-demangles some names: the mangled prefix DF16bLi32E
    # (bf16, then the integer 32) comes out as "bool _Accum, int, E".
    kernel = kernel.replace("<bool _Accum, int, E", "IDF16bLi32E")
    for pat, slot in PSA_SLOTS:
        if pat in kernel:
            m = re.search(pat + r"I(DF16b|DF16_|f)((?:Li\d+E)*)", kernel)
            if m:
                dt = {"DF16b": "bf16", "DF16_": "f16"}.get(m.group(1), "f32")
                dims = re.findall(r"Li(\d+)E", m.group(2))
                return f"{slot}<{','.join([dt] + dims)}>"
            # fully demangled (fp32 instances): psa_fwd_kernel<float, 16, 16, ...>
            m = re.search(pat + r"<(float|__bf16|_Float16)((?:, \d+)*)", kernel)
            if m:
                dt = {"__bf16": "bf16", "_Float16": "f16"}.get(m.group(1), "f32")
                dims = re.findall(r"\d+", m.group(2))
                return f"{slot}<{','.join([dt] + dims)}>"
            return slot
    return kernel[:60]


def stats(path: str, out: str, command: str, trace: str | None = None) -> None:
    """One row per kernel from the stats CSV; with the kernel-trace CSV, one
    row per (kernel, grid size), so that one instance used by two workloads
    shows as two rows."""
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{command}`", ""]
    if trace:
        per = defaultdict(list)
        for r in csv.DictReader(open(trace)):
            grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            per[(short_name(r["Kernel_Name"]), grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        tot = sum(sum(v) for v in per.values())
        lines += ["| kernel | workgroups | calls | total us | avg us | min us | max us | % |",
                  "|---|---|---|---|---|---|---|---|"]
        for (name, grid), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {name} | {grid} | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                         f"{max(v):.1f} | {100 * sum(v) / tot:.1f} |")
    else:
        lines += ["| kernel | calls | total us | avg us | min us | max us | % |",
                  "|---|---|---|---|---|---|---|"]
        for r in csv.DictReader(open(path)):
            name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
            ns = lambda k: float(r[k]) / 1000.0
            lines.append(f"| {short_name(name)} | {r['Calls']} | {ns('TotalDurationNs'):.1f} | "
                         f"{ns('AverageNs'):.1f} | {ns('MinNs'):.1f} | {ns('MaxNs'):.1f} | "
                         f"{float(r['Percentage']):.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def per_dispatch(path: str, counter: str) -> dict:
    """{kernel name: [value per dispatch]} for one counter."""
    acc = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def _instance_prefixes(workload: str) -> dict:
    """Short-name prefix of the kernel instance each slot runs for `workload`
    (attention kernels carry (dk, dv), the preprocessing kernel dv)."""
    from vision_transformer_attention_psa_amd.inputs import WORKLOADS
    wl = WORKLOADS[workload]
    return {"fwd": f"fwd<{wl.dtype},{wl.dk},{wl.dv},", "bwd_main": f"bwd_main<{wl.dtype},{wl.dk},{wl.dv},",
            "bwd_pre": f"bwd_pre<{wl.dtype},{wl.dv}>"}


def traffic(fetch_csv: str, write_csv: str, workload: str, copy_mib: int, out_json: str,
            out_md: str, command: str, fingerprint: str) -> None:
    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w = per_dispatch(write_csv, "WRITE_SIZE")
    calib = [k for k in f if "MulFunctor" in k]
    if not calib:
        sys.exit("no calibration kernel (MulFunctor) in the FETCH_SIZE run")
    known = copy_mib * float(1 << 20)
    f_cal = max(f[calib[0]])
    w_cal = max(w[[k for k in w if "MulFunctor" in k][0]])
    f_scale, w_scale = known / f_cal, known / w_cal
    res, lines = {}, []
    wanted = _instance_prefixes(workload)
    for k in f:
        slot = next((s for p, s in PSA_SLOTS if p in k), None)
        if slot is None:
            continue
        fb = sum(f[k]) / len(f[k]) * f_scale
        wb = sum(w.get(k, [0.0])) / max(1, len(w.get(k, []))) * w_scale
        # Several instances of one slot can run in the same program (the
        # V-slice calls use other head dims): record the workload's own.
        pre = wanted.get(slot)
        if slot not in res and (pre is None or short_name(k).startswith(pre)):
            res[slot] = fb + wb
        lines.append(f"| {short_name(k)} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {(fb + wb) / 1e6:.2f} |")
    rec = {}
    if os.path.exists(out_json):
        rec = json.load(open(out_json))
    if rec.get("fingerprint") != fingerprint:
        rec = {"fingerprint": fingerprint, "workloads": {}}
    rec["workloads"][workload] = res
    rec["calibration"] = {"copy_mib": copy_mib, "fetch_kib_read": f_cal, "write_kib_read": w_cal,
                          "fetch_scale": f_scale, "write_scale": w_scale}
    json.dump(rec, open(out_json, "w"), indent=1)
    md = [f"# HBM traffic per launch, {workload}", "",
          f"Commands: `{command}` (one run with `--pmc FETCH_SIZE`, one with `--pmc WRITE_SIZE`).", "",
          f"Calibration: dst = src * 1 over {copy_mib} MiB float32; FETCH_SIZE read {f_cal:.0f} and "
          f"WRITE_SIZE {w_cal:.0f} for {known / 1024:.0f} KiB moved each way, so the counters are "
          f"scaled by {f_scale:.4f} (fetch) and {w_scale:.4f} (write) bytes per unit.", "",
          f"Kernel source fingerprint: `{fingerprint}`", "",
          "| kernel | fetch MB | write MB | total MB |", "|---|---|---|---|", *lines]
    with open(out_md, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def pmc(csvs: list, out: str, command: str, cus: int = 256, xccs: int = 8) -> None:
    """Per-kernel averages of the counters in one or more --pmc runs and the
    ratios derived from them.  Utilisation expressions follow rocprofv3's own
    derived metrics: MFMA busy = sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE
    of one XCC x SIMDs); GRBM_GUI_ACTIVE in the CSV is the sum over the XCCs."""
    vals = defaultdict(lambda: defaultdict(list))  # short name -> counter -> per-dispatch values
    dur = defaultdict(dict)
    for path in csvs:
        per = defaultdict(lambda: defaultdict(float))
        for r in csv.DictReader(open(path)):
            if not any(p in r["Kernel_Name"] for p, _ in PSA_SLOTS):
                continue
            # one row per (kernel, workgroups): an instance shared by two workloads shows twice
            wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            name = f"{short_name(r['Kernel_Name'])} x{wg}"
            key = (name, r["Dispatch_Id"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            dur[name][(path, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        for (name, _), cs in per.items():
            for c, v in cs.items():
                vals[name][f"{c}@{path}" if c == "GRBM_GUI_ACTIVE" else c].append(v)
    avg = {n: {c: sum(v) / len(v) for c, v in cs.items()} for n, cs in vals.items()}
    simds = cus * 4

    def div(x, y):
        return x / y if y else float("nan")

    def gui(a, counter_file):
        return a.get(f"GRBM_GUI_ACTIVE@{counter_file}", float("nan")) / xccs

    rows = []
    for name in sorted(avg, key=lambda n: -sum(dur[n].values()) / max(1, len(dur[n]))):
        a = avg[name]
        f1 = next((p for p in csvs if f"GRBM_GUI_ACTIVE@{p}" in a and "SQ_INSTS_MFMA" in a), csvs[0])
        mf = a.get("SQ_INSTS_MFMA", float("nan"))
        g = gui(a, f1)
        rows.append((name, sum(dur[name].values()) / len(dur[name]),
                     100 * div(a.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")), g * simds),
                     div(a.get("SQ_INSTS_VALU", float("nan")), mf),
                     div(a.get("SQ_INSTS_VALU_TRANS_F32", float("nan")), mf),
                     div(a.get("SQ_INSTS_LDS", float("nan")), mf),
                     100 * div(a.get("SQ_LDS_BANK_CONFLICT", float("nan")), g * cus),
                     100 * div(a.get("SQ_ACTIVE_INST_VALU", float("nan")), a.get("SQ_WAVE_CYCLES", float("nan"))),
                     100 * div(a.get("SQ_ACTIVE_INST_LDS", float("nan")), a.get("SQ_WAVE_CYCLES", float("nan"))),
                     100 * div(a.get("SQ_WAIT_ANY", float("nan")), a.get("SQ_WAVE_CYCLES", float("nan"))),
                     100 * div(a.get("TCC_HIT_sum", float("nan")),
                               a.get("TCC_HIT_sum", float("nan")) + a.get("TCC_MISS_sum", float("nan")))))
    lines = ["# rocprofv3 counters per kernel", "", f"Commands: `{command}`", "",
             "Columns: MFMA busy = sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC x "
             f"{simds} SIMDs); VALU/MFMA, TRANS/MFMA, LDS/MFMA = issued instructions per MFMA "
             "instruction (SQ_INSTS_VALU counts MFMA too); LDS conflict = SQ_LDS_BANK_CONFLICT / "
             f"(GRBM_GUI_ACTIVE per XCC x {cus} CUs); VALU / LDS active and waiting = SQ_ACTIVE_INST_VALU, "
             "SQ_ACTIVE_INST_LDS and SQ_WAIT_ANY as a share of SQ_WAVE_CYCLES (wave-cycles, all in quad-cycles); "
             "L2 hit = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum), all L2 requests of the dispatch. Counters "
             "come from separate runs; durations are per dispatch under the profiler.", "",
             "| kernel x workgroups | us | MFMA busy % | VALU/MFMA | TRANS/MFMA | LDS/MFMA | LDS conflict % | "
             "VALU active % | LDS active % | waiting % | L2 hit % |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| " + r[0] + " | " + " | ".join(f"{x:.1f}" if i in (0, 1, 5, 6, 7, 8, 9) else f"{x:.2f}"
                                                    for i, x in enumerate(r[1:])) + " |")
    # Where the wave-cycles go, when the run also holds these counters.
    att = [n for n in avg if "SQ_WAIT_INST_ANY" in avg[n] and "SQ_ACTIVE_INST_ANY" in avg[n]]
    if att:
        lines += ["", "Wave-cycle attribution (shares of SQ_WAVE_CYCLES): active = SQ_ACTIVE_INST_ANY (the wave "
                  "has an instruction executing), issue wait = SQ_WAIT_INST_ANY (an instruction is ready but "
                  "not issued: the SIMD's issue slots or the unit it needs are taken), dependency wait = "
                  "SQ_WAIT_ANY (s_waitcnt on memory results, barriers), of which LDS issue wait = "
                  "SQ_WAIT_INST_LDS; VALU with MFMA = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES "
                  "(share of matrix-busy cycles in which a VALU instruction also executes).", "",
                  "| kernel x workgroups | active % | issue wait % | dependency wait % | LDS issue wait % | "
                  "VALU with MFMA % |", "|---|---|---|---|---|---|"]
        for name in sorted(att, key=lambda n: -sum(dur[n].values()) / max(1, len(dur[n]))):
            a = avg[name]
            wc = a.get("SQ_WAVE_CYCLES", float("nan"))
            vals_ = (100 * div(a["SQ_ACTIVE_INST_ANY"], wc), 100 * div(a["SQ_WAIT_INST_ANY"], wc),
                     100 * div(a.get("SQ_WAIT_ANY", float("nan")), wc),
                     100 * div(a.get("SQ_WAIT_INST_LDS", float("nan")), wc),
                     100 * div(a.get("SQ_VALU_MFMA_COEXEC_CYCLES", float("nan")),
                               a.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))))
            lines.append(f"| {name} | " + " | ".join(f"{x:.1f}" for x in vals_) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--trace", help="kernel_trace.csv of the same run: one row per (kernel, grid size)")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--out-json", required=True)
    t.add_argument("--out-md", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--fingerprint", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("csv", nargs="+")
    m.add_argument("--out", required=True)
    m.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "pmc":
        pmc(a.csv, a.out, a.command)
    elif a.cmd == "stats":
        stats(a.csv, a.out, a.command, a.trace)
    else:
        traffic(a.fetch_csv, a.write_csv, a.workload, a.copy_mib, a.out_json, a.out_md, a.command,
                a.fingerprint)


if __name__ == "__main__":
    main()
