"""Summaries of rocprofv3 output for profiles/ (text only), and the HBM
traffic per launch that bench.py reports.

    python -m bit_quantization_block_amd.profiling stats  STATS_CSV  OUT_MD  "COMMAND"
    python -m bit_quantization_block_amd.profiling traffic FETCH_CSV WRITE_CSV COPY_BYTES OUT_JSON "CMD_FETCH" "CMD_WRITE"
    python -m bit_quantization_block_amd.profiling counters COUNTER_CSV OUT_MD "COMMAND"

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, from two separate
--pmc runs) are each scaled by the factor that makes the same counter read
the known byte count of a plain elementwise copy in the same run (torch.neg
on fp32: COPY_BYTES read and COPY_BYTES written).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_MARK = "neg_kernel"   # torch.neg on fp32: reads and writes the calibration size


def _code_only(text: str) -> str:
    """C/C++/Python source with comments and blank space removed, so that a
    comment-only edit keeps the digest."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest() -> str:
    """Digest of everything that decides the kernels' code (comments aside)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "bit_quantization_block_amd", "csrc", "*")))
    files += [os.path.join(ROOT, "bit_quantization_block_amd", "build.py"), os.path.join(ROOT, "include", "lq.h")]
    for p in files:
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel summary", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines.append("")
    lines.append(f"Kernel source digest: {kernel_source_digest()}")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


# MI355X: 256 CUs of 4 SIMDs, 16 lanes each (a wave64 VALU instruction issues
# over 4 cycles), 2.4 GHz peak engine clock.
SIMDS = 256 * 4
CYCLES_PER_VALU = 4
CLOCK_HZ = 2.4e9


def summarize_counters(counter_csv: str, out_md: str, command: str) -> dict:
    """Per-kernel averages per dispatch of every counter in one --pmc run,
    with what follows from them: VALU instructions per wave, the time the
    VALU instructions alone take to issue over the whole chip (a lower bound
    on the kernel's duration), and the share of wave-cycles spent waiting."""
    acc = defaultdict(lambda: defaultdict(list))
    meta = {}
    for r in csv.DictReader(open(counter_csv)):
        k = r["Kernel_Name"]
        acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        meta[k] = (int(r["Grid_Size"]), int(r["Workgroup_Size"]), int(r["VGPR_Count"]), int(r["Scratch_Size"]))
    names = sorted({c for k in acc for c in acc[k]})
    lines = ["# rocprofv3 counter summary", "", f"Command: `{command}`", "",
             "Averages per dispatch. VALU issue us = SQ_INSTS_VALU x 4 cycles / 1024 SIMDs / 2.4 GHz. "
             "Wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.", "",
             "| kernel | dispatches | grid | wg | VGPR | scratch | " + " | ".join(names) +
             " | VALU per wave | VALU issue us | wait share |",
             "|---|---|---|---|---|---|" + "---|" * len(names) + "---|---|---|"]
    out = {}
    for k in sorted(acc):
        avg = {c: sum(v) / len(v) for c, v in acc[k].items()}
        nd = max(len(v) for v in acc[k].values())
        g, wg, vgpr, scr = meta[k]
        waves = avg.get("SQ_WAVES", 0.0)
        valu = avg.get("SQ_INSTS_VALU")
        per_wave = valu / waves if valu is not None and waves else None
        issue_us = valu * CYCLES_PER_VALU / SIMDS / CLOCK_HZ * 1e6 if valu is not None else None
        wait = (avg["SQ_WAIT_INST_ANY"] / avg["SQ_WAVE_CYCLES"]
                if avg.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in avg else None)
        f = lambda v, fmt: "" if v is None else format(v, fmt)
        lines.append(f"| `{k}` | {nd} | {g} | {wg} | {vgpr} | {scr} | " +
                     " | ".join(f(avg.get(c), ".0f") for c in names) +
                     f" | {f(per_wave, '.1f')} | {f(issue_us, '.2f')} | {f(wait, '.3f')} |")
        out[k] = {"avg": avg, "valu_per_wave": per_wave, "valu_issue_us": issue_us, "wait_share": wait}
    lines += ["", f"Kernel source digest: {kernel_source_digest()}"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


def _counter_avgs(path: str, counter: str) -> dict:
    acc = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int, out_json: str, cmd_fetch: str, cmd_write: str) -> dict:
    fetch = _counter_avgs(fetch_csv, "FETCH_SIZE")
    write = _counter_avgs(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if COPY_MARK in k]
    if len(copy) != 1 or copy[0] not in write:
        raise SystemExit(f"calibration kernel not found uniquely: {copy}")
    cf = copy_bytes / (fetch[copy[0]] * 1024.0)
    cw = copy_bytes / (write[copy[0]] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k == copy[0]:
            continue
        fb = fetch[k] * 1024.0 * cf
        wb = write[k] * 1024.0 * cw
        kernels[k] = {"fetch_kib": fetch[k], "write_kib": write[k], "fetch_bytes": round(fb),
                      "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    out = {"kernel_source_digest": kernel_source_digest(), "copy_bytes": copy_bytes,
           "fetch_scale": cf, "write_scale": cw, "commands": {"fetch": cmd_fetch, "write": cmd_write},
           "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    return out


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "stats":
        summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif cmd == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7]),
                         indent=1))
    elif cmd == "counters":
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        raise SystemExit(__doc__)
