"""Summaries of rocprofv3 output for profiles/ (text only), and the HBM
traffic per launch that bench.py reports.

    python -m bit_quantization_block_amd.profiling stats  STATS_CSV  OUT_MD  "COMMAND"
    python -m bit_quantization_block_amd.profiling traffic FETCH_CSV WRITE_CSV COPY_BYTES OUT_JSON "CMD_FETCH" "CMD_WRITE"

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


# k_flat / k_lc modes: per block, per tensor, two-level
MODE_BLOCK, MODE_TENSOR, MODE_TWO = 0, 1, 2


def flat_kernel_name(in_dtype: int, fmt: int, out_dtype: int, mode: int) -> str:
    return f"void lqd::k_flat<{in_dtype}, {fmt}, {out_dtype}, {mode}>(lqd::Args)"


def fast_kernel_name(dtype: int, fmt: int, scale_fmt: int, sym: bool, had: bool, wide: bool,
                     two: bool = False) -> str:
    b = lambda v: "true" if v else "false"
    return (f"void lqd::k_fast<{dtype}, {fmt}, {dtype}, {scale_fmt}, {b(sym)}, {b(had)}, {b(wide)}, "
            f"{b(two)}>(lqd::FastArgs)")


FINISH_KERNEL = "lqd::k_finish(lqd::Workspace const*, int, lq_result*)"


# (format, scale format, symmetric, rotation) combinations that have a
# specialised per-block kernel (the table filled in lq_fast.hip)
_FMT = {"int8": 0, "int4": 1, "e4m3": 2, "e5m2": 3, "e2m1": 4, "e2m3": 5, "e3m2": 6}
_SF = {"f32": 0, "f16": 1, "ue8m0": 2, "e4m3": 3}
_DT = {"f32": 0, "bf16": 1, "f16": 2}
FAST_SET = ({(f, sf, True, False) for f in range(7) for sf in range(4)}
            | {(f, sf, False, False) for f in (0, 1) for sf in (0, 1)}
            | {(1, 3, True, True), (4, 3, True, True), (0, 2, True, True), (2, 2, True, True), (3, 2, True, True)})


def balanced_grid(needed: int, cap: int) -> int:
    """Workgroups the host launches for `needed` under `cap` (lq_api.hip):
    the fewest that give every workgroup the same number of passes."""
    if needed <= cap:
        return needed
    passes = -(-needed // cap)
    return -(-needed // passes)


INLINE_FINISH_MAX_WG = 1024   # narrow grids up to this size finish the QSNR in their last workgroup
SIX_LC_MAX_WG = 1024          # narrow lane-contiguous grids for FP6


def call_kernel_names(v: dict, in_dtype: str, rows: int, cols: int, cus: int = 256) -> list:
    """Names (as rocprofv3 prints them) of the kernels one fake-quant call with
    data-driven scales and every output launches, in order; [] for the
    per-channel path. Mirrors the dispatch in lq_api.hip: grid cap
    min(32 * CUs, 8192) workgroups of 256; the wide shape (a quarter as many
    1024-thread workgroups, no finishing kernel) when it covers the tensor in
    one pass; bf16 with symmetric scales and a multiple of 1024 elements takes
    the lane-contiguous kernels (per-tensor: fp32 scales; fp32 block scales
    and FP6 only narrow, FP6 on at most 1024 workgroups); narrow and general
    grids of at most 1024 workgroups finish the QSNR in their last one. Per-tensor and two-level calls start with the statistic pass."""
    fmt, sf, out = _FMT[v["fmt"]], _SF[v["scale"]], v.get("out", "bf16")
    sym, had = bool(v.get("sym", True)), bool(v.get("hadamard", 0))
    two = bool(v.get("two_level", False))
    rne = v.get("round", "rne") == "rne"
    if v["gran"] == "tile" and v["tile_rows"] == 1:
        v = dict(v, gran="block")                       # one-row tiles are blocks
    if v["gran"] == "channel":
        return []
    if v["gran"] == "tile":
        # one workgroup per tile, then the finishing kernel
        units = v["tile_rows"] * v["block"] // 16
        per_lane = -(-units // 256)
        nch = 1 if per_lane <= 1 else 2 if per_lane <= 2 else 4 if per_lane <= 4 else 0
        if nch and rne and sym and not had and in_dtype == out and in_dtype != "f16" and fmt < 5:
            return [f"void lqd::k_tile<{_DT[in_dtype]}, {fmt}, {sf}, {nch}>(lqd::Args)", FINISH_KERNEL]
        return [f"void lqd::k_row<{_DT[in_dtype]}, {fmt}, {_DT[out]}, {nch}>(lqd::Args)", FINISH_KERNEL]
    b = lambda x: "true" if x else "false"
    n = rows * cols
    ntiles = (n + 15) // 16
    cap = min(32 * cus, 8192)
    lc_ok = rne and in_dtype == out == "bf16" and sym and not had and n % 1024 == 0

    def lc(mode):
        chunks = n // 1024
        wide = fmt < 5 and (mode != MODE_BLOCK or sf != _SF["f32"]) and chunks <= max(1, cap // 4) * 16
        waves, capl = (16, max(1, cap // 4)) if wide else (4, min(cap, SIX_LC_MAX_WG) if fmt >= 5 else cap)
        nwg = balanced_grid(-(-chunks // waves), capl)
        if chunks > 32 * nwg * waves:
            return None
        k = f"void lqd::k_lc<{fmt}, {sf}, {mode}, {b(wide)}>(lqd::FastArgs)"
        return [k] if wide or nwg <= INLINE_FINISH_MAX_WG else [k, FINISH_KERNEL]

    nwg = balanced_grid(-(-ntiles // 256), cap)
    flat_tail = [] if nwg <= INLINE_FINISH_MAX_WG else [FINISH_KERNEL]
    nrot = int(v.get("hadamard", 0) or 0)
    stat = f"void lqd::k_stat<{_DT[in_dtype]}, {0 if not nrot else 16 if nrot == 16 else 1024}>(lqd::Args)"
    if v["gran"] == "tensor":
        if lc_ok and sf == _SF["f32"]:
            ks = lc(MODE_TENSOR)
            if ks is not None:
                return [stat] + ks
        return [stat, flat_kernel_name(_DT[in_dtype], fmt, _DT[out], MODE_TENSOR)] + flat_tail
    head = [stat] if two else []
    if lc_ok and (two or (fmt, sf, sym, had) in FAST_SET):
        ks = lc(MODE_TWO if two else MODE_BLOCK)
        if ks is not None:
            return head + ks
    if (rne and in_dtype == out and in_dtype != "f16" and (two or (fmt, sf, sym, had) in FAST_SET)):
        wide = in_dtype != "f32" and not had and fmt < 5 and ntiles <= max(1, cap // 4) * 1024
        nt, capf = (1024, max(1, cap // 4)) if wide else (256, cap)
        nwgf = balanced_grid(-(-ntiles // nt), capf)
        if ntiles <= 32 * nwgf * nt:
            if nrot > 256:      # rotations of 512 and 1024 columns: their own kernel, narrow
                dt = _DT[in_dtype]
                k = f"void lqd::k_fast_wrot<{dt}, {fmt}, {dt}, {sf}, {b(sym)}, {b(two)}>(lqd::FastArgs)"
            else:
                k = fast_kernel_name(_DT[in_dtype], fmt, sf, sym, had, wide, two)
            return head + ([k] if wide or nwgf <= INLINE_FINISH_MAX_WG else [k, FINISH_KERNEL])
    return head + [flat_kernel_name(_DT[in_dtype], fmt, _DT[out], MODE_TWO if two else MODE_BLOCK)] + flat_tail


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
    else:
        raise SystemExit(__doc__)
