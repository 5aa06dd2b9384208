#!/usr/bin/env python3
"""Fake-quant + QSNR throughput on one MI355X, through the C ABI of liblq.

One step = one pass of the whole path over one synthetic tensor: every
variant the workload names (for the default workload, 8192x4096 bf16
activations with outlier columns, MXINT8 / MXFP8-E4M3 / MXFP8-E5M2 with
32-element blocks and UE8M0 scales), each a single fused launch that reads x
and writes codes, scales, the dequantized tensor and the QSNR.

value = algorithmic bytes per step (one read of x, one write of codes, scales,
zero points and dequant, per variant) / time per step, inputs resident in HBM.
Input copies are rotated so that consecutive steps never find x in the
256 MB Infinity Cache.

Prints ONE JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fake-quant+QSNR GB/s and % of HBM peak on 1 MI355X (bit-exact vs oracle)"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20

DESCRIPTIONS = {
    "c1": "fp32 1024x1024 N(0,1): per-tensor INT8 and E4M3, fp32 scale and dequant",
    "c2": "bf16 8192x4096 N(0,1) with 8 outlier columns x100: MXINT8, MXFP8-E4M3, MXFP8-E5M2 "
          "(blocks of 32, UE8M0 scales, bf16 dequant)",
    "c3": "bf16 11008x4096 N(0,0.02^2): INT4 group 64 symmetric and group 128 asymmetric, fp16 scales/zeros",
    "c4": "bf16 16384x8192 Student-t(3): E2M1 and INT4, blocks of 16, E4M3 scales, without and with H16",
    "c4t": "c4 with two-level scaling (NVFP4 / NVINT4): an FP32 tensor scale above the E4M3 block scales",
    "c4r": "c4's tensor, E2M1 and INT4 blocks of 16 with E4M3 scales under a 256-column randomized Hadamard "
           "rotation (QuaRot; seeded signs), y rotated back",
    "c4q": "c4r with 1024-column rotation groups (one wave of lanes per group)",
    "c7": "c2's tensor as MXFP6: E2M3 and E3M2, blocks of 32 with UE8M0 scales, bf16 dequant",
    "c6": "c3's bf16 11008x4096 weights, DeepSeek-V3 style FP8: E4M3 with fp32 scales per 128x128 tile "
          "(weights) and per 1x128 tile (activations)",
    "c5": "256 bf16 4096x4096 tensors (uniform / normal / t(3) with 0.1% outliers x50): INT8, INT4, E4M3, "
          "E5M2, E2M1 x per-tensor, per-channel, blocks of 16/32/64; QSNR table and INT-vs-FP win counts",
}




def call_kernels(v: dict, in_dtype: str, rows: int, cols: int) -> list:
    """Kernel names one fake-quant call launches (per-block and per-tensor paths)."""
    import torch
    from bit_quantization_block_amd.profiling import call_kernel_names

    return call_kernel_names(v, in_dtype, rows, cols, torch.cuda.get_device_properties(0).multi_processor_count)


def load_traffic(cfg: str, kernels: list):
    """HBM bytes per call from committed rocprofv3 counter runs (profiles/), if
    they were taken on the current kernel sources; otherwise None."""
    from bit_quantization_block_amd.profiling import kernel_source_digest

    p = os.path.join(ROOT, "profiles", f"traffic_{cfg}.json")
    if not kernels or not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    total = 0
    for k in kernels:
        rec = t.get("kernels", {}).get(k)
        if rec is None:
            return None
        total += rec["hbm_bytes_per_launch"]
    return total


def cpu_baseline(cfg, d, variants, budget_elems=1.6e8):
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from bit_quantization_block_amd import workloads as W

    rows, cols = d["x"].shape
    # row spans start at multiples of the largest tile height (whole bands of tiles)
    band = max([v["tile_rows"] for v in variants if v["gran"] == "tile"] + [1])
    sample_rows = int(min(rows, max(band, budget_elems // (len(variants) * cols) // band * band)))
    threads = max(1, min(16, os.cpu_count() or 1))
    chunk = -(-max(1, -(-sample_rows // (threads * 4))) // band) * band
    spans = [(r, min(sample_rows, r + chunk)) for r in range(0, sample_rows, chunk)]
    in_bytes = 4 if d["dtype"] == "f32" else 2
    x = d["x"]
    tstats = {id(v): oracle.tensor_stat(v, x)[0] for v in variants if oracle.needs_stat(v)}

    def work(item):
        v, span = item
        oracle.fake_quant(v, x, rows=span, tstat=tstats.get(id(v)))

    items = [(v, s) for v in variants for s in spans]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, items))
    dt = time.perf_counter() - t0
    nbytes = sum(W.algorithmic_bytes(v, sample_rows, cols, in_bytes) for v in variants)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg}: rows 0..{sample_rows} of {rows} (x{cols}), all {len(variants)} variants, "
                      f"all outputs, {threads} threads over row chunks, {dt:.2f} s wall"}


def run_sweep(args, L) -> dict:
    """The 256-tensor sweep: every tensor resident in HBM first, then 25 calls
    per tensor timed as one region; QSNR table, win counts, oracle checks."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    from bit_quantization_block_amd import lq
    from bit_quantization_block_amd import workloads as W

    n_t = args.tensors
    rows = cols = 4096
    variants = W.c5_variants()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(16) as ex:
        host = list(ex.map(W.c5_input, range(n_t)))
    print(f"# {n_t} tensors generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    xs = [torch.from_numpy(np.ascontiguousarray(h["bits"]).view(np.uint8).reshape(-1).copy()).cuda() for h in host]
    runners = [lq.Runner(v, rows, cols, "bf16", lib=L) for v in variants]
    # one 64-byte result slot per (tensor, variant), written by the finish kernels
    res = torch.zeros((n_t, len(variants), 8), dtype=torch.float64, device="cuda")
    bytes_per_tensor = sum(W.algorithmic_bytes(v, rows, cols, 2) for v in variants)

    def tensor_pass(i):
        for j, r in enumerate(runners):
            r.res = res[i, j].view(torch.uint8)
            r.fake_quant(xs[i])

    tensor_pass(0)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(n_t):
        tensor_pass(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    table = res[:, :, 2].cpu().numpy().reshape(n_t, 5, 5)          # qsnr_db of each call
    wins = lq.lq_sweep_tally(table, 1e-3, lib=L)
    pairs = ("int8-vs-e4m3", "int8-vs-e5m2", "int4-vs-e2m1")
    win_table = {g: {pairs[p]: {"int": int(wins[gi, p, 0]), "fp": int(wins[gi, p, 1]), "tie": int(wins[gi, p, 2])}
                     for p in range(3)} for gi, g in enumerate(W.C5_GRANS)}
    check = None
    if not args.no_parity:
        worst = 0.0
        for i in range(min(3, n_t)):
            for j, v in enumerate(variants):
                _, _, q = oracle.qsnr_full(v, host[i]["x"], threads=16)
                worst = max(worst, abs(q - table.reshape(n_t, -1)[i, j]))
        check = {"tensors_checked": min(3, n_t), "max_qsnr_delta_db": worst, "qsnr_tol_db": 1e-3}
    mean_by_kind = {}
    for k in W.C5_KINDS:
        idx = [i for i in range(n_t) if W.c5_kind(i) == k]
        mean_by_kind[k] = {f"{f}/{g}": round(float(table[idx, fi, gi].mean()), 3)
                           for fi, f in enumerate(W.C5_FORMATS) for gi, g in enumerate(W.C5_GRANS)}
    return {"ms": ms, "bytes": bytes_per_tensor * n_t, "n_tensors": n_t, "calls": n_t * len(variants),
            "win_counts": win_table, "mean_qsnr_db": mean_by_kind, "parity": check}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated across steps (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain elementwise copy (torch.neg on fp32) reading and writing this "
                         "many MiB, for counter calibration")
    ap.add_argument("--lib", default=None, help="path of liblq.so (default: the in-tree build)")
    ap.add_argument("--tensors", type=int, default=256, help="c5: number of sweep tensors")
    ap.add_argument("--grid-limit", type=int, default=0,
                    help="cap on workgroups per launch (lq_set_grid_limit; 0 = the library default)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from bit_quantization_block_amd import lq
    from bit_quantization_block_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    L = lq.load(args.lib) if args.lib else lq.load()
    if args.grid_limit:
        lq.lq_set_grid_limit(args.grid_limit, lib=L)
    if args.config == "c5":
        sw = run_sweep(args, L)
        out = {"metric": METRIC, "value": round(sw["bytes"] / (sw["ms"] * 1e-3) / 1e9, 2), "unit": "GB/s",
               "n_gpus": 1, "steps": 1, "warmup": 1, "ms_per_step": round(sw["ms"], 3), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
               "config": {"workload": f"c5: {DESCRIPTIONS['c5']}", "tensors": sw["n_tensors"],
                          "calls": sw["calls"], "bytes_per_step": sw["bytes"]},
               "win_counts": sw["win_counts"], "mean_qsnr_db": sw["mean_qsnr_db"], "parity": sw["parity"]}
        print(json.dumps(out), flush=True)
        return 0
    spec = W.WORKLOADS[args.config]
    variants = spec["variants"]()
    t0 = time.perf_counter()
    d = spec["input"]()
    print(f"# input {args.config} generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    rows, cols = d["x"].shape
    in_bytes = 4 if d["dtype"] == "f32" else 2
    raw = np.ascontiguousarray(d["bits"]).view(np.uint8).reshape(-1)
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / raw.nbytes))
    x0 = torch.from_numpy(raw.copy()).cuda()
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    runners = [lq.Runner(v, rows, cols, d["dtype"], lib=L) for v in variants]
    bytes_per = [W.algorithmic_bytes(v, rows, cols, in_bytes) for v in variants]
    bytes_per_step = sum(bytes_per)

    def step(k):
        x = xs[k % copies]
        for r in runners:
            r.fake_quant(x)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    K = args.steps
    # timed region: K steps between two events on the launch stream (nothing
    # else is recorded inside it, so no event packet adds to the step time)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for k in range(K):
        step(args.warmup + k)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # per variant: K back-to-back calls (inputs rotated) between two events;
    # the average covers every kernel of a call and the gaps between calls
    per_kernel = []
    for i, (v, r) in enumerate(zip(variants, runners)):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record()
        for k in range(K):
            r.fake_quant(xs[k % copies])
        b_.record()
        torch.cuda.synchronize()
        avg = a_.elapsed_time(b_) / K
        shape = f"{v['tile_rows']}x{v['block']}" if v["gran"] == "tile" else (v.get("block") or "")
        per_kernel.append({"variant": f"{v['fmt']}/{v['gran']}{shape}/{v['scale']}"
                                      f"{'/asym' if not v.get('sym', True) else ''}"
                                      f"{'/h%d' % v['hadamard'] if v.get('hadamard') else ''}"
                                      f"{'/signs' if v.get('signs') is not None else ''}"
                                      f"{'/2level' if v.get('two_level') else ''}",
                           "avg_ms": round(avg, 5), "gbs": round(bytes_per[i] / (avg * 1e-3) / 1e9, 1)})
    dom = max(range(len(variants)), key=lambda i: per_kernel[i]["avg_ms"])
    achieved = bytes_per[dom] / (per_kernel[dom]["avg_ms"] * 1e-3) / 1e9
    dom_kernels = call_kernels(variants[dom], d["dtype"], rows, cols)
    traffic = load_traffic(args.config, dom_kernels)

    if args.calibrate_copy_mib:
        n = (args.calibrate_copy_mib << 20) // 4
        a = torch.zeros(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()

    parity = None
    if not args.no_parity:
        import oracle

        ok = True
        worst = 0.0
        for r, v in zip(runners, variants):
            got = r.host()
            res = r.result()
            cb = oracle.codes_bytes(v, 1, cols)
            tr = v["tile_rows"] if v["gran"] == "tile" else 1
            last = (rows - 1) // tr * tr                   # tiled variants: whole bands
            for a_, b_ in ((0, min(rows, max(4, tr))), (last if tr > 1 else rows - 2, rows)):
                ref = oracle.fake_quant(v, d["x"], rows=(a_, b_))
                ok &= bool(np.array_equal(got["codes"][a_ * cb:b_ * cb], ref["codes"]))
                ok &= bool(np.array_equal(got["y"][a_:b_], ref["y"]))
            _, _, q = oracle.qsnr_full(v, d["x"], threads=16)
            worst = max(worst, abs(res["qsnr"] - q))
        parity = {"sampled_rows_bit_exact": ok, "max_qsnr_delta_db": worst, "qsnr_tol_db": 1e-3}

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config, d, variants)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}", "rows": rows, "cols": cols,
                   "in_dtype": d["dtype"], "variants": [p["variant"] for p in per_kernel],
                   "bytes_per_step": bytes_per_step, "input_copies": copies,
                   "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
                   "grid_limit": args.grid_limit or None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": per_kernel[dom]["variant"], "kernels": dom_kernels,
                     "bytes_per_launch": bytes_per[dom],
                     "timing": "two HIP events on the launch stream around K back-to-back calls of this "
                               "variant (inputs rotated): the average covers every kernel a call launches "
                               "(listed in kernels) and the gaps between calls"},
        "per_kernel": per_kernel,
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_s": round(wall, 3),
        "kernel_source_digest": __import__("bit_quantization_block_amd.profiling",
                                           fromlist=["x"]).kernel_source_digest(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
