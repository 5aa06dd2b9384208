"""CPU checks of the profiling helpers that turn rocprofv3 output into the
summaries under profiles/ and the traffic figure bench.py reports."""
import csv
import json
import subprocess
import sys

from bit_quantization_block_amd import profiling as P
from bit_quantization_block_amd import workloads as W

COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"
FAST = "void lqd::k_lc<0, 2, 0, true>(lqd::FastArgs)"


def _write_stats(path):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([FAST, 25, 875000, 35000, 90.0, 33000, 40000, 0.0])
        w.writerow(["lqd::k_finish(lqd::Workspace const*, int, lq_result*)", 25, 100000, 4000, 10.0, 3900, 4200, 0.0])


def _write_counters(path, counter, copy_kib, fast_kib):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for _ in range(2):
            w.writerow([COPY, counter, copy_kib])
            w.writerow([FAST, counter, fast_kib])


def test_stats_summary(tmp_path):
    _write_stats(tmp_path / "s.csv")
    out = tmp_path / "k.md"
    subprocess.run([sys.executable, "-m", "bit_quantization_block_amd.profiling", "stats", str(tmp_path / "s.csv"),
                    str(out), "the command"], check=True)
    text = out.read_text()
    assert "Command: `the command`" in text
    assert f"| `{FAST}` | 25 | 35.00 | 33.00 | 40.00 | 90.00 |" in text
    assert P.kernel_source_digest() in text


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    copy_bytes = 1 << 28
    # FETCH reads half the bytes on the copy, WRITE reads them exactly
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE", copy_bytes / 2048, 1000.0)
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", copy_bytes / 1024, 3000.0)
    t = P.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy_bytes, str(tmp_path / "t.json"), "a", "b")
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    k = t["kernels"][FAST]
    assert k["fetch_bytes"] == 2 * 1000 * 1024 and k["write_bytes"] == 3000 * 1024
    assert k["hbm_bytes_per_launch"] == 5000 * 1024
    assert json.load(open(tmp_path / "t.json"))["kernel_source_digest"] == P.kernel_source_digest()


def test_counter_summary(tmp_path):
    """Averages per dispatch, VALU instructions per wave, the chip-wide VALU
    issue time (4 cycles per wave64 instruction over 1024 SIMDs at 2.4 GHz)
    and the wait share."""
    path = tmp_path / "c.csv"
    cols = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "VGPR_Count", "Scratch_Size", "Counter_Name",
            "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for valu in (2.4e5 * 1024 / 4 * 0.9, 2.4e5 * 1024 / 4 * 1.1):   # 90 and 110 us of issue: 100 on average
            w.writerow([FAST, 8192, 256, 64, 0, "SQ_INSTS_VALU", valu])
            w.writerow([FAST, 8192, 256, 64, 0, "SQ_WAVES", 32768])
            w.writerow([FAST, 8192, 256, 64, 0, "SQ_WAVE_CYCLES", 1000.0])
            w.writerow([FAST, 8192, 256, 64, 0, "SQ_WAIT_INST_ANY", 250.0])
    out = tmp_path / "c.md"
    subprocess.run([sys.executable, "-m", "bit_quantization_block_amd.profiling", "counters", str(path), str(out),
                    "the command"], check=True)
    r = P.summarize_counters(str(path), str(tmp_path / "d.md"), "x")[FAST]
    assert abs(r["valu_issue_us"] - 100.0) < 1e-9
    assert abs(r["valu_per_wave"] - 2.4e5 * 1024 / 4 / 32768) < 1e-9
    assert abs(r["wait_share"] - 0.25) < 1e-12
    text = out.read_text()
    assert "Command: `the command`" in text and f"| `{FAST}` | 2 | 8192 | 256 | 64 | 0 |" in text
    assert "| 100.00 | 0.250 |" in text and P.kernel_source_digest() in text


FINISH = "lqd::k_finish(lqd::Workspace const*, int, lq_result*)"


def names(v, in_dtype, rows, cols, **kw):
    from bit_quantization_block_amd import lq

    return lq.call_kernels(v, in_dtype, rows, cols, **kw)


def test_call_kernels_follow_the_dispatch():
    """lq_call_kernels reports the kernels of a call from the library's own
    dispatch (on a host without a GPU, for 256 compute units)."""
    c2 = W.c2_variants()[0]
    assert names(c2, "bf16", 8192, 4096) == [FAST]                               # one pass: wide, no finish
    big = names(c2, "bf16", 16384, 8192)                                         # narrow, finishes itself
    assert big == ["void lqd::k_lc<0, 2, 0, false>(lqd::FastArgs)"]
    odd = names(c2, "bf16", 3, 32 * 11)                                          # not a multiple of 1024
    assert odd == ["void lqd::k_fast<1, 0, 1, 2, true, false, true, false>(lqd::FastArgs)"]
    had = dict(W.c4_variants()[2])                                              # NVFP4 under H16
    assert names(had, "bf16", 64, 4096) == ["void lqd::k_h16<4>(lqd::FastArgs)"]
    assert names(had, "bf16", 16384, 8192) == ["void lqd::k_h16<4>(lqd::FastArgs)"]
    assert names(dict(W.c4t_variants()[3]), "bf16", 16384, 8192) == [                # NVINT4, H16, two-level
        "void lqd::k_stat<1, 16>(lqd::Args)", "void lqd::k_h16_two<1>(lqd::FastArgs)"]
    assert names(dict(W.c4t_variants()[3]), "bf16", 3, 1008)[1].startswith("void lqd::k_fast<")   # ragged
    assert names(dict(had, fmt="e4m3", scale="ue8m0"), "bf16", 64, 4096)[0].endswith(
        "true, true, false, false>(lqd::FastArgs)")                             # 8-bit under H16: k_fast
    assert names(W.c1_variants()[0], "f32", 1024, 1024) == [
        "void lqd::k_stat<0, 0>(lqd::Args)", "void lqd::k_flat<0, 0, 0, 1>(lqd::Args)"]   # last workgroup finishes
    t = dict(c2, gran="tensor", scale="f32")
    assert names(t, "bf16", 4096, 4096) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_lc<0, 0, 1, true>(lqd::FastArgs)"]
    # two-level: the statistic pass, then the lane-contiguous or tile-per-lane kernel
    t4 = W.c4t_variants()
    assert names(t4[0], "bf16", 16384, 8192) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_lc<4, 3, 2, false>(lqd::FastArgs)"]
    assert names(t4[2], "bf16", 16384, 8192) == [
        "void lqd::k_stat<1, 16>(lqd::Args)", "void lqd::k_h16_two<4>(lqd::FastArgs)"]
    assert names(dict(t4[1], out="f32"), "bf16", 64, 4096) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_flat<1, 1, 0, 2>(lqd::Args)"]
    assert names(dict(c2, gran="channel", scale="f32"), "bf16", 64, 4096) == [
        "void lqd::k_row_lc<0, 0>(lqd::FastArgs)"]                               # one wave per row
    e2m3 = W.c7_variants()[0]
    assert names(e2m3, "bf16", 8192, 4096) == [
        "void lqd::k_lc<5, 2, 0, false>(lqd::FastArgs)"]        # FP6: narrow, 1024 workgroups, finishes itself
    assert names(e2m3, "bf16", 8191, 4000) == [
        "void lqd::k_fast<1, 5, 1, 2, true, false, false, false>(lqd::FastArgs)"]
    w, a = W.c6_variants()
    assert names(w, "bf16", 11008, 4096) == ["void lqd::k_tile<1, 2, 0, 4>(lqd::Args)"]   # finishes in-kernel
    assert names(dict(w, out="f32"), "bf16", 11008, 4096) == ["void lqd::k_row<1, 2, 0, 4>(lqd::Args)", FINISH]
    assert names(a, "bf16", 11008, 4096) == ["void lqd::k_lc<2, 0, 0, false>(lqd::FastArgs)"]
    # rotations of 512 and 1024 columns: the specialised kernel's wide-rotation build
    q = W.c4q_variants()[0]
    assert names(q, "bf16", 16384, 8192) == [
        "void lqd::k_fast_wrot<1, 4, 1, 3, true, false>(lqd::FastArgs)"]
    assert names(dict(q, sym=False, fmt="int4", scale="f16", block=64), "bf16", 64, 4096)[0] == \
        "void lqd::k_flat<1, 1, 1, 0>(lqd::Args)"                               # zero points: general kernel
    # more than 32 passes per lane: the general kernel
    assert names(c2, "bf16", 1 << 17, 1 << 16)[0].startswith("void lqd::k_flat<")
    assert names(dict(c2, out="f32"), "f32", 64, 4096)[0] == \
        "void lqd::k_fast<0, 0, 0, 2, true, false, false, false>(lqd::FastArgs)"
    # no QSNR, no codes or a given scale: the general kernel, no finishing launch
    assert names(c2, "bf16", 8192, 4096, want=("codes", "scales", "y")) == [
        "void lqd::k_flat<1, 0, 1, 0>(lqd::Args)"]
    assert names(c2, "bf16", 0, 4096, want=("codes", "y")) == []                 # empty: nothing launched
    assert names(c2, "bf16", 0, 4096) == ["lqd::k_empty_result(lq_result*)"]     # ... but the empty QSNR
    from bit_quantization_block_amd import lq

    plan = lq.lq_call_kernels(lq.desc(c2, "bf16"), 16384, 8192, 31)
    assert plan == [("void lqd::k_lc<0, 2, 0, false>(lqd::FastArgs)", 32768, 256)]   # one chunk per wave
    # the general kernels over more than the inline grid of 1024 keep the finishing kernel
    assert names(dict(c2, out="f32", fmt="int8", scale="f32", gran="channel"), "f32", 8192, 4096)[-1] == FINISH
    # the wide one-pass shape: 2048 working workgroups and one that only collects
    assert lq.lq_call_kernels(lq.desc(c2, "bf16"), 8192, 4096, 31)[0][1:] == (2049, 1024)


def test_call_kernels_rejects_what_the_call_rejects():
    from bit_quantization_block_amd import lq

    d = lq.desc(W.c2_variants()[0], "bf16")
    d.block = 48
    L = lq.load()
    assert L.lq_call_kernels(d, 4, 96, 31, 0, None, 0) == -7
    d.block = 32
    assert L.lq_call_kernels(d, 4, 48, 31, 0, None, 0) == -3
    assert L.lq_call_kernels(None, 4, 48, 31, 0, None, 0) == -1
    assert L.lq_call_kernels(d, 4, 64, 31, 0, None, 0) == 1                  # counting only


def test_profiles_name_the_planned_kernels():
    """Every kernel lq_call_kernels plans for a workload's variants appears in
    the committed rocprofv3 summary of that workload's bench run, for each
    summary taken on the current kernel sources."""
    import glob
    import os
    import re

    checked = 0
    for path in sorted(glob.glob(os.path.join(P.ROOT, "profiles", "kernels_c*.md"))):
        text = open(path).read()
        m = re.search(r"Kernel source digest: ([0-9a-f]{16})", text)
        cfg = os.path.basename(path)[len("kernels_"):-len(".md")]
        if not m or m.group(1) != P.kernel_source_digest() or cfg not in W.WORKLOADS:
            continue
        spec = W.WORKLOADS[cfg]
        rows, cols = spec["shape"]
        listed = set(re.findall(r"\| `([^`]+)` \|", text))
        for v in spec["variants"]():
            for k in names(v, spec["dtype"], rows, cols):
                assert k in listed, (cfg, v, k)
        checked += 1
    assert checked >= 0


def test_digest_ignores_comments():
    assert P._code_only("int a; /* one\n two */ int b; // three\n  int c;") == "int a; int b; int c;"


def test_build_reads_kernel_resources():
    """The build's check of the compiler's resource remarks: per-kernel VGPRs,
    scratch and occupancy, and a kernel with scratch is found."""
    from bit_quantization_block_amd import build as B

    text = "\n".join([
        "a.hip:1:1: remark: Function Name: _ZN3lqd1kILi0EEEvv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark: Function Name: _ZN3lqd1kILi1EEEvv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]",
    ])
    r = B.kernel_resources(text)
    assert r == {"_ZN3lqd1kILi0EEEvv": {"vgprs": 64, "scratch": 0, "occupancy": 8},
                 "_ZN3lqd1kILi1EEEvv": {"vgprs": 128, "scratch": 20, "occupancy": 4}}
    assert "-Rpass-analysis=kernel-resource-usage" in B.FLAGS


def test_signed_rotation_grids_keep_each_lane_at_one_column():
    """A tile-per-lane kernel under a rotation with random signs reads each
    lane's sign bits once, so its grid covers the tensor in one pass or has a
    stride (workgroups x 256 threads x 16 elements) that is a multiple of
    cols; with no such grid under the cap the call takes k_flat."""
    from bit_quantization_block_amd import lq

    base = {"fmt": "e2m1", "gran": "block", "block": 16, "scale": "e4m3", "sym": True, "round": "rne",
            "out": "bf16", "hadamard": 256, "unrotate": True}

    def plan(v, rows, cols, signed):
        d = lq.desc(v, "bf16", signs_ptr=64 if signed else None)
        return lq.lq_call_kernels(d, rows, cols, sum(lq.OUT.values()), 1)

    # 11008 columns: m = 11008 / gcd(11008, 4096) = 43
    (name, nwg, nt), = plan(base, 4096, 11008, True)
    assert name.startswith("void lqd::k_fast<") and nt == 256
    assert nwg % 43 == 0 and nwg <= 8192 and (nwg * nt * 16) % 11008 == 0
    ntiles = 4096 * 11008 // 16
    assert nwg * nt < ntiles                                  # several passes
    # unsigned: any balanced grid
    (name_u, nwg_u, _), = plan(base, 4096, 11008, False)
    assert name_u == name
    # C4's shape: m = 2
    (_, nwg4, _), = plan(base, 16384, 8192, True)
    assert nwg4 % 2 == 0 and (nwg4 * 256 * 16) % 8192 == 0
    # one pass: no constraint
    (_, nwg1, nt1), = plan(base, 64, 11008, True)
    assert nwg1 * nt1 * 16 >= 64 * 11008
    # m above the cap: 16 x 8209 columns (gcd with 4096 is 16, m = 8209)
    v16 = dict(base, hadamard=16)
    kernels = [k[0] for k in plan(v16, 512, 16 * 8209, True)]
    assert kernels[0].startswith("void lqd::k_flat<"), kernels


def test_sweep_results_rows_and_resume(tmp_path):
    """The sweep's JSONL results: one row per (tensor, variant) from the
    lq_result words (err2, sig2, qsnr_db, then the non-finite count in the low
    word), read back only for tensors with every variant present."""
    import numpy as np

    import bench

    names = [bench.variant_name(v) for v in W.c5_variants()]
    res = np.zeros((len(names), 8), np.float64)
    res[:, 0], res[:, 1], res[:, 2] = 0.5, 2.0, np.arange(len(names), dtype=np.float64)
    res[3, 2] = np.inf                                   # an exact variant: err2 = 0
    counts = np.zeros((len(names), 2), np.uint32)
    counts[:, 0] = np.arange(len(names), dtype=np.uint32) * 7
    res[:, 3] = counts.view(np.float64).reshape(-1)
    rows = bench.sweep_rows(5, "normal", names, res)
    assert [r["variant"] for r in rows] == names and rows[0]["seed"] == 5005
    assert rows[3]["qsnr_db"] == float("inf") and rows[4]["nonfinite"] == 28 and rows[2]["err2"] == 0.5
    path = tmp_path / "sweep.jsonl"
    with open(path, "w") as f:
        for r in rows:                                   # tensor 5 complete
            f.write(json.dumps(r) + "\n")
        for r in bench.sweep_rows(6, "uniform", names, res)[:-1]:   # tensor 6 missing one variant
            f.write(json.dumps(r) + "\n")
    done = bench.load_sweep_rows(str(path), names)
    assert sorted(done) == [5]
    assert done[5][names[3]]["qsnr_db"] == float("inf") and done[5][names[10]]["qsnr_db"] == 10.0
    assert bench.load_sweep_rows(str(tmp_path / "absent.jsonl"), names) == {}
