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
        w.writerow([P.FINISH_KERNEL, 25, 100000, 4000, 10.0, 3900, 4200, 0.0])


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


def test_call_kernel_names_follow_the_dispatch():
    c2 = W.c2_variants()[0]
    assert P.call_kernel_names(c2, "bf16", 8192, 4096) == [FAST]                 # one pass: wide, no finish
    big = P.call_kernel_names(c2, "bf16", 16384, 8192)                             # several passes: narrow
    assert big == ["void lqd::k_lc<0, 2, 0, false>(lqd::FastArgs)", P.FINISH_KERNEL]
    odd = P.call_kernel_names(c2, "bf16", 3, 32 * 11)                              # not a multiple of 1024
    assert odd == ["void lqd::k_fast<1, 0, 1, 2, true, false, true, false>(lqd::FastArgs)"]
    had = dict(W.c4_variants()[2])
    assert P.call_kernel_names(had, "bf16", 64, 4096)[0].endswith("true, true, false, false>(lqd::FastArgs)")
    assert P.call_kernel_names(W.c1_variants()[0], "f32", 1024, 1024) == [
        "void lqd::k_stat<0, 0>(lqd::Args)", "void lqd::k_flat<0, 0, 0, 1>(lqd::Args)"]   # last workgroup finishes
    t = dict(c2, gran="tensor", scale="f32")
    assert P.call_kernel_names(t, "bf16", 4096, 4096) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_lc<0, 0, 1, true>(lqd::FastArgs)"]
    # two-level: the statistic pass, then the lane-contiguous or tile-per-lane kernel
    t4 = W.c4t_variants()
    assert P.call_kernel_names(t4[0], "bf16", 16384, 8192) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_lc<4, 3, 2, false>(lqd::FastArgs)", P.FINISH_KERNEL]
    assert P.call_kernel_names(t4[2], "bf16", 16384, 8192) == [
        "void lqd::k_stat<1, 16>(lqd::Args)",
        "void lqd::k_fast<1, 4, 1, 3, true, true, false, true>(lqd::FastArgs)", P.FINISH_KERNEL]
    assert P.call_kernel_names(dict(t4[1], out="f32"), "bf16", 64, 4096) == [
        "void lqd::k_stat<1, 0>(lqd::Args)", "void lqd::k_flat<1, 1, 0, 2>(lqd::Args)"]
    assert P.call_kernel_names(dict(c2, gran="channel"), "bf16", 64, 4096) == []
    e2m3 = W.c7_variants()[0]
    assert P.call_kernel_names(e2m3, "bf16", 8192, 4096) == [
        "void lqd::k_lc<5, 2, 0, false>(lqd::FastArgs)"]        # FP6: narrow, 1024 workgroups, finishes itself
    assert P.call_kernel_names(e2m3, "bf16", 8191, 4000) == [
        "void lqd::k_fast<1, 5, 1, 2, true, false, false, false>(lqd::FastArgs)", P.FINISH_KERNEL]
    w, a = W.c6_variants()
    assert P.call_kernel_names(w, "bf16", 11008, 4096) == ["void lqd::k_tile<1, 2, 0, 4>(lqd::Args)", P.FINISH_KERNEL]
    assert P.call_kernel_names(dict(w, out="f32"), "bf16", 11008, 4096) == [
        "void lqd::k_row<1, 2, 0, 4>(lqd::Args)", P.FINISH_KERNEL]
    assert P.call_kernel_names(a, "bf16", 11008, 4096) == ["void lqd::k_lc<2, 0, 0, false>(lqd::FastArgs)",
                                                            P.FINISH_KERNEL]
    # rotations of 512 and 1024 columns: the specialised kernel's wide-rotation build
    q = W.c4q_variants()[0]
    assert P.call_kernel_names(q, "bf16", 16384, 8192) == [
        "void lqd::k_fast_wrot<1, 4, 1, 3, true, false>(lqd::FastArgs)", P.FINISH_KERNEL]
    assert P.call_kernel_names(dict(q, sym=False, fmt="int4", scale="f16", block=64), "bf16", 64, 4096)[0] == \
        "void lqd::k_flat<1, 1, 1, 0>(lqd::Args)"                               # zero points: general kernel
    # more than 32 passes per lane: the general kernel
    assert P.call_kernel_names(c2, "bf16", 1 << 16, 1 << 16)[0].startswith("void lqd::k_flat<")
    assert P.call_kernel_names(dict(c2, out="f32"), "f32", 64, 4096)[0] == \
        "void lqd::k_fast<0, 0, 0, 2, true, false, false, false>(lqd::FastArgs)"


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
