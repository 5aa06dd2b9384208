"""CPU checks of the boundary: liblq.so loads, exports every function that
include/lq.h declares, and rejects bad arguments before touching the GPU
(every failing check returns before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HDR = os.path.join(INCLUDE, "lq.h")
CEILING_HDR = os.path.join(INCLUDE, "lq_ceiling.h")


def declared_functions(hdr=HDR, prefix="lq_"):
    text = open(hdr).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(" + prefix + r"[a-z_0-9]+)\s*\(", text)))


def test_every_header_is_covered():
    """include/ holds the two ABIs checked here and nothing else."""
    assert sorted(os.listdir(INCLUDE)) == ["lq.h", "lq_ceiling.h"]


def _exported(path):
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    return {s for s in syms if not s.startswith("__hip_cuid_") and s not in ("_init", "_fini")}


def test_ceiling_library_exports_exactly_its_header():
    names = declared_functions(CEILING_HDR, "lqc_")
    assert set(names) == set(lq.CEILING_EXPORTS)
    L = lq.load_ceiling()
    for n in names:
        assert hasattr(L, n), n
    assert _exported(lq.CEILING_PATH) == set(names)
    # argument checks return before any HIP call (every case below fails one)
    B = 2048   # bytes of 1024 bf16 elements
    assert L.lqc_copy(None, B, FAKE, B, 1024, 256, 1, None) == -1
    assert L.lqc_copy(FAKE, B, FAKE, B, 1000, 256, 1, None) == -3
    assert L.lqc_copy(FAKE, B, FAKE, B, 1024, 128, 1, None) == -3
    assert L.lqc_copy(FAKE, B - 1, FAKE, B, 1024, 256, 1, None) == -3        # source smaller than 2n
    assert L.lqc_copy(FAKE, B, FAKE, B - 1, 1024, 256, 1, None) == -3        # destination smaller than 2n
    assert L.lqc_copy(FAKE + 4, B, FAKE, B, 1024, 256, 1, None) == -4

    assert L.lqc_read(None, B, B, FAKE, 16, 256, 1, None) == -1
    assert L.lqc_read(FAKE, B, B, None, 16, 256, 1, None) == -1
    assert L.lqc_read(FAKE, B, 1024, FAKE, 16, 256, 1, None) == -3          # bytes a multiple of 2048
    assert L.lqc_read(FAKE, B - 1, B, FAKE, 16, 256, 1, None) == -3         # source smaller than bytes
    assert L.lqc_read(FAKE, B, B, FAKE, 15, 256, 1, None) == -3             # sink: 4 bytes per wave
    assert L.lqc_read(FAKE, B, B, FAKE, 16, 256, 0, None) == -3
    assert L.lqc_read(FAKE + 4, B, B, FAKE, 16, 256, 1, None) == -4
    assert L.lqc_write(None, B, B, 256, 1, None) == -1
    assert L.lqc_write(FAKE, B, 1000, 256, 1, None) == -3                   # bytes a multiple of 1024
    assert L.lqc_write(FAKE, B - 1, B, 256, 1, None) == -3                  # destination smaller than bytes
    assert L.lqc_write(FAKE, B, B, 512, 1, None) == -3
    assert L.lqc_write(FAKE + 4, B, B, 256, 1, None) == -4

    def pattern(x_b=B, codes_b=1024, bits=8, scales_b=64, block=16, y_b=B, codes=FAKE, x=FAKE):
        return L.lqc_pattern(x, x_b, 1024, codes, codes_b, bits, FAKE, scales_b, block, FAKE, y_b, 256, 1, None)

    assert pattern(bits=5) == -3
    assert pattern(block=512) == -3
    assert pattern(codes=None) == -1
    assert pattern(x_b=B - 1) == -3
    assert pattern(y_b=B - 1) == -3
    assert pattern(codes_b=1023) == -3                     # 8-bit codes: n bytes
    assert pattern(bits=6, codes_b=767) == -3              # 6-bit codes: 3n/4 bytes
    assert pattern(bits=4, codes_b=511) == -3              # 4-bit codes: n/2 bytes
    assert pattern(scales_b=63) == -3                      # one byte per block of 16
    assert pattern(block=256, scales_b=3) == -3
    assert pattern(bits=6, codes_b=768, x=FAKE + 4) == -4  # sizes right, misaligned


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("lq_quantize", "lq_dequantize", "lq_fake_quant_qsnr", "lq_hadamard_quant"):
        assert n in names
    assert set(names) == set(lq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = lq.load()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_library_exports_nothing_else():
    """Kernels and helpers stay internal: the dynamic symbol table holds the
    declared entry points and the HIP runtime's per-unit ids only."""
    assert _exported(lq.LIB_PATH) == set(declared_functions())


def V(fmt="int8", gran="block", scale="ue8m0", block=32, sym=True, out="bf16", hadamard=0):
    return {"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": sym, "out": out,
            "hadamard": hadamard}


FAKE = 1 << 20  # an aligned, never dereferenced device address


def call_fq(d, rows=4, cols=64, x=FAKE, codes=FAKE, scales=FAKE, zeros=None, y=FAKE, res=FAKE, ws=FAKE,
            ws_bytes=1 << 20):
    L = lq.load()
    return L.lq_fake_quant_qsnr(ctypes.byref(d), x, rows, cols, codes, scales, zeros, y, res, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("format", 9, -2), ("gran", 5, -2), ("scale_fmt", -1, -2), ("rounding", 3, -2), ("in_dtype", 7, -2),
    ("out_dtype", 3, -2), ("hadamard", 8, -2), ("scale_source", 2, -2), ("symmetric", 2, -2),
    ("block", 0, -2), ("block", 48, -7), ("block", 512, -7)])
def test_bad_descriptor_fields(field, value, status):
    d = lq.desc(V(), "bf16")
    setattr(d, field, value)
    assert call_fq(d) == status


def test_undefined_combinations():
    # zero point only for integer formats with fp32/fp16 scales
    assert call_fq(lq.desc(V(fmt="e4m3", scale="f32", sym=False), "bf16")) == -2
    assert call_fq(lq.desc(V(fmt="int8", scale="ue8m0", sym=False), "bf16")) == -2
    assert call_fq(lq.desc(V(fmt="int4", scale="e4m3", sym=False, block=16), "bf16")) == -2
    # fake_quant_qsnr takes no rotation; hadamard_quant needs it
    assert call_fq(lq.desc(V(hadamard=16), "bf16")) == -2
    L = lq.load()
    d = lq.desc(V(), "bf16")
    assert L.lq_hadamard_quant(ctypes.byref(d), FAKE, 4, 64, FAKE, FAKE, None, FAKE, 1, FAKE, FAKE, 1 << 20,
                               None) == -2


def test_shapes():
    d = lq.desc(V(), "bf16")
    assert call_fq(d, rows=-1) == -3
    assert call_fq(d, cols=48) == -3                    # cols % block
    d4 = lq.desc(V(fmt="int4", gran="channel", scale="f32"), "bf16")
    assert call_fq(d4, cols=33) == -3                   # odd cols, 4-bit
    dh = lq.desc(V(fmt="int4", gran="tensor", scale="f32", hadamard=16), "bf16")
    L = lq.load()
    assert L.lq_hadamard_quant(ctypes.byref(dh), FAKE, 4, 40, FAKE, FAKE, None, FAKE, 0, FAKE, FAKE, 1 << 20,
                               None) == -3
    assert call_fq(d, rows=1 << 40, cols=1 << 30) == -3  # size overflow


def test_pointers_alignment_workspace():
    d = lq.desc(V(), "bf16")
    assert call_fq(d, x=None) == -1
    assert call_fq(d, x=FAKE + 2) == -4
    assert call_fq(d, y=FAKE + 8) == -4
    assert call_fq(d, ws=None) == -5
    assert call_fq(d, ws_bytes=16) == -5
    dg = lq.desc(V(), "bf16", given=True)
    assert call_fq(dg, scales=None) == -1
    L = lq.load()
    assert L.lq_quantize(ctypes.byref(d), FAKE, 4, 64, None, FAKE, None, FAKE, 1 << 20, None) == -1
    assert L.lq_dequantize(ctypes.byref(d), None, FAKE, None, 4, 64, FAKE, None) == -1
    da = lq.desc(V(fmt="int8", scale="f16", sym=False), "bf16")
    assert L.lq_dequantize(ctypes.byref(da), FAKE, FAKE, None, 4, 64, FAKE, None) == -1
    assert L.lq_workspace_init(None, 64, None) == -1
    assert L.lq_workspace_init(FAKE + 4, 64, None) == -4
    assert L.lq_fake_quant_qsnr(None, FAKE, 4, 64, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == -1


def test_buffer_sizes():
    d = lq.desc(V(fmt="e2m1", scale="ue8m0", block=32), "bf16")
    # MXFP4: per 32 values 16 code bytes + 1 scale byte = 136 bits
    assert lq.lq_codes_bytes(d, 1, 32) == 16 and lq.lq_scales_bytes(d, 1, 32) == 1
    d = lq.desc(V(fmt="e2m1", scale="e4m3", block=16), "bf16")
    assert (lq.lq_codes_bytes(d, 1, 16) + lq.lq_scales_bytes(d, 1, 16)) * 8 == 72
    d = lq.desc(V(fmt="int4", scale="f16", block=128, sym=False), "bf16")
    assert lq.lq_scales_bytes(d, 11008, 4096) == 11008 * 32 * 2 == lq.lq_zeros_bytes(d, 11008, 4096)
    d = lq.desc(V(fmt="int8", gran="channel", scale="f32"), "bf16")
    assert lq.lq_scales_bytes(d, 7, 100) == 28 and lq.lq_zeros_bytes(d, 7, 100) == 0
    assert lq.lq_workspace_bytes(d, 7, 100) > 0
    bad = lq.desc(V(), "bf16")
    bad.format = 11
    assert lq.lq_codes_bytes(bad, 4, 64) == 0


def test_status_strings():
    for s in range(-7, 1):
        assert lq.status_string(s) and lq.status_string(s) != "unknown status"


def test_sweep_tally_matches_the_oracle():
    """The library's win counts (host code) against the oracle's on random
    tables whose differences crowd both edges of the band, plus infinities
    and NaN; and the argument checks."""
    import oracle

    rng = np.random.default_rng(0)
    base = rng.uniform(10, 40, (40, 5, 5))
    steps = np.array([0.0, 0.005, 0.0079, 0.008, 0.0081, 0.01, 0.0119, 0.012, 0.0121, 0.3])
    q = base.copy()
    q[:, 2:, :] = base[:, :2, :].repeat([2, 1], axis=1) - rng.choice(steps, (40, 3, 5)) * rng.choice([-1, 1], (40, 3, 5))
    q[0, 0, 0], q[0, 2, 0] = np.inf, np.inf
    q[1, 0, 1], q[1, 3, 1] = np.nan, 20.0
    q[2, 1, 2], q[2, 4, 2] = -np.inf, 5.0
    for tie, margin in ((1e-2, 2e-3), (0.25, 0.0625), (1e-3, 0.0)):
        got = lq.lq_sweep_tally(q, tie, margin)
        want = oracle.sweep_tally(q, tie, margin)
        assert np.array_equal(got, want), (tie, margin, got - want)
        assert got.sum() == 40 * 15
    assert lq.lq_sweep_tally(q, 1e-2, 2e-3)[..., 3].sum() > 0      # some pairs are undecided
    L = lq.load()
    buf = np.zeros(60, np.int32)
    qp = np.ascontiguousarray(q).ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    bp = buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.lq_sweep_tally(qp, -1, 0.01, 0.0, bp) == -3
    assert L.lq_sweep_tally(None, 2, 0.01, 0.0, bp) == -1
    assert L.lq_sweep_tally(qp, 2, 0.01, 0.01, bp) == -2        # margin must be below the band
    assert L.lq_sweep_tally(qp, 2, 0.01, -1.0, bp) == -2
    assert L.lq_sweep_tally(qp, 2, float("nan"), 0.0, bp) == -2


def test_grid_limit_rejects_negative():
    L = lq.load()
    assert L.lq_set_grid_limit(-1) == -3          # LQ_ERR_SHAPE
    assert L.lq_set_grid_limit(0) == 0


def test_bench_pattern_buffers_cover_the_pattern():
    """The ceiling's pattern writes into buffers sized from the pattern's own
    shape: as many code bytes as a call of the variant when its scales are
    per block, never fewer than lqc_pattern checks for."""
    import bench

    for cfg, spec in W.WORKLOADS.items():
        if cfg == "c5":
            continue
        rows, cols = spec["shape"]
        n = rows * cols
        for v in spec["variants"]():
            bits, block = bench.pattern_shape(v)
            nb = bench.pattern_buffer_bytes(n, bits, block)
            assert bits in (4, 6, 8) and block in (16, 32, 64, 128, 256), (cfg, v)
            assert nb == {"codes": n // 8 * bits, "scales": n // block, "y": 2 * n}
            d = lq.desc(v, spec["dtype"], signs_ptr=64 if v.get("signs") is not None else None)
            if v["gran"] == "block" and spec["dtype"] == "bf16":
                assert nb["codes"] == lq.load().lq_codes_bytes(d, rows, cols), (cfg, v)

