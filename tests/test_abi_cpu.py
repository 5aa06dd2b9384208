"""CPU checks of the boundary: liblq.so loads, exports every function that
include/lq.h declares, and rejects bad arguments before touching the GPU
(every failing check returns before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_quantization_block_amd import lq

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lq.h")


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lq_[a-z_0-9]+)\s*\(", text)))


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
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", lq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    syms = {s for s in syms if not s.startswith("__hip_cuid_") and s not in ("_init", "_fini")}
    assert syms == set(declared_functions())


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


def test_sweep_tally():
    rng = np.random.default_rng(0)
    q = rng.uniform(10, 40, (7, 5, 5))
    q[0, 0, 0] = q[0, 2, 0] + 1e-4                      # a tie (within 1e-3 dB)
    w = lq.lq_sweep_tally(q, 1e-3)
    assert w.sum() == 7 * 5 * 3
    pairs = ((0, 2), (0, 3), (1, 4))
    for g in range(5):
        for p, (i, f) in enumerate(pairs):
            d = q[:, i, g] - q[:, f, g]
            tie = np.abs(d) < 1e-3
            assert w[g, p, 2] == tie.sum()
            assert w[g, p, 0] == ((d > 0) & ~tie).sum()
            assert w[g, p, 1] == ((d < 0) & ~tie).sum()


def test_grid_limit_rejects_negative():
    L = lq.load()
    assert L.lq_set_grid_limit(-1) == -3          # LQ_ERR_SHAPE
    assert L.lq_set_grid_limit(0) == 0
