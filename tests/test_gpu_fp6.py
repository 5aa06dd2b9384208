"""GPU parity of the FP6 element formats E2M3 (±7.5) and E3M2 (±28)
(walkerchi.com quantization playbook §4.1 table, MXFP6) against the oracle,
bit-exact: 6-bit codes packed 16 elements to 12 bytes, every scale format and
granularity, ragged tails (a multiple of 4 elements), input and output dtypes,
the specialised per-block kernel over several passes, rotation, two-level
scaling, special values, dequantization, and the c7 workload at full size."""
import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import as_f16, check_variant, run_gpu, say, upload

pytestmark = pytest.mark.gpu

FP6 = ("e2m3", "e3m2")


def V(fmt, gran, scale, block=0, out="bf16", rnd="rne", **kw):
    return dict({"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": True, "round": rnd,
                 "out": out, "hadamard": 0, "unrotate": False}, **kw)


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("scale", ["f32", "f16", "ue8m0", "e4m3"])
def test_fp6_granularities(fmt, scale):
    d = W.c2_input(rows=37, cols=1024, seed=51)
    xdev = upload(d)
    for gran, block, extra in (("block", 16, {}), ("block", 32, {}), ("block", 256, {}), ("tensor", 0, {}),
                               ("channel", 0, {}), ("tile", 128, {"tile_rows": 8})):
        check_variant(V(fmt, gran, scale, block, **extra), d, f"fp6 {gran}{block}", xdev)


@pytest.mark.parametrize("rows,cols", [(3, 36), (5, 100), (1, 4), (7, 1020)])
def test_fp6_ragged_shapes(rows, cols):
    d = W.c1_input(rows=rows, cols=cols)
    for fmt in FP6:
        for v in (V(fmt, "tensor", "f32", out="f32"), V(fmt, "channel", "ue8m0", out="bf16"),
                  V(fmt, "channel", "f16", out="f16")):
            check_variant(v, d, f"fp6 ragged {rows}x{cols}")


@pytest.mark.parametrize("limit", [0, 4, 64])
def test_fp6_fast_path_passes_and_extremes(limit):
    from tests.test_gpu_parity import _extremes_bf16

    try:
        lq.lq_set_grid_limit(limit)
        for rows, cols in ((64, 4096), (63, 3968)):
            d = _extremes_bf16(rows, cols)
            xdev = upload(d)
            for fmt in FP6:
                for scale, block in (("ue8m0", 32), ("e4m3", 16), ("f32", 32), ("f16", 64)):
                    check_variant(V(fmt, "block", scale, block), d, f"fp6 fast limit={limit}", xdev)
    finally:
        lq.lq_set_grid_limit(0)


@pytest.mark.parametrize("src", ["f32", "f16"])
def test_fp6_input_dtypes_rounding_rotation_two_level(src):
    base = W.c4_input(rows=8, cols=1024, seed=52)
    d = as_f16(base) if src == "f16" else {"dtype": "f32", "bits": base["x"].view(np.uint32), "x": base["x"]}
    xdev = upload(d)
    for fmt in FP6:
        for out in ("f32", "bf16", "f16"):
            check_variant(V(fmt, "block", "ue8m0", 32, out=out), d, f"fp6 in-{src}", xdev)
        check_variant(V(fmt, "block", "ue8m0", 32, hadamard=64, unrotate=True), d, f"fp6 h64 in-{src}", xdev)
        check_variant(V(fmt, "block", "e4m3", 16, two_level=True), d, f"fp6 two-level in-{src}", xdev)
    dbf = W.c4_input(rows=8, cols=1024, seed=52)
    xb = upload(dbf)
    for fmt in FP6:
        check_variant(V(fmt, "block", "ue8m0", 32, hadamard=16, unrotate=True), dbf, "fp6 h16 bf16", xb)
        check_variant(V(fmt, "block", "e4m3", 16, two_level=True), dbf, "fp6 two-level bf16", xb)


def test_fp6_special_values_and_dequantize():
    d = W.special_values_input(rows=6, cols=512)
    d["x"][2, 64:96] = 0.0
    d["x"][3, 0:32] = np.float32(1e-30)
    d["bits"] = d["x"].view(np.uint32)
    xdev = upload(d)
    for fmt in FP6:
        for scale in ("f32", "f16", "ue8m0", "e4m3"):
            check_variant(V(fmt, "block", scale, 32, out="f32"), d, "fp6 special", xdev)
    rows, cols = 24, 2048
    d = W.c3_input(rows=rows, cols=cols)
    xdev = upload(d)
    for fmt in FP6:
        v = V(fmt, "block", "ue8m0", 32)
        ref = oracle.fake_quant(v, d["x"])
        r = lq.Runner(v, rows, cols, "bf16", want=("codes", "scales", "y"))
        r.quantize(xdev)
        h = r.host()
        assert np.array_equal(h["codes"], ref["codes"]) and np.array_equal(h["scales"], ref["scales"]), fmt
        r.y.zero_()
        r.dequantize()
        assert np.array_equal(r.host()["y"], ref["y"]), fmt


@pytest.mark.parametrize("i", [0, 1])
def test_full_size_c7(i):
    """C2's tensor as MXFP6 (E2M3, E3M2) at full size, whole tensor."""
    from tests.gpu_helpers import full_size

    full_size("c7", i)

def test_fp6_under_1024_column_rotation():
    """FP6 under a signed 1024-column rotation: block scales (general kernel)
    and two-level scaling (the specialised kernel's 1024-column build)."""
    from tests.test_gpu_rotation import R, signs_for

    d = W.c4_input(rows=12, cols=2048, seed=53)
    xdev = upload(d)
    sg = signs_for(2048, 54)
    for fmt in FP6:
        for v in (V(fmt, "block", "ue8m0", 32), V(fmt, "block", "e4m3", 16, two_level=True)):
            check_variant(R(v, 1024, sg), d, f"fp6 {fmt} rot1024", xdev)
