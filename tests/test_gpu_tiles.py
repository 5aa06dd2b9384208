"""GPU parity of 2-D tile scaling (walkerchi.com quantization playbook §4.4,
DeepSeek-V3: 1x128 activation tiles, 128x128 weight tiles) against the
oracle: codes, scales, zero points and outputs bit-exact, QSNR within
1e-3 dB. Tiles held in registers (1, 2 or 4 units of 16 per lane) and read
twice (larger tiles), ragged last bands, every format and scale format,
zero points, rotation, input and output dtypes, given scales, dequantization,
and the c6 workload at full size on sampled bands."""
import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import as_f16, check_variant, compare, run_gpu, say, upload

pytestmark = pytest.mark.gpu


def T(fmt, scale, block, tile_rows, sym=True, out="bf16", rnd="rne", hadamard=0, unrotate=False):
    return {"fmt": fmt, "gran": "tile", "block": block, "tile_rows": tile_rows, "scale": scale, "sym": sym,
            "round": rnd, "out": out, "hadamard": hadamard, "unrotate": unrotate}


# (tile_rows, block): units of 16 per lane 1, 1, 2, 4 (128x128), 16 (read twice), and
# one-row tiles (the per-block kernels)
SHAPES = [(3, 32), (16, 256), (32, 128), (128, 128), (256, 256), (1, 128)]


@pytest.mark.parametrize("tile_rows,block", SHAPES)
def test_tile_shapes_formats_and_scales(tile_rows, block):
    d = W.c3_input(rows=300, cols=512, seed=31)           # 300 rows: a short last band for every shape
    xdev = upload(d)
    for fmt in ("int8", "int4", "e4m3", "e5m2", "e2m1"):
        for scale in ("f32", "f16", "ue8m0", "e4m3"):
            check_variant(T(fmt, scale, block, tile_rows), d, f"tile {tile_rows}x{block}", xdev)


@pytest.mark.parametrize("tile_rows,block", [(4, 64), (128, 128), (64, 256)])
def test_tile_zero_points_rounding_and_rotation(tile_rows, block):
    d = W.c4_input(rows=200, cols=512, seed=32)
    xdev = upload(d)
    for fmt in ("int8", "int4"):
        for scale in ("f32", "f16"):
            for rnd in ("rne", "rna"):
                check_variant(T(fmt, scale, block, tile_rows, sym=False, rnd=rnd), d, "tile asym", xdev)
    for fmt, scale in (("e4m3", "f32"), ("int4", "e4m3"), ("e2m1", "ue8m0")):
        for un in (False, True):
            check_variant(T(fmt, scale, block, tile_rows, hadamard=16, unrotate=un), d, "tile h16", xdev)


@pytest.mark.parametrize("src", ["f32", "f16"])
def test_tile_dtypes(src):
    base = W.c3_input(rows=130, cols=256, seed=33)
    d = as_f16(base) if src == "f16" else {"dtype": "f32", "bits": base["x"].view(np.uint32), "x": base["x"]}
    xdev = upload(d)
    for out in ("f32", "bf16", "f16"):
        check_variant(T("e4m3", "f32", 128, 128, out=out), d, f"tile in-{src}", xdev)
        check_variant(T("int8", "f16", 64, 8, out=out), d, f"tile in-{src}", xdev)


def test_tile_special_values_and_grid_cap():
    d = W.special_values_input(rows=40, cols=512)
    d["x"][0:8, 0:128] = 0.0                               # an all-zero tile
    d["x"][8:16, 128:256] = np.float32(1e-30)              # a tile whose fp16 / E4M3 scale underflows
    d["bits"] = d["x"].view(np.uint32)
    xdev = upload(d)
    try:
        for limit in (0, 3):                               # 3: every workgroup takes several tiles
            lq.lq_set_grid_limit(limit)
            for fmt in ("int8", "e4m3", "e2m1"):
                for scale in ("f32", "f16", "e4m3"):
                    check_variant(T(fmt, scale, 128, 8, out="f32"), d, f"tile special limit={limit}", xdev)
    finally:
        lq.lq_set_grid_limit(0)


def test_tile_given_scales_and_dequantize():
    rows, cols = 260, 256
    d = W.c3_input(rows=rows, cols=cols, seed=34)
    xdev = upload(d)
    for v in (T("e4m3", "f32", 128, 128), T("int4", "f16", 64, 4, sym=False), T("e2m1", "e4m3", 16, 3),
              T("int8", "ue8m0", 128, 1), T("e4m3", "f32", 128, 32, hadamard=16, unrotate=True)):
        ref = oracle.fake_quant(v, d["x"])
        gpu, _ = run_gpu(v, d, xdev=xdev, given=(ref["scales"], ref["zeros"]))
        compare(v, gpu, ref, what=("codes", "y"), label="tile given")
        r = lq.Runner(v, rows, cols, "bf16", want=("codes", "scales", "zeros", "y"))
        r.quantize(xdev)
        compare(v, r.host(), ref, what=("codes", "scales", "zeros"), qsnr=False, label="tile quantize")
        r.y.zero_()
        r.dequantize()
        ref_y = oracle.fake_quant(dict(v, unrotate=True), d["x"])["y"] if v["hadamard"] else ref["y"]
        assert np.array_equal(r.host()["y"], ref_y), v


@pytest.mark.parametrize("i", [0, 1])
def test_full_size_c6(i):
    """C3's weights under 128x128 and 1x128 E4M3 tiles at full size, whole tensor."""
    from tests.gpu_helpers import full_size

    full_size("c6", i)

