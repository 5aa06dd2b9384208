"""GPU parity of per-tensor scaling from the data (the statistic pass, then
the quantizing kernel) against the oracle: every element format, symmetric
and zero-point scales, input and output dtypes, tails, grids on both sides of
the general kernel's in-kernel QSNR finish, special values."""
import math

import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import as_f16, check_variant, run_gpu, upload

pytestmark = pytest.mark.gpu


def V(fmt, scale, sym=True, out="f32", rnd="rne"):
    return {"fmt": fmt, "gran": "tensor", "block": 0, "scale": scale, "sym": sym, "round": rnd,
            "out": out, "hadamard": 0, "unrotate": False}


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 15), (3, 7), (37, 1000), (1024, 1024)])
def test_every_format_and_tail(rows, cols):
    d = W.c1_input(rows=rows, cols=cols)
    xdev = upload(d)
    for fmt in ("int8", "int4", "e4m3", "e5m2", "e2m1", "e2m3", "e3m2"):
        if fmt in ("e2m3", "e3m2") and cols % 4:
            continue
        if fmt in ("int4", "e2m1") and cols % 2:
            continue
        for scale in ("f32", "ue8m0"):
            check_variant(V(fmt, scale), d, f"per-tensor {fmt} {scale} {rows}x{cols}", xdev)


@pytest.mark.parametrize("fmt", ["int8", "int4"])
@pytest.mark.parametrize("scale", ["f32", "f16"])
def test_zero_point_and_rounding(fmt, scale):
    d = W.c1_input(rows=37, cols=1000)
    xdev = upload(d)
    for rnd in ("rne", "rna"):
        check_variant(V(fmt, scale, sym=False, rnd=rnd), d, f"per-tensor asym {fmt} {scale} {rnd}", xdev)


@pytest.mark.parametrize("src,out", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16")])
def test_input_and_output_dtypes(src, out):
    d = W.c2_input(rows=40, cols=1000)
    if src == "f16":
        d = as_f16(d)
    xdev = upload(d)
    for fmt, scale in (("int8", "f32"), ("e4m3", "e4m3"), ("e2m1", "f16")):
        check_variant(V(fmt, scale, out=out), d, f"per-tensor {src}->{out} {fmt}", xdev)


@pytest.mark.parametrize("cols", [4096, 4112])
def test_finish_in_kernel_and_after(cols):
    """1024 x 4096 fp32 is 1024 workgroups of the general kernel, the most
    whose last workgroup writes the QSNR; 4112 columns need 1028 and the
    finishing kernel."""
    d = W.c1_input(rows=1024, cols=cols)
    xdev = upload(d)
    for v in (V("int8", "f32"), V("e4m3", "f32", out="bf16"), V("int4", "f16", sym=False)):
        check_variant(v, d, f"per-tensor 1024x{cols}", xdev)


def test_special_values_and_repeatable():
    """Zeros, a tensor of zeros (zero scale), subnormals and huge values
    against the oracle; non-finite inputs counted with the QSNR NaN as the
    oracle's (their codes are unspecified); thirty calls in a row give the
    same QSNR bit for bit."""
    x = W.c1_input(rows=64, cols=512)["x"].copy()
    x[0] = 0.0
    x[1, :7] = np.float32(1e-40)
    x[2, 3] = np.float32(3e38)
    for arr, name in ((x, "special"), (np.zeros_like(x), "zeros")):
        dd = W._pack("f32", arr)
        xdev = upload(dd)
        for v in (V("int8", "f32"), V("e4m3", "ue8m0"), V("int4", "f32", sym=False)):
            check_variant(v, dd, f"per-tensor {name}", xdev)
    xn = x.copy()
    xn[5, 5] = np.inf
    xn[6, 6] = np.nan
    dn = W._pack("f32", xn)
    for v in (V("int8", "f32"), V("e4m3", "ue8m0")):
        gpu, _ = run_gpu(v, dn)
        ref = oracle.fake_quant(v, dn["x"])
        assert gpu["nonfinite"] == 2, v
        assert math.isnan(ref["qsnr"]) and math.isnan(gpu["qsnr"]), (v, gpu["qsnr"], ref["qsnr"])
    dd = W._pack("f32", x)
    xdev = upload(dd)
    v = V("e4m3", "f32")
    r = lq.Runner(v, 64, 512, "f32")
    ref = oracle.fake_quant(v, x)["qsnr"]
    seen = set()
    for _ in range(30):
        r.fake_quant(xdev)
        seen.add(r.result()["qsnr"])
    assert len(seen) == 1 and abs(seen.pop() - ref) <= 1e-3
