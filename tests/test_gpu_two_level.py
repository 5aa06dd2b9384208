"""GPU parity of two-level scaling (an FP32 tensor scale S above E4M3 block
scales, walkerchi.com quantization playbook §4.3.1-§4.3.2) against the
oracle: codes, block scales, S and dequantized outputs bit-exact, QSNR within
1e-3 dB, on every kernel that takes it (lane-contiguous bf16, tile-per-lane
with and without rotation, fp32 input, the general kernel), at several grid
caps, with tensors whose S needs the pre-scaled division, given scales, and
dequantization."""
import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import as_f16, check_variant, compare, run_gpu, say, split_two_level, upload

pytestmark = pytest.mark.gpu

FMTS = ("int8", "int4", "e4m3", "e5m2", "e2m1")


def TL(fmt, block=16, out="bf16", hadamard=0, unrotate=False, rnd="rne"):
    return {"fmt": fmt, "gran": "block", "block": block, "scale": "e4m3", "sym": True, "round": rnd,
            "out": out, "hadamard": hadamard, "unrotate": unrotate, "two_level": True}


def _scaled(d: dict, factor: float) -> dict:
    """The same bf16 tensor times a power of two (exact)."""
    x = (d["x"] * np.float32(factor)).astype(np.float32)
    bits, xv = W.to_bf16(x)
    return {"dtype": "bf16", "bits": bits, "x": xv}


def test_c4t_small():
    d = W.c4_input(rows=24, cols=8192)
    xdev = upload(d)
    for v in W.c4t_variants():
        check_variant(v, d, "c4t-small", xdev)
        check_variant(dict(v, unrotate=False), d, "c4t-small-rotated-y", xdev)


@pytest.mark.parametrize("limit", [0, 4, 64])
@pytest.mark.parametrize("block", [16, 32, 64, 128, 256])
def test_every_format_block_and_grid(limit, block):
    """Lane-contiguous (64x4096) and tile-per-lane (63x3840) shapes, with and
    without the rotation, the grid capped so that threads run several
    iterations; limit 4 on the larger tensor exceeds the iterations the
    specialised kernels record and takes the general kernel."""
    shapes = [(64, 4096), (63, 3840)] + ([(128, 8192)] if limit == 4 else [])
    try:
        lq.lq_set_grid_limit(limit)
        for rows, cols in shapes:
            d = W.c4_input(rows=rows, cols=cols, seed=11)
            xdev = upload(d)
            for f in FMTS:
                check_variant(TL(f, block), d, f"two-level limit={limit} {rows}x{cols}", xdev)
            for f in ("int4", "e2m1"):
                check_variant(TL(f, block, hadamard=16, unrotate=True), d, f"two-level h16 limit={limit}", xdev)
    finally:
        lq.lq_set_grid_limit(0)


@pytest.mark.parametrize("k", [-126, -60, -20, 0, 20, 60, 120])
def test_tensor_magnitudes(k):
    """x * 2^k, from tensors whose S is so small that 1/S overflows fp32 (the
    pre-scaled division; 2^-126, much of it bf16 subnormals) to ones near the
    top of the range. The rotation runs only up to 2^60: sums of 16 values
    near FLT_MAX overflow in the rotation itself."""
    base = W.c4_input(rows=32, cols=4096, seed=12)
    d = _scaled(base, 2.0 ** k)
    xdev = upload(d)
    for f in FMTS:
        check_variant(TL(f), d, f"magnitude 2^{k}", xdev)
        if abs(k) <= 60:
            check_variant(TL(f, hadamard=16, unrotate=True), d, f"magnitude 2^{k} h16", xdev)


def test_zero_tiny_and_special_tensors():
    """All-zero tensor (S = 1), a tensor of bf16 subnormals only, and blocks of
    zeros, tiny and huge values inside an ordinary tensor."""
    rows, cols = 16, 2048
    cases = {"zero": np.zeros((rows, cols), np.float32),
             "subnormal": np.full((rows, cols), 1e-40, np.float32) * (1 + np.arange(cols, dtype=np.float32) % 7)}
    x = W.c4_input(rows=rows, cols=cols, seed=13)["x"].copy()
    x[1, 0:64] = 0.0
    x[2, 64:128] = np.float32(1e-30)
    x[3, 128:192] = np.float32(3e35) * np.cos(np.arange(64, dtype=np.float32))
    x[4, 7] = -np.float32(3e36)
    cases["mixed"] = x
    for name, x in cases.items():
        bits, xv = W.to_bf16(x)
        d = {"dtype": "bf16", "bits": bits, "x": xv}
        xdev = upload(d)
        for f in FMTS:
            for out in ("bf16", "f32"):
                check_variant(TL(f, out=out), d, f"special {name}", xdev)
            check_variant(TL(f, hadamard=16), d, f"special {name} h16", xdev)


@pytest.mark.parametrize("src", ["f32", "f16"])
def test_input_dtypes_and_general_kernel(src):
    base = W.c4_input(rows=8, cols=1024, seed=14)
    d = as_f16(base) if src == "f16" else {"dtype": "f32", "bits": base["x"].view(np.uint32), "x": base["x"]}
    xdev = upload(d)
    for f in FMTS:
        for out in ("f32", "bf16"):
            check_variant(TL(f, 32, out=out), d, f"two-level in-{src}", xdev)
            check_variant(TL(f, 32, out=out, rnd="rna"), d, f"two-level in-{src} rna", xdev)
        check_variant(TL(f, 16, hadamard=16, unrotate=True), d, f"two-level in-{src} h16", xdev)


def test_ragged_and_partial_outputs():
    """A tensor that is no multiple of 1024 elements nor of a wave's tiles, and
    calls that skip outputs (the general kernel)."""
    d = W.c4_input(rows=7, cols=48 * 16, seed=15)
    xdev = upload(d)
    for f in FMTS:
        check_variant(TL(f), d, "two-level ragged", xdev)
    v = TL("e2m1")
    ref = oracle.fake_quant(v, d["x"])
    gpu, _ = run_gpu(v, d, xdev=xdev, want=("codes", "scales", "res"))
    compare(v, gpu, ref, what=("codes", "scales"), label="two-level no y")
    gpu, _ = run_gpu(v, d, xdev=xdev, want=("y", "res"))
    compare(v, gpu, ref, what=("y",), label="two-level y only")


def test_given_scales_and_dequantize():
    import torch

    rows, cols = 16, 1024
    d = W.c4_input(rows=rows, cols=cols, seed=16)
    xdev = upload(d)
    for v in (TL("e2m1"), TL("int4", 32), TL("e4m3", 64, out="f32"), TL("int4", hadamard=16, unrotate=True)):
        ref = oracle.fake_quant(v, d["x"])
        # given block scales and S (placed as the library lays them out)
        r = lq.Runner(v, rows, cols, "bf16", given=True)
        nb = ref["scales"].size
        off = (nb + 15) // 16 * 16
        buf = np.zeros(off + 4, np.uint8)
        buf[:nb] = ref["scales"]
        buf[off:off + 4] = np.float32(ref["tscale"]).reshape(1).view(np.uint8)
        r.scales[:buf.size].copy_(torch.from_numpy(buf))
        r.fake_quant(xdev)
        got = r.host()
        got.update(r.result())
        compare(v, got, ref, what=("codes", "y"), label="two-level given")
        # quantize (dynamic), then dequantize from the stored codes, block scales and S
        q = lq.Runner(v, rows, cols, "bf16", want=("codes", "scales", "y"))
        q.quantize(xdev)
        h = q.host()
        compare(v, h, ref, what=("codes", "scales"), qsnr=False, label="two-level quantize")
        q.y.zero_()
        q.dequantize()
        ref_y = oracle.fake_quant(dict(v, unrotate=True), d["x"])["y"] if v["hadamard"] else ref["y"]
        assert np.array_equal(q.host()["y"], ref_y), v
        _, S = split_two_level(h["scales"], nb)
        y2 = oracle.dequant(dict(v, unrotate=bool(v["hadamard"])), ref["codes"], ref["scales"], None, rows, cols,
                            tscale=S)
        assert np.array_equal(y2, ref_y), v


def test_rejects_undefined_combinations():
    import torch

    x = torch.zeros(64 * 16, dtype=torch.uint8, device="cuda")
    for v in (dict(TL("e2m1"), scale="ue8m0"), dict(TL("int4"), gran="channel"),
              dict(TL("int4"), scale="f16", sym=False)):
        with pytest.raises(lq.LQError):
            lq.Runner(v, 8, 64, "bf16").fake_quant(x)


@pytest.mark.parametrize("i", range(4))
def test_full_size_c4t(i):
    """C4 with two-level scaling at full size, whole tensor (the tensor scale too)."""
    from tests.gpu_helpers import full_size

    full_size("c4t", i)
