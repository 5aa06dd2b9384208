"""GPU parity of the n-point randomized Hadamard rotation (walkerchi.com
quantization playbook §5.3, QuaRot: R = H_n D / sqrt(n) per aligned group of
n columns, D random signs; cyqw.cn/news/1000169 §4.2, §7.2) against the
oracle, bit-exact: groups of 16..1024 columns spread over 1..64 lanes, with
and without signs, on every kernel that rotates (per-block specialised and
general, per-tensor with its rotated statistic, per-channel, 2-D tiles,
two-level, fp32 and fp16 inputs), outputs in either domain, dequantization,
grid caps that give several loop passes, and the argument checks."""
import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import as_f16, check_variant, upload

pytestmark = pytest.mark.gpu

SIZES = (16, 32, 64, 128, 256, 512, 1024)


def signs_for(cols, seed):
    bits = np.random.default_rng(seed).integers(0, 2, cols).astype(np.uint64)
    words = np.zeros((cols + 31) // 32, np.uint64)
    for j in range(cols):
        words[j // 32] |= bits[j] << np.uint64(j % 32)
    return words.astype(np.uint32)


def R(v, n, signs, unrotate=True):
    return dict(v, hadamard=n, unrotate=unrotate, signs=signs)


def V(fmt, gran, scale, block=0, sym=True, out="bf16", rnd="rne", **kw):
    return dict({"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": sym, "round": rnd, "out": out},
                **kw)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("signed", [False, True])
def test_block_variants_rotated(n, signed):
    d = W.c4_input(rows=24, cols=2048, seed=41)
    xdev = upload(d)
    sg = signs_for(2048, n) if signed else None
    for v in (V("int4", "block", "e4m3", block=16), V("e2m1", "block", "e4m3", block=16),
              V("int8", "block", "ue8m0", block=32), V("e4m3", "block", "ue8m0", block=32),
              V("int4", "block", "f16", block=64, sym=False), V("e5m2", "block", "f32", block=128)):
        for un in (False, True):
            check_variant(R(v, n, sg, un), d, f"rot{n} signed={signed}", xdev)


@pytest.mark.parametrize("n", SIZES)
def test_tensor_channel_tile_and_two_level_rotated(n):
    d = W.c2_input(rows=40, cols=1024, seed=42)
    xdev = upload(d)
    sg = signs_for(1024, 7 * n)
    # tiles are at most 256 columns wide, so they take rotations up to 256
    # (a narrower tile than its rotation is LQ_ERR_UNSUPPORTED)
    tiles = (V("e4m3", "tile", "f32", block=256, tile_rows=16),
             V("int4", "tile", "e4m3", block=256, tile_rows=3)) if n <= 256 else ()
    for v in (V("int8", "tensor", "f32"), V("e4m3", "tensor", "f32", out="f32"),
              V("int4", "channel", "f32"), V("int8", "channel", "f16", sym=False), *tiles,
              V("e2m1", "block", "e4m3", block=16, two_level=True), V("int4", "block", "e4m3", block=16, two_level=True)):
        check_variant(R(v, n, sg), d, f"rot{n}", xdev)


@pytest.mark.parametrize("limit", [0, 3, 64])
def test_rotation_over_several_passes(limit):
    d = W.c4_input(rows=64, cols=4096, seed=43)
    xdev = upload(d)
    sg = signs_for(4096, 44)
    try:
        lq.lq_set_grid_limit(limit)
        for n in (32, 256, 1024):
            for v in (V("int4", "block", "e4m3", block=16), V("int8", "tensor", "f32"),
                      V("e2m1", "block", "e4m3", block=16, two_level=True)):
                check_variant(R(v, n, sg), d, f"rot{n} limit={limit}", xdev)
    finally:
        lq.lq_set_grid_limit(0)


@pytest.mark.parametrize("limit", [100, 40])
def test_signed_rotation_grid_columns(limit):
    """Signed rotations over several passes on 11008 = 43 x 256 columns. The
    specialised kernel reads each lane's sign bits once, so its grid stride
    must be a multiple of cols: under a limit of 100 workgroups the grid is 86
    (a multiple of 43); under 40 there is no such grid and the call takes the
    general kernel. Both against the oracle. (Zero points under a rotation
    always take the general kernel.)"""
    rows, cols = 48, 11008
    d = W.c3_input(rows=rows, cols=cols, seed=45)
    xdev = upload(d)
    sg = signs_for(cols, 46)
    try:
        lq.lq_set_grid_limit(limit)
        for n in (16, 256):
            for v in (V("int4", "block", "e4m3", block=16), V("e2m1", "block", "e4m3", block=16),
                      V("int8", "block", "ue8m0", block=32), V("int4", "block", "f16", block=64, sym=False)):
                ks = lq.call_kernels(R(v, n, sg), "bf16", rows, cols)
                fast = limit == 100 and v["sym"]
                assert ks[0].startswith("void lqd::k_fast<" if fast else "void lqd::k_flat<"), ks
                check_variant(R(v, n, sg), d, f"rot{n} signed limit={limit}", xdev)
    finally:
        lq.lq_set_grid_limit(0)


@pytest.mark.parametrize("src", ["f32", "f16"])
def test_rotation_input_dtypes(src):
    base = W.c4_input(rows=8, cols=1024, seed=45)
    d = as_f16(base) if src == "f16" else {"dtype": "f32", "bits": base["x"].view(np.uint32), "x": base["x"]}
    xdev = upload(d)
    sg = signs_for(1024, 46)
    for n in (64, 256, 1024):
        for v in (V("int4", "block", "e4m3", block=16), V("int8", "block", "ue8m0", block=32),
                  V("e4m3", "block", "f32", block=32, rnd="rna", out="bf16")):
            check_variant(R(v, n, sg), d, f"rot{n} in-{src}", xdev)


def test_rotated_quantize_then_dequantize():
    rows, cols = 16, 1024
    d = W.c4_input(rows=rows, cols=cols, seed=47)
    xdev = upload(d)
    sg = signs_for(cols, 48)
    for n in SIZES:
        for v in (V("e2m1", "block", "e4m3", block=16), V("int8", "channel", "f32")):
            v = R(v, n, sg)
            ref = oracle.fake_quant(v, d["x"])
            r = lq.Runner(v, rows, cols, "bf16", want=("codes", "scales", "zeros", "y"))
            r.quantize(xdev)
            h = r.host()
            assert np.array_equal(h["codes"], ref["codes"]), (n, v)
            r.y.zero_()
            r.dequantize()
            assert np.array_equal(r.host()["y"], ref["y"]), (n, v)


def test_rotation_argument_checks():
    """Sizes other than the powers of two 16..1024 are undefined (LQ_ERR_BAD_DESC); a tile
    narrower than its rotation groups is defined but not built
    (LQ_ERR_UNSUPPORTED); columns not a multiple of n (LQ_ERR_SHAPE)."""
    import torch

    ok = R(V("e4m3", "tile", "f32", block=256, tile_rows=4), 16, None)
    r = lq.Runner(ok, 8, 512, "bf16")
    x = torch.zeros(8 * 512 * 2, dtype=torch.uint8, device="cuda")
    for change, cols, code in ((dict(hadamard=48), 512, -2), (dict(hadamard=2048), 512, -2),
                               (dict(hadamard=512), 512, -7),
                               (dict(block=64, hadamard=128), 512, -7), (dict(hadamard=256), 384, -3)):
        d = lq.desc(dict(ok, **change), "bf16")
        with pytest.raises(lq.LQError) as e:
            lq.lq_hadamard_quant(d, x, 8, cols, r.codes, r.scales, r.zeros, r.y, 1, r.res, r.ws, r.ws_bytes)
        assert e.value.status == code, (change, e.value.status)


@pytest.mark.parametrize("name", ["c4r", "c4q"])
@pytest.mark.parametrize("i", [0, 1])
def test_full_size_c4r(name, i):
    """C4's tensor under 256- and 1024-column signed rotations at full size,
    whole tensor."""
    from tests.gpu_helpers import full_size

    full_size(name, i)

@pytest.mark.parametrize("n", [16, 256, 1024])
def test_given_scales_under_rotation(n):
    """Scales (and zero points) given by the caller, quantizing the rotated
    values: the codes and outputs of the oracle fed the same scales."""
    from tests.gpu_helpers import compare, run_gpu

    d = W.c4_input(rows=16, cols=2048, seed=49)
    xdev = upload(d)
    sg = signs_for(2048, 50 + n)
    for v in (V("int4", "block", "e4m3", block=16), V("int4", "block", "f16", block=64, sym=False),
              V("e4m3", "channel", "f32"), V("int8", "tensor", "f32")):
        v = R(v, n, sg)
        ref = oracle.fake_quant(v, d["x"])
        gpu, _ = run_gpu(v, d, xdev=xdev, given=(ref["scales"], ref["zeros"]))
        compare(v, gpu, ref, what=("codes", "y"), label=f"given rot{n}")
