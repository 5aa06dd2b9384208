"""Pins for the oracle's quantizer: an independent brute-force model on tiny
tensors, the pages' own INT4 group example run in torch, the AbsMax formula in
torch, invariants (power-of-two scaling, zero-point, rotation), the pages'
closed form for QSNR, the qualitative orderings the pages report, and the
storage sizes they print."""
import itertools
import math
import zlib

import numpy as np
import pytest
import scipy.linalg
import torch

from bit_quantization_block_amd import workloads as W
from tests import bruteforce as bf


def V(fmt, gran, scale, block=0, sym=True, out="bf16", rnd="rne", hadamard=0, unrotate=False):
    return {"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": sym, "round": rnd,
            "out": out, "hadamard": hadamard, "unrotate": unrotate}


def scale_bits(o, arr):
    return [int(v) for v in np.asarray(arr).reshape(-1)]


def check_against_bruteforce(o, v, x):
    rows, cols = x.shape
    got = o.fake_quant(v, x)
    ref = bf.fake_quant(v, x)
    codes = bf.unpack_codes(v["fmt"], got["codes"], rows, cols)
    assert np.array_equal(codes, ref["codes"]), (v, np.argwhere(codes != ref["codes"])[:5])
    assert scale_bits(o, got["scales"]) == ref["sbits"], v
    if not v["sym"]:
        assert scale_bits(o, got["zeros"]) == ref["zbits"], v
    assert np.array_equal(got["xhat"].view(np.uint32), ref["xhat"].view(np.uint32)), v
    assert np.array_equal(got["y"], ref["y"]), v
    assert math.isclose(got["err2"], ref["err2"], rel_tol=1e-12, abs_tol=1e-300), v
    assert math.isclose(got["sig2"], ref["sig2"], rel_tol=1e-12), v


def tiny_input(seed, rows=3, cols=64, special=True):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 2.0 ** rng.uniform(-6, 6, (rows, 1))).astype(np.float32)
    if special:
        x[0, :16] = np.float32([0.0, -0.0, 1e-45, -3e-41, 0.5, -0.5, 1.5, 2.5, -3.5, 7.49, -7.5, 100.0,
                                -100.0, 2.0 ** -20, 3.0, -0.25])
        x[1, 16:32] = 0.0  # an all-zero group
    return x


SYM_CASES = [(f, s) for f in ("int8", "int4", "e4m3", "e5m2", "e2m1", "e2m3", "e3m2")
             for s in ("f32", "f16", "ue8m0", "e4m3")]


@pytest.mark.parametrize("fmt,scale", SYM_CASES)
@pytest.mark.parametrize("gran,block", [("block", 16), ("block", 32), ("channel", 0), ("tensor", 0)])
def test_symmetric_matches_bruteforce(oracle_mod, fmt, scale, gran, block):
    x = tiny_input(zlib.crc32(f"{fmt}/{scale}/{gran}".encode()) % 1000)
    check_against_bruteforce(oracle_mod, V(fmt, gran, scale, block=block), x)


@pytest.mark.parametrize("fmt,scale,gran,block,rnd", [
    (f, s, g, b, r) for f in ("int8", "int4") for s in ("f32", "f16")
    for g, b in (("block", 16), ("block", 64), ("channel", 0), ("tensor", 0)) for r in ("rne", "rna")])
def test_asymmetric_matches_bruteforce(oracle_mod, fmt, scale, gran, block, rnd):
    x = tiny_input(7, cols=128)
    x[2] = np.abs(x[2]) + 0.5  # a row with no negative values (range extends to 0)
    check_against_bruteforce(oracle_mod, V(fmt, gran, scale, block=block, sym=False, rnd=rnd), x)


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_rna_and_output_dtypes_match_bruteforce(oracle_mod, out):
    x = tiny_input(9)
    for fmt in ("int8", "int4"):
        check_against_bruteforce(oracle_mod, V(fmt, "block", "f32", block=32, rnd="rna", out=out), x)
    check_against_bruteforce(oracle_mod, V("e5m2", "block", "ue8m0", block=16, out=out), x)


def test_page_int4_group_example(oracle_mod):
    """guijiagi.com "INT4量化" (group-wise INT4): every 64 consecutive weights of
    a row share one fp32 scale s = absmax / 7; a weight's code is its quotient
    by s rounded half to even and clipped to [-8, 7]; the reconstruction is
    code * s. Computed here in numpy binary32 from that statement, the oracle's
    INT4 group-64 symmetric path with fp32 scales must agree bit for bit."""
    rows, cols, g = 48, 256, 64
    w = W.c3_input(rows=rows, cols=cols)["x"]
    groups = w.reshape(rows * cols // g, g)
    s = (np.abs(groups).max(axis=1) / np.float32(7.0)).astype(np.float32)
    code = np.clip(np.rint(groups / s[:, None]), -8, 7).astype(np.int64)
    recon = (code.astype(np.float32) * s[:, None]).astype(np.float32)

    got = oracle_mod.fake_quant(V("int4", "block", "f32", block=g, out="f32"), w)
    nib = bf.unpack_codes("int4", got["codes"], rows, cols)
    assert np.array_equal(np.where(nib >= 8, nib - 16, nib).reshape(-1, g), code)
    assert np.array_equal(got["scales"].view(np.float32), s)
    assert np.array_equal(got["xhat"].reshape(-1, g).view(np.uint32), recon.view(np.uint32))


def test_absmax_per_tensor_int8_formula(oracle_mod):
    """cyqw.cn/news/1000169 §2.1: Xq = clip(round(X/s), -127, 127) * s with
    s = max|X| / 127, in torch."""
    d = W.c1_input(rows=64, cols=256)
    x = torch.from_numpy(d["x"])
    s = x.abs().max() / 127.0
    q = torch.round(x / s).clamp(-127, 127)
    got = oracle_mod.fake_quant(V("int8", "tensor", "f32", out="f32"), d["x"])
    assert np.array_equal(got["codes"].view(np.int8).reshape(64, 256), q.numpy().astype(np.int8))
    assert np.array_equal(got["xhat"], (q * s).numpy())


@pytest.mark.parametrize("fmt", ["int8", "int4", "e4m3", "e5m2", "e2m1"])
def test_power_of_two_input_scaling(oracle_mod, fmt):
    """With UE8M0 scales, multiplying the input by 2^k shifts every scale code by
    k and leaves every element code unchanged."""
    x = W.c2_input(rows=8, cols=256)["x"]
    v = V(fmt, "block", "ue8m0", block=32)
    base = oracle_mod.fake_quant(v, x)
    for k in (5, -7):
        got = oracle_mod.fake_quant(v, (x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(got["codes"], base["codes"])
        assert np.array_equal(got["scales"].astype(int), base["scales"].astype(int) + k)


def test_asymmetric_invariants(oracle_mod):
    x = W.c3_input(rows=16, cols=512)["x"]
    for fmt in ("int8", "int4"):
        v = V(fmt, "block", "f32", block=128, sym=False, out="f32")
        got = oracle_mod.fake_quant(v, x)
        qmin, qmax = (-128, 127) if fmt == "int8" else (-8, 7)
        zp = got["zeros"].view(np.float32)
        s = got["scales"].view(np.float32)
        assert np.all(zp == np.round(zp)) and zp.min() >= qmin and zp.max() <= qmax
        err = np.abs(x.reshape(-1, 128) - got["xhat"].reshape(-1, 128))
        assert np.all(err <= s[:, None] * (0.5 + 1e-5))  # nothing clips: error at most half a step
        # zero is representable exactly
        z = np.zeros_like(x)
        z[:, 1:] = x[:, 1:]
        assert np.all(oracle_mod.fake_quant(v, z)["xhat"][:, 0] == 0.0)


def test_hadamard_butterfly(oracle_mod):
    """walkerchi.com playbook §5.3: the rotation is an orthogonal ±1 matrix. The
    butterfly equals scipy's Sylvester H16 / 4 (binary64) within binary32
    rounding, is its own inverse, and preserves the 2-norm."""
    H = scipy.linalg.hadamard(16).astype(np.float64) / 4.0
    assert np.allclose(H.T @ H, np.eye(16))
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        y = oracle_mod.hadamard16(x)
        assert np.allclose(y, H @ x.astype(np.float64), rtol=0, atol=4e-7 * np.abs(x).sum())
        assert np.allclose(oracle_mod.hadamard16(y), x, atol=1e-6)
        assert math.isclose(np.linalg.norm(y), np.linalg.norm(x), rel_tol=1e-6)
    xi = rng.integers(-50, 50, 16).astype(np.float32)
    assert np.array_equal(oracle_mod.hadamard16(oracle_mod.hadamard16(xi)), xi)
    e0 = np.zeros(16, np.float32)
    e0[5] = 4.0
    assert np.array_equal(oracle_mod.hadamard16(e0), (H[:, 5] * 4.0).astype(np.float32))


def test_hadamard_variant_rotates_then_quantizes(oracle_mod):
    x = W.c4_input(rows=4, cols=64)["x"]
    xr = np.stack([np.concatenate([oracle_mod.hadamard16(r[j:j + 16]) for j in range(0, 64, 16)])
                   for r in x])
    for fmt in ("e2m1", "int4"):
        plain = V(fmt, "block", "e4m3", block=16)
        rot = V(fmt, "block", "e4m3", block=16, hadamard=16)
        a = oracle_mod.fake_quant(rot, x)
        b = oracle_mod.fake_quant(plain, xr)
        for k in ("codes", "scales", "xhat", "y"):
            assert np.array_equal(a[k], b[k]), k
        # un-rotated output, and QSNR in either domain agree
        c = oracle_mod.fake_quant(dict(rot, unrotate=True, out="f32"), x)
        back = np.stack([np.concatenate([oracle_mod.hadamard16(r[j:j + 16]) for j in range(0, 64, 16)])
                         for r in a["xhat"]])
        assert np.array_equal(c["y"].view(np.float32), back)
        d = x.astype(np.float64) - back.astype(np.float64)
        q_orig = -10 * math.log10(np.sum(d * d) / np.sum(x.astype(np.float64) ** 2))
        assert abs(q_orig - a["qsnr"]) < 1e-4


def _rho_kappa(scales_f, x, bits, G):
    """cyqw.cn/news/1000169 §4.1 terms, aggregated over groups: the step s of a
    b-bit symmetric code covers absmax with 2^(b-1) steps when rho = 1, so
    rho*kappa = sqrt(mean_group(s^2) * 4^(b-1) / mean(x^2))."""
    s2 = np.mean(np.asarray(scales_f, np.float64) ** 2)
    return math.sqrt(s2 * 4.0 ** (bits - 1) / np.mean(x.astype(np.float64) ** 2))


@pytest.mark.parametrize("fmt,bits,gran,block,scale", [
    ("int8", 8, "tensor", 0, "f32"), ("int8", 8, "block", 32, "ue8m0"), ("int8", 8, "channel", 0, "f32"),
    ("int4", 4, "block", 64, "f32"), ("int4", 4, "block", 16, "f32"), ("int4", 4, "block", 16, "e4m3")])
def test_qsnr_closed_form(oracle_mod, fmt, bits, gran, block, scale):
    """QSNR_INT ≈ 4.78 + 6.02 b - 20 log10(rho*kappa) (cyqw.cn/news/1000169 §4.1;
    the '+' is lost in the page text) on Gaussian data, within 0.5 dB."""
    x = W.c1_input(rows=512, cols=1024)["x"]
    got = oracle_mod.fake_quant(V(fmt, gran, scale, block=block, out="f32"), x)
    if scale == "ue8m0":
        sf = 2.0 ** (got["scales"].astype(np.float64) - 127)
    elif scale == "e4m3":
        sf = np.array([oracle_mod.fp_decode("e4m3", int(c)) for c in got["scales"]])
    else:
        sf = got["scales"].view(np.float32)
    pred = 4.78 + 6.02 * bits - 20 * math.log10(_rho_kappa(sf, x, bits, block))
    assert abs(got["qsnr"] - pred) < 0.5, (got["qsnr"], pred)


def test_qualitative_orderings(oracle_mod):
    """m.youleyou.com/wenzhang/3165839 §3.1: uniform data favours INT8 over FP8-E4,
    t-distributed data with outliers favours FP8-E4 (per-tensor); cyqw.cn/news/1000169
    §4.2: at 32-element blocks MXINT8 beats MXFP8."""
    q = lambda v, x: oracle_mod.fake_quant(v, x, want=())["qsnr"]
    u = W.c5_input(0, rows=256, cols=512)["x"]
    t = W.c5_input(2, rows=256, cols=512)["x"]
    n = W.c5_input(1, rows=256, cols=512)["x"]
    pt = lambda f: V(f, "tensor", "f32")
    assert q(pt("int8"), u) > q(pt("e4m3"), u) + 3
    assert q(pt("e4m3"), t) > q(pt("int8"), t) + 3
    mx = lambda f: V(f, "block", "ue8m0", block=32)
    assert q(mx("int8"), n) > q(mx("e4m3"), n) + 3
    assert q(mx("e4m3"), n) > q(mx("e5m2"), n) + 3
    # E4M3 keeps ~31.5 dB on Gaussian data whatever the scale (printed MXFP8 mean 31.50 dB)
    assert abs(q(mx("e4m3"), n) - 31.5) < 1.0


def test_storage_sizes_match_printed(oracle_mod):
    """walkerchi.com playbook §4.3.1: MXFP4 stores 4x32+8 = 136 bit per 32 values,
    NVFP4 4x16+8 = 72 bit per 16 values."""
    x = np.random.default_rng(0).standard_normal((1, 32)).astype(np.float32)
    mx = oracle_mod.fake_quant(V("e2m1", "block", "ue8m0", block=32), x)
    assert (mx["codes"].nbytes + mx["scales"].nbytes) * 8 == 136
    nv = oracle_mod.fake_quant(V("e2m1", "block", "e4m3", block=16), x[:, :16])
    assert (nv["codes"].nbytes + nv["scales"].nbytes) * 8 == 72
    # INT4 codes are a quarter of the FP16 bytes (guijiagi.com introduction: 144 GB -> 36 GB)
    assert oracle_mod.codes_bytes(V("int4", "block", "f16", block=64), 64, 64) * 4 == 64 * 64 * 2


def test_zero_and_degenerate_groups(oracle_mod):
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = -0.0
    for fmt, sc in itertools.product(("int8", "int4", "e4m3", "e5m2", "e2m1"), ("f32", "f16", "ue8m0", "e4m3")):
        got = oracle_mod.fake_quant(V(fmt, "block", sc, block=32), x)
        codes = bf.unpack_codes(fmt, got["codes"], 2, 64)
        y = got["y"].reshape(2, 64)
        codes_neg0, y_neg0 = codes[1, 40], y[1, 40]
        codes[1, 40] = y[1, 40] = 0
        assert not np.any(codes) and not np.any(y)
        if sc == "ue8m0" and fmt not in ("int8", "int4"):
            # a power-of-two scale is never 0 (an all-zero block takes 2^-127), so
            # -0 keeps its sign: the negative-zero code and a -0 dequant
            assert codes_neg0 == (0x8 if fmt == "e2m1" else 0x80) and y_neg0 == 0x8000
        else:
            # a zero stored scale (or an integer code) gives code 0 and +0
            assert codes_neg0 == 0 and y_neg0 == 0
        assert got["qsnr"] == math.inf
    # a group whose fp16 scale underflows: codes 0, dequant +0
    tiny = np.full((1, 32), 1e-12, np.float32)
    got = oracle_mod.fake_quant(V("int8", "block", "f16", block=32), tiny)
    assert got["scales"][0] == 0 and not np.any(got["codes"]) and not np.any(got["y"])


def test_given_scales_reproduce_dynamic(oracle_mod):
    x = W.c3_input(rows=8, cols=256)["x"]
    for v in (V("int4", "block", "f16", block=64), V("int4", "block", "f16", block=128, sym=False),
              V("e4m3", "channel", "f32"), V("e2m1", "block", "e4m3", block=16)):
        a = oracle_mod.fake_quant(v, x)
        b = oracle_mod.fake_quant(v, x, given_scales=a["scales"], given_zeros=a["zeros"])
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["y"], b["y"])
        y = oracle_mod.dequant(v, a["codes"], a["scales"], a["zeros"], 8, 256)
        assert np.array_equal(y, a["y"])


def test_sampled_rows_equal_full(oracle_mod):
    x = W.c5_input(2, rows=64, cols=256)["x"]
    for v in W.c5_variants()[::3]:
        full = oracle_mod.fake_quant(v, x)
        part = oracle_mod.fake_quant(v, x, rows=(10, 20))
        cb = oracle_mod.codes_bytes(v, 1, 256)
        assert np.array_equal(part["codes"], full["codes"][10 * cb:20 * cb])
        assert np.array_equal(part["y"], full["y"][10:20])
        e2, s2, qs = oracle_mod.qsnr_full(v, x, threads=4, chunk_rows=7)
        assert math.isclose(qs, full["qsnr"], rel_tol=1e-12)


def test_algorithmic_bytes_match_config_arithmetic():
    # 8192x4096 bf16, MX block 32: 64 MiB + 32 MiB + 1 MiB + 64 MiB
    assert W.algorithmic_bytes(W.c2_variants()[0], 8192, 4096, 2) == 168_820_736
    for v in W.c3_variants():
        assert W.algorithmic_bytes(v, 11008, 4096, 2) == 204_308_480
    for v in W.c4_variants():
        assert W.algorithmic_bytes(v, 16384, 8192, 2) == 612_368_384
    assert W.algorithmic_bytes(W.c1_variants()[0], 1024, 1024, 4) == 9_437_188


@pytest.mark.parametrize("fmt,sym,lo,hi", [("int8", True, -127, 127), ("int8", False, -128, 127),
                                           ("int4", True, -8, 7), ("int4", False, -8, 7)])
def test_clamp_ranges_with_given_scales(oracle_mod, fmt, sym, lo, hi):
    """Code ranges: symmetric INT8 [-127,127] (cyqw.cn/news/1000169 §2.1), INT8
    [-128,127] (guijiagi.com "INT8量化"), INT4 [-8,7] (guijiagi.com "INT4量化").
    A caller-supplied scale smaller than absmax/Qmax makes the clamp visible."""
    x = np.float32([[-1e30, -200.0, -128.4, -8.6, 0.0, 8.6, 127.6, 3e38]])
    v = V(fmt, "tensor", "f32", sym=sym, out="f32")
    zeros = None if sym else np.zeros(1, np.float32)
    got = oracle_mod.fake_quant(v, x, given_scales=np.ones(1, np.float32), given_zeros=zeros)
    codes = bf.unpack_codes(fmt, got["codes"], 1, 8)[0]
    signed = np.where(codes >= (128 if fmt == "int8" else 8), codes - (256 if fmt == "int8" else 16), codes)
    want = np.clip(np.rint(x[0].astype(np.float64)), lo, hi)     # clip(round(x / 1), Qmin, Qmax)
    assert np.array_equal(signed, want) and np.array_equal(got["xhat"][0], want)
    assert signed.min() == lo and signed.max() == hi


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
def test_fp_saturation_with_given_scales(oracle_mod, fmt):
    big = oracle_mod.fp_max(fmt) * 4
    x = np.float32([[-big, big, 0.0, -0.0]])
    got = oracle_mod.fake_quant(V(fmt, "tensor", "f32", out="f32"), x, given_scales=np.ones(1, np.float32))
    assert list(got["xhat"][0]) == [-oracle_mod.fp_max(fmt), oracle_mod.fp_max(fmt), 0.0, 0.0]
    assert np.signbit(got["xhat"][0, 3]) and not np.signbit(got["xhat"][0, 2])


def test_fp6_orderings_and_storage(oracle_mod):
    """walkerchi.com playbook §4.1 table: FP6 E2M3 is MXFP6's high-precision
    layout, E3M2 its wide-range one (for training activations). Under MX block
    scaling (32 values, UE8M0) E2M3's extra significand bit wins and FP6 sits
    between FP4 and FP8; under one scale for a heavy-tailed tensor E3M2's range
    wins. A 32-value MXFP6 block stores 6x32 + 8 = 200 bits."""
    g = W.c2_input(rows=64, cols=1024)["x"]
    t = W.c4_input(rows=64, cols=1024)["x"]
    mx = lambda f, x: oracle_mod.fake_quant(V(f, "block", "ue8m0", block=32), x)["qsnr"]
    for x in (g, t):
        assert mx("e2m1", x) < mx("e3m2", x) < mx("e2m3", x) < mx("e4m3", x)
    per_tensor = lambda f: oracle_mod.fake_quant(V(f, "tensor", "f32"), t)["qsnr"]
    assert per_tensor("e3m2") > per_tensor("e2m3") + 5.0
    x = np.random.default_rng(0).standard_normal((1, 32)).astype(np.float32)
    b = oracle_mod.fake_quant(V("e2m3", "block", "ue8m0", block=32), x)
    assert (b["codes"].nbytes + b["scales"].nbytes) * 8 == 200
