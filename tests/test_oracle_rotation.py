"""Pins for the oracle's n-point randomized Hadamard rotation (walkerchi.com
quantization playbook §5.3: an orthogonal rotation R, R^T R = I, applied as
y' = y R and undone with R^T; QuaRot's R is a Hadamard matrix with random
signs; cyqw.cn/news/1000169 §4.2, §7.2: rotation before 4-bit quantization).
Reading: R is block diagonal over aligned groups of n columns, each block
H_n D / sqrt(n) with D the random ±1 signs of those columns (passed in as a
bit vector), butterflies in binary32 and 1/sqrt(n) rounded to binary32.

Independent checks: scipy's Hadamard matrix in float64; the binary32
rounding of 1/sqrt(n) from a 60-digit decimal value; orthogonality (the
inverse undoes the rotation); the signs as negated inputs; the 16-point case
against the unsigned 16-point rotation already pinned; rotation before
quantization; QuaRot's effect on channel outliers."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg

from bit_quantization_block_amd import workloads as W
from tests.test_oracle_method import V

SIZES = (16, 32, 64, 128, 256, 512, 1024)


def _signs(n_cols, seed):
    bits = np.random.default_rng(seed).integers(0, 2, n_cols)
    words = np.zeros((n_cols + 31) // 32, np.uint32)
    for j, b in enumerate(bits):
        words[j // 32] |= np.uint32(int(b) << (j % 32))
    return words, np.where(bits == 1, -1.0, 1.0)


def _f32_nearest(x: Decimal) -> np.float32:
    """The binary32 value nearest to x (ties to even), by exact comparison."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Decimal(float(c)) - x)
        if best is None or d < best[0] or (d == best[0] and int(c.view(np.uint32)) % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("n", SIZES + (1024,))
def test_rotation_scale_is_rounded_inverse_sqrt(oracle_mod, n):
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(n).sqrt()
    assert oracle_mod.rotation_scale(n) == _f32_nearest(exact)
    if round(math.log(n, 4)) == math.log(n, 4):
        assert float(oracle_mod.rotation_scale(n)) == 2.0 ** (-math.log2(n) / 2)


@pytest.mark.parametrize("n", SIZES)
def test_rotation_matches_signed_hadamard_matrix(oracle_mod, n):
    rng = np.random.default_rng(n)
    words, d = _signs(3 * n, n)
    H = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    for g in range(3):
        x = rng.standard_normal(n).astype(np.float32)
        got = oracle_mod.rotate(x, words, col0=g * n)
        ref = H @ (d[g * n:(g + 1) * n] * x.astype(np.float64))
        assert np.max(np.abs(got - ref)) <= 4e-6 * math.sqrt(n) * np.max(np.abs(x)), (n, g)


@pytest.mark.parametrize("n", SIZES)
def test_inverse_undoes_rotation(oracle_mod, n):
    rng = np.random.default_rng(100 + n)
    words, _ = _signs(2 * n, n + 1)
    x = rng.standard_normal(n).astype(np.float32) * 10
    y = oracle_mod.rotate(x, words, col0=n)
    z = oracle_mod.rotate(y, words, col0=n, inverse=True)
    assert np.max(np.abs(z - x)) <= 1e-5 * np.max(np.abs(x))
    assert math.isclose(float(np.sum(y.astype(np.float64) ** 2)), float(np.sum(x.astype(np.float64) ** 2)),
                        rel_tol=1e-5)


def test_signs_are_negated_inputs(oracle_mod):
    rng = np.random.default_rng(7)
    n = 64
    x = rng.standard_normal(n).astype(np.float32)
    words, d = _signs(n, 8)
    a = oracle_mod.rotate(x, words)
    b = oracle_mod.rotate((x * d).astype(np.float32))
    assert np.array_equal(a, b)                     # negation is exact: bit for bit
    allneg = np.full(2, 0xFFFFFFFF, np.uint32)
    assert np.array_equal(oracle_mod.rotate(x, allneg), oracle_mod.rotate(-x))


def test_sixteen_points_without_signs_is_the_plain_rotation(oracle_mod):
    x = np.random.default_rng(9).standard_normal(16).astype(np.float32)
    assert np.array_equal(oracle_mod.rotate(x), oracle_mod.hadamard16(x))
    v = V("int4", "block", "e4m3", block=16, hadamard=16)
    xx = W.c4_input(rows=4, cols=256)["x"]
    a = oracle_mod.fake_quant(v, xx)
    b = oracle_mod.fake_quant(dict(v, signs=np.zeros(8, np.uint32)), xx)
    for k in ("codes", "scales", "y"):
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("n", (32, 128, 256, 512))
def test_rotation_then_quantize_equals_quantizing_rotated(oracle_mod, n):
    rows, cols = 6, 512
    x = W.c4_input(rows=rows, cols=cols)["x"]
    words, _ = _signs(cols, 3 * n)
    xr = x.copy()
    for r in range(rows):
        for j in range(0, cols, n):
            xr[r, j:j + n] = oracle_mod.rotate(x[r, j:j + n], words, col0=j)
    for v in (V("int4", "block", "e4m3", block=16), V("e4m3", "channel", "f32"), V("int8", "tensor", "f32")):
        a = oracle_mod.fake_quant(dict(v, hadamard=n, signs=words), x)
        b = oracle_mod.fake_quant(v, xr)
        for k in ("codes", "scales", "xhat"):
            assert np.array_equal(a[k], b[k]), (n, v, k)
        # un-rotated output: the inverse rotation of xhat, column by column
        u = oracle_mod.fake_quant(dict(v, hadamard=n, signs=words, unrotate=True, out="f32"), x)["y"]
        back = np.stack([np.concatenate([oracle_mod.rotate(a["xhat"][r, j:j + n], words, col0=j, inverse=True)
                                         for j in range(0, cols, n)]) for r in range(rows)])
        assert np.array_equal(u.view(np.float32), back)


def test_quarot_spreads_channel_outliers(oracle_mod):
    """Channel outliers (8 columns x100): per-channel INT4 gains from rotating
    over wider groups, which spread each outlier over more columns; random
    signs keep the gain."""
    x = W.c2_input(rows=32, cols=1024)["x"]
    v = V("int4", "channel", "f32", out="f32")
    q = {0: oracle_mod.fake_quant(v, x)["qsnr"]}
    for n in SIZES:
        q[n] = oracle_mod.fake_quant(dict(v, hadamard=n), x)["qsnr"]
    words, _ = _signs(1024, 11)
    qs = oracle_mod.fake_quant(dict(v, hadamard=256, signs=words), x)["qsnr"]
    assert q[0] < q[16] < q[64] < q[256], q
    assert abs(qs - q[256]) < 1.5, (qs, q[256])


def test_dequant_unrotates_with_signs(oracle_mod):
    x = W.c4_input(rows=4, cols=256)["x"]
    words, _ = _signs(256, 5)
    v = dict(V("e2m1", "block", "e4m3", block=16, hadamard=64, unrotate=True), signs=words)
    a = oracle_mod.fake_quant(v, x)
    y = oracle_mod.dequant(v, a["codes"], a["scales"], None, 4, 256)
    assert np.array_equal(y, a["y"])


def test_rejects_bad_sizes(oracle_mod):
    x = np.ones((1, 64), np.float32)
    for n in (8, 48, 2048):
        with pytest.raises(ValueError):
            oracle_mod.fake_quant(V("int8", "block", "f32", block=32, hadamard=n), x)
    with pytest.raises(ValueError):                   # 64 columns do not hold a 128-group
        oracle_mod.fake_quant(V("int8", "block", "f32", block=32, hadamard=128), x)
