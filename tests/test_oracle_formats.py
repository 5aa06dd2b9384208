"""Pins for the oracle's number formats: the pages' printed ranges, library
casts (torch float8 / bfloat16, numpy float16), exhaustive round trips and
brute-force nearest-value search at every midpoint."""
import math
import os

import numpy as np
import pytest
import torch

from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.tsv")


def golden():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, val, tol, cite = line.rstrip("\n").split("\t")
        out[name] = (float(val), float(tol), cite)
    return out


def close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


def test_golden_file_has_citations():
    g = golden()
    assert len(g) >= 20
    for name, (_, _, cite) in g.items():
        assert "§" in cite or "guijiagi" in cite, name


def test_printed_ranges(oracle_mod):
    o, g = oracle_mod, golden()
    for kind in ("e4m3", "e5m2", "e2m1", "fp16", "bf16", "e2m3", "e3m2"):
        key = f"{kind}_max"
        val, tol, _ = g[key]
        assert close(o.fp_max(kind), val, tol), (kind, o.fp_max(kind))
    # smallest positive code (subnormal for the 8/4-bit formats, printed as such)
    for kind in ("e4m3", "e5m2", "e2m1"):
        val, tol, _ = g[f"{kind}_min_pos"]
        assert close(o.fp_decode(kind, 1), val, tol), kind
    # smallest normal for FP16/BF16 (that table column mixes the two notions)
    for kind, code in (("fp16", 0x0400), ("bf16", 0x0080)):
        val, tol, _ = g[f"{kind}_min_normal"]
        assert close(o.fp_decode(kind, code), val, tol), kind
    # E2M1: 16 codes, all finite, +-0 among them
    vals = [o.fp_decode("e2m1", c) for c in range(16)]
    assert len(vals) == int(g["e2m1_n_values"][0]) and all(math.isfinite(v) for v in vals)
    assert sorted({abs(v) for v in vals}) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    # FP6: 64 codes, all finite, 32 magnitudes with 8 (E2M3) or 4 (E3M2) per binade
    for kind, per_binade in (("e2m3", 8), ("e3m2", 4)):
        vals = [o.fp_decode(kind, c) for c in range(64)]
        assert all(math.isfinite(v) for v in vals) and len({abs(v) for v in vals}) == 32
        assert sum(1 for v in vals if 1.0 <= v < 2.0) == per_binade, kind


@pytest.mark.parametrize("kind,dtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decode_matches_torch(oracle_mod, kind, dtype):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dtype).float().numpy()
    for c in range(256):
        got = oracle_mod.fp_decode(kind, c)
        r = float(ref[c])
        if math.isnan(r):
            assert math.isnan(got), (kind, c)
        else:
            assert got == r and math.copysign(1, got) == math.copysign(1, r), (kind, c, got, r)


def test_e4m3_has_no_infinity(oracle_mod):
    vals = [oracle_mod.fp_decode("e4m3", c) for c in range(256)]
    assert not any(math.isinf(v) for v in vals)
    assert sum(math.isnan(v) for v in vals) == 2  # s.1111.111 only


def test_fp16_bf16_decode_match_libraries(oracle_mod):
    codes = np.arange(65536, dtype=np.uint32)
    f16 = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    bf = torch.from_numpy(codes.astype(np.int32)).to(torch.int16).view(torch.bfloat16).double().numpy()
    for c in list(range(0, 65536, 97)) + [0x7BFF, 0xFBFF, 0x0001, 0x8001, 0x7C00, 0x7F7F, 0xFF80]:
        for kind, ref in (("fp16", f16), ("bf16", bf)):
            got, r = oracle_mod.fp_decode(kind, c), ref[c]
            assert (math.isnan(got) and math.isnan(r)) or got == r, (kind, hex(c), got, r)


def test_fp6_decode_matches_layout_model(oracle_mod):
    for kind in ("e2m3", "e3m2"):
        for c in range(64):
            got, want = oracle_mod.fp_decode(kind, c), bf.TABLES[kind][c]
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (kind, c)


@pytest.mark.parametrize("kind,ncodes", [("e4m3", 256), ("e5m2", 256), ("e2m1", 16), ("e2m3", 64), ("e3m2", 64)])
def test_round_trip_every_code(oracle_mod, kind, ncodes):
    for c in range(ncodes):
        v = oracle_mod.fp_decode(kind, c)
        if not math.isfinite(v):
            continue
        assert oracle_mod.fp_encode(kind, v) == c, (kind, c, v)


def test_e2m1_hand_ties(oracle_mod):
    # midpoints between adjacent E2M1 magnitudes and the even code each goes to
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in cases.items():
        for sgn in (1.0, -1.0):
            got = oracle_mod.fp_decode("e2m1", oracle_mod.fp_encode("e2m1", sgn * v))
            assert got == sgn * want and math.copysign(1, got) == sgn, (v, sgn, got)
    assert oracle_mod.fp_encode("e2m1", -0.2) == 0x8   # negative zero code
    assert oracle_mod.fp_encode("e2m1", 1e9) == 0x7    # saturates at 6
    assert oracle_mod.fp_encode("e2m1", -7.0) == 0xF


@pytest.mark.parametrize("kind", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_every_midpoint_brute_force(oracle_mod, kind):
    """At each midpoint between adjacent codes, and one binary32 ulp either
    side, the oracle agrees with an exhaustive exact nearest search."""
    pos = sorted(bf.positive_codes(kind), key=lambda cv: cv[1])
    probes = []
    for (c0, v0), (c1, v1) in zip(pos, pos[1:]):
        m = np.float32((v0 + v1) / 2.0)
        assert float(m) == (v0 + v1) / 2.0
        probes += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))]
    top = pos[-1][1]
    probes += [np.float32(top), np.nextafter(np.float32(top), np.float32(np.inf)), np.float32(top * 4)]
    for p in probes:
        for s in (1.0, -1.0):
            v = float(np.float32(s) * p)
            assert oracle_mod.fp_encode(kind, v) == bf.nearest_code(kind, v), (kind, v)


@pytest.mark.parametrize("kind", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_random_values_brute_force(oracle_mod, kind):
    rng = np.random.default_rng(11)
    mags = np.float32(2.0) ** rng.uniform(-22, 17, size=400).astype(np.float32)
    vals = (mags * rng.choice([-1, 1], size=400)).astype(np.float32)
    for v in vals:
        assert oracle_mod.fp_encode(kind, float(v)) == bf.nearest_code(kind, float(v)), (kind, v)


@pytest.mark.parametrize("kind,dtype,lim", [("e4m3", torch.float8_e4m3fn, 464.0),
                                            ("e5m2", torch.float8_e5m2, 61440.0)])
def test_fp8_encode_matches_torch_in_range(oracle_mod, kind, dtype, lim):
    """torch's float8 casts round to nearest-even but do not saturate, so the
    comparison stays strictly below the overflow threshold."""
    rng = np.random.default_rng(5)
    mags = np.float32(2.0) ** rng.uniform(-20, math.log2(lim) - 1e-3, size=20000).astype(np.float32)
    vals = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    vals = np.concatenate([vals, np.float32([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -17])])
    ref = torch.from_numpy(vals).to(dtype).view(torch.uint8).numpy()
    for v, r in zip(vals, ref):
        assert oracle_mod.fp_encode(kind, float(v)) == int(r), (kind, v)


def test_fp16_bf16_encode_match_library_casts(oracle_mod):
    rng = np.random.default_rng(6)
    mags = np.float32(2.0) ** rng.uniform(-30, 17, size=5000).astype(np.float32)
    vals = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    vals = np.concatenate([vals, np.float32([65504.0, 65519.0, 65520.0, 1e6, 3e-8, -0.0])])
    with np.errstate(over="ignore"):
        f16 = vals.astype(np.float16).view(np.uint16)
    b16 = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, a, b in zip(vals, f16, b16):
        assert oracle_mod.fp_encode("fp16", float(v), saturate=False) == int(a), v
        assert oracle_mod.fp_encode("bf16", float(v), saturate=False) == int(b), v
    assert oracle_mod.fp_encode("fp16", 1e6, saturate=True) == 0x7BFF


def test_ue8m0_exponent_brute_force(oracle_mod):
    rng = np.random.default_rng(3)
    amaxes = list(np.float32(2.0) ** rng.uniform(-140, 127, size=300).astype(np.float32))
    amaxes += [np.float32(0.0), np.float32(1e-45), np.float32(127.0), np.float32(127.00001),
               np.float32(448.0), np.float32(3.4e38), np.float32(6.0 * 2.0 ** -127)]
    for qmax in (127.0, 7.0, 448.0, 57344.0, 6.0):
        for a in amaxes:
            e = oracle_mod.ue8m0_exponent(float(a), qmax)
            assert e == bf.ue8m0_exp(float(a), qmax), (a, qmax, e)
            af = float(a)
            if 0 < af and -127 < e < 127:
                assert qmax * 2.0 ** (e - 1) < af <= qmax * 2.0 ** e


def test_integer_rounding_modes(oracle_mod):
    for v, rne, rna in ((0.5, 0, 1), (1.5, 2, 2), (2.5, 2, 3), (-0.5, 0, -1), (-2.5, -2, -3),
                        (2.4999998, 2, 2), (-7.5, -8, -8), (126.5, 126, 127)):
        assert oracle_mod.round_int(v, "rne") == rne, v
        assert oracle_mod.round_int(v, "rna") == rna, v
    rng = np.random.default_rng(1)
    for v in (rng.standard_normal(2000) * 50).astype(np.float32):
        assert oracle_mod.round_int(float(v), "rne") == float(torch.round(torch.tensor(v)))
        assert oracle_mod.round_int(float(v), "rna") == bf.round_int(float(v), "rna")
