"""Brute-force model of the quantizer for tiny inputs, used to pin the oracle.

It shares nothing with ``oracle/``: float element formats come from torch's
float8 dtypes (E4M3, E5M2) or from the E2M1 bit layout, encoding scans every
code for the exact nearest value (Fractions), the power-of-two scale exponent
is found by scanning all 255 exponents, fp16/bf16 roundings are numpy/torch
casts, and binary32 division/multiplication are numpy float32 operations.
"""
from __future__ import annotations

import math
from fractions import Fraction as Fr

import numpy as np
import torch

F32 = np.float32


def _torch_table(dtype):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(dtype).float().numpy()
    return {c: float(vals[c]) for c in range(256)}


def _e2m1_table():
    # [s][ee][m], bias 1: e=0 -> 0.m * 2^0 ; else 1.m * 2^(e-1)
    t = {}
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m * 0.5) if e == 0 else (1.0 + m * 0.5) * 2.0 ** (e - 1)
        t[c] = -mag if s else mag
    return t


def _fp6_table(ebits, mbits):
    """FP6 values from the bit layout [s][e..][m..] the playbook's §4.1 table
    prints; every code is a number, the bias puts the largest at the printed
    maximum (E2M3 7.5 = 1.875 * 2^2, E3M2 28 = 1.75 * 2^4)."""
    bias = {(2, 3): 1, (3, 2): 3}[(ebits, mbits)]
    t = {}
    for c in range(64):
        s, e, m = c >> 5, (c >> mbits) & ((1 << ebits) - 1), c & ((1 << mbits) - 1)
        if e == 0:
            mag = Fr(m, 1 << mbits) * Fr(2) ** (1 - bias)
        else:
            mag = (1 + Fr(m, 1 << mbits)) * Fr(2) ** (e - bias)
        t[c] = -float(mag) if s else float(mag)
    return t


TABLES = {
    "e4m3": _torch_table(torch.float8_e4m3fn),
    "e5m2": _torch_table(torch.float8_e5m2),
    "e2m1": _e2m1_table(),
    "e2m3": _fp6_table(2, 3),
    "e3m2": _fp6_table(3, 2),
}
SIGN_BIT = {"e4m3": 0x80, "e5m2": 0x80, "e2m1": 0x8, "e2m3": 0x20, "e3m2": 0x20}


def positive_codes(kind):
    sb = SIGN_BIT[kind]
    return [(c, v) for c, v in TABLES[kind].items() if not (c & sb) and math.isfinite(v)]


def fmt_max(kind):
    return max(v for _, v in positive_codes(kind))


def nearest_code(kind: str, v: float) -> int:
    """Exact nearest finite code to |v| (ties: even code), sign bit from v."""
    a = Fr(abs(float(v)))
    best, bestd = None, None
    for c, val in positive_codes(kind):
        d = abs(a - Fr(val))
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    if math.copysign(1.0, float(v)) < 0:
        best |= SIGN_BIT[kind]
    return best


def ue8m0_exp(absmax: float, qmax: float) -> int:
    A, Q = Fr(float(absmax)), Fr(float(qmax))
    for e in range(-127, 128):
        if Q * Fr(2) ** e >= A:
            return e
    return 127


def round_int(v: float, mode: str) -> int:
    if mode == "rne":
        return round(float(v))  # Python rounds half to even, exactly
    a = Fr(abs(float(v)))
    q = math.floor(a + Fr(1, 2))
    return -q if v < 0 else q


QMAX = {"int8": 127, "int4": 7}


def qrange(fmt, sym):
    if fmt == "int8":
        return (-127 if sym else -128), 127
    return -8, 7


def fp16_sat(t):
    return F32(np.float16(min(float(t), 65504.0)))


def store_scale(scale, t):
    t = F32(t)
    if scale == "f16":
        s = fp16_sat(t)
        return s, int(np.float16(s).view(np.uint16))
    if scale == "e4m3":
        c = nearest_code("e4m3", float(t))
        return F32(TABLES["e4m3"][c]), c
    return t, int(np.array(t, np.float32).view(np.uint32))


def quantize_group(v: dict, vals: np.ndarray, stat=None):
    """Quantize one group of fp32 values. Returns (codes, sbits, zbits, xhat)."""
    fmt, scale, sym = v["fmt"], v["scale"], v.get("sym", True)
    rnd = v.get("round", "rne")
    vals = vals.astype(np.float32)
    if stat is None:
        amax = F32(np.max(np.abs(vals))) if vals.size else F32(0)
        mn, mx = F32(np.min(vals)), F32(np.max(vals))
    else:
        amax, mn, mx = (F32(s) for s in stat)
    is_int = fmt in ("int8", "int4")
    qmax = QMAX[fmt] if is_int else fmt_max(fmt)
    zp, zbits = 0, None
    if sym:
        if scale == "ue8m0":
            e = ue8m0_exp(float(amax), qmax)
            s, sbits = F32(2.0 ** e), e + 127
        else:
            s, sbits = store_scale(scale, F32(amax) / F32(qmax))
    else:
        qmin, qmx = qrange(fmt, False)
        lo, hi = min(mn, F32(0)), max(mx, F32(0))
        s, sbits = store_scale(scale, F32(F32(hi) - F32(lo)) / F32(qmx - qmin))
        if s != 0:
            zp = qmin - round_int(float(F32(lo) / s), rnd)
            zp = min(max(zp, qmin), qmx)
        zbits = (int(np.float16(zp).view(np.uint16)) if scale == "f16"
                 else int(np.array(F32(zp), np.float32).view(np.uint32)))
    codes, xhat = [], []
    for x in vals:
        if s == 0:
            codes.append(0)
            xhat.append(F32(0.0))
            continue
        q = F32(x) / s
        if is_int:
            lo_, hi_ = qrange(fmt, sym)
            qi = round_int(float(q), rnd) + (0 if sym else zp)
            qi = min(max(qi, lo_), hi_)
            xhat.append(F32(F32(qi) * s) if sym else F32(s * F32(qi - zp)))
            codes.append(qi & (0xFF if fmt == "int8" else 0xF))
        else:
            c = nearest_code(fmt, float(q))
            codes.append(c)
            xhat.append(F32(F32(TABLES[fmt][c]) * s))
    return codes, sbits, zbits, np.array(xhat, np.float32)


def y_bits(out: str, xhat: np.ndarray) -> np.ndarray:
    if out == "f32":
        return xhat.astype(np.float32).view(np.uint32)
    if out == "f16":
        with np.errstate(over="ignore"):
            return xhat.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(xhat.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def two_level_scale(fmt: str, amax) -> np.float32:
    """NVFP4-style tensor scale: the largest magnitude over the product of the
    E4M3 maximum (read from torch's table) and the element Qmax, one binary32
    quotient; a zero quotient becomes 1."""
    qmax = QMAX[fmt] if fmt in QMAX else fmt_max(fmt)
    with np.errstate(under="ignore"):
        S = F32(amax) / (F32(fmt_max("e4m3")) * F32(qmax))
    return F32(1.0) if S == 0 else S


def fake_quant(v: dict, x: np.ndarray):
    """Whole tiny tensor (no rotation). Returns dict like the oracle's, codes unpacked.
    Two-level variants divide the tensor by S first and multiply each group's
    dequantized values by S."""
    rows, cols = x.shape
    g = v["gran"]
    if g == "tile":
        return _fake_quant_tiles(v, x)
    G = v["block"] if g == "block" else cols
    stat = None
    if g == "tensor":
        stat = (np.max(np.abs(x)), np.min(x), np.max(x))
    two = bool(v.get("two_level", False))
    S = two_level_scale(v["fmt"], np.max(np.abs(x))) if two else F32(1.0)
    codes = np.zeros((rows, cols), np.int64)
    xhat = np.zeros((rows, cols), np.float32)
    sb, zb = [], []
    for r in range(rows):
        for g0 in range(0, cols, G):
            vals = x[r, g0:g0 + G].astype(np.float32)
            if two:
                with np.errstate(under="ignore"):
                    vals = np.array([F32(a) / S for a in vals], np.float32)
            c, s, z, xh = quantize_group(v, vals, stat)
            if two:
                with np.errstate(under="ignore"):
                    xh = np.array([F32(a) * S for a in xh], np.float32)
            codes[r, g0:g0 + G] = c
            xhat[r, g0:g0 + G] = xh
            sb.append(s)
            zb.append(z)
    if g == "tensor":
        sb, zb = sb[:1], zb[:1]
    d = x.astype(np.float64) - xhat.astype(np.float64)
    return {"codes": codes, "sbits": sb, "zbits": zb, "xhat": xhat, "tscale": S if two else None,
            "y": y_bits(v.get("out", "bf16"), xhat),
            "err2": float(np.sum(d * d)), "sig2": float(np.sum(x.astype(np.float64) ** 2))}


def _fake_quant_tiles(v: dict, x: np.ndarray):
    """2-D tiles of tile_rows x block elements: each tile's values (row-major)
    form one group; the last band of rows may be shorter."""
    rows, cols = x.shape
    TR, TC = v["tile_rows"], v["block"]
    codes = np.zeros((rows, cols), np.int64)
    xhat = np.zeros((rows, cols), np.float32)
    sb, zb = [], []
    for r0 in range(0, rows, TR):
        for c0 in range(0, cols, TC):
            t = x[r0:r0 + TR, c0:c0 + TC]
            c, s, z, xh = quantize_group(v, t.reshape(-1))
            codes[r0:r0 + TR, c0:c0 + TC] = np.array(c).reshape(t.shape)
            xhat[r0:r0 + TR, c0:c0 + TC] = xh.reshape(t.shape)
            sb.append(s)
            zb.append(z)
    d = x.astype(np.float64) - xhat.astype(np.float64)
    return {"codes": codes, "sbits": sb, "zbits": zb, "xhat": xhat, "tscale": None,
            "y": y_bits(v.get("out", "bf16"), xhat),
            "err2": float(np.sum(d * d)), "sig2": float(np.sum(x.astype(np.float64) ** 2))}


def unpack_codes(fmt: str, packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    if fmt in ("e2m3", "e3m2"):
        # element e: bits 6e .. 6e+5 of the byte stream, low bits first
        bits = np.unpackbits(np.asarray(packed, np.uint8), bitorder="little")
        six = bits[:rows * cols * 6].reshape(-1, 6).astype(np.int64)
        return (six << np.arange(6)).sum(axis=1).reshape(rows, cols)
    if fmt in ("int4", "e2m1"):
        lo = packed & 0xF
        hi = packed >> 4
        return np.stack([lo, hi], axis=-1).reshape(rows, cols).astype(np.int64)
    return packed.reshape(rows, cols).astype(np.int64)
