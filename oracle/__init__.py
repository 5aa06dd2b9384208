"""Python face of the CPU oracle (``lq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``; the product package never imports it.

A quantization variant is a plain dict of strings and ints, for example::

    {"fmt": "e4m3", "gran": "block", "block": 32, "scale": "ue8m0",
     "sym": True, "round": "rne", "out": "bf16", "hadamard": 0}

The oracle parses it into its own descriptor; the HIP binding parses the same
dict into the library's descriptor. Nothing else is shared.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lq_oracle.c")
_LIB = os.path.join(_HERE, "liblq_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
             "-fno-fast-math", "-fPIC", "-shared"]

FMT = {"int8": 0, "int4": 1, "e4m3": 2, "e5m2": 3, "e2m1": 4, "e2m3": 5, "e3m2": 6}
KIND = {"e4m3": 0, "e5m2": 1, "e2m1": 2, "fp16": 3, "bf16": 4, "e2m3": 5, "e3m2": 6}
GRAN = {"tensor": 0, "channel": 1, "block": 2, "tile": 3}
SCALE = {"f32": 0, "f16": 1, "ue8m0": 2, "e4m3": 3}
ROUND = {"rne": 0, "rna": 1}
DTYPE = {"f32": 0, "bf16": 1, "f16": 2}

SCALE_BYTES = {"f32": 4, "f16": 2, "ue8m0": 1, "e4m3": 1}
OUT_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", _LIB, "-lm"], check=True)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "fmt", "gran", "block", "scale_fmt", "symmetric", "rounding",
        "out_dtype", "hadamard", "unrotate_y", "given_scales", "two_level", "tile_rows")] + [
        ("signs", ctypes.c_void_p)]


_lib = None


class swap_library:
    """Context manager: route every oracle call through another build of
    lq_oracle.c (used by the tests that plant mistakes in a copy of it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = None
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _load(_LIB)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    c_f = ctypes.POINTER(ctypes.c_float)
    c_d = ctypes.POINTER(ctypes.c_double)
    c_u8 = ctypes.POINTER(ctypes.c_uint8)
    dp = ctypes.POINTER(_Desc)
    L.or_fp_decode.argtypes = [ctypes.c_int, ctypes.c_uint32]
    L.or_fp_decode.restype = ctypes.c_double
    L.or_fp_encode.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_int]
    L.or_fp_encode.restype = ctypes.c_uint32
    L.or_fp_max.argtypes = [ctypes.c_int]
    L.or_fp_max.restype = ctypes.c_double
    L.or_ue8m0_exponent.argtypes = [ctypes.c_double, ctypes.c_double]
    L.or_ue8m0_exponent.restype = ctypes.c_int
    L.or_round_int.argtypes = [ctypes.c_double, ctypes.c_int]
    L.or_round_int.restype = ctypes.c_double
    L.or_hadamard16.argtypes = [c_f]
    L.or_hadamard16.restype = None
    L.or_rotate.argtypes = [c_f, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
    L.or_rotate.restype = None
    L.or_unrotate.argtypes = [c_f, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
    L.or_unrotate.restype = None
    L.or_rotation_scale.argtypes = [ctypes.c_int]
    L.or_rotation_scale.restype = ctypes.c_float
    L.or_tensor_stat.argtypes = [dp, c_f, ctypes.c_int64, ctypes.c_int64, c_f]
    L.or_tensor_stat.restype = ctypes.c_int64
    L.or_tensor_scale.argtypes = [dp, ctypes.c_float]
    L.or_tensor_scale.restype = ctypes.c_float
    L.or_fake_quant_rows.argtypes = [dp, c_f, ctypes.c_int64, ctypes.c_int64, c_f, c_f, c_u8,
                                     ctypes.c_void_p, ctypes.c_void_p, c_f, ctypes.c_void_p,
                                     c_d, c_d]
    L.or_fake_quant_rows.restype = ctypes.c_int
    L.or_dequant_rows.argtypes = [dp, c_u8, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    L.or_dequant_rows.restype = ctypes.c_int
    L.or_sweep_tally.argtypes = [c_d, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                 ctypes.POINTER(ctypes.c_int32)]
    L.or_sweep_tally.restype = ctypes.c_int
    return L


# ---------------------------------------------------------------- formats
def fp_decode(kind: str, code: int) -> float:
    return lib().or_fp_decode(KIND[kind], code)


def fp_encode(kind: str, v: float, saturate: bool = True) -> int:
    return lib().or_fp_encode(KIND[kind], float(v), 1 if saturate else 0)


def fp_max(kind: str) -> float:
    return lib().or_fp_max(KIND[kind])


def ue8m0_exponent(absmax: float, qmax: float) -> int:
    return lib().or_ue8m0_exponent(float(absmax), float(qmax))


def round_int(v: float, mode: str = "rne") -> float:
    return lib().or_round_int(float(v), ROUND[mode])


def hadamard16(v) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).copy())
    assert a.size == 16
    lib().or_hadamard16(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return a


def _signs_ptr(signs):
    return None if signs is None else np.ascontiguousarray(signs, np.uint32).ctypes.data


def rotate(v, signs=None, col0: int = 0, inverse: bool = False) -> np.ndarray:
    """n-point rotation (n = len(v)) of values whose first is column col0;
    signs: uint32 words, bit j = column j negated (None: no signs)."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).copy())
    sg = None if signs is None else np.ascontiguousarray(signs, np.uint32)
    f = lib().or_unrotate if inverse else lib().or_rotate
    f(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.size, _signs_ptr(sg), col0)
    return a


def rotation_scale(n: int) -> np.float32:
    return np.float32(lib().or_rotation_scale(n))


# ---------------------------------------------------------------- variants
def qmax_of(fmt: str) -> float:
    return {"int8": 127.0, "int4": 7.0}.get(fmt) or fp_max(fmt)


def is_4bit(fmt: str) -> bool:
    return fmt in ("int4", "e2m1")


def _desc(v: dict, given: bool = False) -> _Desc:
    """The oracle's descriptor of a variant; "signs" (uint32 words of the random
    ±1 diagonal) must stay referenced by the variant while the call runs."""
    sg = v.get("signs")
    if sg is not None:
        assert isinstance(sg, np.ndarray) and sg.dtype == np.uint32 and sg.flags.c_contiguous
    return _Desc(FMT[v["fmt"]], GRAN[v["gran"]], int(v.get("block", 0) or 0), SCALE[v["scale"]],
                 1 if v.get("sym", True) else 0, ROUND[v.get("round", "rne")],
                 DTYPE[v.get("out", "bf16")], int(v.get("hadamard", 0)),
                 1 if v.get("unrotate", False) else 0, 1 if given else 0,
                 1 if v.get("two_level", False) else 0, int(v.get("tile_rows", 0) or 0),
                 None if sg is None else sg.ctypes.data)


def n_scales(v: dict, rows: int, cols: int) -> int:
    if v["gran"] == "tensor":
        return 1
    if v["gran"] == "channel":
        return rows
    if v["gran"] == "tile":
        return -(-rows // v["tile_rows"]) * (cols // v["block"])
    return rows * (cols // v["block"])


def is_6bit(fmt: str) -> bool:
    return fmt in ("e2m3", "e3m2")


def codes_bytes(v: dict, rows: int, cols: int) -> int:
    if is_6bit(v["fmt"]):
        return rows * cols * 3 // 4
    return rows * cols // 2 if is_4bit(v["fmt"]) else rows * cols


def _ptr(a, t=ctypes.c_float):
    return a.ctypes.data_as(ctypes.POINTER(t))


def needs_stat(v: dict) -> bool:
    """Whether the variant uses the whole-tensor statistic."""
    return v["gran"] == "tensor" or bool(v.get("two_level", False))


def tensor_scale(v: dict, amax: float) -> np.float32:
    """Two-level tensor scale S for a tensor maximum magnitude ``amax``."""
    return np.float32(lib().or_tensor_scale(ctypes.byref(_desc(v)), float(np.float32(amax))))


def tensor_stat(v: dict, x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(3, np.float32)
    bad = lib().or_tensor_stat(ctypes.byref(_desc(v)), _ptr(x), x.shape[0], x.shape[1], _ptr(out))
    return out, int(bad)


def fake_quant(v: dict, x: np.ndarray, rows=None, tstat=None, want=("codes", "scales", "zeros", "xhat", "y"),
               given_scales=None, given_zeros=None, given_tscale=None) -> dict:
    """Fake-quantize ``x`` (2-D fp32 values). ``rows`` = optional (begin, end) to
    process only those rows (for sampled checks of large tensors); the
    per-tensor statistic is always taken over the whole of ``x``. Two-level
    variants return the tensor scale as ``tscale`` (np.float32) and read it
    from ``given_tscale`` with given scales."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    r0, r1 = (0, R) if rows is None else rows
    n = r1 - r0
    if v["gran"] == "tile" and r0 % v["tile_rows"] != 0:
        raise ValueError("a row block of a tiled variant must start at a multiple of tile_rows")
    if tstat is None:
        tstat = tensor_stat(v, x)[0] if needs_stat(v) else np.zeros(3, np.float32)
    tstat = np.asarray(tstat, np.float32)
    out = {}
    codes = np.zeros(codes_bytes(v, n, C), np.uint8) if "codes" in want else None
    nsc = 1 if v["gran"] == "tensor" else n_scales(v, n, C)
    sdt = {4: np.uint32, 2: np.uint16, 1: np.uint8}[SCALE_BYTES[v["scale"]]]
    given = given_scales is not None
    if given:
        scales = np.ascontiguousarray(given_scales).view(sdt).copy()
    else:
        scales = np.zeros(nsc, sdt) if "scales" in want else None
    sym = v.get("sym", True)
    zdt = np.uint16 if v["scale"] == "f16" else np.uint32
    if given and not sym:
        zeros = np.ascontiguousarray(given_zeros).view(zdt).copy()
    else:
        zeros = np.zeros(nsc, zdt) if ("zeros" in want and not sym) else None
    xhat = np.zeros((n, C), np.float32) if "xhat" in want else None
    ob = OUT_BYTES[v.get("out", "bf16")]
    y = np.zeros((n, C), np.uint32 if ob == 4 else np.uint16) if "y" in want else None
    e2 = ctypes.c_double(0.0)
    s2 = ctypes.c_double(0.0)
    ts = np.array([1.0 if given_tscale is None else given_tscale], np.float32)
    rc = lib().or_fake_quant_rows(
        ctypes.byref(_desc(v, given)), _ptr(x[r0:r1]), n, C, _ptr(tstat), _ptr(ts),
        None if codes is None else _ptr(codes, ctypes.c_uint8),
        None if scales is None else scales.ctypes.data,
        None if zeros is None else zeros.ctypes.data,
        None if xhat is None else _ptr(xhat),
        None if y is None else y.ctypes.data,
        ctypes.byref(e2), ctypes.byref(s2))
    if rc != 0:
        raise ValueError(f"oracle rejected variant {v} on shape {x.shape}: rc={rc}")
    out.update(codes=codes, scales=scales, zeros=zeros, xhat=xhat, y=y,
               err2=e2.value, sig2=s2.value, qsnr=qsnr_db(e2.value, s2.value),
               tscale=ts[0] if v.get("two_level", False) else None)
    return out


def qsnr_db(err2: float, sig2: float) -> float:
    """QSNR = -10 log10(|X - Xq|^2 / |X|^2) (cyqw.cn/news/1000169 §4.1);
    +inf when the error is zero."""
    if err2 == 0.0:
        return math.inf
    return -10.0 * math.log10(err2 / sig2)


def qsnr_full(v: dict, x: np.ndarray, threads: int = 0, chunk_rows: int = 0):
    """err2, sig2 and QSNR over the whole tensor, the row chunks computed in
    parallel threads (ctypes releases the GIL); partial sums are added in
    binary64 in chunk order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R = x.shape[0]
    threads = threads or min(16, os.cpu_count() or 1)
    tstat = tensor_stat(v, x)[0] if needs_stat(v) else np.zeros(3, np.float32)
    chunk_rows = chunk_rows or max(1, -(-R // (threads * 4)))
    if v["gran"] == "tile":                       # whole bands of tiles per chunk
        chunk_rows = -(-chunk_rows // v["tile_rows"]) * v["tile_rows"]
    spans = [(r, min(R, r + chunk_rows)) for r in range(0, R, chunk_rows)]

    def one(span):
        o = fake_quant(v, x, rows=span, tstat=tstat, want=())
        return o["err2"], o["sig2"]

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(one, spans))
    e2 = sum(p[0] for p in parts)
    s2 = sum(p[1] for p in parts)
    return e2, s2, qsnr_db(e2, s2)


def dequant(v: dict, codes: np.ndarray, scales: np.ndarray, zeros, rows: int, cols: int,
            tscale: float = 1.0) -> np.ndarray:
    ob = OUT_BYTES[v.get("out", "bf16")]
    y = np.zeros((rows, cols), np.uint32 if ob == 4 else np.uint16)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales)
    zp = None if zeros is None else np.ascontiguousarray(zeros)
    rc = lib().or_dequant_rows(ctypes.byref(_desc(v, True)), _ptr(codes, ctypes.c_uint8), scales.ctypes.data,
                               None if zp is None else zp.ctypes.data, float(np.float32(tscale)),
                               rows, cols, y.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected variant {v}: rc={rc}")
    return y


# ---------------------------------------------------------------- sweep
SWEEP_FORMATS = ("int8", "int4", "e4m3", "e5m2", "e2m1")
SWEEP_GRANS = ("tensor", "channel", "b16", "b32", "b64")
SWEEP_PAIRS = (("int8", "e4m3"), ("int8", "e5m2"), ("int4", "e2m1"))
# the sweep's tie band and the margin around its edges (tie_db, margin_db):
# QSNRs within 0.01 dB tie; a pair is decided only when its difference is
# more than twice the 1e-3 dB QSNR tolerance away from that edge
SWEEP_TIE_DB = 1e-2
SWEEP_MARGIN_DB = 2e-3


def sweep_tally(qsnr: np.ndarray, tie_db: float = SWEEP_TIE_DB, margin_db: float = SWEEP_MARGIN_DB) -> np.ndarray:
    """qsnr [n_tensors, 5 formats, 5 granularities] -> counts [5 granularities,
    3 pairs, 4] = (INT wins, FP wins, ties, undecided); the tensor-level
    analogue of the win counts of cyqw.cn/news/1000169 §5.1."""
    q = np.ascontiguousarray(qsnr, dtype=np.float64).reshape(-1, 25)
    out = np.zeros(60, np.int32)
    rc = lib().or_sweep_tally(q.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), q.shape[0], float(tie_db),
                              float(margin_db), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != 0:
        raise ValueError(f"oracle rejected the tally arguments (tie {tie_db}, margin {margin_db})")
    return out.reshape(5, 3, 4)
