"""Thin ctypes binding of liblq (include/lq.h): argument marshalling only.

Every computation runs in the HIP library. torch is used for device memory
and streams: tensors are passed as device pointers, the current torch stream
as the hipStream_t. There is no fallback: if liblq.so is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblq.so")

LQ_OK = 0
STATUS = {0: "LQ_OK", -1: "LQ_ERR_NULL", -2: "LQ_ERR_BAD_DESC", -3: "LQ_ERR_SHAPE", -4: "LQ_ERR_ALIGN",
          -5: "LQ_ERR_WORKSPACE", -6: "LQ_ERR_HIP", -7: "LQ_ERR_UNSUPPORTED"}
FORMAT = {"int8": 0, "int4": 1, "e4m3": 2, "e5m2": 3, "e2m1": 4, "e2m3": 5, "e3m2": 6}
GRAN = {"tensor": 0, "channel": 1, "block": 2, "tile": 3}
SCALE_FMT = {"f32": 0, "f16": 1, "ue8m0": 2, "e4m3": 3}
ROUND = {"rne": 0, "rna": 1}
DTYPE = {"f32": 0, "bf16": 1, "f16": 2}

EXPORTS = ("lq_quantize", "lq_dequantize", "lq_fake_quant_qsnr", "lq_hadamard_quant", "lq_workspace_bytes",
           "lq_codes_bytes", "lq_scales_bytes", "lq_zeros_bytes", "lq_workspace_init", "lq_sweep_tally",
           "lq_call_kernels", "lq_set_grid_limit", "lq_status_string", "lq_fake_quant_qsnr_static")
# output bits of lq_call_kernels
OUT = {"codes": 1, "scales": 2, "zeros": 4, "y": 8, "res": 16}


class LQError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')}): {status_string(status)}")


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("format", "gran", "block", "scale_fmt", "symmetric", "rounding",
                                               "in_dtype", "out_dtype", "hadamard", "scale_source", "two_level",
                                               "tile_rows")] + [("signs", ctypes.c_void_p)]


class Result(ctypes.Structure):
    _fields_ = [("err2", ctypes.c_double), ("sig2", ctypes.c_double), ("qsnr_db", ctypes.c_double),
                ("nonfinite", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None


def load(path: str | None = None):
    """Load liblq.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"liblq not built: {p} is missing (run __graft_entry__.build())")
    L = ctypes.CDLL(p)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    L.lq_quantize.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, sz, vp]
    L.lq_dequantize.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp]
    L.lq_fake_quant_qsnr.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lq_hadamard_quant.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp]
    L.lq_fake_quant_qsnr_static.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.lq_fake_quant_qsnr_static.restype = ctypes.c_int
    for f in ("lq_quantize", "lq_dequantize", "lq_fake_quant_qsnr", "lq_hadamard_quant", "lq_workspace_init",
              "lq_sweep_tally", "lq_set_grid_limit"):
        getattr(L, f).restype = ctypes.c_int
    L.lq_set_grid_limit.argtypes = [ctypes.c_int]
    for f in ("lq_workspace_bytes", "lq_codes_bytes", "lq_scales_bytes", "lq_zeros_bytes"):
        getattr(L, f).argtypes = [dp, i64, i64]
        getattr(L, f).restype = sz
    L.lq_workspace_init.argtypes = [vp, sz, vp]
    L.lq_sweep_tally.argtypes = [ctypes.POINTER(ctypes.c_double), i64, ctypes.c_double, ctypes.c_double,
                                 ctypes.POINTER(ctypes.c_int32)]
    L.lq_call_kernels.argtypes = [dp, i64, i64, ctypes.c_uint32, ctypes.c_int, ctypes.c_char_p, sz]
    L.lq_call_kernels.restype = ctypes.c_int
    L.lq_status_string.argtypes = [ctypes.c_int]
    L.lq_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = L
    return L


def status_string(status: int) -> str:
    return load().lq_status_string(status).decode()


def desc(variant: dict, in_dtype: str, given: bool = False, signs_ptr: int | None = None) -> Desc:
    """Descriptor from a variant dict (fmt, gran, block, scale, sym, round, out, hadamard, two_level,
    tile_rows); signs_ptr: device address of the rotation's sign bits, or None."""
    return Desc(FORMAT[variant["fmt"]], GRAN[variant["gran"]], int(variant.get("block", 0) or 0),
                SCALE_FMT[variant["scale"]], 1 if variant.get("sym", True) else 0,
                ROUND[variant.get("round", "rne")], DTYPE[in_dtype], DTYPE[variant.get("out", "bf16")],
                int(variant.get("hadamard", 0)), 1 if given else 0, 1 if variant.get("two_level", False) else 0,
                int(variant.get("tile_rows", 0) or 0), signs_ptr)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(fn, rc):
    if rc != LQ_OK:
        raise LQError(fn, rc)


# ------------------------------------------------------------------ the ABI
def lq_quantize(d: Desc, x, rows, cols, codes, scales, zeros, ws, ws_bytes, stream=None, lib=None):
    L = lib or load()
    _check("lq_quantize", L.lq_quantize(ctypes.byref(d), _ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                        _ptr(zeros), _ptr(ws), ws_bytes, _stream(stream)))


def lq_dequantize(d: Desc, codes, scales, zeros, rows, cols, y, stream=None, lib=None):
    L = lib or load()
    _check("lq_dequantize", L.lq_dequantize(ctypes.byref(d), _ptr(codes), _ptr(scales), _ptr(zeros), rows, cols,
                                            _ptr(y), _stream(stream)))


def lq_fake_quant_qsnr(d: Desc, x, rows, cols, codes, scales, zeros, y, res, ws, ws_bytes, stream=None, lib=None):
    L = lib or load()
    _check("lq_fake_quant_qsnr", L.lq_fake_quant_qsnr(ctypes.byref(d), _ptr(x), rows, cols, _ptr(codes),
                                                      _ptr(scales), _ptr(zeros), _ptr(y), _ptr(res), _ptr(ws),
                                                      ws_bytes, _stream(stream)))


def lq_fake_quant_qsnr_static(d: Desc, x, rows, cols, codes, scales, zeros, y, res, stream=None, lib=None):
    L = lib or load()
    _check("lq_fake_quant_qsnr_static", L.lq_fake_quant_qsnr_static(ctypes.byref(d), _ptr(x), rows, cols,
                                                                    _ptr(codes), _ptr(scales), _ptr(zeros),
                                                                    _ptr(y), _ptr(res), _stream(stream)))


def lq_hadamard_quant(d: Desc, x, rows, cols, codes, scales, zeros, y, unrotate_y, res, ws, ws_bytes, stream=None,
                      lib=None):
    L = lib or load()
    _check("lq_hadamard_quant", L.lq_hadamard_quant(ctypes.byref(d), _ptr(x), rows, cols, _ptr(codes),
                                                    _ptr(scales), _ptr(zeros), _ptr(y), int(unrotate_y), _ptr(res),
                                                    _ptr(ws), ws_bytes, _stream(stream)))


def lq_workspace_bytes(d: Desc, rows, cols, lib=None) -> int:
    return (lib or load()).lq_workspace_bytes(ctypes.byref(d), rows, cols)


def lq_codes_bytes(d: Desc, rows, cols, lib=None) -> int:
    return (lib or load()).lq_codes_bytes(ctypes.byref(d), rows, cols)


def lq_scales_bytes(d: Desc, rows, cols, lib=None) -> int:
    return (lib or load()).lq_scales_bytes(ctypes.byref(d), rows, cols)


def lq_zeros_bytes(d: Desc, rows, cols, lib=None) -> int:
    return (lib or load()).lq_zeros_bytes(ctypes.byref(d), rows, cols)


def lq_workspace_init(ws, ws_bytes, stream=None, lib=None):
    L = lib or load()
    _check("lq_workspace_init", L.lq_workspace_init(_ptr(ws), ws_bytes, _stream(stream)))


def lq_set_grid_limit(max_workgroups: int, lib=None):
    L = lib or load()
    _check("lq_set_grid_limit", L.lq_set_grid_limit(int(max_workgroups)))


def lq_sweep_tally(qsnr: np.ndarray, tie_db: float, margin_db: float, lib=None) -> np.ndarray:
    """qsnr: [n_tensors, 5 formats, 5 granularities] -> counts [5 granularities, 3 pairs,
    4] = (INT wins, FP wins, ties, undecided)."""
    L = lib or load()
    q = np.ascontiguousarray(qsnr, dtype=np.float64).reshape(-1, 25)
    counts = np.zeros(60, np.int32)
    _check("lq_sweep_tally", L.lq_sweep_tally(q.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), q.shape[0],
                                              float(tie_db), float(margin_db),
                                              counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return counts.reshape(5, 3, 4)


def lq_call_kernels(d: Desc, rows, cols, outputs: int, unrotate_y: int = 0, lib=None) -> list:
    """[(kernel name, workgroups, threads per workgroup)] one call would launch, in order."""
    L = lib or load()
    n = L.lq_call_kernels(ctypes.byref(d), rows, cols, outputs, int(unrotate_y), None, 0)
    if n < 0:
        raise LQError("lq_call_kernels", n)
    buf = ctypes.create_string_buffer(512 * (n + 1))
    _check_count = L.lq_call_kernels(ctypes.byref(d), rows, cols, outputs, int(unrotate_y), buf, len(buf))
    assert _check_count == n
    out = []
    for line in buf.value.decode().splitlines():
        name, nwg, nt = line.rsplit("\t", 2)
        out.append((name, int(nwg), int(nt)))
    return out


def call_kernels(variant: dict, in_dtype: str, rows: int, cols: int,
                 want=("codes", "scales", "zeros", "y", "res"), lib=None) -> list:
    """Kernel names a fake-quant call of this variant with these outputs launches."""
    d = desc(variant, in_dtype, signs_ptr=64 if variant.get("signs") is not None else None)
    bits = sum(OUT[k] for k in want)
    un = bool(variant.get("unrotate", False)) if int(variant.get("hadamard", 0)) else 0
    return [k[0] for k in lq_call_kernels(d, rows, cols, bits, un, lib=lib)]


# ------------------------------------------------------------------ buffers
class Runner:
    """Device buffers for one (variant, shape, input dtype) and calls into the
    ABI. Buffers are torch tensors; sizes come from the library."""

    def __init__(self, variant: dict, rows: int, cols: int, in_dtype: str, device="cuda", given=False,
                 want=("codes", "scales", "zeros", "y", "res"), lib=None):
        import torch

        self.torch = torch
        self.lib = lib or load()
        self.v = variant
        self.rows, self.cols = rows, cols
        # the rotation's random signs (uint32 words, one bit per column) live on the device
        sg = variant.get("signs")
        self.signs = None if sg is None else torch.from_numpy(
            np.ascontiguousarray(sg, np.uint32).view(np.int32).copy()).to(device)
        self.d = desc(variant, in_dtype, given, None if self.signs is None else self.signs.data_ptr())
        self.given = given
        u8 = dict(dtype=torch.uint8, device=device)
        nb = lambda f: f(self.d, rows, cols, lib=self.lib)
        self.codes = torch.zeros(max(16, nb(lq_codes_bytes)), **u8) if "codes" in want else None
        self.scales = torch.zeros(max(16, nb(lq_scales_bytes)), **u8) if ("scales" in want or given) else None
        zb = nb(lq_zeros_bytes)
        self.zeros = torch.zeros(max(16, zb), **u8) if (zb and ("zeros" in want or given)) else None
        ob = {"f32": 4, "bf16": 2, "f16": 2}[variant.get("out", "bf16")]
        self.y = torch.zeros(max(16, rows * cols * ob), **u8) if "y" in want else None
        self.res = torch.zeros(64, **u8) if "res" in want else None
        self.ws_bytes = nb(lq_workspace_bytes)
        self.ws = torch.zeros(self.ws_bytes, **u8)
        lq_workspace_init(self.ws, self.ws_bytes, lib=self.lib)

    def fake_quant(self, x, unrotate=None, stream=None):
        if int(self.v.get("hadamard", 0)):
            un = self.v.get("unrotate", False) if unrotate is None else unrotate
            lq_hadamard_quant(self.d, x, self.rows, self.cols, self.codes, self.scales, self.zeros, self.y, un,
                              self.res, self.ws, self.ws_bytes, stream, lib=self.lib)
        else:
            lq_fake_quant_qsnr(self.d, x, self.rows, self.cols, self.codes, self.scales, self.zeros, self.y,
                               self.res, self.ws, self.ws_bytes, stream, lib=self.lib)

    def quantize(self, x, stream=None):
        lq_quantize(self.d, x, self.rows, self.cols, self.codes, self.scales, self.zeros, self.ws, self.ws_bytes,
                    stream, lib=self.lib)

    def dequantize(self, y=None, stream=None):
        lq_dequantize(self.d, self.codes, self.scales, self.zeros, self.rows, self.cols,
                      self.y if y is None else y, stream, lib=self.lib)

    def result(self) -> dict:
        """Read the device result struct (synchronises the current stream).
        `failed`: the library could not complete the sum (a partial record
        never arrived); the values are then NaN."""
        self.torch.cuda.current_stream().synchronize()
        raw = self.res[:ctypes.sizeof(Result)].cpu().numpy().tobytes()
        r = Result.from_buffer_copy(raw)
        return {"err2": r.err2, "sig2": r.sig2, "qsnr": r.qsnr_db, "nonfinite": r.nonfinite,
                "failed": r.reserved != 0}

    def host(self) -> dict:
        """Copy the outputs to host numpy arrays (bytes trimmed to their sizes)."""
        self.torch.cuda.current_stream().synchronize()
        n = lambda f: f(self.d, self.rows, self.cols, lib=self.lib)
        out = {}
        if self.codes is not None:
            out["codes"] = self.codes[:n(lq_codes_bytes)].cpu().numpy()
        if self.scales is not None:
            out["scales"] = self.scales[:n(lq_scales_bytes)].cpu().numpy()
        if self.zeros is not None:
            out["zeros"] = self.zeros[:n(lq_zeros_bytes)].cpu().numpy()
        if self.y is not None:
            ob = {"f32": 4, "bf16": 2, "f16": 2}[self.v.get("out", "bf16")]
            raw = self.y[:self.rows * self.cols * ob].cpu().numpy()
            out["y"] = raw.view(np.uint32 if ob == 4 else np.uint16).reshape(self.rows, self.cols)
        return out


# ------------------------------------------------------------------ ceilings
CEILING_PATH = os.path.join(_HERE, "liblq_ceiling.so")
CEILING_EXPORTS = ("lqc_copy", "lqc_pattern", "lqc_read", "lqc_write")
_ceiling = None


def load_ceiling(path: str | None = None):
    """Load liblq_ceiling.so (include/lq_ceiling.h): the copy, pattern, read-only and write-only kernels."""
    global _ceiling
    if _ceiling is not None and path is None:
        return _ceiling
    p = path or CEILING_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"liblq_ceiling not built: {p} is missing (run __graft_entry__.build())")
    L = ctypes.CDLL(p)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.lqc_copy.argtypes = [vp, sz, vp, sz, i64, ci, ci, vp]
    L.lqc_copy.restype = ci
    L.lqc_pattern.argtypes = [vp, sz, i64, vp, sz, ci, vp, sz, ci, vp, sz, ci, ci, vp]
    L.lqc_pattern.restype = ci
    L.lqc_read.argtypes = [vp, sz, i64, vp, sz, ci, ci, vp]
    L.lqc_read.restype = ci
    L.lqc_write.argtypes = [vp, sz, i64, ci, ci, vp]
    L.lqc_write.restype = ci
    if path is None:
        _ceiling = L
    return L


def _nbytes(t) -> int:
    """Byte size of a contiguous torch tensor from its data pointer on (the
    buffer the library may touch)."""
    if not t.is_contiguous():
        raise ValueError("the ceiling kernels take contiguous buffers")
    return t.numel() * t.element_size()


def lqc_copy(src, dst, n: int, threads: int, workgroups: int, stream=None, lib=None):
    L = lib or load_ceiling()
    rc = L.lqc_copy(_ptr(src), _nbytes(src), _ptr(dst), _nbytes(dst), n, threads, workgroups, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"lqc_copy returned {rc}")


def lqc_read(src, nbytes: int, sink, threads: int, workgroups: int, stream=None, lib=None):
    L = lib or load_ceiling()
    rc = L.lqc_read(_ptr(src), _nbytes(src), nbytes, _ptr(sink), _nbytes(sink), threads, workgroups, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"lqc_read returned {rc}")


def lqc_write(dst, nbytes: int, threads: int, workgroups: int, stream=None, lib=None):
    L = lib or load_ceiling()
    rc = L.lqc_write(_ptr(dst), _nbytes(dst), nbytes, threads, workgroups, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"lqc_write returned {rc}")


def lqc_pattern(x, n: int, codes, code_bits: int, scales, block: int, y, threads: int, workgroups: int,
                stream=None, lib=None):
    L = lib or load_ceiling()
    rc = L.lqc_pattern(_ptr(x), _nbytes(x), n, _ptr(codes), _nbytes(codes), code_bits, _ptr(scales), _nbytes(scales),
                       block, _ptr(y), _nbytes(y), threads, workgroups, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"lqc_pattern returned {rc}")
