"""Shared helpers of the GPU parity tests: upload seeded inputs, run one
variant through the C ABI, run the oracle on the same values, compare."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
from bit_quantization_block_amd import lq

QSNR_TOL_DB = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(d: dict):
    import torch

    raw = np.ascontiguousarray(d["bits"]).view(np.uint8).reshape(-1)
    return torch.from_numpy(raw.copy()).cuda()


def as_f16(d: dict) -> dict:
    """The same values as fp16 (inputs whose values fp16 holds exactly)."""
    x16 = d["x"].astype(np.float16)
    return {"dtype": "f16", "bits": x16.view(np.uint16), "x": x16.astype(np.float32)}


def run_gpu(v: dict, d: dict, xdev=None, given=None, want=("codes", "scales", "zeros", "y", "res")):
    rows, cols = d["x"].shape
    r = lq.Runner(v, rows, cols, d["dtype"], given=given is not None, want=want)
    if given is not None:
        import torch

        sc, zp = given
        r.scales[:sc.nbytes].copy_(torch.from_numpy(np.ascontiguousarray(sc).view(np.uint8).reshape(-1)))
        if zp is not None:
            r.zeros[:zp.nbytes].copy_(torch.from_numpy(np.ascontiguousarray(zp).view(np.uint8).reshape(-1)))
    xdev = upload(d) if xdev is None else xdev
    r.fake_quant(xdev)
    out = r.host()
    if r.res is not None:
        out.update(r.result())
    return out, r


def first_mismatch(a: np.ndarray, b: np.ndarray):
    idx = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
    if idx.size == 0:
        return None
    i = int(idx[0])
    return f"{idx.size} mismatches, first at flat index {i}: gpu={a.reshape(-1)[i]!r} oracle={b.reshape(-1)[i]!r}"


def split_two_level(scales: np.ndarray, n_blocks: int):
    """A two-level scales buffer: the E4M3 block scales, then the fp32 tensor
    scale at the next multiple of 16 bytes."""
    raw = np.ascontiguousarray(scales).view(np.uint8).reshape(-1)
    off = (n_blocks + 15) // 16 * 16
    return raw[:n_blocks], raw[off:off + 4].view(np.float32)[0]


def compare(v: dict, gpu: dict, ref: dict, what=("codes", "scales", "zeros", "y"), qsnr=True, label=""):
    for k in what:
        if k == "zeros" and v.get("sym", True):
            continue
        if ref.get(k) is None or k not in gpu:
            continue
        a = np.ascontiguousarray(gpu[k]).view(np.uint8).reshape(-1)
        b = np.ascontiguousarray(ref[k]).view(np.uint8).reshape(-1)
        if k == "scales" and v.get("two_level", False):
            a, ts = split_two_level(a, b.size)
            assert ts.view(np.uint32) == np.float32(ref["tscale"]).view(np.uint32), \
                f"{label} tensor scale of {v}: gpu {ts!r} oracle {ref['tscale']!r}"
        assert a.size == b.size, f"{label} {k}: size {a.size} vs {b.size}"
        mm = first_mismatch(a, b)
        assert mm is None, f"{label} {k} of {v}: {mm}"
    if qsnr:
        g, o = gpu["qsnr"], ref["qsnr"]
        if math.isinf(o):
            # +inf: no error at all; -inf: an x-hat that overflowed fp32 (the
            # error sum is infinite on both sides)
            assert g == o, (label, g, o)
        else:
            assert abs(g - o) <= QSNR_TOL_DB, f"{label} QSNR gpu {g} vs oracle {o} ({v})"
            assert math.isclose(gpu["sig2"], ref["sig2"], rel_tol=1e-5), (label, gpu["sig2"], ref["sig2"])


def check_variant(v: dict, d: dict, label="", xdev=None):
    say(f"[gpu] {label} {v} shape={d['x'].shape} dtype={d['dtype']}")
    gpu, _ = run_gpu(v, d, xdev=xdev)
    assert not gpu.get("failed", False), f"{label}: the QSNR sum did not complete"
    ref = oracle.fake_quant(v, d["x"])
    compare(v, gpu, ref, label=label)
    stat_bad = oracle.tensor_stat(v, d["x"])[1]
    assert gpu["nonfinite"] == stat_bad
    return gpu, ref
