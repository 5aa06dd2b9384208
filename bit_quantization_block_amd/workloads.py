"""Seeded synthetic inputs and the variant lists of the five workloads.

This module holds no quantization arithmetic: it draws seeded random tensors
(numpy), rounds them to bf16 with torch's round-to-nearest-even cast, and names
the quantization variants each workload runs. Both the CPU oracle and the HIP
path read the exact same values from here.

Shapes and distributions stand in for the pages' missing real tensors
(10,752 LLM tensors in cyqw.cn/news/1000169 §4.2): LLM layer shapes (hidden
4096, MLP 11008 as in Llama-7B), near-normal weights, activation outlier
channels (x100), Student-t heavy tails and uniform data (the distributions
compared in m.youleyou.com/wenzhang/3165839 §3.1).
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------ inputs


def to_bf16(x32: np.ndarray):
    """Round fp32 values to bf16 (RNE, torch cast). Returns (bits uint16, values fp32)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = t.float().numpy().copy()
    return bits, vals


def _pack(dtype: str, x32: np.ndarray) -> dict:
    if dtype == "bf16":
        bits, vals = to_bf16(x32)
        return {"dtype": "bf16", "bits": bits, "x": vals}
    x = np.ascontiguousarray(x32, dtype=np.float32)
    return {"dtype": "f32", "bits": x.view(np.uint32), "x": x}


def c1_input(rows: int = 1024, cols: int = 1024, seed: int = 0) -> dict:
    """fp32 N(0,1)."""
    rng = np.random.default_rng(seed)
    return _pack("f32", rng.standard_normal((rows, cols), dtype=np.float32))


def c2_input(rows: int = 8192, cols: int = 4096, seed: int = 2, n_outlier_cols: int = 8,
             factor: float = 100.0) -> dict:
    """bf16 activations: N(0,1) with `n_outlier_cols` seeded columns scaled x100."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    cols_sel = rng.choice(cols, size=min(n_outlier_cols, cols), replace=False)
    x[:, cols_sel] *= np.float32(factor)
    return _pack("bf16", x)


def c3_input(rows: int = 11008, cols: int = 4096, seed: int = 3, sigma: float = 0.02) -> dict:
    """bf16 weights N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
    return _pack("bf16", x)


def c4_input(rows: int = 16384, cols: int = 8192, seed: int = 4, nu: float = 3.0) -> dict:
    """bf16 Student-t(nu) activations (drawn in float64, then fp32, then bf16)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(nu, size=(rows, cols)).astype(np.float32)
    return _pack("bf16", x)


C5_KINDS = ("uniform", "normal", "t3_outliers")


def c5_kind(i: int) -> str:
    """Tensor i of the sweep: kind i mod 3 (86 uniform, 85 normal, 85 t(3) of 256)."""
    return C5_KINDS[i % 3]


def c5_input(i: int, rows: int = 4096, cols: int = 4096, seed_base: int = 5000,
             outlier_frac: float = 0.001, outlier_factor: float = 50.0) -> dict:
    """bf16 tensor i of the 256-tensor sweep: U(-1,1), N(0,1), or t(3) with a
    fraction of entries (chosen without replacement) scaled x50."""
    rng = np.random.default_rng(seed_base + i)
    kind = c5_kind(i)
    if kind == "uniform":
        x = rng.uniform(-1.0, 1.0, size=(rows, cols)).astype(np.float32)
    elif kind == "normal":
        x = rng.standard_normal((rows, cols), dtype=np.float32)
    else:
        x = rng.standard_t(3.0, size=(rows, cols)).astype(np.float32)
        n = rows * cols
        k = max(1, int(round(n * outlier_frac)))
        idx = rng.choice(n, size=k, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_factor)
    out = _pack("bf16", x)
    out["kind"] = kind
    return out


def special_values_input(rows: int, cols: int, seed: int = 7) -> dict:
    """fp32 tensor mixing edge values: exact zeros, negative zeros, tiny and
    subnormal magnitudes, ties of common grids, and large values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    flat = x.reshape(-1)
    n = flat.size
    pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38, -2.5e-39, 0.25, -0.75, 1.25,
                     2.5, -3.5, 5.0, 448.0, -464.0, 57344.0, 6.0, 1e30, -1e-30],
                    dtype=np.float32)
    idx = rng.choice(n, size=min(n, n // 4), replace=False)
    flat[idx] = pool[rng.integers(0, pool.size, size=idx.size)]
    return _pack("f32", x)


# ---------------------------------------------------------------- variants
def _v(fmt, gran, scale, block=0, sym=True, out="bf16", hadamard=0, unrotate=False, rnd="rne"):
    return {"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": sym,
            "round": rnd, "out": out, "hadamard": hadamard, "unrotate": unrotate}


def c1_variants():
    """Per-tensor symmetric INT8 (absmax/127) and E4M3 (absmax/448), fp32 scale and dequant."""
    return [_v("int8", "tensor", "f32", out="f32"), _v("e4m3", "tensor", "f32", out="f32")]


def c2_variants():
    """MXINT8, MXFP8-E4M3, MXFP8-E5M2: blocks of 32, UE8M0 scales, bf16 dequant."""
    return [_v(f, "block", "ue8m0", block=32) for f in ("int8", "e4m3", "e5m2")]


def c3_variants():
    """INT4 group 64 symmetric and group 128 asymmetric, fp16 scales (and zeros)."""
    return [_v("int4", "block", "f16", block=64), _v("int4", "block", "f16", block=128, sym=False)]


def c4_variants():
    """E2M1 and INT4, blocks of 16 with E4M3 scales, without and with the H16 rotation
    (dequant written back in the original domain)."""
    out = []
    for had in (0, 16):
        for f in ("e2m1", "int4"):
            out.append(_v(f, "block", "e4m3", block=16, hadamard=had, unrotate=bool(had)))
    return out


def c4t_variants():
    """C4 with NVFP4's two-level scaling (an FP32 tensor scale above the E4M3
    block scales; walkerchi.com playbook §4.3.1-§4.3.2): E2M1 and INT4, blocks
    of 16, without and with the H16 rotation."""
    return [dict(v, two_level=True) for v in c4_variants()]


def rotation_signs(cols: int, seed: int = 1234) -> np.ndarray:
    """Random ±1 signs for a rotation, one bit per column (bit j of word j//32
    set: column j negated), drawn from numpy's generator with `seed`."""
    bits = np.random.default_rng(seed).integers(0, 2, cols, dtype=np.uint64)
    words = np.zeros((cols + 31) // 32, np.uint64)
    np.bitwise_or.at(words, np.arange(cols) // 32, bits << (np.arange(cols, dtype=np.uint64) % 32))
    return words.astype(np.uint32)


def c4r_variants():
    """C4's NVINT4 / NVFP4 blocks under QuaRot's randomized Hadamard rotation
    (walkerchi.com playbook §5.3) of 256 columns, dequantized output rotated
    back."""
    signs = rotation_signs(8192)
    return [dict(_v(f, "block", "e4m3", block=16), hadamard=256, unrotate=True, signs=signs)
            for f in ("e2m1", "int4")]


def c4q_variants():
    """As c4r with rotation groups of 1024 columns (a whole wave of lanes)."""
    signs = rotation_signs(8192)
    return [dict(_v(f, "block", "e4m3", block=16), hadamard=1024, unrotate=True, signs=signs)
            for f in ("e2m1", "int4")]


def c7_variants():
    """MXFP6 (walkerchi.com playbook §4.1 table): E2M3 and E3M2, blocks of 32
    with UE8M0 scales."""
    return [_v(f, "block", "ue8m0", block=32) for f in ("e2m3", "e3m2")]


def c6_variants():
    """DeepSeek-V3 style FP8 tiles (walkerchi.com playbook §4.4): E4M3 elements
    with fp32 scales, 128x128 tiles (weights) and 1x128 tiles (activations)."""
    return [dict(_v("e4m3", "tile", "f32", block=128), tile_rows=128),
            dict(_v("e4m3", "tile", "f32", block=128), tile_rows=1)]


C5_FORMATS = ("int8", "int4", "e4m3", "e5m2", "e2m1")
C5_GRANS = ("tensor", "channel", "b16", "b32", "b64")


def c5_variants():
    """5 formats x {tensor, channel, block 16/32/64}: fp32 scales per tensor and per
    channel; UE8M0 block scales for 8-bit formats (MX style), E4M3 for 4-bit
    (NV style). Order: format-major, matching lq_sweep_tally's table."""
    out = []
    for f in C5_FORMATS:
        four = f in ("int4", "e2m1")
        for g in C5_GRANS:
            if g == "tensor":
                out.append(_v(f, "tensor", "f32"))
            elif g == "channel":
                out.append(_v(f, "channel", "f32"))
            else:
                out.append(_v(f, "block", "e4m3" if four else "ue8m0", block=int(g[1:])))
    return out


WORKLOADS = {
    "c1": {"input": c1_input, "variants": c1_variants, "shape": (1024, 1024), "dtype": "f32"},
    "c2": {"input": c2_input, "variants": c2_variants, "shape": (8192, 4096), "dtype": "bf16"},
    "c3": {"input": c3_input, "variants": c3_variants, "shape": (11008, 4096), "dtype": "bf16"},
    "c4": {"input": c4_input, "variants": c4_variants, "shape": (16384, 8192), "dtype": "bf16"},
    "c4t": {"input": c4_input, "variants": c4t_variants, "shape": (16384, 8192), "dtype": "bf16"},
    "c6": {"input": c3_input, "variants": c6_variants, "shape": (11008, 4096), "dtype": "bf16"},
    "c4r": {"input": c4_input, "variants": c4r_variants, "shape": (16384, 8192), "dtype": "bf16"},
    "c4q": {"input": c4_input, "variants": c4q_variants, "shape": (16384, 8192), "dtype": "bf16"},
    "c7": {"input": c2_input, "variants": c7_variants, "shape": (8192, 4096), "dtype": "bf16"},
}


def algorithmic_bytes(v: dict, rows: int, cols: int, in_bytes: int) -> int:
    """Bytes the method must move for one fake-quant call: read x once, write
    codes, scales, zeros (asymmetric) and the dequantized y once."""
    n = rows * cols
    codes = n * 3 // 4 if v["fmt"] in ("e2m3", "e3m2") else n // 2 if v["fmt"] in ("int4", "e2m1") else n
    sb = {"f32": 4, "f16": 2, "ue8m0": 1, "e4m3": 1}[v["scale"]]
    if v["gran"] == "tensor":
        ns = 1
    elif v["gran"] == "channel":
        ns = rows
    elif v["gran"] == "tile":
        ns = -(-rows // v["tile_rows"]) * (cols // v["block"])
    else:
        ns = n // v["block"]
    zeros = 0 if v.get("sym", True) else ns * sb
    ob = {"f32": 4, "bf16": 2, "f16": 2}[v.get("out", "bf16")]
    tensor_scale = 4 if v.get("two_level", False) else 0
    return n * in_bytes + codes + ns * sb + zeros + tensor_scale + n * ob
