"""The specialised kernel for 4-bit blocks of 16 with E4M3 scales under the
16-point rotation (NVFP4 / NVINT4 with H16, cyqw.cn/news/1000169 §4.2, §7.2):
bit-exact against the oracle on the values where its shortcuts need care
(zero quotients of either sign, all-zero and all-negative-zero blocks, tiny
blocks whose scale underflows to 0, tiny values beside large ones, saturated
scales and codes, exact ties of the element grids), with the rotation back
and without, over one and several chunks per wave, and with non-finite
inputs counted."""
import numpy as np
import pytest

import oracle
from bit_quantization_block_amd import lq
from bit_quantization_block_amd import workloads as W
from tests.gpu_helpers import check_variant, compare, run_gpu, say, upload

pytestmark = pytest.mark.gpu


def V(fmt, unrotate=True):
    return {"fmt": fmt, "gran": "block", "block": 16, "scale": "e4m3", "sym": True, "round": "rne", "out": "bf16",
            "hadamard": 16, "unrotate": unrotate}


def bf16_input(x32: np.ndarray) -> dict:
    return W._pack("bf16", x32)


def kernel_of(v, rows, cols):
    return lq.call_kernels(v, "bf16", rows, cols)[0]


def kernels_of(v, rows, cols):
    """Every kernel of a call (two-level: the statistic pass first)."""
    return " ".join(lq.call_kernels(v, "bf16", rows, cols))


def edge_values(rows, cols, seed):
    """t(3) data with planted blocks of edge values (every block is one row's
    16 consecutive columns)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (rows, cols)).astype(np.float32)
    blocks = x.reshape(-1, 16)
    nb = blocks.shape[0]
    pick = rng.permutation(nb)
    k = 0

    def take(m):
        nonlocal k
        out = pick[k:k + m]
        k += m
        return out

    blocks[take(8)] = 0.0                                              # zero scale
    blocks[take(8)] = -0.0                                             # zero scale, negative zeros
    for b in take(16):                                                 # zeros of both signs beside values
        blocks[b, rng.integers(0, 16, 6)] = rng.choice(np.float32([0.0, -0.0]), 6)
    for b in take(16):                                                 # scale underflows E4M3: codes 0
        blocks[b] = rng.standard_normal(16).astype(np.float32) * np.float32(1e-6)
    for b in take(16):                                                 # tiny next to large: zero codes, signs
        blocks[b] = rng.standard_normal(16).astype(np.float32) * np.float32(1e-30)
        blocks[b, rng.integers(0, 16)] = np.float32(rng.choice([-3.0, 5.0]))
    for b in take(16):                                                 # bf16 subnormals and the normal minimum
        blocks[b] = rng.choice(np.float32([1e-40, -1e-40, 1.1754944e-38, -2.3e-39, 0.0]), 16)
    for b in take(16):                                                 # scale saturates at 448
        blocks[b] = rng.standard_normal(16).astype(np.float32) * np.float32(3e4)
    for b in take(16):                                                 # values on exact grid midpoints
        blocks[b] = rng.choice(np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, 6.0, 7.5, -8.5]), 16)
    for b in take(16):                                                 # one value per block, the rest zero
        blocks[b] = 0.0
        blocks[b, rng.integers(0, 16)] = np.float32(rng.choice([-1.0, 2.0, 1e-3, -1e5]))
    return bf16_input(x)


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
@pytest.mark.parametrize("unrotate", [True, False])
def test_h16_edge_values(fmt, unrotate):
    v = V(fmt, unrotate)
    d = edge_values(64, 4096, seed=71 if fmt == "e2m1" else 72)
    assert "k_h16" in kernel_of(v, 64, 4096)
    check_variant(v, d, f"h16 {fmt} unrotate={unrotate}")


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
@pytest.mark.parametrize("limit", [0, 4, 1])
def test_h16_chunks_per_wave(fmt, limit):
    """One chunk of 1024 elements per wave, and several (a capped grid), with
    shapes whose element count is a multiple of 1024 but whose rows are not."""
    lq.lq_set_grid_limit(limit)
    try:
        for rows, cols in ((16, 4096), (3, 1024 * 7), (40, 1536)):
            d = edge_values(rows, cols, seed=rows + cols)
            v = V(fmt)
            assert "k_h16" in kernel_of(v, rows, cols), (rows, cols)
            check_variant(v, d, f"h16 {fmt} {rows}x{cols} limit {limit}")
    finally:
        lq.lq_set_grid_limit(0)


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
def test_h16_nonfinite_counted(fmt):
    """NaN and infinities are outside the contract: their blocks' outputs are
    unspecified, but every other block is exact and the count is right."""
    d = edge_values(32, 2048, seed=73)
    x = d["x"].copy()
    bad = [(3, 17), (9, 1000), (30, 2047)]
    for (r, c), val in zip(bad, (np.inf, -np.inf, np.nan)):
        x[r, c] = val
    d = bf16_input(x)
    v = V(fmt)
    gpu, _ = run_gpu(v, d)
    assert gpu["nonfinite"] == 3
    ref = oracle.fake_quant(v, d["x"])
    cb = oracle.codes_bytes(v, 1, 2048)
    for r in range(32):
        if r in [b[0] for b in bad]:
            continue
        assert np.array_equal(gpu["codes"][r * cb:(r + 1) * cb], ref["codes"][r * cb:(r + 1) * cb]), r
        assert np.array_equal(gpu["y"][r], ref["y"][r]), r


def test_h16_not_taken_outside_its_case():
    """Signs, other block sizes, other scale formats, 8-bit elements and fp32
    inputs take the general kernels."""
    base = V("e2m1")
    for change in (dict(block=32), dict(scale="ue8m0"), dict(fmt="int8", scale="ue8m0"),
                   dict(block=32, two_level=True)):
        assert "k_h16" not in kernels_of(dict(base, **change), 8, 4096), change
    assert "k_h16" not in lq.call_kernels(base, "f32", 8, 4096)[0]
    signed = dict(base, signs=W.rotation_signs(4096))
    assert "k_h16" not in kernel_of(signed, 8, 4096)
    assert "k_h16" not in kernel_of(base, 1, 1008)            # not a multiple of 1024 elements


# ---------------------------------------------------------------- two-level
def V2(fmt, unrotate=True):
    return dict(V(fmt, unrotate), two_level=True)


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
@pytest.mark.parametrize("unrotate", [True, False])
def test_h16_two_level_edge_values(fmt, unrotate):
    """NVFP4 / NVINT4 under H16 with an fp32 tensor scale above the E4M3 block
    scales (walkerchi.com playbook §4.3.2): the same planted blocks."""
    v = V2(fmt, unrotate)
    d = edge_values(64, 4096, seed=81 if fmt == "e2m1" else 82)
    assert "k_h16_two" in kernels_of(v, 64, 4096)
    check_variant(v, d, f"h16 two-level {fmt} unrotate={unrotate}")


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
@pytest.mark.parametrize("magnitude", [0.0, 1e-37, 1e-20, 3e4])
def test_h16_two_level_tensor_scales(fmt, magnitude):
    """Tensor scales at their edges: an all-zero tensor (S becomes 1), one so
    small that 1/S overflows (the divisions by S are taken on operands scaled
    by 2^64), tiny values and large ones."""
    rng = np.random.default_rng(83)
    x = (rng.standard_t(3, (16, 2048)) * magnitude).astype(np.float32)
    v = V2(fmt)
    assert "k_h16_two" in kernels_of(v, 16, 2048)
    check_variant(v, bf16_input(x), f"h16 two-level {fmt} magnitude {magnitude}")


@pytest.mark.parametrize("fmt", ["e2m1", "int4"])
@pytest.mark.parametrize("limit", [0, 4, 1])
def test_h16_two_level_chunks_per_wave(fmt, limit):
    """The two-level kernel over one and several chunks per wave."""
    lq.lq_set_grid_limit(limit)
    try:
        for rows, cols in ((16, 4096), (3, 1024 * 7), (40, 1536)):
            d = edge_values(rows, cols, seed=rows + cols + 1)
            v = V2(fmt)
            assert "k_h16_two" in kernels_of(v, rows, cols), (rows, cols)
            check_variant(v, d, f"h16 two-level {fmt} {rows}x{cols} limit {limit}")
    finally:
        lq.lq_set_grid_limit(0)
