"""Pins for the oracle's sweep post-processing (INT-vs-FP win counts, the
tensor-level analogue of cyqw.cn/news/1000169 §5.1) and for the 6-bit branch
of its dequantizer.

The win-count tables below are written by hand: every expected count is a
literal, so a wrong pair, a transposed table index, a swapped winner or a
band edge on the wrong side fails one of them."""
import math

import numpy as np
import pytest

from tests import bruteforce as bf

INT8, INT4, E4M3, E5M2, E2M1 = range(5)
PAIR = {"int8-e4m3": 0, "int8-e5m2": 1, "int4-e2m1": 2}
WIN_INT, WIN_FP, TIE, UNDECIDED = range(4)


def table(n):
    """n tensors, every QSNR 30 dB (all pairs tie) until set."""
    return np.full((n, 5, 5), 30.0, np.float64)


def test_tally_pairs_and_slots(oracle_mod):
    """One tensor, different outcomes per pair and per granularity slot."""
    q = table(1)
    q[0, INT8, :] = 40.0
    q[0, E4M3, :] = 31.0           # INT8 beats E4M3 everywhere ...
    q[0, E5M2, :] = 45.0           # ... and loses to E5M2 everywhere
    q[0, INT4, :] = 20.0
    q[0, E2M1, :] = 20.001         # INT4 vs E2M1: within 0.01 dB, a tie
    q[0, INT8, 3] = 10.0           # slot 3 (blocks of 32): INT8 now loses both
    q[0, E2M1, 1] = 25.0           # slot 1 (per channel): E2M1 wins
    got = oracle_mod.sweep_tally(q)
    want = np.zeros((5, 3, 4), np.int32)
    for g in range(5):
        want[g, 0] = [1, 0, 0, 0]
        want[g, 1] = [0, 1, 0, 0]
        want[g, 2] = [0, 0, 1, 0]
    want[3, 0] = [0, 1, 0, 0]
    want[1, 2] = [0, 1, 0, 0]
    assert np.array_equal(got, want), got


def test_tally_band_edges(oracle_mod):
    """tie 0.25 dB, margin 0.0625 dB (both exact in binary): the band edge sits
    at 0.25, undecided from 0.1875 to 0.3125 inclusive. Differences placed
    exactly on, just inside and just outside each edge, both signs."""
    diffs_and_class = [
        (0.0, TIE), (0.1, TIE), (0.1875 - 2 ** -20, TIE),
        (0.1875, UNDECIDED), (0.2, UNDECIDED), (0.25, UNDECIDED), (0.3, UNDECIDED), (0.3125, UNDECIDED),
        (0.3125 + 2 ** -20, WIN_INT), (1.0, WIN_INT),
        (-0.1875 + 2 ** -20, TIE), (-0.1875, UNDECIDED), (-0.3125, UNDECIDED),
        (-0.3125 - 2 ** -20, WIN_FP), (-7.0, WIN_FP),
    ]
    n = len(diffs_and_class)
    q = table(n)
    for t, (d, _) in enumerate(diffs_and_class):
        q[t, INT8, 2] = 40.0 + d       # only (slot 2, INT8 vs E4M3) varies
        q[t, E4M3, 2] = 40.0
    got = oracle_mod.sweep_tally(q, tie_db=0.25, margin_db=0.0625)
    # 2 INT wins, 2 FP wins, 4 ties, 7 undecided, counted by hand from the list
    assert list(got[2, PAIR["int8-e4m3"]]) == [2, 2, 4, 7]
    # the same INT8 values beat E5M2's 30 dB at slot 2 in all 15 tensors
    assert list(got[2, PAIR["int8-e5m2"]]) == [15, 0, 0, 0]
    # every other pair of every slot: 30 vs 30, a tie in each tensor
    rest = got.copy()
    rest[2, :2] = 0
    assert rest[..., TIE].sum() == 13 * n and rest[..., [WIN_INT, WIN_FP, UNDECIDED]].sum() == 0


def test_tally_infinities_and_nan(oracle_mod):
    """+inf is an error-free quantization: equal to another +inf, better than
    any finite QSNR; -inf (an overflowed x-hat) loses to anything finite; a
    NaN QSNR decides nothing."""
    inf, nan = math.inf, math.nan
    cases = [((inf, inf), TIE), ((inf, 50.0), WIN_INT), ((50.0, inf), WIN_FP), ((-inf, -inf), TIE),
             ((-inf, 3.0), WIN_FP), ((nan, 30.0), UNDECIDED), ((30.0, nan), UNDECIDED), ((nan, nan), UNDECIDED)]
    q = table(len(cases))
    for t, ((qi, qf), _) in enumerate(cases):
        q[t, INT4, 4] = qi             # slot 4 (blocks of 64), INT4 vs E2M1
        q[t, E2M1, 4] = qf
    got = oracle_mod.sweep_tally(q)
    assert list(got[4, PAIR["int4-e2m1"]]) == [1, 2, 2, 3]


def test_tally_antisymmetric(oracle_mod):
    """Swapping each pair's two QSNRs swaps INT and FP wins and keeps ties and
    undecided pairs (random tables with differences crowding the band)."""
    rng = np.random.default_rng(11)
    q = 30.0 + rng.choice([-1.0, 1.0], (64, 5, 5)) * rng.choice([0.0, 0.005, 0.0079, 0.0101, 0.0119, 0.02, 2.0],
                                                               (64, 5, 5))
    sw = q.copy()
    sw[:, [INT8, INT4]] = q[:, [E4M3, E2M1]]
    sw[:, [E4M3, E2M1]] = q[:, [INT8, INT4]]
    a = oracle_mod.sweep_tally(q)
    b = oracle_mod.sweep_tally(sw)
    # pairs 0 and 2 swap their operands exactly; pair 1 (INT8 vs E5M2) changed INT8 only
    for p in (0, 2):
        assert np.array_equal(a[:, p, [WIN_INT, WIN_FP, TIE, UNDECIDED]], b[:, p, [WIN_FP, WIN_INT, TIE, UNDECIDED]])
    assert a.sum() == b.sum() == 64 * 15


def test_tally_rejects_bad_arguments(oracle_mod):
    q = table(2)
    for tie, margin in ((0.01, 0.01), (0.01, 0.02), (0.01, -1e-3), (0.0, 0.0)):
        with pytest.raises(ValueError):
            oracle_mod.sweep_tally(q, tie_db=tie, margin_db=margin)
    assert oracle_mod.sweep_tally(np.zeros((0, 5, 5))).sum() == 0


# ---------------------------------------------------------------- FP6 dequant
def pack6(codes: np.ndarray) -> np.ndarray:
    """Element e's six bits at bits 6e .. 6e+5 of the byte stream, low bits
    first: written bit by bit, independently of the oracle."""
    bits = ((codes.reshape(-1, 1) >> np.arange(6)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bits, bitorder="little")


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("scale", ["ue8m0", "e4m3", "f32"])
def test_fp6_dequant_bit_by_bit(oracle_mod, fmt, scale):
    """Every 6-bit code in every position of a group, under random stored
    scales: value from the layout-derived table times the scale in binary32,
    rounded to bf16 (and to fp32 / fp16 for the other outputs)."""
    rng = np.random.default_rng(5)
    rows, cols, block = 6, 128, 32
    codes = rng.integers(0, 64, (rows, cols))
    codes[0, :64] = np.arange(64)
    nsc = rows * cols // block
    if scale == "ue8m0":
        sc = rng.integers(127 - 30, 127 + 30, nsc).astype(np.uint8)
        s32 = np.ldexp(np.float32(1.0), sc.astype(np.int32) - 127).astype(np.float32)
    elif scale == "e4m3":
        sc = rng.integers(0, 0x7F, nsc).astype(np.uint8)        # every finite positive E4M3 scale but NaN
        s32 = np.array([bf.TABLES["e4m3"][int(c)] for c in sc], np.float32)
    else:
        s32 = (rng.standard_normal(nsc) ** 2 + 1e-3).astype(np.float32)
        sc = s32.view(np.uint32)
    vals = np.array([[bf.TABLES[fmt][int(c)] for c in row] for row in codes], np.float32)
    xhat = (vals.reshape(-1, block) * np.repeat(s32, 1).reshape(-1, 1)).astype(np.float32).reshape(rows, cols)
    for out in ("bf16", "f32", "f16"):
        v = {"fmt": fmt, "gran": "block", "block": block, "scale": scale, "sym": True, "out": out}
        y = oracle_mod.dequant(v, pack6(codes), sc, None, rows, cols)
        assert np.array_equal(y, bf.y_bits(out, xhat)), (fmt, scale, out)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_dequant_round_trip(oracle_mod, fmt):
    """Dequantizing the oracle's own FP6 codes and scales reproduces the y its
    fake-quant wrote (per block, per channel, per tensor)."""
    x = np.random.default_rng(8).standard_t(3, (16, 256)).astype(np.float32)
    for gran, block, scale in (("block", 32, "ue8m0"), ("block", 16, "e4m3"), ("channel", 0, "f32"),
                               ("tensor", 0, "f32")):
        v = {"fmt": fmt, "gran": gran, "block": block, "scale": scale, "sym": True, "out": "bf16"}
        o = oracle_mod.fake_quant(v, x)
        y = oracle_mod.dequant(v, o["codes"], o["scales"], None, 16, 256)
        assert np.array_equal(y, o["y"]), (fmt, gran)
