"""The ceiling kernels (include/lq_ceiling.h) write exactly what the header
says and nothing past the sizes they are given: every output byte against a
numpy model of the pattern, and guard bytes after each buffer unchanged, for
4-, 6- and 8-bit codes, small and large blocks, both workgroup sizes and
grids that give a wave several chunks."""
import numpy as np
import pytest

from bit_quantization_block_amd import lq
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5


def guarded(torch, nbytes):
    """A buffer of nbytes followed by GUARD sentinel bytes; returns (whole, view)."""
    whole = torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    return whole, whole[:nbytes]


def expected(xbits: np.ndarray, code_bits: int, block: int):
    """Codes and scales of the pattern for bf16 bit patterns xbits (uint16)."""
    n = xbits.size
    hb = (xbits >> 8).astype(np.uint8)                      # each element's high byte
    if code_bits == 8:
        codes = hb.copy()
    elif code_bits == 4:
        nib = hb >> 4
        codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    else:
        # per chunk, half and lane: 6 bytes at 384 * half + 6 * lane, from the
        # high bytes of the lane's 8 elements: even lanes hb0..hb5, odd lanes
        # hb4 hb5 hb0 hb1 hb2 hb3
        g = hb.reshape(-1, 2, 64, 8)                          # chunk, half, lane, element
        six = np.empty((g.shape[0], 2, 64, 6), np.uint8)
        six[:, :, 0::2, :] = g[:, :, 0::2, :6]
        six[:, :, 1::2, :2] = g[:, :, 1::2, 4:6]
        six[:, :, 1::2, 2:] = g[:, :, 1::2, :4]
        codes = six.reshape(-1)
    scales = hb[1::block][: n // block].copy()             # high byte of element 1 of each block
    return codes, scales


@pytest.mark.parametrize("code_bits", [4, 6, 8])
@pytest.mark.parametrize("block,threads,workgroups", [(16, 256, 5), (32, 1024, 1), (256, 256, 64)])
def test_pattern_writes_exactly_its_buffers(code_bits, block, threads, workgroups):
    import torch

    n = 1024 * 37
    say(f"lqc_pattern n={n} code_bits={code_bits} block={block} threads={threads} workgroups={workgroups}")
    rng = np.random.default_rng(code_bits * 1000 + block)
    xbits = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    x = torch.from_numpy(xbits.view(np.uint8).copy()).cuda()
    cw, cv = guarded(torch, n // 8 * code_bits)
    sw, sv = guarded(torch, n // block)
    yw, yv = guarded(torch, 2 * n)
    lq.lqc_pattern(x, n, cv, code_bits, sv, block, yv, threads, workgroups)
    torch.cuda.synchronize()
    codes, scales = expected(xbits, code_bits, block)
    assert np.array_equal(cv.cpu().numpy(), codes)
    assert np.array_equal(sv.cpu().numpy(), scales)
    assert np.array_equal(yv.cpu().numpy(), xbits.view(np.uint8))
    for w, size in ((cw, cv.numel()), (sw, sv.numel()), (yw, yv.numel())):
        assert bool((w[size:] == SENTINEL).all()), "a guard byte changed"


@pytest.mark.parametrize("threads,workgroups", [(256, 3), (1024, 40)])
def test_copy_writes_exactly_its_buffer(threads, workgroups):
    import torch

    n = 1024 * 29
    say(f"lqc_copy n={n} threads={threads} workgroups={workgroups}")
    src = torch.randint(0, 256, (2 * n,), dtype=torch.uint8, device="cuda")
    dw, dv = guarded(torch, 2 * n)
    lq.lqc_copy(src, dv, n, threads, workgroups)
    torch.cuda.synchronize()
    assert torch.equal(dv, src)
    assert bool((dw[2 * n:] == SENTINEL).all())


@pytest.mark.parametrize("threads,workgroups", [(256, 3), (1024, 5)])
def test_write_writes_exactly_its_bytes(threads, workgroups):
    """Every 16-byte unit of the write stream holds the values the header
    describes (made from its 1 KB unit's index), and nothing past `bytes`."""
    import torch

    nbytes = 1024 * 37
    say(f"lqc_write bytes={nbytes} threads={threads} workgroups={workgroups}")
    dw, dv = guarded(torch, nbytes)
    lq.lqc_write(dv, nbytes, threads, workgroups)
    torch.cuda.synchronize()
    got = dv.cpu().numpy().view(np.uint32).reshape(-1, 64, 4)
    u = np.arange(nbytes // 1024, dtype=np.uint32)[:, None]
    lane = np.arange(64, dtype=np.uint32)[None, :]
    assert np.array_equal(got[:, :, 0], np.broadcast_to(u, (u.size, 64)))
    assert np.array_equal(got[:, :, 1], u ^ lane)
    assert np.array_equal(got[:, :, 2], np.broadcast_to(u + 1, (u.size, 64)))
    assert np.array_equal(got[:, :, 3], np.broadcast_to(~u, (u.size, 64)))
    assert bool((dw[nbytes:] == SENTINEL).all())


@pytest.mark.parametrize("threads,workgroups", [(256, 3), (1024, 5)])
def test_read_touches_only_its_sink(threads, workgroups):
    """The read stream writes nothing but (at most) its sink's words, and
    nothing at all when no lane's fold equals the fixed value."""
    import torch

    nbytes = 2048 * 29
    say(f"lqc_read bytes={nbytes} threads={threads} workgroups={workgroups}")
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")        # every fold is 0
    sink_bytes = 4 * workgroups * (threads // 64)
    sw, sv = guarded(torch, sink_bytes)
    lq.lqc_read(src, nbytes, sv, threads, workgroups)
    torch.cuda.synchronize()
    assert bool((sw == SENTINEL).all())
    assert bool((src == 0).all())


def test_undersized_buffers_are_refused_before_launch():
    import torch

    n = 2048
    x = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
    y = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(n // 16, dtype=torch.uint8, device="cuda")
    short = torch.zeros(n // 8 * 6 - 16, dtype=torch.uint8, device="cuda")   # 6-bit codes need 3n/4
    with pytest.raises(RuntimeError, match="returned -3"):
        lq.lqc_pattern(x, n, short, 6, scales, 16, y, 256, 2)
    with pytest.raises(RuntimeError, match="returned -3"):
        lq.lqc_copy(x, y[: 2 * n - 16], n, 256, 2)
    with pytest.raises(RuntimeError, match="returned -3"):
        lq.lqc_write(y[: 2 * n - 1024], 2 * n, 256, 2)
    with pytest.raises(RuntimeError, match="returned -3"):
        lq.lqc_read(x, 2 * n, scales[:31], 256, 8)                       # 8 workgroups of 4 waves: 128 sink bytes
    assert bool((short == 0).all()) and bool((y == 0).all())
