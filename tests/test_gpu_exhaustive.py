"""Every float32 in [-1, 1] through the quantisers at unit scale, against the
oracle: 2,130,706,434 values (+0 .. 1 and -0 .. -1 by bit pattern), each in a
block of 64 whose first element is 1.0, so the block absmax is exactly 1 and
the decision for x is "how many level midpoints lie below x".  Checked on the
first-level NF4 route, the one-pass quantise + DQ route and the single INT4
quantiser, every packed byte bit-exact.

The NF4 levels and their nearest-level rule follow "QLoRAの理論と実装",
§5-1 (NormalFloat, the argmin over the 16 levels); INT4 is the page's uniform
comparison code.  The oracle runs on the host in a thread pool over whole
blocks."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from oracle.quant import quantize_nf4
from oracle.variants import INT4, quantize_4bit

from support import f32_bits, host_threads, say, u8

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")

ONE_BITS = 0x3F800000
HALF = ONE_BITS + 1            # +0 .. 1.0 (and -0 .. -1.0) by bit pattern
TOTAL = 2 * HALF
PER_BLOCK = 63                 # values per block besides the leading 1.0
CHUNK_BLOCKS = 1 << 21
CHUNK = PER_BLOCK * CHUNK_BLOCKS
SUB_BLOCKS = 1 << 17           # oracle work item: 8,388,608 elements


def _chunk(c):
    """Flat float32 weight of chunk c: blocks [1.0, 63 enumerated values]; the
    last chunk's tail is zero-filled."""
    lo, hi = c * CHUNK, min((c + 1) * CHUNK, TOTAL)
    nb = -(-(hi - lo) // PER_BLOCK)
    v = np.zeros(nb * PER_BLOCK, np.uint32)
    # the part of [lo, hi) below HALF holds positive patterns, the rest negative ones
    cut = min(max(HALF - lo, 0), hi - lo)
    v[:cut] = np.arange(lo, lo + cut, dtype=np.uint32)
    v[cut:hi - lo] = np.arange(0x80000000 + max(lo - HALF, 0),
                               0x80000000 + (hi - HALF), dtype=np.uint32)[: hi - lo - cut]
    blocks = np.empty((nb, 64), np.float32)
    blocks[:, 0] = 1.0
    blocks[:, 1:] = v.view(np.float32).reshape(nb, PER_BLOCK)
    return blocks.ravel(), hi - lo


def _oracle(flat, ex):
    starts = range(0, flat.size, SUB_BLOCKS * 64)

    def one(s):
        part = flat[s:s + SUB_BLOCKS * 64]
        return quantize_nf4(part)[0], quantize_4bit(part, INT4)[0]

    parts = list(ex.map(one, starts))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def _first_bad(got, ref, what, c):
    bad = np.nonzero(got != ref)[0]
    if bad.size:
        raise AssertionError(f"chunk {c} {what}: {bad.size} bytes differ, first at byte "
                             f"{bad[:4]} (got {got[bad[:4]]}, oracle {ref[bad[:4]]})")


NCHUNKS = -(-TOTAL // CHUNK)


@pytest.mark.parametrize("c", range(NCHUNKS))
def test_every_float32_in_unit_interval(c):
    """Chunk c of the 17 (132,120,576 values each, the last one shorter)."""
    flat, nvals = _chunk(c)
    say(f"[exhaustive] chunk {c + 1}/{NCHUNKS}: {nvals} values, {flat.size // 64} blocks")
    w = torch.from_numpy(flat).to("cuda:0")
    p1, a1 = q.quantize_nf4(w)
    p2, _, _ = q.quantize_nf4_dq(w, one_pass=True)
    p3, a3 = q.quantize_4bit(w, "int4")
    with threadpool_limits(1), ThreadPoolExecutor(host_threads()) as ex:
        ref_nf4, ref_int4 = _oracle(flat, ex)
    assert np.all(f32_bits(a1) == ONE_BITS) and np.all(f32_bits(a3) == ONE_BITS)
    _first_bad(u8(p1), ref_nf4, "NF4 first level", c)
    _first_bad(u8(p2), ref_nf4, "NF4 one-pass quantise + DQ", c)
    _first_bad(u8(p3), ref_int4, "INT4", c)
