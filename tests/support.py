"""Helpers shared by the GPU parity tests (imports the oracle: test-side only)."""

import sys

import numpy as np
import torch

from oracle.quant import (
    bf16_to_f64,
    block_absmax,
    dequantize_nf4,
    double_quant,
    quantize_nf4,
)

TOL = 1e-2  # max |gpu - ref| <= TOL * max |ref|, per tensor


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu()


def u8(t):
    return host(t).numpy().view(np.uint8)


def bf16_bits(t):
    return host(t).contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_bits(t):
    return host(t).numpy().view(np.uint32)


def assert_close(name, got, ref, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    assert np.all(np.isfinite(got)), name
    rel = err / scale if scale > 0 else err
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {rel:.2e}")
    assert err <= tol * scale or (scale == 0 and err == 0), (name, err, scale)
    return rel


def oracle_weight(W):
    """Oracle NF4 + DQ of a float32 [n_out][k_in]: dict of the storage arrays and
    the decoded bf16 weight (uint16 bits) and its float64 values."""
    flat = np.ascontiguousarray(W, dtype=np.float32).ravel()
    packed, absmax = quantize_nf4(flat)
    q, c2 = double_quant(absmax)
    w_hat = dequantize_nf4(packed, q, c2, flat.size).reshape(W.shape)
    return dict(packed=packed, absmax=absmax, q=q, c2=c2, w_hat=w_hat, w64=bf16_to_f64(w_hat))


def host_threads():
    """Host threads the parity harness may use (the CPU share this process has,
    at most 16)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_weight_parallel(W, threads=None, chunk_groups=64):
    """oracle_weight(W) computed over flat ranges of whole DQ groups (16384
    elements each) in a thread pool, then joined.  DQ groups are independent
    of each other (each has its own absmax values, c2 and codes), so the
    joined arrays are exactly the whole-weight oracle's; a CPU test checks
    that on a ragged weight."""
    from concurrent.futures import ThreadPoolExecutor

    flat = np.ascontiguousarray(W, dtype=np.float32).ravel()
    step = 64 * 256 * chunk_groups
    starts = list(range(0, flat.size, step)) or [0]

    def one(s0):
        part = flat[s0:s0 + step]
        packed, absmax = quantize_nf4(part)
        q, c2 = double_quant(absmax)
        return packed, absmax, q, c2, dequantize_nf4(packed, q, c2, part.size)

    with ThreadPoolExecutor(threads or host_threads()) as ex:
        parts = list(ex.map(one, starts))
    packed, absmax, q, c2, w_hat = (np.concatenate([p[i] for p in parts]) for i in range(5))
    w_hat = w_hat.reshape(W.shape)
    return dict(packed=packed, absmax=absmax, q=q, c2=c2, w_hat=w_hat)


def oracle_rows(W, r0, r1):
    """Oracle decode of rows [r0, r1) of W computed from whole DQ groups only
    (groups are independent), so a full-size weight can be spot-checked."""
    n_out, k_in = W.shape
    flat = W.reshape(-1)
    e0, e1 = r0 * k_in, r1 * k_in
    g0, g1 = e0 // (64 * 256), -(-e1 // (64 * 256))
    s0, s1 = g0 * 64 * 256, min(g1 * 64 * 256, flat.size)
    part = np.ascontiguousarray(flat[s0:s1])
    packed, absmax = quantize_nf4(part)
    q, c2 = double_quant(absmax)
    w_hat = dequantize_nf4(packed, q, c2, part.size)
    sl = slice(e0 - s0, e1 - s0)
    return dict(w_hat=w_hat[sl].reshape(r1 - r0, k_in),
                packed=packed[(e0 - s0) // 2:(e1 - s0) // 2],
                q=q[(e0 - s0) // 64:(e1 - s0) // 64],
                c2=c2, g0=g0, g1=g1)


def guarded(shape, dtype, fill, margin=4096):
    """A device tensor viewed inside a larger buffer whose margins hold `fill`;
    returns (view, check) where check() asserts the margins are untouched."""
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.full((n + 2 * margin,), fill, dtype=dtype, device=dev())
    view = buf[margin:margin + n].view(*shape)

    def check():
        h = host(buf)
        lo, hi = h[:margin], h[margin + n:]
        ref = torch.full((margin,), fill, dtype=dtype)
        assert torch.equal(lo, ref) and torch.equal(hi, ref), "write outside the output"
    return view, check
