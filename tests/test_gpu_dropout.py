"""GPU parity of the LoRA dropout path against the oracle: the mask and the
dropped input bit-exact; outputs and gradients of the dropout linear within
1e-2 · max |ref| per tensor (the float64 oracle with the same mask)."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.dropout import keep_mask, linear_bwd_dropout, linear_fwd_dropout
from oracle.linear import lora_scale

from support import assert_close, bf16_bits, guarded, host, oracle_weight, say, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _f64(t):
    return host(t).to(torch.float64).numpy()


def _inputs(M, K, N, r, seed):
    key = 950 + seed
    W = wl.weight_f32(key, N, K)
    A = wl.bf16_normal(key, (r, K), 0.01, tensor=wl.T_A)
    B = wl.bf16_normal(key, (N, r), 0.01, tensor=wl.T_B)
    X = wl.bf16_normal(key, (M, K), 1.0, tensor=wl.T_X)
    dY = wl.bf16_normal(key, (M, N), 1.0, tensor=wl.T_DY)
    return W, A, B, X, dY


@pytest.mark.parametrize("M,K,p,seed,offset", [
    (1, 64, 0.05, 1, 0),
    (7, 192, 0.05, 2 ** 64 - 1, 2 ** 63 + 5),
    (130, 512, 0.5, 12345, 77),
    (64, 4096, 0.05, 0, 1),
    (33, 1024, 0.0, 9, 9),
    (8, 256, 0.999, 3, 4),
])
def test_dropped_input_bit_exact(M, K, p, seed, offset):
    say(f"[dropout] mask M={M} K={K} p={p} seed={seed} offset={offset}")
    X = wl.bf16_normal(960, (M, K), 1.0)
    X[0, :8] = torch.tensor([-0.0, 0.0, 1.0, -1.0, 0.0, -0.0, 2.0, 3.0], dtype=torch.bfloat16)
    Xd, check = guarded((M, K), torch.bfloat16, 7.0)
    q.lora_dropout(to_dev(X), p, seed, offset, Xd=Xd)
    keep = keep_mask(M, K, p, seed, offset)
    ref = np.where(keep, X.view(torch.int16).numpy().view(np.uint16), np.uint16(0))
    assert np.array_equal(bf16_bits(Xd), ref)
    check()


def _run_case(M, K, N, r, alpha, p, seed, offset, dseed):
    say(f"[dropout] linear M={M} K={K} N={N} r={r} p={p}")
    W, A, B, X, dY = _inputs(M, K, N, r, dseed)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    Xg, Ag, Bg, dYg = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    Y, cy = guarded((M, N), torch.bfloat16, -3.0)
    U, cu = guarded((M, r), torch.bfloat16, -3.0)
    Xd, cd = guarded((M, K), torch.bfloat16, -3.0)
    q.linear_fwd_dropout(wq, Xg, Ag, Bg, alpha, p, seed, offset, Y=Y, U=U, Xd=Xd)
    keep = keep_mask(M, K, p, seed, offset)
    s = lora_scale(alpha, r)
    X64, A64, B64, dY64 = _f64(X), _f64(A), _f64(B), _f64(dY)
    Yr, Ur = linear_fwd_dropout(X64, o["w64"], A64, B64, s, p, keep)
    assert np.array_equal(bf16_bits(Xd), np.where(keep, bf16_bits(Xg), np.uint16(0)))
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)
    dX, cx = guarded((M, K), torch.bfloat16, 5.0)
    dA, ca = guarded((r, K), torch.float32, 5.0)
    dB, cb = guarded((N, r), torch.float32, 5.0)
    q.linear_bwd_dropout(wq, Xd, dYg, Ag, Bg, U, alpha, p, seed, offset, dX=dX, dA=dA, dB=dB)
    dXr, dAr, dBr = linear_bwd_dropout(X64, dY64, o["w64"], A64, B64, s, p, keep)
    assert_close("dX", _f64(dX), dXr)
    assert_close("dA", _f64(dA), dAr)
    assert_close("dB", _f64(dB), dBr)
    for c in (cy, cu, cd, cx, ca, cb):
        c()


@pytest.mark.parametrize("M,K,N,r,alpha,p", [
    (1, 64, 8, 1, 2.0, 0.05),
    (8, 128, 72, 8, 16.0, 0.05),      # few tokens: U from the dropped input, then the GEMV
    (16, 192, 264, 16, 32.0, 0.3),
    (100, 320, 264, 3, 16.0, 0.05),   # split-K backward, rank not a multiple of 8
    (130, 64, 16, 16, 16.0, 0.05),    # many-token path
    (300, 192, 520, 8, 16.0, 0.5),
    (513, 128, 1032, 72, 16.0, 0.05),
    (257, 448, 256, 64, 16.0, 0.05),
])
def test_small_shapes(M, K, N, r, alpha, p):
    _run_case(M, K, N, r, alpha, p, seed=1000 + M, offset=r, dseed=M)


def _sweep(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 128)),
                            int(rng.integers(128, 600))]))
        out.append((M, 64 * int(rng.integers(1, 25)), int(rng.integers(1, 2000)),
                    int(rng.integers(1, 100)), float(rng.choice([0.05, 0.1, 0.5]))))
    return out


@pytest.mark.parametrize("M,K,N,r,p", _sweep(8, 515))
def test_dropout_sweep(M, K, N, r, p):
    """Seeded shapes and rates across the dropout paths, against the oracle
    (mask bit-exact, outputs and gradients within tolerance)."""
    _run_case(M, K, N, r, 16.0, p, seed=7 + M, offset=M * K, dseed=M + N)


def test_masked_input_gradient_zero_pattern():
    """With a zero weight dX is the masked adapter term alone: every dropped
    element is exactly +0 and (generically) every kept one is not."""
    M, K, N, r, p = 256, 512, 128, 16, 0.3
    _, A, B, X, dY = _inputs(M, K, N, r, 7)
    wq = q.quantize_weight(torch.zeros(N, K, dtype=torch.float32, device="cuda"))
    Xg, Ag, Bg, dYg = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    _, U, Xd = q.linear_fwd_dropout(wq, Xg, Ag, Bg, 16.0, p, 5, 6)
    dX, _, _ = q.linear_bwd_dropout(wq, Xd, dYg, Ag, Bg, U, 16.0, p, 5, 6)
    keep = keep_mask(M, K, p, 5, 6)
    bits = bf16_bits(dX)
    assert np.all(bits[~keep] == 0)
    assert np.mean(bits[keep] != 0) > 0.99


def test_zero_rate_equals_plain_layer_bitwise():
    M, K, N, r = 256, 448, 264, 16
    W, A, B, X, dY = _inputs(M, K, N, r, 8)
    wq = q.quantize_weight(to_dev(W))
    Xg, Ag, Bg, dYg = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    Y0, U0 = q.linear_fwd(wq, Xg, Ag, Bg, 16.0)
    dX0, dA0, dB0 = q.linear_bwd(wq, Xg, dYg, Ag, Bg, U0, 16.0)
    Y1, U1, Xd = q.linear_fwd_dropout(wq, Xg, Ag, Bg, 16.0, 0.0, 1, 2)
    dX1, dA1, dB1 = q.linear_bwd_dropout(wq, Xd, dYg, Ag, Bg, U1, 16.0, 0.0, 1, 2)
    assert torch.equal(Xd.view(torch.int16), Xg.view(torch.int16))
    for a, b in ((Y0, Y1), (U0, U1), (dX0, dX1)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for a, b in ((dA0, dA1), (dB0, dB1)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_repeatable_and_offset_changes_mask():
    M, K, N, r = 300, 256, 264, 8
    W, A, B, X, dY = _inputs(M, K, N, r, 9)
    wq = q.quantize_weight(to_dev(W))
    Xg, Ag, Bg, dYg = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    outs = []
    for offset in (3, 3, 4):
        Y, U, Xd = q.linear_fwd_dropout(wq, Xg, Ag, Bg, 16.0, 0.05, 11, offset)
        dX, dA, dB = q.linear_bwd_dropout(wq, Xd, dYg, Ag, Bg, U, 16.0, 0.05, 11, offset)
        torch.cuda.synchronize()
        outs.append([host(t).view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
                     for t in (Y, U, Xd, dX, dA, dB)])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    assert not torch.equal(outs[0][2], outs[2][2])


def test_llama7b_mlp_full_with_dropout():
    """4096 tokens, 4096 -> 11008, r = 64, p = 0.05: every element."""
    wlc = wl.LLAMA7B_MLP
    say(f"[dropout] full {wlc.name}")
    inp = wlc.inputs()
    o = oracle_weight(inp["W"])
    wq = q.quantize_weight(to_dev(inp["W"]))
    Xg, Ag, Bg, dYg = (to_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    p, seed, offset = 0.05, 2024, 31
    Y, U, Xd = q.linear_fwd_dropout(wq, Xg, Ag, Bg, wlc.alpha, p, seed, offset)
    dX, dA, dB = q.linear_bwd_dropout(wq, Xd, dYg, Ag, Bg, U, wlc.alpha, p, seed, offset)
    keep = keep_mask(wlc.M, wlc.k_in, p, seed, offset)
    assert np.array_equal(bf16_bits(Xd), np.where(keep, bf16_bits(Xg), np.uint16(0)))
    s = lora_scale(wlc.alpha, wlc.r)
    X64, A64, B64, dY64 = (_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    Yr, Ur = linear_fwd_dropout(X64, o["w64"], A64, B64, s, p, keep)
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)
    del Yr
    dXr, dAr, dBr = linear_bwd_dropout(X64, dY64, o["w64"], A64, B64, s, p, keep)
    assert_close("dX", _f64(dX), dXr)
    assert_close("dA", _f64(dA), dAr)
    assert_close("dB", _f64(dB), dBr)
