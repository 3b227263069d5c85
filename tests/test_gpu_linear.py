"""GPU parity of the QLoRA linear forward / backward against the float64 oracle.

Outputs and gradients: max |gpu - ref| <= 1e-2 · max |ref| per tensor.  The
identity cases pin the in-GEMM dequantisation bit-exactly through the GEMM's
own output."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.linear import linear_bwd, linear_fwd, lora_scale
from oracle.quant import bf16_to_f64

from support import (TOL, assert_close, bf16_bits, guarded, host, oracle_rows, oracle_weight, say,
                     to_dev)

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _f64(t):
    return host(t).to(torch.float64).numpy()


def _inputs(M, K, N, r, seed, fwd_only=False):
    key = 900 + seed
    W = wl.weight_f32(key, N, K)
    A = wl.bf16_normal(key, (r, K), 0.01, tensor=wl.T_A)
    B = wl.bf16_normal(key, (N, r), 0.01, tensor=wl.T_B)
    X = wl.bf16_normal(key, (M, K), 1.0, tensor=wl.T_X)
    dY = None if fwd_only else wl.bf16_normal(key, (M, N), 1.0, tensor=wl.T_DY)
    return W, A, B, X, dY


def _run_case(M, K, N, r, alpha, seed, bwd=True):
    say(f"[linear] M={M} K={K} N={N} r={r} alpha={alpha}")
    W, A, B, X, dY = _inputs(M, K, N, r, seed, fwd_only=not bwd)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    assert np.array_equal(bf16_bits(q.dequantize_nf4(wq)), o["w_hat"])
    Xd, Ad, Bd = to_dev(X), to_dev(A), to_dev(B)
    Y, check_y = guarded((M, N), torch.bfloat16, -3.0)
    U, check_u = guarded((M, r), torch.bfloat16, -3.0)
    q.linear_fwd(wq, Xd, Ad, Bd, alpha, Y=Y, U=U)
    s = lora_scale(alpha, r)
    Yr, Ur = linear_fwd(_f64(X), o["w64"], _f64(A), _f64(B), s)
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)
    check_y()
    check_u()
    if not bwd:
        return
    dYd = to_dev(dY)
    dX, cx = guarded((M, K), torch.bfloat16, 5.0)
    dA, ca = guarded((r, K), torch.float32, 5.0)
    dB, cb = guarded((N, r), torch.float32, 5.0)
    q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, alpha, dX=dX, dA=dA, dB=dB)
    dXr, dAr, dBr = linear_bwd(_f64(X), _f64(dY), o["w64"], _f64(A), _f64(B), s)
    assert_close("dX", _f64(dX), dXr)
    assert_close("dA", _f64(dA), dAr)
    assert_close("dB", _f64(dB), dBr)
    cx(), ca(), cb()


@pytest.mark.parametrize("M,K,N,r,alpha", [
    (1, 64, 8, 1, 2.0),
    (5, 128, 72, 8, 16.0),
    (16, 192, 264, 16, 32.0),
    (100, 320, 264, 3, 16.0),     # few-token path, rank not a multiple of 8
    (130, 64, 16, 16, 16.0),      # many-token path, one column tile
    (300, 192, 520, 8, 16.0),     # ragged in M and N, several tiles each way
    (513, 128, 1032, 72, 16.0),   # rank above 64: prologue over two 64-chunks
    (257, 448, 256, 64, 16.0),
    (3, 8448, 64, 8, 16.0),       # few-token path split over k (partial sums + reduction)
    (12, 4096, 40, 16, 32.0),     # few tokens in two groups of 8
    (6, 4096, 40, 32, 16.0),      # few tokens, rank 32
    (2, 1088, 48, 8, 16.0),       # few tokens, byte-wise scale codes, k split in two
    (9, 8448, 40, 8, 16.0),       # two token groups, k split (partial sums + reduction)
    (13, 1088, 48, 8, 16.0),      # two token groups, byte-wise scale codes
    (256, 512, 264, 256, 16.0),   # largest rank, many-token path
    (40, 256, 96, 256, 64.0),     # largest rank, split-K path
    (3, 512, 64, 256, 16.0),      # largest rank, few-token path
])
def test_small_shapes(M, K, N, r, alpha):
    _run_case(M, K, N, r, alpha, seed=M + K + N + r)


def test_zero_tokens():
    W, A, B, X, dY = _inputs(1, 64, 16, 4, 7)
    wq = q.quantize_weight(to_dev(W))
    Ad, Bd = to_dev(A), to_dev(B)
    X0 = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    dY0 = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    Y, U = q.linear_fwd(wq, X0, Ad, Bd, 8.0)
    dA = torch.full((4, 64), 9.0, device="cuda")
    dB = torch.full((16, 4), 9.0, device="cuda")
    dX, dA, dB = q.linear_bwd(wq, X0, dY0, Ad, Bd, U, 8.0, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, 16) and dX.shape == (0, 64)
    assert torch.all(dA == 0) and torch.all(dB == 0)


@pytest.mark.parametrize("K,N", [(256, 264), (64, 72)])
def test_identity_input_exposes_decoded_weight(K, N):
    """X = I (M = K), B = 0: Y = Ŵᵀ bit-exactly (one non-zero term per output)."""
    say(f"[identity] K={K} N={N}")
    W = wl.weight_f32(950, N, K)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    X = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    A = to_dev(wl.bf16_normal(950, (8, K), 0.01, tensor=wl.T_A))
    B = torch.zeros(N, 8, dtype=torch.bfloat16, device="cuda")
    Y, U = q.linear_fwd(wq, X, A, B, 16.0)
    assert np.array_equal(bf16_bits(Y), o["w_hat"].T.copy())


@pytest.mark.parametrize("K,N", [(192, 256), (128, 64)])
def test_identity_grad_exposes_decoded_weight(K, N):
    """dY = I (M = N), A = 0: dX = Ŵ bit-exactly through the transposed traversal."""
    say(f"[identity-grad] K={K} N={N}")
    W = wl.weight_f32(951, N, K)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    dY = torch.eye(N, dtype=torch.bfloat16, device="cuda")
    X = to_dev(wl.bf16_normal(951, (N, K), 1.0))
    A = torch.zeros(8, K, dtype=torch.bfloat16, device="cuda")
    B = to_dev(wl.bf16_normal(951, (N, 8), 0.01, tensor=wl.T_B))
    U = torch.zeros(N, 8, dtype=torch.bfloat16, device="cuda")
    dX, dA, dB = q.linear_bwd(wq, X, dY, A, B, U, 16.0)
    assert np.array_equal(bf16_bits(dX), o["w_hat"])
    # U = 0 gives dB = 0; dA = s·(dY·B)ᵀ·X = s·Bᵀ·X does not vanish
    torch.cuda.synchronize()
    assert torch.all(dB == 0)
    assert_close("dA", _f64(dA), lora_scale(16.0, 8) * (_f64(B).T @ _f64(X)))


def test_deterministic_repeat():
    W, A, B, X, dY = _inputs(200, 256, 264, 16, 31)
    wq = q.quantize_weight(to_dev(W))
    Xd, Ad, Bd, dYd = map(to_dev, (X, A, B, dY))
    outs = []
    for _ in range(2):
        Y, U = q.linear_fwd(wq, Xd, Ad, Bd, 16.0)
        dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, 16.0)
        outs.append([host(t).clone() for t in (Y, U, dX, dA, dB)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_workspace_too_small_is_rejected():
    W, A, B, X, dY = _inputs(16, 64, 16, 4, 8)
    wq = q.quantize_weight(to_dev(W))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QloraError) as e:
        q.linear_fwd(wq, to_dev(X), to_dev(A), to_dev(B), 8.0, workspace=ws)
    assert e.value.status == 5


# ---- full-size workloads ---------------------------------------------------------

def test_single_linear_full():
    wlc = wl.SINGLE_LINEAR
    _run_case_full_fwd(wlc)


def _run_case_full_fwd(wlc, M=None):
    inp = wlc.inputs(M=M)
    W = inp["W"]
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    Y, U = q.linear_fwd(wq, to_dev(inp["X"]), to_dev(inp["A"]), to_dev(inp["B"]), wlc.alpha)
    s = lora_scale(wlc.alpha, wlc.r)
    Yr, Ur = linear_fwd(_f64(inp["X"]), o["w64"], _f64(inp["A"]), _f64(inp["B"]), s)
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)


def test_llama7b_mlp_full_fwd_bwd():
    """4096 tokens, 4096 -> 11008, r = 64: every output and gradient in full."""
    wlc = wl.LLAMA7B_MLP
    say(f"[full] {wlc.name}")
    inp = wlc.inputs()
    o = oracle_weight(inp["W"])
    wq = q.quantize_weight(to_dev(inp["W"]))
    assert np.array_equal(bf16_bits(q.dequantize_nf4(wq)), o["w_hat"])
    Xd, Ad, Bd, dYd = (to_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    Y, U = q.linear_fwd(wq, Xd, Ad, Bd, wlc.alpha)
    dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, wlc.alpha)
    s = lora_scale(wlc.alpha, wlc.r)
    X64, A64, B64, dY64 = (_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    Yr, Ur = linear_fwd(X64, o["w64"], A64, B64, s)
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)
    del Yr
    dXr, dAr, dBr = linear_bwd(X64, dY64, o["w64"], A64, B64, s)
    assert_close("dX", _f64(dX), dXr)
    assert_close("dA", _f64(dA), dAr)
    assert_close("dB", _f64(dB), dBr)


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_gemv_70b_full_sampled_outputs(M):
    """8192 -> 28672, r = 16, few tokens: the GPU computes every output; the
    oracle checks all tokens on output rows sampled over whole DQ groups."""
    wlc = wl.GEMV_70B
    say(f"[full] {wlc.name} M={M}")
    inp = wlc.inputs(M=M)
    W = inp["W"]
    wq = q.quantize_weight(to_dev(W))
    Y, U = q.linear_fwd(wq, to_dev(inp["X"]), to_dev(inp["A"]), to_dev(inp["B"]), wlc.alpha)
    Yh = _f64(Y)
    s = lora_scale(wlc.alpha, wlc.r)
    X64, A64, B64 = (_f64(inp[k]) for k in ("X", "A", "B"))
    Ur = X64 @ A64.T
    assert_close("U", _f64(U), Ur)
    rng = np.random.default_rng(M)
    rows = sorted(set([0, wlc.n_out - 2] + [int(x) * 2 for x in rng.integers(0, wlc.n_out // 2, 24)]))
    for r0 in rows:
        o = oracle_rows(W, r0, r0 + 2)
        Yr, _ = linear_fwd(X64, bf16_to_f64(o["w_hat"]), A64, B64[r0:r0 + 2], s)
        ref_scale = np.max(np.abs(Yh))  # the per-tensor bound uses the whole output's scale
        err = np.max(np.abs(Yh[:, r0:r0 + 2] - Yr))
        assert err <= TOL * ref_scale, (r0, err, ref_scale)


@pytest.mark.parametrize("proj", [3, 6])  # o 8192x8192, down 22016->8192
def test_llama65b_projection_full(proj):
    """2048 tokens, r = 64: Y and dX on sampled token rows, dA, dB and U in full."""
    wlc = wl.LLAMA65B_LAYER[proj]
    say(f"[full] {wlc.name}")
    inp = wlc.inputs()
    o = oracle_weight(inp["W"])
    wq = q.quantize_weight(to_dev(inp["W"]))
    Xd, Ad, Bd, dYd = (to_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    Y, U = q.linear_fwd(wq, Xd, Ad, Bd, wlc.alpha)
    dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, wlc.alpha)
    s = lora_scale(wlc.alpha, wlc.r)
    X64, A64, B64, dY64 = (_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    rows = np.random.default_rng(proj).choice(wlc.M, 64, replace=False)
    rows = np.sort(np.concatenate([rows, [0, wlc.M - 1]]))
    Yr, _ = linear_fwd(X64[rows], o["w64"], A64, B64, s)
    Yf = _f64(Y)
    assert np.max(np.abs(Yf[rows] - Yr)) <= TOL * np.max(np.abs(Yr))
    Ur = X64 @ A64.T
    assert_close("U", _f64(U), Ur)
    V = dY64 @ B64
    dXr = dY64[rows] @ o["w64"] + s * (V[rows] @ A64)
    dXf = _f64(dX)
    assert np.max(np.abs(dXf[rows] - dXr)) <= TOL * np.max(np.abs(dXr))
    assert_close("dA", _f64(dA), s * (V.T @ X64))
    assert_close("dB", _f64(dB), s * (dY64.T @ Ur))
