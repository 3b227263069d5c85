"""GPU parity of the QLoRA linear forward / backward against the float64 oracle.

Outputs and gradients: max |gpu - ref| <= 1e-2 · max |ref| per tensor.  The
identity cases pin the in-GEMM dequantisation bit-exactly through the GEMM's
own output."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.linear import linear_bwd, linear_fwd, lora_scale

from support import assert_close, bf16_bits, guarded, host, oracle_weight, say, to_dev

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
    (3, 256, 75, 8, 16.0),        # n_out not a multiple of 8: few-token path
    (40, 192, 75, 8, 16.0),       # ... split-K path
    (300, 128, 75, 16, 16.0),     # ... many-token path
    (257, 320, 1001, 64, 16.0),   # ... many-token path, several column tiles
    (130, 64, 13, 3, 16.0),       # ... with a rank that is not a multiple of 8
    (21, 128, 1, 1, 2.0),         # a single output column
    (1, 11008, 4096, 16, 32.0),   # small weight split over k, U formed in the pass (ragged split)
    (9, 2048, 1000, 72, 16.0),    # ... two token groups, five rank groups
    (16, 4096, 4096, 256, 16.0),  # ... largest rank
    (5, 3072, 75, 3, 16.0),       # ... rank and n_out not multiples of 8
    (300, 256, 264, 129, 16.0),   # two groups of ranks, the second holding one rank
    (40, 192, 96, 200, 16.0),     # ... split-K path, a rank that is not a multiple of 8
    (7, 512, 72, 129, 16.0),      # ... few-token path
    # one-launch path for small weights (<= 16 tokens, r <= 16, k_in <= 4096,
    # one workgroup of 16 columns per compute unit)
    (16, 4096, 4096, 16, 32.0),   # largest rank, two 128-k chunks per wave
    (1, 64, 16, 1, 2.0),          # one chunk, half of it past k_in, one rank
    (7, 4032, 75, 5, 16.0),       # last chunk half past k_in; n_out and r ragged
    (16, 2112, 4096, 16, 16.0),   # two chunks per wave, most waves' second chunk empty
    (3, 128, 4096, 9, 16.0),      # rank group of 4 rows only partly used
    (12, 4096, 17, 3, 16.0),      # one column past a workgroup of 16
    (5, 1984, 33, 13, 8.0),       # token and rank groups partly used, ragged k
])
def test_small_shapes(M, K, N, r, alpha):
    _run_case(M, K, N, r, alpha, seed=M + K + N + r)


def _sweep_shapes(n, seed, k_max, n_max, r_max):
    """n seeded (M, K, N, r) of at most 16 tokens: K a multiple of 64 up to
    k_max, N up to n_max, r up to r_max."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 17))
        K = 64 * int(rng.integers(1, k_max // 64 + 1))
        N = int(rng.integers(1, n_max + 1))
        r = int(rng.integers(1, r_max + 1))
        out.append((M, K, N, r))
    return out


@pytest.mark.parametrize("M,K,N,r", _sweep_shapes(16, 2026, 4096, 4096, 16))
def test_one_launch_forward_sweep(M, K, N, r):
    """Seeded shapes inside the one-launch forward's range (<= 16 tokens, r <=
    16, k_in <= 4096, n_out <= 4096): every output against the oracle."""
    _run_case(M, K, N, r, 16.0, seed=M * 7 + K + N + r, bwd=False)


@pytest.mark.parametrize("M,K,N,r", _sweep_shapes(6, 77, 4096, 9000, 48))
def test_few_token_forward_sweep(M, K, N, r):
    """Seeded few-token shapes over both forward kernels (wider weights, larger
    ranks and k_in take the GEMV): every output against the oracle."""
    _run_case(M, K, N, r, 16.0, seed=M * 7 + K + N + r, bwd=False)


def _fwd_bwd_shapes(n, seed):
    """n seeded (M, K, N, r) across every path: tokens from the few-token to
    the many-token range, ragged n_out, k_in a multiple of 64, r up to 130."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 128)),
                            int(rng.integers(128, 700))]))
        K = 64 * int(rng.integers(1, 33))
        N = int(rng.integers(1, 3000))
        r = int(rng.integers(1, 131))
        out.append((M, K, N, r))
    return out


@pytest.mark.parametrize("M,K,N,r", _fwd_bwd_shapes(12, 4242))
def test_fwd_bwd_sweep(M, K, N, r):
    """Seeded shapes across all forward and backward paths: every output and
    gradient against the oracle."""
    _run_case(M, K, N, r, 16.0, seed=M * 3 + K + N * 5 + r)


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


@pytest.mark.parametrize("M,K,N,r", [
    (5, 1984, 33, 13),    # n_out and rank padded in the backward, few tokens
    (5, 1984, 40, 16),    # the same unpadded
    (40, 192, 75, 8),     # split-K path, n_out padded, rank a multiple of 8 (B not copied)
    (300, 128, 75, 16),   # many-token path
    (130, 64, 13, 3),
    (12, 4096, 17, 3),    # one-launch forward
    (3, 8448, 64, 8),     # few-token forward split over k (partial sums in the workspace)
])
def test_workspace_contents_do_not_matter(M, K, N, r):
    """Every output is the same whether the workspace starts as zeros or as
    0xFF bytes (NaN for every float type): nothing is read from it before it
    is written, and no padding is read from past a buffer's rows."""
    say(f"[workspace] M={M} K={K} N={N} r={r}")
    W, A, B, X, dY = _inputs(M, K, N, r, seed=7 + M + N)
    wq = q.quantize_weight(to_dev(W))
    Xd, Ad, Bd, dYd = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    outs = []
    for fill in (0, 255):
        wf = torch.full((q.workspace_size(0, M, N, K, r),), fill, dtype=torch.uint8, device="cuda")
        wb = torch.full((q.workspace_size(1, M, N, K, r),), fill, dtype=torch.uint8, device="cuda")
        Y, U = q.linear_fwd(wq, Xd, Ad, Bd, 16.0, workspace=wf)
        dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, 16.0, workspace=wb)
        outs.append([host(t) for t in (Y, U, dX, dA, dB)])
    for name, a, b in zip(("Y", "U", "dX", "dA", "dB"), *outs):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), name


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


def test_offsets_past_2_31_bytes():
    """A 2.16 GB streamed operand: X [33000][32768] bf16, n_out = 64, r = 16.
    The adapter-gradient kernel's splits then cap their rows so that buffer
    offsets stay below 2^31 bytes (two splits of at most 32704 rows), and
    every other kernel addresses rows far past 2^31 bytes.  U and dB in full;
    Y, dX on sampled token rows; dA on sampled columns (whole NF4 blocks)."""
    M, K, N, r, alpha = 33000, 32768, 64, 16, 16.0
    say(f"[linear] M={M} K={K} N={N} r={r}: offsets past 2^31 bytes")
    key = 960
    W = wl.weight_f32(key, N, K)
    A = wl.bf16_normal(key, (r, K), 0.01, tensor=wl.T_A)
    B = wl.bf16_normal(key, (N, r), 0.01, tensor=wl.T_B)
    X = wl.bf16_normal(key, (M, K), 1.0, tensor=wl.T_X)
    dY = wl.bf16_normal(key, (M, N), 1.0, tensor=wl.T_DY)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    Xd, Ad, Bd, dYd = to_dev(X), to_dev(A), to_dev(B), to_dev(dY)
    Y, U = q.linear_fwd(wq, Xd, Ad, Bd, alpha)
    dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, alpha)
    torch.cuda.synchronize()
    del Xd
    s = lora_scale(alpha, r)
    A64, B64, dY64 = _f64(A), _f64(B), _f64(dY)
    # U = X·Aᵀ and V = dY·B in float64, X in row chunks
    Ur = np.empty((M, r))
    for r0 in range(0, M, 2048):
        Ur[r0:r0 + 2048] = _f64(X[r0:r0 + 2048]) @ A64.T
    assert_close("U", _f64(U), Ur)
    assert_close("dB", _f64(dB), s * (dY64.T @ Ur))
    rows = np.r_[0:3, 16380:16390, 32700:32710, M - 5:M]
    Xr = _f64(X[torch.from_numpy(rows)])
    Yr, _ = linear_fwd(Xr, o["w64"], A64, B64, s)
    assert_close("Y rows", _f64(Y)[rows], Yr)
    dXr, _, _ = linear_bwd(Xr, dY64[rows], o["w64"], A64, B64, s)
    assert_close("dX rows", _f64(dX[torch.as_tensor(rows, device=dX.device)]), dXr)
    cols = np.r_[0:64, 16384:16448, K - 64:K]
    V = dY64 @ B64
    dAr = s * (V.T @ _f64(X[:, torch.from_numpy(cols)]))
    assert_close("dA cols", _f64(dA)[:, cols], dAr)
