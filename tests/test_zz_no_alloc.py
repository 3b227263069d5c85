"""The forward for callers that cannot allocate (qlora_linear_fwd_noalloc),
called through the C ABI: the same outputs, bit for bit, as qlora_linear_fwd
with a caller workspace, on consecutive calls that reuse the library's
per-GPU scratch (each smaller than the one before, so stale contents from a
larger call sit in the buffer), and the float64 oracle's tolerance on top."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.linear import linear_fwd, lora_scale

from support import assert_close, bf16_bits, host, oracle_weight, say, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _noalloc_fwd(wq, X, A, B, alpha):
    M, r = X.shape[0], A.shape[0]
    Y = torch.full((M, wq.n_out), -7.0, dtype=torch.bfloat16, device=X.device)
    U = torch.full((M, r), -7.0, dtype=torch.bfloat16, device=X.device)
    st = wq.c_struct()
    s = q.lib().qlora_linear_fwd_noalloc(ctypes.byref(st), q._ptr(X), M, q._ptr(A), q._ptr(B), r,
                                         alpha, q._ptr(Y), q._ptr(U), q._stream(X.device))
    assert s == 0, q.status_string(s)
    return Y, U


def test_noalloc_forward_matches_workspace_forward():
    K, N, r, alpha = 320, 1032, 20, 16.0  # r % 8 != 0: padded copies of U and B too
    W = wl.weight_f32(970, N, K)
    o = oracle_weight(W)
    wq = q.quantize_weight(to_dev(W))
    A = wl.bf16_normal(970, (r, K), 0.01, tensor=wl.T_A)
    B = wl.bf16_normal(970, (N, r), 0.01, tensor=wl.T_B)
    Ad, Bd = to_dev(A), to_dev(B)
    # many tokens (U partial sums + padded U, B), then split-K (larger partial
    # sums of Y), then the few-token path, each call smaller than the last
    for M in (700, 100, 9):
        say(f"[noalloc] M={M} K={K} N={N} r={r}")
        X = wl.bf16_normal(970 + M, (M, K), 1.0, tensor=wl.T_X)
        Xd = to_dev(X)
        Y, U = _noalloc_fwd(wq, Xd, Ad, Bd, alpha)
        Yw, Uw = q.linear_fwd(wq, Xd, Ad, Bd, alpha)
        assert np.array_equal(bf16_bits(Y), bf16_bits(Yw)), M
        assert np.array_equal(bf16_bits(U), bf16_bits(Uw)), M
        Yr, Ur = linear_fwd(host(Xd).to(torch.float64).numpy(), o["w64"],
                            A.to(torch.float64).numpy(), B.to(torch.float64).numpy(),
                            lora_scale(alpha, r))
        assert_close("Y", host(Y).to(torch.float64).numpy(), Yr)
        assert_close("U", host(U).to(torch.float64).numpy(), Ur)


def test_noalloc_forward_rejects_a_workspace_beyond_its_buffer():
    """127 tokens, n_out = 262144: the split-K partial sums need more than the
    buffer holds; the call returns QLORA_ERR_WORKSPACE and launches nothing."""
    M, K, N, r = 127, 64, 262144, 8
    need = q.workspace_size(0, M, N, K, r)
    limit = 64 << 20
    assert need > limit
    wq = q.NF4Tensor(torch.zeros(N * K // 2, dtype=torch.uint8, device="cuda"),
                     torch.zeros(N * K // 64, dtype=torch.int8, device="cuda"),
                     torch.zeros(-(-N * K // 16384), dtype=torch.float32, device="cuda"), N, K)
    X = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(r, K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(N, r, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    U = torch.full((M, r), 3.0, dtype=torch.bfloat16, device="cuda")
    st = wq.c_struct()
    s = q.lib().qlora_linear_fwd_noalloc(ctypes.byref(st), q._ptr(X), M, q._ptr(A), q._ptr(B), r,
                                         16.0, q._ptr(Y), q._ptr(U), q._stream(X.device))
    assert s == 5
    torch.cuda.synchronize()
    assert torch.all(Y == 3.0) and torch.all(U == 3.0)
