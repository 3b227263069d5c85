"""Reads stay inside the inputs' rows and the workspace.

Every input is placed at the start of its own buffer whose bytes past the
input are 0xFF (NaN as bf16 and fp32, code 15 and scale code -1 as NF4 + DQ
bytes), and the workspace is filled with 0xFF too.  On every path of the
linear forward and backward (one-launch small weights, few-token GEMV with
and without a k split, split-K, many-token; ragged n_out, ranks that are not
a multiple of 8, dropout) the outputs must equal, bit for bit, those of the
same inputs in ordinary allocations with a zeroed workspace: a read past an
input's end or of workspace bytes not yet written would change them."""

import pytest
import torch

import workloads as wl
from support import host, say, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _tail(t):
    """A copy of t at the start of a buffer whose remaining bytes are 0xFF."""
    t = t.contiguous()
    n = t.numel() * t.element_size()
    buf = torch.full(((n + 15) // 16 * 16 + 4096,), 255, dtype=torch.uint8, device=t.device)
    buf[:n] = t.view(-1).view(torch.uint8)
    return buf[:n].view(t.dtype).view(t.shape)


def _ws(op, M, N, K, r, fill):
    return torch.full((q.workspace_size(op, M, N, K, r),), fill, dtype=torch.uint8, device="cuda")


def _run(wq, X, A, B, dY, alpha, M, N, K, r, fill, dropout, wrap):
    """Forward then backward; wrap places the forward's U (and Xd) for the backward."""
    if dropout:
        p, seed, off = 0.1, 77, 5
        Y, U, Xd = q.linear_fwd_dropout(wq, X, A, B, alpha, p, seed, off,
                                        workspace=_ws(0, M, N, K, r, fill))
        dX, dA, dB = q.linear_bwd_dropout(wq, wrap(Xd), dY, A, B, wrap(U), alpha, p, seed, off,
                                          workspace=_ws(2, M, N, K, r, fill))
        outs = (Y, U, Xd, dX, dA, dB)
    else:
        Y, U = q.linear_fwd(wq, X, A, B, alpha, workspace=_ws(0, M, N, K, r, fill))
        dX, dA, dB = q.linear_bwd(wq, X, dY, A, B, wrap(U), alpha,
                                  workspace=_ws(1, M, N, K, r, fill))
        outs = (Y, U, dX, dA, dB)
    return [host(t) for t in outs]


@pytest.mark.parametrize("M,K,N,r,dropout", [
    (16, 4096, 4096, 8, False),   # one-launch forward (the single-linear shape)
    (7, 1984, 75, 5, False),      # ... ragged k, n_out and rank
    (3, 8448, 64, 8, False),      # few-token GEMV split over k
    (5, 4096, 8200, 13, False),   # few-token GEMV (too wide for one launch), rank padded
    (7, 512, 72, 129, False),     # few-token GEMV, two rank groups
    (40, 192, 75, 8, False),      # split-K, n_out padded, B not copied
    (40, 256, 96, 200, False),    # split-K, large rank
    (300, 128, 75, 16, False),    # many-token
    (257, 320, 1001, 64, False),  # many-token, several column tiles
    (130, 64, 13, 3, False),
    (6, 1984, 33, 13, True),      # dropout: few tokens
    (130, 256, 75, 5, True),      # dropout: many tokens
])
def test_no_reads_past_inputs_or_unwritten_workspace(M, K, N, r, dropout):
    say(f"[bounds] M={M} K={K} N={N} r={r} dropout={dropout}")
    key = 4000 + M + K + N + r
    W = wl.weight_f32(key, N, K)
    A = to_dev(wl.bf16_normal(key, (r, K), 0.01, tensor=wl.T_A))
    B = to_dev(wl.bf16_normal(key, (N, r), 0.01, tensor=wl.T_B))
    X = to_dev(wl.bf16_normal(key, (M, K), 1.0, tensor=wl.T_X))
    dY = to_dev(wl.bf16_normal(key, (M, N), 1.0, tensor=wl.T_DY))
    wq = q.quantize_weight(to_dev(W))
    clean = _run(wq, X, A, B, dY, 16.0, M, N, K, r, 0, dropout, lambda t: t)
    wt = q.NF4Tensor(_tail(wq.packed), _tail(wq.qabsmax), _tail(wq.c2), wq.n_out, wq.k_in)
    dirty = _run(wt, _tail(X), _tail(A), _tail(B), _tail(dY), 16.0, M, N, K, r, 255, dropout, _tail)
    names = ("Y", "U", "Xd", "dX", "dA", "dB") if dropout else ("Y", "U", "dX", "dA", "dB")
    for name, a, b in zip(names, clean, dirty):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), name
