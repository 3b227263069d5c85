"""The library's calls captured into HIP graphs (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between
replays, gives the same bits as the same calls run eagerly.  Buffers and
workspaces are allocated before capture; only library launches are captured
(the library issues no memset, allocation or synchronisation)."""

import numpy as np
import pytest
import torch

import workloads as wl

from support import say, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _bits(t):
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().clone()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().clone()
    if t.dtype == torch.float64:
        return t.view(torch.int64).cpu().clone()
    return t.cpu().clone()


def _replay_and_compare(run, outputs, refresh, replays=3):
    """Capture run(), then for each replay: refresh the inputs eagerly, replay,
    and compare every output with an eager run() on the same inputs."""
    run()  # eager warm-up (caches device properties, loads the kernels)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(replays):
        refresh(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(o) for o in outputs]
        run()  # eager, same inputs
        torch.cuda.synchronize()
        for k, (a, o) in enumerate(zip(got, outputs)):
            assert torch.equal(a, _bits(o)), (i, k)


def _layer(M, K, N, r, seed):
    key = 1100 + seed
    W = to_dev(wl.weight_f32(key, N, K))
    wq = q.quantize_weight(W)
    A = to_dev(wl.bf16_normal(key, (r, K), 0.01, tensor=wl.T_A))
    B = to_dev(wl.bf16_normal(key, (N, r), 0.01, tensor=wl.T_B))
    X = to_dev(wl.bf16_normal(key, (M, K), 1.0, tensor=wl.T_X))
    dY = to_dev(wl.bf16_normal(key, (M, N), 1.0, tensor=wl.T_DY))
    return wq, A, B, X, dY


@pytest.mark.parametrize("M,r", [
    (1, 16),    # one-launch small-weight forward
    (8, 16),    # ... with the split-K backward
    (4, 32),    # few-token GEMV + U launch (rank above the one-launch limit)
    (40, 16),   # split-K forward
    (256, 16),  # many-token forward and backward
])
def test_training_step_graph(M, r):
    K, N, alpha = 512, 1024, 32.0
    say(f"[graph] fwd + bwd M={M} r={r}")
    wq, A, B, X, dY = _layer(M, K, N, r, M)
    dev = X.device
    ws_f = torch.empty(q.workspace_size(0, M, N, K, r), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(q.workspace_size(1, M, N, K, r), dtype=torch.uint8, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, dtype=torch.float32, device=dev)
    dB = torch.empty(N, r, dtype=torch.float32, device=dev)

    def run():
        q.linear_fwd(wq, X, A, B, alpha, workspace=ws_f, Y=Y, U=U)
        q.linear_bwd(wq, X, dY, A, B, U, alpha, workspace=ws_b, dX=dX, dA=dA, dB=dB)

    gen = torch.Generator(device=dev).manual_seed(5)

    def refresh(i):
        X.copy_(torch.randn(X.shape, generator=gen, device=dev).to(torch.bfloat16))
        dY.copy_(torch.randn(dY.shape, generator=gen, device=dev).to(torch.bfloat16))

    _replay_and_compare(run, [Y, U, dX, dA, dB], refresh)


def test_dropout_step_graph():
    M, K, N, r, alpha = 300, 448, 264, 8, 16.0
    wq, A, B, X, dY = _layer(M, K, N, r, 7)
    dev = X.device
    ws_f = torch.empty(q.workspace_size(0, M, N, K, r), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(q.workspace_size(2, M, N, K, r), dtype=torch.uint8, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    Xd = torch.empty_like(X)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, dtype=torch.float32, device=dev)
    dB = torch.empty(N, r, dtype=torch.float32, device=dev)

    def run():
        q.linear_fwd_dropout(wq, X, A, B, alpha, 0.05, 9, 3, workspace=ws_f, Y=Y, U=U, Xd=Xd)
        q.linear_bwd_dropout(wq, Xd, dY, A, B, U, alpha, 0.05, 9, 3, workspace=ws_b, dX=dX, dA=dA,
                             dB=dB)

    gen = torch.Generator(device=dev).manual_seed(6)

    def refresh(i):
        X.copy_(torch.randn(X.shape, generator=gen, device=dev).to(torch.bfloat16))

    _replay_and_compare(run, [Y, U, Xd, dX, dA, dB], refresh)


def test_adamw_and_quantiser_graph():
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    sizes = [4096 * 16, 1000, 37]
    P = [torch.randn(n, generator=gen, device=dev) * 0.02 for n in sizes]
    G = [torch.randn(n, generator=gen, device=dev) * 1e-3 for n in sizes]
    Mo = [torch.zeros(n, device=dev) for n in sizes]
    V = [torch.zeros(n, device=dev) for n in sizes]
    PB = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    lst = q.AdamWList(P, G, Mo, V, PB)
    ws = torch.empty(q.adamw_workspace_size(len(sizes)), dtype=torch.uint8, device=dev)
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    W = torch.randn(64 * 1000 + 5, generator=gen, device=dev) * 0.02
    packed = torch.empty(((W.numel() + 63) // 64) * 32, dtype=torch.uint8, device=dev)
    qa = torch.empty((W.numel() + 63) // 64, dtype=torch.int8, device=dev)
    c2 = torch.empty(((W.numel() + 63) // 64 + 255) // 256, dtype=torch.float32, device=dev)
    lib = q.lib()

    # the optimizer step updates its own state, so each replay is compared with
    # an eager step from a copy of the state the replay started from
    def run_opt():
        q.adamw_step_list(lst, 3, grad_norm=norm, workspace=ws)

    def run_quant():
        lib.qlora_quantize_nf4_dq(q._ptr(W), W.numel(), q._ptr(packed), q._ptr(qa), q._ptr(c2),
                                  None, None, q._stream(dev))

    run_opt()
    run_quant()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_opt()
        run_quant()
    torch.cuda.synchronize()
    for i in range(3):
        state = [[t.clone() for t in ts] for ts in (P, Mo, V)]
        W.copy_(torch.randn(W.shape, generator=gen, device=dev) * 0.02)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in P + Mo + V + PB + [norm, packed, qa, c2]]
        for dst, src in zip(P + Mo + V, state[0] + state[1] + state[2]):
            dst.copy_(src)
        run_opt()
        run_quant()
        torch.cuda.synchronize()
        ref = [_bits(t) for t in P + Mo + V + PB + [norm, packed, qa, c2]]
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (i, k)
