"""Full-size parity on the quantiser and linear workloads: every stored byte,
code, scale and decoded value of the 224-matrix LLaMA-7B weight set; every
output of the few-token 8192 -> 28672 forward at 1..8 tokens; every output and
gradient of the 7 projections of a LLaMA-65B decoder layer (2048 tokens).

The oracle runs on the host in a thread pool (its numpy steps release the
GIL); the GPU path runs through the library's entry points.  Tolerance for
the linear outputs: max |gpu - ref| <= 1e-2 · max |ref| per tensor, with the
scale taken from the oracle's reference."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import workloads as wl
from oracle.linear import linear_bwd, linear_fwd, lora_scale
from oracle.quant import bf16_to_f64, dequantize_nf4, double_quant, quantize_nf4

from support import (assert_close, bf16_bits, f32_bits, host, host_threads, oracle_weight_parallel,
                     say, to_dev, u8)

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _f64(t):
    return host(t).to(torch.float64).numpy()


# ---- LLaMA-7B weight set: 32 layers x 7 matrices ---------------------------------

def _oracle_storage(layer, matrix):
    """Seeded weight and its oracle storage: packed codes, float32 absmax, DQ
    codes, c2 and the decoded bf16 bits (one thread per matrix)."""
    W = wl.llama7b_weight(layer, matrix)
    flat = W.ravel()
    packed, absmax = quantize_nf4(flat)
    qa, c2 = double_quant(absmax)
    return W, dict(packed=packed, absmax=absmax, q=qa, c2=c2,
                   w_hat=dequantize_nf4(packed, qa, c2, flat.size))


LAYERS_PER_TEST = 4


@pytest.mark.parametrize("part", range(wl.LLAMA7B_LAYERS // LAYERS_PER_TEST))
def test_llama7b_weight_set_every_matrix(part):
    """Layers 4·part .. 4·part + 3, each as one batch of its 7 matrices through
    the batched quantiser (both levels) and the batched decoder: every packed
    byte, float32 absmax, DQ code, c2 and decoded bf16 value bit-exact."""
    layers = list(range(part * LAYERS_PER_TEST, (part + 1) * LAYERS_PER_TEST))
    nmat = len(wl.LLAMA7B_MATRICES)
    with threadpool_limits(1), ThreadPoolExecutor(host_threads()) as ex:
        pending = [ex.submit(_oracle_storage, layers[0], m) for m in range(nmat)]
        for li, layer in enumerate(layers):
            res = [f.result() for f in pending]
            pending = ([ex.submit(_oracle_storage, layers[li + 1], m) for m in range(nmat)]
                       if li + 1 < len(layers) else [])
            say(f"[weight set] layer {layer}")
            ws = [to_dev(W.ravel()) for W, _ in res]
            got = q.quantize_nf4_dq_batch(ws)
            wqs = [q.NF4Tensor(g[0], g[1], g[2], W.shape[0], W.shape[1])
                   for g, (W, _) in zip(got, res)]
            outs = q.dequantize_nf4_batch(wqs)
            torch.cuda.synchronize()
            for m, (g, o, (W, ref)) in enumerate(zip(got, outs, res)):
                where = (layer, wl.LLAMA7B_MATRICES[m][0])
                gp = u8(g[0])
                if not np.array_equal(gp, ref["packed"]):
                    bad = np.nonzero(gp != ref["packed"])[0]
                    raise AssertionError(f"{where}: packed differs at {bad[:8]} ({bad.size} bytes)")
                assert np.array_equal(f32_bits(g[3]), ref["absmax"].view(np.uint32)), where
                assert np.array_equal(u8(g[1]).view(np.int8), ref["q"]), where
                assert np.array_equal(f32_bits(g[2]), ref["c2"].view(np.uint32)), where
                assert np.array_equal(bf16_bits(o).ravel(), ref["w_hat"]), where
            del res, ws, got, wqs, outs


# ---- few-token forward, 8192 -> 28672, r = 16, 1..8 tokens ----------------------

@pytest.fixture(scope="module")
def gemv70b():
    wlc = wl.GEMV_70B
    say(f"[full] {wlc.name}: weight and oracle")
    W = wl.weight_f32(wlc.workload, wlc.n_out, wlc.k_in)
    with threadpool_limits(1):
        o = oracle_weight_parallel(W)
    wq = q.quantize_weight(to_dev(W))
    # the codes of this shape, bit-exact as well
    assert np.array_equal(u8(wq.packed), o["packed"])
    assert np.array_equal(u8(wq.qabsmax).view(np.int8), o["q"])
    assert np.array_equal(f32_bits(wq.c2), o["c2"].view(np.uint32))
    w64 = bf16_to_f64(o["w_hat"])
    inp = wlc.inputs(M=1, with_w=False)
    return dict(wlc=wlc, wq=wq, w64=w64, A=inp["A"], B=inp["B"])


@pytest.mark.parametrize("M", wl.GEMV_TOKENS)
def test_gemv_70b_every_output(gemv70b, M):
    """Every element of Y [M][28672] and U [M][16] against the float64 oracle,
    the bound scaled by the oracle's own max |Y|."""
    wlc = gemv70b["wlc"]
    say(f"[full] {wlc.name} M={M}")
    X = wlc.inputs(M=M, with_w=False)["X"]
    A, B = gemv70b["A"], gemv70b["B"]
    Y, U = q.linear_fwd(gemv70b["wq"], to_dev(X), to_dev(A), to_dev(B), wlc.alpha)
    with threadpool_limits(host_threads()):
        Yr, Ur = linear_fwd(_f64(X), gemv70b["w64"], _f64(A), _f64(B), lora_scale(wlc.alpha, wlc.r))
    assert_close("Y", _f64(Y), Yr)
    assert_close("U", _f64(U), Ur)


# ---- one LLaMA-65B decoder layer: 7 projections, 2048 tokens, fwd + bwd ---------

@pytest.mark.parametrize("proj", range(len(wl.LLAMA65B_LAYER)))
def test_llama65b_projection_every_output(proj):
    """2048 tokens, r = 64: every element of Y, U, dX, dA and dB against the
    float64 oracle; the quantised weight bit-exact."""
    wlc = wl.LLAMA65B_LAYER[proj]
    say(f"[full] {wlc.name}")
    inp = wlc.inputs()
    with threadpool_limits(1):
        o = oracle_weight_parallel(inp["W"])
    wq = q.quantize_weight(to_dev(inp["W"]))
    assert np.array_equal(u8(wq.packed), o["packed"])
    assert np.array_equal(u8(wq.qabsmax).view(np.int8), o["q"])
    Xd, Ad, Bd, dYd = (to_dev(inp[k]) for k in ("X", "A", "B", "dY"))
    Y, U = q.linear_fwd(wq, Xd, Ad, Bd, wlc.alpha)
    dX, dA, dB = q.linear_bwd(wq, Xd, dYd, Ad, Bd, U, wlc.alpha)
    s = lora_scale(wlc.alpha, wlc.r)
    X64, A64, B64, dY64 = (_f64(inp[k]) for k in ("X", "A", "B", "dY"))
    w64 = bf16_to_f64(o["w_hat"])
    del o
    with threadpool_limits(host_threads()):
        Yr, Ur = linear_fwd(X64, w64, A64, B64, s)
        assert_close("Y", _f64(Y), Yr)
        assert_close("U", _f64(U), Ur)
        del Yr
        dXr, dAr, dBr = linear_bwd(X64, dY64, w64, A64, B64, s)
    assert_close("dX", _f64(dX), dXr)
    assert_close("dA", _f64(dA), dAr)
    assert_close("dB", _f64(dB), dBr)
