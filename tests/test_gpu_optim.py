"""GPU parity of the 32-bit AdamW step against the oracle.

Each step is checked on its own: the oracle (float64) starts from the GPU's
previous float32 state, so the bound covers one step's float32 arithmetic.
With D = sqrt(v_ref)/sqrt(1-β2^t) + eps and
|u| = lr/(1-β1^t) · (β1·|m_prev| + (1-β1)·|g|) / D the update term taken at
the magnitudes of the two terms that make up m (the new m can nearly cancel,
so its float32 rounding error is relative to those magnitudes, not to m):
  |p - p_ref| <= 16·2^-24·|u| + 2·2^-24·(|p_prev| + |p_ref|)
  |m - m_ref| <= 4·2^-24·(β1·|m_prev| + (1-β1)·|g|)
  |v - v_ref| <= 6·2^-24·(β2·v_prev + (1-β2)·g²)
(a few roundings each: the products, the sum, sqrt, the division, and the
float32 step size, bias correction and clipping coefficient).  The oracle is
given the hyperparameters as the float32 values the entry point receives
(0.9 as a float32 is 0.89999998, and 1 - β1 then differs from 0.1 by 4 ulp).
The bf16 copy must be RNE_bf16 of the float32 result, bit for bit."""

import numpy as np
import pytest
import torch

from oracle.optim import BETA1, BETA2, EPS, adamw_step, clip_coefficient, global_grad_norm

from support import host, say

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")

ULP = 2.0 ** -24


def f32(x):
    return float(np.float32(x))


B1, B2, E = f32(BETA1), f32(BETA2), f32(EPS)


def _state(rng, n, step0):
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * rng.uniform(0.01, 2.0)).astype(np.float32)
    if step0 == 0:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    else:  # a state as after some steps
        m = (rng.standard_normal(n) * 0.05).astype(np.float32)
        v = (np.abs(rng.standard_normal(n)) * 0.01).astype(np.float32)
    return p, g, m, v


def _np(t):
    return host(t).numpy()


def _run(sizes, steps, lr=2e-4, wd=0.001, max_norm=0.3, seed=0, step0=0, plan=False):
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    st = [_state(rng, n, step0) for n in sizes]
    P = [torch.from_numpy(s[0].copy()).to(dev) for s in st]
    M = [torch.from_numpy(s[2].copy()).to(dev) for s in st]
    V = [torch.from_numpy(s[3].copy()).to(dev) for s in st]
    G = [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]
    PB = [torch.empty(n, dtype=torch.bfloat16, device=dev) if i % 2 == 0 else None
          for i, n in enumerate(sizes)]
    norm_t = torch.zeros(4, dtype=torch.float32, device=dev)
    pl = q.AdamWPlan(P, G, M, V, PB) if plan else None
    for k, step in enumerate(steps):
        grads = [(rng.standard_normal(n) * (0.1 + i)).astype(np.float32)
                 for i, n in enumerate(sizes)]
        for t, g in zip(G, grads):
            t.copy_(torch.from_numpy(g))
        p0 = [_np(x).astype(np.float64) for x in P]
        m0 = [_np(x).astype(np.float64) for x in M]
        v0 = [_np(x).astype(np.float64) for x in V]
        say(f"[adamw] sizes={sizes} step={step} max_norm={max_norm} plan={plan}")
        if plan:
            q.adamw_step_plan(pl, step, lr=lr, weight_decay=wd, max_grad_norm=max_norm,
                              grad_norm=norm_t[:1])
        else:
            q.adamw_step(P, G, M, V, step, lr=lr, weight_decay=wd, max_grad_norm=max_norm,
                         params_bf16=PB, grad_norm=norm_t[:1])
        torch.cuda.synchronize()
        norm = global_grad_norm(grads)
        assert abs(float(_np(norm_t)[0]) - norm) <= 1e-6 * norm + 1e-30
        coef = clip_coefficient(norm, f32(max_norm))
        for i in range(len(sizes)):
            pr, mr, vr = adamw_step(p0[i], grads[i], m0[i], v0[i], step, f32(lr), beta1=B1,
                                    beta2=B2, eps=E, weight_decay=f32(wd), coef=coef)
            gp, gm, gv = (_np(x).astype(np.float64) for x in (P[i], M[i], V[i]))
            g = np.asarray(grads[i], np.float64) * coef
            u = ((f32(lr) / (1 - B1 ** step)) * (B1 * np.abs(m0[i]) + (1 - B1) * np.abs(g))
                 / (np.sqrt(vr / (1 - B2 ** step)) + E))
            bp = 16 * ULP * np.abs(u) + 2 * ULP * (np.abs(p0[i]) + np.abs(pr)) + 1e-30
            worst = np.max(np.abs(gp - pr) / bp) if gp.size else 0.0
            assert worst <= 1.0, (i, worst)
            assert np.all(np.abs(gm - mr) <= 4 * ULP * (B1 * np.abs(m0[i]) + (1 - B1) * np.abs(g))
                          + 1e-30), i
            assert np.all(np.abs(gv - vr) <= 6 * ULP * (B2 * v0[i] + (1 - B2) * g * g) + 1e-38), i
            if PB[i] is not None:
                ref = P[i].to(torch.bfloat16)  # RNE of the float32 master
                assert torch.equal(PB[i].view(torch.int16), ref.view(torch.int16)), i


@pytest.mark.parametrize("plan", [False, True])
@pytest.mark.parametrize("max_norm", [0.3, 0.0, 1e6])
def test_multi_tensor_steps(max_norm, plan):
    _run([1, 3, 4, 5, 257, 4096 * 64 + 3, 0, 11008], [1, 2, 3], max_norm=max_norm, plan=plan)


@pytest.mark.parametrize("plan", [False, True])
def test_late_step_and_existing_moments(plan):
    _run([64 * 4096, 11008 * 64], [1000, 1001], step0=1, seed=3, plan=plan)


@pytest.mark.parametrize("plan", [False, True])
def test_more_tensors_than_one_launch_holds(plan):
    # 100 tensors: three kernel-argument launches share one global norm; one
    # launch over the prepared list
    _run([17 + (i * 37) % 300 for i in range(100)], [1, 2], seed=5, plan=plan)


def test_prepared_list_of_the_page_sized_adapter_set():
    # 256 tensors as in LLaMA-7B's attention adapters, shrunk to 4096 x 8 each
    _run([4096 * 8] * 256, [1, 2], seed=8, plan=True)


def test_no_decay_no_clip_repeatable():
    dev = torch.device("cuda:0")
    outs = []
    for _ in range(2):
        state = _state(np.random.default_rng(9), 100003, 0)
        p, g, m, v = (torch.from_numpy(x).to(dev) for x in state)
        q.adamw_step([p], [g], [m], [v], 1, lr=1e-3, weight_decay=0.0, max_grad_norm=0.0)
        torch.cuda.synchronize()
        outs.append((_np(p).view(np.uint32), _np(m).view(np.uint32), _np(v).view(np.uint32)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_empty_list_and_zero_sizes():
    dev = torch.device("cuda:0")
    q.adamw_step([], [], [], [], 1)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    q.adamw_step([e], [e], [e], [e], 1)
    pl = q.AdamWPlan([e], [e], [e], [e])
    norm = torch.full((1,), 7.0, device=dev)
    q.adamw_step_plan(pl, 1, grad_norm=norm)
    torch.cuda.synchronize()
    assert float(norm.cpu()[0]) == 0.0


def test_prepared_list_repeatable():
    dev = torch.device("cuda:0")
    outs = []
    for _ in range(2):
        state = _state(np.random.default_rng(9), 100003, 0)
        p, g, m, v = (torch.from_numpy(x).to(dev) for x in state)
        pl = q.AdamWPlan([p], [g], [m], [v])
        q.adamw_step_plan(pl, 1, lr=1e-3, max_grad_norm=0.3)
        torch.cuda.synchronize()
        outs.append((_np(p).view(np.uint32), _np(m).view(np.uint32), _np(v).view(np.uint32)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def _paged_vs_resident(sizes, steps, max_norm, seed):
    """The paged step (m, v in pinned host memory, updated there across the
    host link) against the resident step from the same state: p, m, v, the
    bf16 copies and the norm bit for bit, step after step."""
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    st = [_state(rng, n, 1) for n in sizes]
    P1 = [torch.from_numpy(s[0].copy()).to(dev) for s in st]
    P2 = [x.clone() for x in P1]
    M1 = [torch.from_numpy(s[2].copy()).to(dev) for s in st]
    V1 = [torch.from_numpy(s[3].copy()).to(dev) for s in st]
    M2 = [torch.from_numpy(s[2].copy()).pin_memory() for s in st]
    V2 = [torch.from_numpy(s[3].copy()).pin_memory() for s in st]
    G = [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]
    PB1 = [torch.empty(n, dtype=torch.bfloat16, device=dev) if i % 2 == 0 else None
           for i, n in enumerate(sizes)]
    PB2 = [torch.empty_like(x) if x is not None else None for x in PB1]
    n1, n2 = (torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(2))
    for step in steps:
        say(f"[adamw paged] {len(sizes)} tensors step={step} max_norm={max_norm}")
        for t in G:
            t.copy_(torch.from_numpy((rng.standard_normal(t.numel()) * 0.3).astype(np.float32)))
        q.adamw_step(P1, G, M1, V1, step, max_grad_norm=max_norm, params_bf16=PB1, grad_norm=n1)
        q.adamw_step_paged(P2, G, M2, V2, step, max_grad_norm=max_norm, params_bf16=PB2,
                           grad_norm=n2)
        torch.cuda.synchronize()
        assert torch.equal(n1.view(torch.int32), n2.view(torch.int32))
        for i in range(len(sizes)):
            assert torch.equal(P1[i].view(torch.int32), P2[i].view(torch.int32)), i
            assert torch.equal(host(M1[i]).view(torch.int32), M2[i].view(torch.int32)), i
            assert torch.equal(host(V1[i]).view(torch.int32), V2[i].view(torch.int32)), i
            if PB1[i] is not None:
                assert torch.equal(PB1[i].view(torch.int16), PB2[i].view(torch.int16)), i


@pytest.mark.parametrize("max_norm", [0.3, 0.0])
def test_paged_step_equals_resident_step(max_norm):
    # ragged sizes (tails of 1-3 elements, a partial last chunk, an empty tensor)
    _paged_vs_resident([1, 3, 4, 5, 257, 4096 * 64 + 3, 0, 11008, 100003], [1, 2, 3], max_norm,
                       seed=7)


def test_paged_step_more_tensors_than_one_launch_holds():
    # 100 small tensors: three launches of at most 48 descriptors
    _paged_vs_resident([17 + (i * 37) % 300 for i in range(100)], [1, 2], 0.3, seed=11)


def test_paged_step_states_at_an_offset_into_their_allocation():
    # m and v as views into larger pinned buffers (the device address of each
    # view, not of its allocation, must be used)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(13)
    n = 5000
    p0, m0, v0 = (rng.standard_normal(n).astype(np.float32) * s for s in (0.01, 1e-4, 1e-6))
    v0 = np.abs(v0)
    g = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 0.3).to(dev)
    P1, P2 = torch.from_numpy(p0).to(dev), torch.from_numpy(p0).to(dev)
    M1, V1 = torch.from_numpy(m0).to(dev), torch.from_numpy(v0).to(dev)
    mbuf = torch.zeros(n + 1024).pin_memory()
    vbuf = torch.zeros(n + 4096).pin_memory()
    M2, V2 = mbuf[512:512 + n], vbuf[2048:2048 + n]
    M2.copy_(torch.from_numpy(m0))
    V2.copy_(torch.from_numpy(v0))
    q.adamw_step([P1], [g], [M1], [V1], 1, max_grad_norm=0.3)
    q.adamw_step_paged([P2], [g], [M2], [V2], 1, max_grad_norm=0.3)
    torch.cuda.synchronize()
    assert torch.equal(P1.view(torch.int32), P2.view(torch.int32))
    assert torch.equal(host(M1).view(torch.int32), M2.view(torch.int32))
    assert torch.equal(host(V1).view(torch.int32), V2.view(torch.int32))
    assert torch.all(mbuf[:512] == 0) and torch.all(mbuf[512 + n:] == 0)
    assert torch.all(vbuf[:2048] == 0) and torch.all(vbuf[2048 + n:] == 0)


def test_paged_step_rejects_unpinned_states():
    dev = torch.device("cuda:0")
    p = torch.zeros(100, device=dev)
    g = torch.ones(100, device=dev)
    v_pin = torch.zeros(100).pin_memory()
    m_pageable = torch.zeros(100)
    with pytest.raises(q.QloraError) as e:
        q.adamw_step_paged([p], [g], [m_pageable], [v_pin], 1)
    assert e.value.status == 4
    with pytest.raises(ValueError):  # device memory is not a host state either
        q.adamw_step_paged([p], [g], [torch.zeros(100, device=dev)], [v_pin], 1)
    torch.cuda.synchronize()
    assert torch.all(p == 0)  # nothing ran
