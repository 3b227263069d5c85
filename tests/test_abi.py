"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching a device.

The device pointers here are fake: every call must fail validation, or be
one that expects QLORA_ERR_DEVICE and is skipped where a GPU is present
(with a GPU such a call would launch on the fake pointers)."""

import ctypes
import re

import numpy as np
import pytest

import bit_nf4_quantized_blockwise_amd as q
from oracle.codebook import nf4_codebook_f32

OK, NULL, SHAPE, ALIGN, UNSUP, WS, DEV = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
MIS = 0x10002


@pytest.fixture(scope="module")
def L():
    return q.lib()


def _header_functions():
    txt = open(q.HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(L):
    names = _header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q._SIGNATURES), set(names) ^ set(q._SIGNATURES)


def test_abi_version_and_strings(L):
    assert q.abi_version() == 3
    for s in range(8):
        assert q.status_string(s).startswith(q.STATUS[s])


def test_codebook_matches_oracle_bitwise(L):
    got = np.array(q.codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4_codebook_f32().view(np.uint32))


def test_workspace_size(L):
    assert q.workspace_size(0, 4096, 11008, 4096, 64) > 0
    assert q.workspace_size(1, 4096, 11008, 4096, 64) > 0
    assert q.workspace_size(3, 16, 64, 64, 8) == 0
    assert q.workspace_size(2, 4096, 11008, 4096, 64) >= \
        q.workspace_size(1, 4096, 11008, 4096, 64) + 4096 * 4096 * 4
    assert q.workspace_size(0, 16, 64, 64, 0) == 0
    assert q.workspace_size(0, 16, 64, 64, 257) == 0
    assert q.workspace_size(0, 0, 64, 64, 8) >= 256
    # zero tokens plan every backward product without dividing by zero
    for op in (1, 2):
        assert q.workspace_size(op, 0, 16, 64, 4) >= 256
        assert q.workspace_size(op, 0, 75, 128, 3) >= 256


def test_quantize_argument_errors(L):
    f = L.qlora_quantize_nf4
    assert f(FAKE, 100, 32, FAKE, FAKE, None, None) == UNSUP
    assert f(FAKE, -1, 64, FAKE, FAKE, None, None) == SHAPE
    assert f(None, 100, 64, FAKE, FAKE, None, None) == NULL
    assert f(FAKE, 100, 64, None, FAKE, None, None) == NULL
    assert f(MIS, 100, 64, FAKE, FAKE, None, None) == ALIGN
    assert f(FAKE, 100, 64, FAKE, FAKE, FAKE + 2, None) == ALIGN  # the flag is an int32
    assert f(FAKE, 0, 64, None, None, None, None) == OK  # nothing to do
    g = L.qlora_double_quant
    assert g(FAKE, 10, 128, FAKE, FAKE, None) == UNSUP
    assert g(FAKE, 10, 256, MIS, FAKE, None) == ALIGN
    assert g(FAKE, -5, 256, FAKE, FAKE, None) == SHAPE
    h = L.qlora_quantize_nf4_dq
    assert h(FAKE, 10, FAKE, FAKE, None, None, None, None) == NULL
    assert h(FAKE, 10, FAKE, FAKE, FAKE, MIS, None, None) == ALIGN
    assert h(FAKE, 10, FAKE, FAKE, FAKE, None, FAKE + 1, None) == ALIGN


def _weight(n_out=64, k_in=128, packed=FAKE):
    return ctypes.byref(q.NF4Weight(packed, FAKE, FAKE, n_out, k_in))


def test_linear_argument_errors(L):
    f = L.qlora_linear_fwd
    args = lambda **kw: dict(dict(w=_weight(), X=FAKE, M=16, A=FAKE, B=FAKE, r=8, alpha=16.0,
                                  Y=FAKE, U=FAKE, ws=FAKE, wsb=1 << 30, st=None), **kw)
    call = lambda d: f(*d.values())
    assert call(args(r=0)) == UNSUP
    assert call(args(r=257)) == UNSUP
    assert call(args(M=-1)) == SHAPE
    assert call(args(w=_weight(k_in=100))) == SHAPE
    assert call(args(w=_weight(n_out=0))) == SHAPE
    assert call(args(w=_weight(n_out=-3))) == SHAPE
    assert call(args(w=_weight(packed=None))) == NULL
    assert call(args(w=_weight(packed=MIS))) == ALIGN
    assert call(args(X=None)) == NULL
    assert call(args(Y=MIS)) == ALIGN
    assert call(args(ws=None)) == WS
    assert call(args(wsb=16)) == WS
    assert f(None, FAKE, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE, FAKE, 1 << 30, None) == NULL
    b = L.qlora_linear_bwd
    assert b(_weight(), FAKE, FAKE, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE, FAKE, None, FAKE,
             1 << 30, None) == NULL
    assert b(_weight(), FAKE, FAKE, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
             None) == WS
    n = L.qlora_linear_fwd_noalloc
    assert n(_weight(), FAKE, 16, FAKE, FAKE, 0, 16.0, FAKE, FAKE, None) == UNSUP
    assert n(_weight(), None, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE, None) == NULL
    assert n(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, MIS, FAKE, None) == ALIGN
    assert n(_weight(), FAKE, 0, None, None, 8, 16.0, None, None, None) == OK  # no tokens
    # 127 tokens into 262144 outputs: the split-K partial sums exceed the buffer
    assert q.workspace_size(0, 127, 262144, 64, 8) > (64 << 20)
    assert n(_weight(n_out=262144, k_in=64), FAKE, 127, FAKE, FAKE, 8, 16.0, FAKE, FAKE,
             None) == WS
    d = L.qlora_dequantize_nf4
    assert d(ctypes.byref(q.NF4Weight(FAKE, FAKE, FAKE, 3, 5)), FAKE, None) == SHAPE
    assert d(ctypes.byref(q.NF4Weight(FAKE, FAKE, FAKE, 4, 16)), MIS, None) == ALIGN


def test_forward_parts_argument_errors(L):
    down = L.qlora_lora_down
    dargs = lambda **kw: dict(dict(X=FAKE, M=200, K=128, A=FAKE, r=8, U=FAKE, ws=FAKE,
                                   wsb=1 << 30, st=None), **kw)
    dcall = lambda d: down(*d.values())
    assert dcall(dargs(r=0)) == UNSUP
    assert dcall(dargs(r=257)) == UNSUP
    assert dcall(dargs(M=-1)) == SHAPE
    assert dcall(dargs(K=100)) == SHAPE
    assert dcall(dargs(K=0)) == SHAPE
    assert dcall(dargs(M=0, X=None, A=None, U=None, ws=None)) == OK  # no tokens
    assert dcall(dargs(X=None)) == NULL
    assert dcall(dargs(A=MIS)) == ALIGN
    assert dcall(dargs(U=MIS)) == ALIGN
    assert dcall(dargs(ws=None)) == WS  # many tokens: split partial sums in the workspace
    assert dcall(dargs(wsb=16)) == WS
    mm = L.qlora_nf4_matmul_fwd
    margs = lambda **kw: dict(dict(w=_weight(), X=FAKE, M=16, U=FAKE, B=FAKE, r=8, alpha=16.0,
                                   Y=FAKE, ws=FAKE, wsb=1 << 30, st=None), **kw)
    mcall = lambda d: mm(*d.values())
    assert mcall(margs(r=0)) == UNSUP
    assert mcall(margs(M=-1)) == SHAPE
    assert mcall(margs(w=_weight(k_in=100))) == SHAPE
    assert mcall(margs(w=None)) == NULL
    assert mcall(margs(w=_weight(packed=MIS))) == ALIGN
    assert mcall(margs(M=0, X=None, U=None, B=None, Y=None, ws=None)) == OK  # no tokens
    assert mcall(margs(U=None)) == NULL
    assert mcall(margs(B=MIS)) == ALIGN
    assert mcall(margs(Y=None)) == NULL
    assert mcall(margs(ws=None)) == WS
    assert mcall(margs(wsb=16)) == WS


def test_batch_argument_errors(L):
    qb, db = L.qlora_quantize_nf4_dq_batch, L.qlora_dequantize_nf4_batch
    assert qb(None, 0, None) == OK
    assert qb(None, -1, None) == SHAPE
    assert qb(None, 2, None) == NULL
    jobs = (q.QuantJob * 2)(q.QuantJob(FAKE, 100, FAKE, FAKE, FAKE, FAKE, None),
                            q.QuantJob(FAKE, 64, FAKE, FAKE, FAKE, None, None))
    assert qb(jobs, 2, None) == NULL  # the first-level scales need a buffer
    jobs[1] = q.QuantJob(FAKE, 64, FAKE, MIS, FAKE, FAKE, None)
    assert qb(jobs, 2, None) == ALIGN
    jobs[1] = q.QuantJob(FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE + 2)
    assert qb(jobs, 2, None) == ALIGN
    jobs[1] = q.QuantJob(FAKE, -5, FAKE, FAKE, FAKE, FAKE, None)
    assert qb(jobs, 2, None) == SHAPE
    assert db(None, None, 0, None) == OK
    assert db(None, None, -1, None) == SHAPE
    assert db(None, None, 1, None) == NULL
    ws = (q.NF4Weight * 2)(q.NF4Weight(FAKE, FAKE, FAKE, 4, 16), q.NF4Weight(FAKE, FAKE, FAKE, 3, 5))
    outs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert db(ws, outs, 2, None) == SHAPE
    ws[1] = q.NF4Weight(FAKE, FAKE, FAKE, 4, 16)
    outs[1] = MIS
    assert db(ws, outs, 2, None) == ALIGN
    ws[1] = q.NF4Weight(None, FAKE, FAKE, 4, 16)
    outs[1] = FAKE
    assert db(ws, outs, 2, None) == NULL


def test_valid_arguments_without_gpu_report_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.qlora_quantize_nf4(FAKE, 100, 64, FAKE, FAKE, None, None) == DEV
    assert L.qlora_quantize_nf4(FAKE, 100, 64, FAKE, FAKE, FAKE, None) == DEV
    jobs = (q.QuantJob * 2)(q.QuantJob(FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE),
                            q.QuantJob(None, 0, None, None, None, None, None))  # an empty job is skipped
    assert L.qlora_quantize_nf4_dq_batch(jobs, 2, None) == DEV
    ws = (q.NF4Weight * 1)(q.NF4Weight(FAKE, FAKE, FAKE, 4, 16))
    assert L.qlora_dequantize_nf4_batch(ws, (ctypes.c_void_p * 1)(FAKE), 1, None) == DEV
    assert L.qlora_linear_fwd(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE, FAKE, 1 << 30,
                              None) == DEV
    assert L.qlora_linear_fwd_noalloc(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, FAKE, FAKE,
                                      None) == DEV
    # few tokens: U needs no workspace
    assert L.qlora_lora_down(FAKE, 8, 128, FAKE, 8, FAKE, None, 0, None) == DEV
    # an 8-byte aligned sum is accepted (it is one double)
    assert L.qlora_quant_sq_error(FAKE, 100, 0, FAKE, FAKE, FAKE + 8, FAKE, 4096, None) == DEV


def test_adamw_argument_errors(L):
    T = q.AdamWTensor
    good = T(FAKE, FAKE, FAKE, FAKE, None, 8)
    arr = (T * 2)(good, good)
    f = L.qlora_adamw_step
    args = dict(lr=2e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.001, step=1, clip=0.3)

    def call(a=arr, n=2, ws=FAKE, wsb=1 << 20, gn=None, **kw):
        p = dict(args, **kw)
        return f(a, n, p["lr"], p["b1"], p["b2"], p["eps"], p["wd"], p["step"], p["clip"], gn, ws,
                 wsb, None)

    assert call(n=-1) == SHAPE
    assert call(step=0) == SHAPE
    assert call(b1=1.0) == UNSUP
    assert call(b2=-0.1) == UNSUP
    assert call(eps=0.0) == UNSUP
    assert call(lr=-1.0) == UNSUP
    assert call(wd=float("nan")) == UNSUP
    assert call(ws=None) == WS                     # clipping needs the workspace
    assert call(wsb=8) == WS
    assert call(gn=MIS) == ALIGN
    bad = (T * 1)(T(MIS, FAKE, FAKE, FAKE, None, 8))
    assert call(a=bad, n=1) == ALIGN
    bad = (T * 1)(T(FAKE, None, FAKE, FAKE, None, 8))
    assert call(a=bad, n=1) == NULL
    bad = (T * 1)(T(FAKE, FAKE, FAKE, FAKE, None, -1))
    assert call(a=bad, n=1) == SHAPE
    pg = L.qlora_adamw_step_paged

    def paged(ws=FAKE, wsb=1 << 20, **kw):
        p = dict(args, **kw)
        return pg(arr, 2, p["lr"], p["b1"], p["b2"], p["eps"], p["wd"], p["step"], p["clip"], None,
                  ws, wsb, None)
    assert paged(ws=None) == WS  # clipping needs the workspace
    assert paged(wsb=8) == WS
    assert paged(step=0) == SHAPE
    assert paged(b1=1.0) == UNSUP
    assert L.qlora_adamw_workspace_size(-1) == 0
    assert L.qlora_adamw_workspace_size(0) >= 256
    assert L.qlora_adamw_workspace_size(200) >= 5 * 256 * 8


def test_quantizer_variant_argument_errors(L):
    f = L.qlora_quantize_4bit
    assert f(FAKE, 100, 2, FAKE, FAKE, None) == UNSUP
    assert f(FAKE, -1, 1, FAKE, FAKE, None) == SHAPE
    assert f(None, 100, 1, FAKE, FAKE, None) == NULL
    assert f(FAKE, 100, 1, FAKE, MIS, None) == ALIGN
    assert f(None, 0, 1, None, None, None) == OK
    d = L.qlora_dequantize_4bit
    assert d(FAKE, FAKE, 100, -1, FAKE, None) == UNSUP
    assert d(FAKE, FAKE, -3, 0, FAKE, None) == SHAPE
    assert d(FAKE, None, 100, 0, FAKE, None) == NULL
    assert d(FAKE, FAKE, 100, 1, MIS, None) == ALIGN
    assert d(None, None, 0, 1, None, None) == OK
    e = L.qlora_quant_sq_error
    ws = L.qlora_quant_error_workspace_size
    assert ws(-1) == 0 and ws(0) >= 256 and ws(10 ** 9) >= 2048 * 8
    assert e(FAKE, 100, 3, FAKE, FAKE, FAKE, FAKE, 4096, None) == UNSUP
    assert e(FAKE, 100, 0, FAKE, FAKE, None, FAKE, 4096, None) == NULL
    assert e(FAKE, 100, 0, FAKE, FAKE, FAKE + 4, FAKE, 4096, None) == ALIGN
    assert e(FAKE, 100, 0, FAKE, FAKE, FAKE, None, 4096, None) == WS
    assert e(FAKE, 100, 0, FAKE, FAKE, FAKE, FAKE, 8, None) == WS
    assert e(MIS, 100, 0, FAKE, FAKE, FAKE, FAKE, 4096, None) == ALIGN


def test_dropout_argument_errors(L):
    d = L.qlora_lora_dropout
    assert d(FAKE, 16, 64, 1.0, 1, 2, FAKE, None) == UNSUP
    assert d(FAKE, 16, 64, -0.1, 1, 2, FAKE, None) == UNSUP
    assert d(FAKE, 16, 64, float("nan"), 1, 2, FAKE, None) == UNSUP
    assert d(FAKE, 16, 60, 0.05, 1, 2, FAKE, None) == SHAPE
    assert d(FAKE, 16, 64, 0.05, 1, 2, MIS, None) == ALIGN
    assert d(None, 0, 64, 0.05, 1, 2, None, None) == OK
    f = L.qlora_linear_fwd_dropout
    assert f(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, 1.5, 1, 2, FAKE, FAKE, FAKE, FAKE, 1 << 30,
             None) == UNSUP
    assert f(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, 0.05, 1, 2, FAKE, FAKE, None, FAKE, 1 << 30,
             None) == NULL
    assert f(_weight(), FAKE, 16, FAKE, FAKE, 8, 16.0, 0.05, 1, 2, FAKE, FAKE, FAKE, FAKE, 8,
             None) == WS
    b = L.qlora_linear_bwd_dropout
    ws1 = q.workspace_size(1, 16, 64, 128, 8)
    assert b(_weight(), FAKE, FAKE, 16, FAKE, FAKE, 8, 16.0, 0.05, 1, 2, FAKE, FAKE, FAKE, FAKE,
             FAKE, ws1, None) == WS  # needs the op-2 size
    assert b(_weight(), FAKE, FAKE, 16, FAKE, FAKE, 8, 16.0, 1.0, 1, 2, FAKE, FAKE, FAKE, FAKE,
             FAKE, 1 << 30, None) == UNSUP
    assert b(_weight(), None, FAKE, 16, FAKE, FAKE, 8, 16.0, 0.05, 1, 2, FAKE, FAKE, FAKE, FAKE,
             FAKE, 1 << 30, None) == NULL


def test_merge_argument_errors(L):
    m = L.qlora_merge_adapter
    w4 = _weight(64, 128)
    assert m(None, None, 64, 128, FAKE, FAKE, 8, 16.0, FAKE, None, None, None, None) == NULL
    assert m(FAKE, w4, 64, 128, FAKE, FAKE, 8, 16.0, FAKE, None, None, None, None) == UNSUP
    assert m(FAKE, None, 64, 100, FAKE, FAKE, 8, 16.0, FAKE, None, None, None, None) == SHAPE
    assert m(FAKE, None, 64, 128, FAKE, FAKE, 0, 16.0, FAKE, None, None, None, None) == UNSUP
    assert m(FAKE, None, 64, 128, FAKE, FAKE, 257, 16.0, FAKE, None, None, None, None) == UNSUP
    assert m(None, _weight(32, 128), 64, 128, FAKE, FAKE, 8, 16.0, FAKE, None, None, None,
             None) == SHAPE
    assert m(FAKE, None, 64, 128, FAKE, FAKE, 8, 16.0, None, None, None, None, None) == NULL
    assert m(FAKE, None, 64, 128, FAKE, FAKE, 8, 16.0, FAKE, FAKE, MIS, FAKE, None) == ALIGN
    assert m(FAKE, None, 0, 128, FAKE, FAKE, 8, 16.0, None, None, None, None, None) == OK


def test_adamw_plan_argument_errors(L):
    T = q.AdamWTensor
    good = T(FAKE, FAKE, FAKE, FAKE, None, 5000)
    arr = (T * 2)(good, good)
    assert L.qlora_adamw_plan_size(arr, 2) >= 2 * 56 + 4 * 2 * 3
    assert L.qlora_adamw_plan_size(arr, -1) == 0
    bad = (T * 1)(T(FAKE, FAKE, FAKE, FAKE, None, -3))
    assert L.qlora_adamw_plan_size(bad, 1) == 0
    plan = q.AdamWPlanC()
    init = L.qlora_adamw_plan_init
    assert init(arr, 2, FAKE, 8, ctypes.byref(plan), None) == WS
    assert init(arr, 2, None, 1 << 20, ctypes.byref(plan), None) == WS
    assert init(arr, 2, FAKE, 1 << 20, None, None) == NULL
    mis = (T * 1)(T(MIS, FAKE, FAKE, FAKE, None, 8))
    assert init(mis, 1, FAKE, 1 << 20, ctypes.byref(plan), None) == ALIGN
    step = L.qlora_adamw_step_plan
    p = q.AdamWPlanC(FAKE, 2, 5)
    assert L.qlora_adamw_plan_workspace_size(ctypes.byref(p)) >= 256 + 8 * 5
    assert step(None, 2e-4, 0.9, 0.999, 1e-8, 0.0, 1, 0.3, None, FAKE, 1 << 20, None) == NULL
    assert step(ctypes.byref(p), 2e-4, 0.9, 0.999, 1e-8, 0.0, 0, 0.3, None, FAKE, 1 << 20,
                None) == SHAPE
    assert step(ctypes.byref(p), 2e-4, 1.0, 0.999, 1e-8, 0.0, 1, 0.3, None, FAKE, 1 << 20,
                None) == UNSUP
    assert step(ctypes.byref(p), 2e-4, 0.9, 0.999, 1e-8, 0.0, 1, 0.3, None, FAKE, 8, None) == WS
    assert step(ctypes.byref(q.AdamWPlanC(None, 2, 5)), 2e-4, 0.9, 0.999, 1e-8, 0.0, 1, 0.0,
                None, None, 0, None) == NULL
