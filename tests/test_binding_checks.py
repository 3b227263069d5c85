"""The Python binding checks every tensor it hands to the library (dtype,
contiguity, shape or size, device) and raises ValueError before any library
call, so a mismatched tensor cannot make the library read or write past it."""

import pytest
import torch

import bit_nf4_quantized_blockwise_amd as q


def _raises(fn, fragment):
    with pytest.raises(ValueError, match=fragment):
        fn()


def test_need_checks_type_dtype_layout_shape_size_and_device():
    t = torch.zeros(4, 8, dtype=torch.bfloat16)
    _raises(lambda: q._need([1, 2], "x", torch.bfloat16), "expected a torch.Tensor")
    _raises(lambda: q._need(t.float(), "x", torch.bfloat16), "expected torch.bfloat16")
    _raises(lambda: q._need(t.t(), "x", torch.bfloat16), "contiguous")
    _raises(lambda: q._need(t, "x", torch.bfloat16, shape=(8, 4)), r"shape \(8, 4\)")
    _raises(lambda: q._need(t, "x", torch.bfloat16, min_numel=33), "at least 33")
    _raises(lambda: q._need(t, "x", torch.bfloat16, shape=(4, 8)), "CUDA tensor")
    assert q._opt(None, "x", torch.bfloat16) is None


def _cpu_weight(n_out=16, k_in=64):
    n = n_out * k_in
    return q.NF4Tensor(torch.zeros(n // 2, dtype=torch.uint8), torch.zeros(n // 64, dtype=torch.int8),
                       torch.zeros(1, dtype=torch.float32), n_out, k_in)


def test_weight_arrays_checked_against_their_shape():
    w = _cpu_weight()
    short = q.NF4Tensor(w.packed[:-1], w.qabsmax, w.c2, w.n_out, w.k_in)
    _raises(short.validate, "packed: expected at least 512")
    wrong = q.NF4Tensor(w.packed, w.qabsmax.to(torch.uint8), w.c2, w.n_out, w.k_in)
    _raises(wrong.validate, "qabsmax: expected torch.int8")
    no_c2 = q.NF4Tensor(w.packed, w.qabsmax, torch.zeros(0, dtype=torch.float32), w.n_out, w.k_in)
    _raises(no_c2.validate, "c2: expected at least 1")
    _raises(w.validate, "CUDA tensor")


def test_linear_operands_checked_before_any_library_call():
    w = _cpu_weight()
    w.validate = lambda: w  # the weight's own checks are covered above
    M, r = 3, 8
    X = torch.zeros(M, 64, dtype=torch.bfloat16)
    A = torch.zeros(r, 64, dtype=torch.bfloat16)
    B = torch.zeros(16, r, dtype=torch.bfloat16)
    _raises(lambda: q._linear_inputs(w, M, r, X=X.float()), "X: expected torch.bfloat16")
    _raises(lambda: q._linear_inputs(w, M, r, A=torch.zeros(r, 32, dtype=torch.bfloat16)),
            r"A: expected shape \(8, 64\)")
    _raises(lambda: q._linear_inputs(w, M, r, B=B.t().contiguous()), r"B: expected shape \(16, 8\)")
    _raises(lambda: q._linear_inputs(w, M, r, dA=torch.zeros(r, 64, dtype=torch.bfloat16)),
            "dA: expected torch.float32")
    _raises(lambda: q._linear_inputs(w, M, r, X=X), "X: expected a CUDA tensor")
    # the entry points run these checks first: CPU tensors never reach the library
    _raises(lambda: q.linear_fwd(w, X, A, B, 16.0), "CUDA tensor")
    _raises(lambda: q.linear_bwd(w, X, torch.zeros(M, 16, dtype=torch.bfloat16), A, B,
                                 torch.zeros(M, r, dtype=torch.bfloat16), 16.0), "CUDA tensor")


def test_quantiser_and_merge_inputs_checked():
    _raises(lambda: q.quantize_nf4(torch.zeros(64, dtype=torch.float16)), "w: expected torch.float32")
    _raises(lambda: q.quantize_nf4_dq(torch.zeros(64, 2).t()), "contiguous")
    _raises(lambda: q.quantize_4bit(torch.zeros(64)), "CUDA tensor")
    _raises(lambda: q.quantize_weight(torch.zeros(64)), "2-D")
    _raises(lambda: q.merge_adapter(torch.zeros(16, 64, dtype=torch.float32),
                                    torch.zeros(8, 64, dtype=torch.bfloat16),
                                    torch.zeros(16, 8, dtype=torch.bfloat16), 16.0),
            "base: expected torch.bfloat16")
    _raises(lambda: q.lora_dropout(torch.zeros(4, 64, dtype=torch.bfloat16), 0.1, 1, 0), "CUDA tensor")
