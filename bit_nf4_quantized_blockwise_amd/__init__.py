"""Thin Python binding of libqlora.so (the gfx950 QLoRA NF4 linear library).

Argument marshalling only: torch provides device memory and the current HIP
stream; every computation runs in the library's HIP kernels.  The library must
have been built (``python -m bit_nf4_quantized_blockwise_amd.build``); there is
no fallback of any kind — a missing library raises.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qlora.h")

BLOCKSIZE = 64
DQ_GROUP = 256

STATUS = {
    0: "QLORA_OK", 1: "QLORA_ERR_NULL", 2: "QLORA_ERR_SHAPE", 3: "QLORA_ERR_ALIGN",
    4: "QLORA_ERR_UNSUPPORTED", 5: "QLORA_ERR_WORKSPACE", 6: "QLORA_ERR_DEVICE",
    7: "QLORA_ERR_LAUNCH",
}


class QloraError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class QuantJob(ctypes.Structure):
    """qlora_quant_job: one weight of a batched quantisation."""
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("packed", ctypes.c_void_p),
        ("qabsmax", ctypes.c_void_p),
        ("c2", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("nonfinite_flag", ctypes.c_void_p),
    ]


class NF4Weight(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("qabsmax", ctypes.c_void_p),
        ("c2", ctypes.c_void_p),
        ("n_out", ctypes.c_int64),
        ("k_in", ctypes.c_int64),
    ]


class AdamWTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("m", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("param_bf16", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


class AdamWPlanC(ctypes.Structure):
    _fields_ = [("device", ctypes.c_void_p), ("count", ctypes.c_int32), ("chunks", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_U64 = ctypes.c_uint64
_W = ctypes.POINTER(NF4Weight)

_SIGNATURES = {
    "qlora_quantize_nf4": ([_P, _I64, _I32, _P, _P, _P, _P], _I32),
    "qlora_double_quant": ([_P, _I64, _I32, _P, _P, _P], _I32),
    "qlora_quantize_nf4_dq": ([_P, _I64, _P, _P, _P, _P, _P, _P], _I32),
    "qlora_dequantize_nf4": ([_W, _P, _P], _I32),
    "qlora_quantize_nf4_dq_batch": ([_P, _I32, _P], _I32),
    "qlora_dequantize_nf4_batch": ([_P, _P, _I32, _P], _I32),
    "qlora_linear_fwd": ([_W, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _SZ, _P], _I32),
    "qlora_linear_fwd_noalloc": ([_W, _P, _I64, _P, _P, _I32, _F, _P, _P, _P], _I32),
    "qlora_linear_bwd": ([_W, _P, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "qlora_lora_down": ([_P, _I64, _I64, _P, _I32, _P, _P, _SZ, _P], _I32),
    "qlora_nf4_matmul_fwd": ([_W, _P, _I64, _P, _P, _I32, _F, _P, _P, _SZ, _P], _I32),
    "qlora_workspace_size": ([_I32, _I64, _I64, _I64, _I32], _SZ),
    "qlora_adamw_step": ([ctypes.POINTER(AdamWTensor), _I32, _F, _F, _F, _F, _F, _I64, _F, _P, _P,
                          _SZ, _P], _I32),
    "qlora_adamw_workspace_size": ([_I32], _SZ),
    "qlora_adamw_step_paged": ([ctypes.POINTER(AdamWTensor), _I32, _F, _F, _F, _F, _F, _I64, _F, _P,
                                _P, _SZ, _P], _I32),
    "qlora_adamw_plan_size": ([ctypes.POINTER(AdamWTensor), _I32], _SZ),
    "qlora_adamw_plan_init": ([ctypes.POINTER(AdamWTensor), _I32, _P, _SZ,
                               ctypes.POINTER(AdamWPlanC), _P], _I32),
    "qlora_adamw_plan_workspace_size": ([ctypes.POINTER(AdamWPlanC)], _SZ),
    "qlora_adamw_step_plan": ([ctypes.POINTER(AdamWPlanC), _F, _F, _F, _F, _F, _I64, _F, _P, _P,
                               _SZ, _P], _I32),
    "qlora_lora_dropout": ([_P, _I64, _I64, _F, _U64, _U64, _P, _P], _I32),
    "qlora_linear_fwd_dropout": ([_W, _P, _I64, _P, _P, _I32, _F, _F, _U64, _U64, _P, _P, _P, _P,
                                  _SZ, _P], _I32),
    "qlora_linear_bwd_dropout": ([_W, _P, _P, _I64, _P, _P, _I32, _F, _F, _U64, _U64, _P, _P, _P,
                                  _P, _P, _SZ, _P], _I32),
    "qlora_merge_adapter": ([_P, _W, _I64, _I64, _P, _P, _I32, _F, _P, _P, _P, _P, _P], _I32),
    "qlora_quantize_4bit": ([_P, _I64, _I32, _P, _P, _P], _I32),
    "qlora_dequantize_4bit": ([_P, _P, _I64, _I32, _P, _P], _I32),
    "qlora_quant_sq_error": ([_P, _I64, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
    "qlora_quant_error_workspace_size": ([_I64], _SZ),
    "qlora_nf4_codebook": ([_P], None),
    "qlora_status_string": ([_I32], ctypes.c_char_p),
    "qlora_abi_version": ([], _I32),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m bit_nf4_quantized_blockwise_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status, where):
    if status != 0:
        raise QloraError(status, where)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, shape=None, min_numel=None, cuda=True):
    """t, checked to be a contiguous CUDA tensor of dtype with the given shape
    (or at least min_numel elements): the library reads and writes through
    raw pointers over exactly these sizes, so a mismatch is an error here."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: expected at least {min_numel} elements, got {t.numel()}")
    if cuda and t.device.type != "cuda":
        raise ValueError(f"{name}: expected a CUDA tensor, got one on {t.device}")
    return t


def _opt(t, name, dtype, shape=None, min_numel=None):
    """_need for an optional argument (None passes)."""
    return None if t is None else _need(t, name, dtype, shape, min_numel)


def _ws_need(t, name="workspace"):
    """A caller's workspace: a contiguous CUDA uint8 tensor (the library checks its size)."""
    return _need(t, name, torch.uint8)


@dataclass
class NF4Tensor:
    """A frozen weight W[n_out][k_in] in NF4 + Double Quantization storage."""
    packed: torch.Tensor   # uint8 [n_out * k_in / 2]
    qabsmax: torch.Tensor  # int8  [n_out * k_in / 64]
    c2: torch.Tensor       # float32 [ceil(n_out * k_in / 64 / 256)]
    n_out: int
    k_in: int

    def validate(self):
        """self, with its three arrays checked against n_out · k_in weights."""
        nb = _nblocks(self.n_out * self.k_in)
        arrays = (("packed", self.packed, torch.uint8, nb * 32),
                  ("qabsmax", self.qabsmax, torch.int8, nb),
                  ("c2", self.c2, torch.float32, (nb + DQ_GROUP - 1) // DQ_GROUP))
        for name, t, dtype, n in arrays:
            _need(t, name, dtype, min_numel=n, cuda=False)
        for name, t, dtype, n in arrays:
            _need(t, name, dtype, min_numel=n)
        if not (self.packed.device == self.qabsmax.device == self.c2.device):
            raise ValueError("packed, qabsmax and c2 must be on one device")
        return self

    def c_struct(self):
        self.validate()
        return NF4Weight(self.packed.data_ptr(), self.qabsmax.data_ptr(), self.c2.data_ptr(),
                         self.n_out, self.k_in)

    @property
    def nbytes(self):
        return self.packed.numel() + self.qabsmax.numel() + self.c2.numel() * 4


def abi_version():
    return lib().qlora_abi_version()


def codebook():
    out = (ctypes.c_float * 16)()
    lib().qlora_nf4_codebook(ctypes.cast(out, ctypes.c_void_p))
    return [out[i] for i in range(16)]


def status_string(s):
    return lib().qlora_status_string(s).decode()


def workspace_size(op, M, n_out, k_in, r):
    return lib().qlora_workspace_size(op, M, n_out, k_in, r)


def _nblocks(n):
    return (n + BLOCKSIZE - 1) // BLOCKSIZE


def quantize_nf4(w, nonfinite_flag=None):
    """First level: (packed uint8, absmax float32) of a float32 CUDA tensor.
    nonfinite_flag: optional int32 CUDA tensor, set to 1 on NaN / Inf input."""
    _need(w, "w", torch.float32)
    _opt(nonfinite_flag, "nonfinite_flag", torch.int32, min_numel=1)
    n = w.numel()
    nb = _nblocks(n)
    packed = torch.empty(nb * 32, dtype=torch.uint8, device=w.device)
    absmax = torch.empty(nb, dtype=torch.float32, device=w.device)
    _check(lib().qlora_quantize_nf4(_ptr(w), n, BLOCKSIZE, _ptr(packed), _ptr(absmax),
                                    _ptr(nonfinite_flag), _stream(w.device)), "qlora_quantize_nf4")
    return packed, absmax


def double_quant(absmax):
    """Second level: (qabsmax int8, c2 float32)."""
    _need(absmax, "absmax", torch.float32)
    nb = absmax.numel()
    q = torch.empty(nb, dtype=torch.int8, device=absmax.device)
    c2 = torch.empty((nb + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=absmax.device)
    _check(lib().qlora_double_quant(_ptr(absmax), nb, DQ_GROUP, _ptr(q), _ptr(c2),
                                    _stream(absmax.device)), "qlora_double_quant")
    return q, c2


def quantize_nf4_dq(w, want_absmax=False, one_pass=False, nonfinite_flag=None):
    """Both levels: (packed, qabsmax, c2[, absmax]).  The first-level scales
    are always given a buffer (the faster two-launch route) unless one_pass.
    nonfinite_flag: optional int32 CUDA tensor, set to 1 on NaN / Inf input."""
    _need(w, "w", torch.float32)
    _opt(nonfinite_flag, "nonfinite_flag", torch.int32, min_numel=1)
    n = w.numel()
    nb = _nblocks(n)
    dev = w.device
    packed = torch.empty(nb * 32, dtype=torch.uint8, device=dev)
    q = torch.empty(nb, dtype=torch.int8, device=dev)
    c2 = torch.empty((nb + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=dev)
    absmax = None if one_pass else torch.empty(nb, dtype=torch.float32, device=dev)
    _check(lib().qlora_quantize_nf4_dq(_ptr(w), n, _ptr(packed), _ptr(q), _ptr(c2),
                                       _ptr(absmax), _ptr(nonfinite_flag), _stream(dev)),
           "qlora_quantize_nf4_dq")
    return (packed, q, c2, absmax) if want_absmax else (packed, q, c2)


def quantize_weight(w):
    """NF4Tensor of a float32 CUDA weight [n_out][k_in]."""
    if w.dim() != 2:
        raise ValueError(f"w: expected a 2-D weight, got shape {tuple(w.shape)}")
    n_out, k_in = w.shape
    packed, q, c2 = quantize_nf4_dq(w)
    return NF4Tensor(packed, q, c2, n_out, k_in)


def quantize_nf4_dq_batch(ws, nonfinite_flags=None):
    """Both levels for a list of float32 CUDA tensors in batched launches:
    [(packed, qabsmax, c2, absmax)], the same bytes as quantize_nf4_dq on each.
    nonfinite_flags: optional list (entries may be None) of int32 CUDA tensors."""
    outs, jobs = [], (QuantJob * max(1, len(ws)))()
    for i, w in enumerate(ws):
        _need(w, f"ws[{i}]", torch.float32)
        if w.device != ws[0].device:
            raise ValueError("all weights must be on one device")
        n = w.numel()
        nb = _nblocks(n)
        dev = w.device
        o = (torch.empty(nb * 32, dtype=torch.uint8, device=dev),
             torch.empty(nb, dtype=torch.int8, device=dev),
             torch.empty((nb + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=dev),
             torch.empty(nb, dtype=torch.float32, device=dev))
        flag = _opt(nonfinite_flags[i] if nonfinite_flags is not None else None,
                    f"nonfinite_flags[{i}]", torch.int32, min_numel=1)
        jobs[i] = QuantJob(_ptr(w), n, *(_ptr(t) for t in o), _ptr(flag))
        outs.append(o)
    if ws:
        _check(lib().qlora_quantize_nf4_dq_batch(jobs, len(ws), _stream(ws[0].device)),
               "qlora_quantize_nf4_dq_batch")
    return outs


def dequantize_nf4_batch(wqs, outs=None):
    """bf16 decoded weights of a list of NF4Tensors in batched launches."""
    if outs is None:
        outs = [torch.empty(w.n_out, w.k_in, dtype=torch.bfloat16, device=w.packed.device)
                for w in wqs]
    if len(outs) != len(wqs):
        raise ValueError("outs must have one tensor per weight")
    for i, (w, o) in enumerate(zip(wqs, outs)):
        _need(o, f"outs[{i}]", torch.bfloat16, min_numel=w.n_out * w.k_in)
    structs = (NF4Weight * max(1, len(wqs)))(*[w.c_struct() for w in wqs])
    ptrs = (ctypes.c_void_p * max(1, len(wqs)))(*[_ptr(o) for o in outs])
    if wqs:
        _check(lib().qlora_dequantize_nf4_batch(structs, ptrs, len(wqs), _stream(outs[0].device)),
               "qlora_dequantize_nf4_batch")
    return outs


def dequantize_nf4(wq, out=None):
    """bf16 [n_out][k_in] decoded weight."""
    if out is None:
        out = torch.empty(wq.n_out, wq.k_in, dtype=torch.bfloat16, device=wq.packed.device)
    _need(out, "out", torch.bfloat16, min_numel=wq.n_out * wq.k_in)
    ws = wq.c_struct()
    _check(lib().qlora_dequantize_nf4(ctypes.byref(ws), _ptr(out), _stream(out.device)),
           "qlora_dequantize_nf4")
    return out


CODES = {"nf4": 0, "int4": 1}


def _code(code):
    if code not in CODES:
        raise ValueError(f"code must be one of {sorted(CODES)}")
    return CODES[code]


def quantize_4bit(w, code="nf4"):
    """Single quantisation with either code: (packed uint8, absmax float32)."""
    _need(w, "w", torch.float32)
    n = w.numel()
    nb = _nblocks(n)
    packed = torch.empty(nb * 32, dtype=torch.uint8, device=w.device)
    absmax = torch.empty(nb, dtype=torch.float32, device=w.device)
    _check(lib().qlora_quantize_4bit(_ptr(w), n, _code(code), _ptr(packed), _ptr(absmax),
                                     _stream(w.device)), "qlora_quantize_4bit")
    return packed, absmax


def dequantize_4bit(packed, absmax, n, code="nf4", out=None):
    """bf16 [n] decoded from single-quantised storage."""
    nb = _nblocks(n)
    _need(packed, "packed", torch.uint8, min_numel=(n + 1) // 2)
    _need(absmax, "absmax", torch.float32, min_numel=nb)
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=packed.device)
    _need(out, "out", torch.bfloat16, min_numel=n)
    _check(lib().qlora_dequantize_4bit(_ptr(packed), _ptr(absmax), n, _code(code), _ptr(out),
                                       _stream(out.device)), "qlora_dequantize_4bit")
    return out


def quant_error_workspace_size(n):
    return lib().qlora_quant_error_workspace_size(n)


def quant_sq_error(w, packed, absmax, code="nf4", out=None, workspace=None):
    """float64 device tensor [1]: Σ (w − RN32(level·absmax))² over w."""
    _need(w, "w", torch.float32)
    n = w.numel()
    _need(packed, "packed", torch.uint8, min_numel=(n + 1) // 2)
    _need(absmax, "absmax", torch.float32, min_numel=_nblocks(n))
    dev = w.device
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = torch.empty(quant_error_workspace_size(n), dtype=torch.uint8, device=dev)
    _need(out, "out", torch.float64, min_numel=1)
    _ws_need(workspace)
    _check(lib().qlora_quant_sq_error(_ptr(w), n, _code(code), _ptr(packed), _ptr(absmax),
                                      _ptr(out), _ptr(workspace), workspace.numel(),
                                      _stream(dev)), "qlora_quant_sq_error")
    return out


def _workspace(op, M, wq, r, device):
    nbytes = workspace_size(op, M, wq.n_out, wq.k_in, r)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _linear_inputs(wq, M, r, **ts):
    """Checks the named operands of a linear call against its shapes: X, Xd
    and dX [M][k_in], A [r][k_in], B [n_out][r], U [M][r], Y and dY
    [M][n_out] bf16; dA [r][k_in], dB [n_out][r] float32."""
    wq.validate()
    K, N = wq.k_in, wq.n_out
    shapes = {"X": ((M, K), torch.bfloat16), "Xd": ((M, K), torch.bfloat16),
              "dX": ((M, K), torch.bfloat16), "A": ((r, K), torch.bfloat16),
              "B": ((N, r), torch.bfloat16), "U": ((M, r), torch.bfloat16),
              "Y": ((M, N), torch.bfloat16), "dY": ((M, N), torch.bfloat16),
              "dA": ((r, K), torch.float32), "dB": ((N, r), torch.float32)}
    for name, t in ts.items():
        shape, dtype = shapes[name]
        _need(t, name, dtype, shape)


def linear_fwd(wq, X, A, B, alpha, workspace=None, Y=None, U=None):
    """(Y, U): Y = X·Ŵᵀ + (alpha/r)·(X·Aᵀ)·Bᵀ, U = X·Aᵀ, bf16."""
    M, r = X.shape[0], A.shape[0]
    dev = X.device
    _linear_inputs(wq, M, r, X=X, A=A, B=B)
    Y = torch.empty(M, wq.n_out, dtype=torch.bfloat16, device=dev) if Y is None else Y
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev) if U is None else U
    _linear_inputs(wq, M, r, Y=Y, U=U)
    ws = _ws_need(_workspace(0, M, wq, r, dev) if workspace is None else workspace)
    st = wq.c_struct()
    _check(lib().qlora_linear_fwd(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, alpha,
                                  _ptr(Y), _ptr(U), _ptr(ws), ws.numel(), _stream(dev)),
           "qlora_linear_fwd")
    return Y, U


def lora_down(X, A, workspace=None, U=None):
    if X.dim() != 2 or A.dim() != 2:
        raise ValueError("X and A must be 2-D")
    M, K = X.shape
    r = A.shape[0]
    dev = X.device
    _need(X, "X", torch.bfloat16, (M, K))
    _need(A, "A", torch.bfloat16, (r, K))
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev) if U is None else U
    _need(U, "U", torch.bfloat16, (M, r))
    if workspace is None:
        workspace = torch.empty(max(workspace_size(0, M, 8, K, r), 256), dtype=torch.uint8,
                                device=dev)
    _ws_need(workspace)
    _check(lib().qlora_lora_down(_ptr(X), M, K, _ptr(A), r, _ptr(U), _ptr(workspace),
                                 workspace.numel(), _stream(dev)), "qlora_lora_down")
    return U


def nf4_matmul_fwd(wq, X, U, B, alpha, workspace=None, Y=None):
    M, r = X.shape[0], B.shape[-1]
    dev = X.device
    Y = torch.empty(M, wq.n_out, dtype=torch.bfloat16, device=dev) if Y is None else Y
    _linear_inputs(wq, M, r, X=X, U=U, B=B, Y=Y)
    ws = _ws_need(_workspace(0, M, wq, r, dev) if workspace is None else workspace)
    st = wq.c_struct()
    _check(lib().qlora_nf4_matmul_fwd(ctypes.byref(st), _ptr(X), M, _ptr(U), _ptr(B), r, alpha,
                                      _ptr(Y), _ptr(ws), ws.numel(), _stream(dev)),
           "qlora_nf4_matmul_fwd")
    return Y


def linear_bwd(wq, X, dY, A, B, U, alpha, workspace=None, dX=None, dA=None, dB=None):
    """(dX bf16, dA fp32, dB fp32)."""
    M, r = dY.shape[0], A.shape[0]
    dev = dY.device
    dX = torch.empty(M, wq.k_in, dtype=torch.bfloat16, device=dev) if dX is None else dX
    dA = torch.empty(r, wq.k_in, dtype=torch.float32, device=dev) if dA is None else dA
    dB = torch.empty(wq.n_out, r, dtype=torch.float32, device=dev) if dB is None else dB
    _linear_inputs(wq, M, r, X=X, dY=dY, A=A, B=B, U=U, dX=dX, dA=dA, dB=dB)
    ws = _ws_need(_workspace(1, M, wq, r, dev) if workspace is None else workspace)
    st = wq.c_struct()
    _check(lib().qlora_linear_bwd(ctypes.byref(st), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r,
                                  alpha, _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                  ws.numel(), _stream(dev)), "qlora_linear_bwd")
    return dX, dA, dB


# ---- adapter merge ----------------------------------------------------------------

def merge_adapter(base, A, B, alpha, requantize=True, merged=None):
    """(merged bf16 [n_out][k_in], NF4Tensor of it or None).  base: a bf16
    tensor [n_out][k_in] (the 16-bit base) or an NF4Tensor (the 4-bit base)."""
    r = A.shape[0]
    if isinstance(base, NF4Tensor):
        n_out, k_in, dev = base.n_out, base.k_in, base.packed.device
        w16, st = None, base.c_struct()
        w4 = ctypes.byref(st)
    else:
        if base.dim() != 2:
            raise ValueError(f"base: expected a 2-D weight, got shape {tuple(base.shape)}")
        (n_out, k_in), dev = base.shape, base.device
        w16, w4 = _need(base, "base", torch.bfloat16, (n_out, k_in)), None
    _need(A, "A", torch.bfloat16, (r, k_in))
    _need(B, "B", torch.bfloat16, (n_out, r))
    merged = torch.empty(n_out, k_in, dtype=torch.bfloat16, device=dev) if merged is None else merged
    _need(merged, "merged", torch.bfloat16, (n_out, k_in))
    out = None
    packed = qa = c2 = None
    if requantize:
        n = n_out * k_in
        packed = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        qa = torch.empty(n // 64, dtype=torch.int8, device=dev)
        c2 = torch.empty((n // 64 + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=dev)
        out = NF4Tensor(packed, qa, c2, n_out, k_in)
    _check(lib().qlora_merge_adapter(_ptr(w16), w4, n_out, k_in, _ptr(A), _ptr(B), r, alpha,
                                     _ptr(merged), _ptr(packed), _ptr(qa), _ptr(c2),
                                     _stream(dev)), "qlora_merge_adapter")
    return merged, out


# ---- LoRA dropout ---------------------------------------------------------------

def lora_dropout(X, p, seed, offset, Xd=None):
    """Xd = mask ⊙ X (bf16) for the dropout rate p and the (seed, offset) mask."""
    if X.dim() != 2:
        raise ValueError(f"X: expected 2-D, got shape {tuple(X.shape)}")
    M, K = X.shape
    _need(X, "X", torch.bfloat16, (M, K))
    Xd = torch.empty_like(X) if Xd is None else Xd
    _need(Xd, "Xd", torch.bfloat16, (M, K))
    _check(lib().qlora_lora_dropout(_ptr(X), M, K, p, seed, offset, _ptr(Xd), _stream(X.device)),
           "qlora_lora_dropout")
    return Xd


def linear_fwd_dropout(wq, X, A, B, alpha, p, seed, offset, workspace=None, Y=None, U=None,
                       Xd=None):
    """(Y, U, Xd) with dropout on the adapter input: Xd = mask ⊙ X,
    U = Xd·Aᵀ, Y = X·Ŵᵀ + (alpha/r)/(1 − p)·U·Bᵀ."""
    M, r = X.shape[0], A.shape[0]
    dev = X.device
    _linear_inputs(wq, M, r, X=X, A=A, B=B)
    Y = torch.empty(M, wq.n_out, dtype=torch.bfloat16, device=dev) if Y is None else Y
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev) if U is None else U
    Xd = torch.empty_like(X) if Xd is None else Xd
    _linear_inputs(wq, M, r, Y=Y, U=U, Xd=Xd)
    ws = _ws_need(_workspace(0, M, wq, r, dev) if workspace is None else workspace)
    st = wq.c_struct()
    _check(lib().qlora_linear_fwd_dropout(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, alpha,
                                          p, seed, offset, _ptr(Y), _ptr(U), _ptr(Xd), _ptr(ws),
                                          ws.numel(), _stream(dev)), "qlora_linear_fwd_dropout")
    return Y, U, Xd


def linear_bwd_dropout(wq, Xd, dY, A, B, U, alpha, p, seed, offset, workspace=None, dX=None,
                       dA=None, dB=None):
    """(dX bf16, dA fp32, dB fp32) of the dropout forward (same p, seed, offset)."""
    M, r = dY.shape[0], A.shape[0]
    dev = dY.device
    dX = torch.empty(M, wq.k_in, dtype=torch.bfloat16, device=dev) if dX is None else dX
    dA = torch.empty(r, wq.k_in, dtype=torch.float32, device=dev) if dA is None else dA
    dB = torch.empty(wq.n_out, r, dtype=torch.float32, device=dev) if dB is None else dB
    _linear_inputs(wq, M, r, Xd=Xd, dY=dY, A=A, B=B, U=U, dX=dX, dA=dA, dB=dB)
    ws = _ws_need(_workspace(2, M, wq, r, dev) if workspace is None else workspace)
    st = wq.c_struct()
    _check(lib().qlora_linear_bwd_dropout(ctypes.byref(st), _ptr(Xd), _ptr(dY), M, _ptr(A), _ptr(B),
                                          r, alpha, p, seed, offset, _ptr(U), _ptr(dX), _ptr(dA),
                                          _ptr(dB), _ptr(ws), ws.numel(), _stream(dev)),
           "qlora_linear_bwd_dropout")
    return dX, dA, dB


# ---- optimizer step on the adapter factors ------------------------------------

def adamw_workspace_size(count):
    return lib().qlora_adamw_workspace_size(count)


class AdamWList:
    """The descriptor array of one AdamW tensor list (float32 params, grads, ms,
    vs and optional bf16 copies), checked and built once so that a training
    loop can step the same tensors without re-marshalling them.  The tensors
    must stay alive and keep their storage while the list is used."""

    def __init__(self, params, grads, ms, vs, params_bf16=None):
        n = len(params)
        if not (len(grads) == len(ms) == len(vs) == n):
            raise ValueError("params, grads, ms and vs must have the same length")
        pbs = params_bf16 if params_bf16 is not None else [None] * n
        if len(pbs) != n:
            raise ValueError("params_bf16 must have one entry (or None) per param")
        arr = (AdamWTensor * max(n, 1))()
        for i in range(n):
            p = _need(params[i], f"params[{i}]", torch.float32)
            for name, t in (("grads", grads[i]), ("ms", ms[i]), ("vs", vs[i])):
                _need(t, f"{name}[{i}]", torch.float32)
                if t.numel() != p.numel():
                    raise ValueError(f"tensor {i}: sizes differ")
            _opt(pbs[i], f"params_bf16[{i}]", torch.bfloat16)
            if pbs[i] is not None and pbs[i].numel() != p.numel():
                raise ValueError(f"tensor {i}: bf16 copy size differs")
            arr[i] = AdamWTensor(p.data_ptr(), grads[i].data_ptr(), ms[i].data_ptr(),
                                 vs[i].data_ptr(),
                                 pbs[i].data_ptr() if pbs[i] is not None else None, p.numel())
        self.arr, self.count = arr, n
        self.device = params[0].device if n else torch.device("cuda")
        self._keep = (list(params), list(grads), list(ms), list(vs), list(pbs))


def adamw_step_list(lst, step, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.001,
                    max_grad_norm=0.3, grad_norm=None, workspace=None):
    """adamw_step over a prebuilt AdamWList."""
    _opt(grad_norm, "grad_norm", torch.float32, min_numel=1)
    if workspace is None:
        workspace = torch.empty(adamw_workspace_size(lst.count), dtype=torch.uint8,
                                device=lst.device)
    _ws_need(workspace)
    _check(lib().qlora_adamw_step(lst.arr, lst.count, lr, beta1, beta2, eps, weight_decay, step,
                                  max_grad_norm, _ptr(grad_norm), _ptr(workspace),
                                  workspace.numel(), _stream(lst.device)),
           "qlora_adamw_step")


def adamw_step_paged(params, grads, ms_host, vs_host, step, lr=2e-4, beta1=0.9,
                     beta2=0.999, eps=1e-8, weight_decay=0.001, max_grad_norm=0.3,
                     params_bf16=None, grad_norm=None, workspace=None):
    """adamw_step with the states m, v in pinned host memory (CPU tensors made
    with pin_memory=True), which the update reads and writes in place across
    the host link.  It runs on the current stream: synchronise it before
    reading m or v on the host."""
    n = len(params)
    pbs = params_bf16 if params_bf16 is not None else [None] * n
    arr = (AdamWTensor * max(n, 1))()
    for i in range(n):
        p = _need(params[i], f"params[{i}]", torch.float32)
        _need(grads[i], f"grads[{i}]", torch.float32)
        _opt(pbs[i], f"params_bf16[{i}]", torch.bfloat16)
        for name, t in (("ms_host", ms_host[i]), ("vs_host", vs_host[i])):
            if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or \
                    t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError(f"{name}[{i}]: expected a contiguous float32 CPU tensor")
        for t in (grads[i], ms_host[i], vs_host[i]):
            if t.numel() != p.numel():
                raise ValueError(f"tensor {i}: sizes differ")
        if pbs[i] is not None and pbs[i].numel() != p.numel():
            raise ValueError(f"tensor {i}: bf16 copy size differs")
        arr[i] = AdamWTensor(p.data_ptr(), grads[i].data_ptr(), ms_host[i].data_ptr(),
                             vs_host[i].data_ptr(),
                             pbs[i].data_ptr() if pbs[i] is not None else None, p.numel())
    _opt(grad_norm, "grad_norm", torch.float32, min_numel=1)
    dev = params[0].device if n else torch.device("cuda", torch.cuda.current_device())
    if workspace is None:
        workspace = torch.empty(adamw_workspace_size(n), dtype=torch.uint8, device=dev)
    _ws_need(workspace)
    _check(lib().qlora_adamw_step_paged(arr, n, lr, beta1, beta2, eps, weight_decay, step,
                                        max_grad_norm, _ptr(grad_norm), _ptr(workspace),
                                        workspace.numel(), _stream(dev)),
           "qlora_adamw_step_paged")


class AdamWPlan:
    """An AdamW tensor list prepared once in device memory (one launch per pass
    for any number of tensors).  Keeps the tensors and its device buffer."""

    def __init__(self, params, grads, ms, vs, params_bf16=None):
        lst = AdamWList(params, grads, ms, vs, params_bf16)
        n = lst.count
        nbytes = lib().qlora_adamw_plan_size(lst.arr, n)
        if nbytes == 0:
            raise ValueError("invalid tensor list")
        self.device = lst.device
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.c = AdamWPlanC()
        _check(lib().qlora_adamw_plan_init(lst.arr, n, _ptr(self.buf), nbytes, ctypes.byref(self.c),
                                           _stream(self.device)), "qlora_adamw_plan_init")
        self._list = lst  # keeps the tensors alive
        self.workspace = torch.empty(lib().qlora_adamw_plan_workspace_size(ctypes.byref(self.c)),
                                     dtype=torch.uint8, device=self.device)


def adamw_step_plan(plan, step, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.001,
                    max_grad_norm=0.3, grad_norm=None):
    """adamw_step over an AdamWPlan."""
    _opt(grad_norm, "grad_norm", torch.float32, min_numel=1)
    _check(lib().qlora_adamw_step_plan(ctypes.byref(plan.c), lr, beta1, beta2, eps, weight_decay,
                                       step, max_grad_norm, _ptr(grad_norm), _ptr(plan.workspace),
                                       plan.workspace.numel(), _stream(plan.device)),
           "qlora_adamw_step_plan")


def adamw_step(params, grads, ms, vs, step, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.001, max_grad_norm=0.3, params_bf16=None, grad_norm=None,
               workspace=None):
    """One 32-bit AdamW step over lists of float32 tensors (updated in place):
    params (master weights), grads, ms, vs; params_bf16 (optional list, entries
    may be None) receives the bf16 copies; grad_norm (optional float32 device
    tensor of one element) the global gradient norm before clipping.  The
    defaults are the page's training settings (lr 2e-4, weight decay 0.001,
    max_grad_norm 0.3) and the usual AdamW betas and eps."""
    adamw_step_list(AdamWList(params, grads, ms, vs, params_bf16), step, lr=lr, beta1=beta1,
                    beta2=beta2, eps=eps, weight_decay=weight_decay,
                    max_grad_norm=max_grad_norm, grad_norm=grad_norm, workspace=workspace)
