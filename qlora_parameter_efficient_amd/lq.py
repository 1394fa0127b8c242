"""ctypes binding of liblq.so (include/lq.h): argument marshalling only.

Each function here has the name of the C entry point it calls and does
nothing but check tensor placement / dtype, allocate outputs with torch (device
memory plumbing), pass raw pointers and the current HIP stream, and turn a
negative status into an exception.  All arithmetic runs in the library's
kernels; if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lq.h")

LQ_F32, LQ_BF16 = 0, 1
LQ_WEIGHT_DENSE, LQ_WEIGHT_NF4 = 0, 1
LQ_OP_FWD, LQ_OP_BWD, LQ_OP_FWD_MULTI, LQ_OP_FWD_FUSED, LQ_OP_BWD_FUSED = 0, 1, 2, 3, 4
LQ_OP_FWD_MULTI_FUSED = 5
LQ_OP_FWD_DROPOUT, LQ_OP_FWD_DROPOUT_FUSED, LQ_OP_BWD_DROPOUT, LQ_OP_BWD_DROPOUT_FUSED = 6, 7, 8, 9
LQ_OP_DORA_FWD, LQ_OP_DORA_FWD_FUSED, LQ_OP_DORA_BWD, LQ_OP_DORA_BWD_FUSED = 10, 11, 12, 13
LQ_DQ_NONE, LQ_DQ_INT8, LQ_DQ_FP8 = 0, 1, 2
LQ_NOALLOC_SCRATCH_BYTES = 64 << 20
LQ_CB_NF4, LQ_CB_NF4_SYMMETRIC = 0, 1
DQ_FORMATS = {"int8": LQ_DQ_INT8, "fp8": LQ_DQ_FP8}
CODEBOOKS = {"nf4": LQ_CB_NF4, "nf4_symmetric": LQ_CB_NF4_SYMMETRIC}
STATUS = {0: "LQ_OK", -1: "LQ_ERR_INVALID_ARG", -2: "LQ_ERR_UNSUPPORTED",
          -3: "LQ_ERR_WORKSPACE", -4: "LQ_ERR_HIP"}


class LqError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class LqWeightStruct(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("dense", ctypes.c_void_p), ("codes", ctypes.c_void_p),
        ("q8", ctypes.c_void_p), ("c2", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
        ("double_quant", ctypes.c_int32), ("codebook", ctypes.c_int32),
    ]


class LqAdamwTensor(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("grad", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("n", ctypes.c_int64)]


_lib = None
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_WP = ctypes.POINTER(LqWeightStruct)

_SIGS = {
    "lq_nf4_codebook": (ctypes.c_int, [_i32, _vp]),
    "lq_nf4_quantize": (ctypes.c_int, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "lq_nf4_dequantize": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _i32, _vp]),
    "lq_lora_fwd": (ctypes.c_int, [_vp, _i64, _WP, _vp, _vp, _i64, _f32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "lq_lora_bwd": (ctypes.c_int, [_vp, _vp, _i64, _WP, _vp, _vp, _i64, _f32, _i32, _vp, _vp, _vp,
                                   _vp, _i32, _vp, _sz, _vp]),
    "lq_lora_bwd_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _WP, _vp, _vp, _i64, _f32, _i32, _vp,
                                           _vp, _vp, _vp, _i32, _vp]),
    "lq_lora_merge": (ctypes.c_int, [_WP, _vp, _vp, _i64, _f32, _i32, _vp, _vp]),
    "lq_dora_fwd": (ctypes.c_int, [_vp, _i64, _WP, _vp, _vp, _i64, _f32, _vp, _i32, _vp, _vp, _vp,
                                   _vp, _vp, _sz, _vp]),
    "lq_dora_bwd": (ctypes.c_int, [_vp, _vp, _i64, _WP, _vp, _vp, _i64, _f32, _vp, _i32, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "lq_dora_saved_floats": (_i64, [_i64, _i64]),
    "lq_lora_fwd_dropout": (ctypes.c_int, [_vp, _i64, _WP, _vp, _vp, _i64, _f32, _vp, _f32, _i32,
                                           _vp, _vp, _vp, _sz, _vp]),
    "lq_lora_bwd_dropout": (ctypes.c_int, [_vp, _vp, _i64, _WP, _vp, _vp, _i64, _f32, _vp, _f32,
                                           _i32, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "lq_lora_fwd_multi": (ctypes.c_int, [_vp, _i64, _WP, _vp, _vp, _i32, _i64, _f32, _vp, _vp, _i32,
                                         _i32, _vp, _vp, _sz, _vp]),
    "lq_lora_fwd_multi_ranks": (ctypes.c_int, [_vp, _i64, _WP, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                               _i32, _i32, _vp, _vp, _sz, _vp]),
    "lq_lora_fwd_decode_layers": (ctypes.c_int, [_vp, _i64, _i32, _WP, _vp, _vp, _i64, _vp, _vp,
                                                 _vp, _vp]),
    "lq_adamw_step": (ctypes.c_int, [ctypes.POINTER(LqAdamwTensor), _i32, _i32, _f32, _f32, _f32,
                                     _f32, _f32, _i64, _f32, _vp]),
    "lq_check_segments": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i32]),
    "lq_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i64, _i32]),
    "lq_lora_num_params": (_i64, [_i64, _i64, _i64]),
    "lq_last_error": (ctypes.c_char_p, []),
    "lq_timing_enable": (ctypes.c_int, [_i32]),
    "lq_debug_set_wait_limit": (ctypes.c_int, [_i32]),
    "lq_debug_wait_giveups": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int64)]),
    "lq_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]),
}


def declared_symbols(header: str = HEADER):
    """Function names declared in include/lq.h."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lq_[a-z0-9_]+)\s*\(", text)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run qlora_parameter_efficient_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise LqError(rc, lib().lq_last_error().decode())


def _ptr(t):
    # ctypes turns a Python int (or None) into the void* argument itself
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _dt(t):
    if t.dtype == torch.float32:
        return LQ_F32
    if t.dtype == torch.bfloat16:
        return LQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dt(dt):
    return torch.float32 if dt == LQ_F32 else torch.bfloat16


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


@dataclass
class NF4Weight:
    """Device buffers of an NF4 weight (N x K, flattened row-major)."""
    codes: torch.Tensor
    N: int
    K: int
    q8: torch.Tensor | None = None
    c2: torch.Tensor | None = None
    absmax: torch.Tensor | None = None
    double_quant: bool = True
    dq_format: str = "int8"        # "int8" or "fp8" (second-level constants)
    codebook: str = "nf4"          # "nf4" or "nf4_symmetric"

    def dq_code(self):
        return DQ_FORMATS[self.dq_format] if self.double_quant else LQ_DQ_NONE


def weight_struct(W0, dtype):
    s = LqWeightStruct()
    s.dtype = dtype
    if isinstance(W0, NF4Weight):
        _dev(W0.codes, W0.q8, W0.c2, W0.absmax)
        s.kind = LQ_WEIGHT_NF4
        s.N, s.K = W0.N, W0.K
        s.codes = W0.codes.data_ptr()
        s.q8 = W0.q8.data_ptr() if W0.q8 is not None else None
        s.c2 = W0.c2.data_ptr() if W0.c2 is not None else None
        s.absmax = W0.absmax.data_ptr() if W0.absmax is not None else None
        s.double_quant = W0.dq_code()
        s.codebook = CODEBOOKS[W0.codebook]
    else:
        _dev(W0)
        s.kind = LQ_WEIGHT_DENSE
        s.N, s.K = W0.shape
        s.dense = W0.data_ptr()
        s.double_quant = 0
    return s


# ------------------------------------------------------------------ calls

def lq_nf4_codebook(codebook="nf4"):
    buf = (ctypes.c_float * 16)()
    _check(lib().lq_nf4_codebook(CODEBOOKS[codebook], ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)


def lq_nf4_quantize(W: torch.Tensor, double_quant: bool = True, dq_format: str = "int8",
                    codebook: str = "nf4") -> NF4Weight:
    _dev(W)
    n = W.numel()
    nb = -(-n // 64)
    dev = W.device
    codes = torch.empty(-(-n // 2), dtype=torch.uint8, device=dev)
    q8 = c2 = absmax = None
    if double_quant:
        q8 = torch.empty(nb, dtype=torch.uint8, device=dev)
        c2 = torch.empty(-(-nb // 256), dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
    out = NF4Weight(codes, *(W.shape if W.dim() == 2 else (1, n)), q8, c2, absmax,
                    double_quant, dq_format, codebook)
    _check(lib().lq_nf4_quantize(_ptr(W), _dt(W), n, out.dq_code(), CODEBOOKS[codebook],
                                 _ptr(codes), _ptr(q8), _ptr(c2), _ptr(absmax), _stream()))
    return out


def lq_nf4_dequantize(q: NF4Weight, dtype=torch.bfloat16, n: int | None = None) -> torch.Tensor:
    n = q.N * q.K if n is None else n
    out = torch.empty(n, dtype=dtype, device=q.codes.device)
    _check(lib().lq_nf4_dequantize(_ptr(q.codes), _ptr(q.q8), _ptr(q.c2), _ptr(q.absmax),
                                   q.dq_code(), CODEBOOKS[q.codebook], n, _ptr(out),
                                   LQ_F32 if dtype == torch.float32 else LQ_BF16, _stream()))
    return out


def lq_workspace_size(op, M, N, K, r, n_adapters=0):
    return int(lib().lq_workspace_size(op, M, N, K, r, n_adapters))


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def lq_lora_fwd(X, W0, A, B, scale, T_out=None, ws=None, Y=None, fused=False, no_ws=False):
    """``fused``: allocate the LQ_OP_FWD_FUSED workspace instead of the
    LQ_OP_FWD one; ``no_ws``: pass no workspace at all."""
    _dev(X, A, B, T_out)
    dt = _dt(X)
    M = X.shape[0]
    ws_struct = weight_struct(W0, dt)
    if Y is None:
        Y = torch.empty((M, ws_struct.N), dtype=X.dtype, device=X.device)
    r = A.shape[0]
    if ws is None and not no_ws:
        need = lq_workspace_size(LQ_OP_FWD_FUSED if fused else LQ_OP_FWD, M, ws_struct.N,
                                 ws_struct.K, r)
        if need:
            ws = _ws(need, X.device)
    _check(lib().lq_lora_fwd(_ptr(X), M, ctypes.byref(ws_struct), _ptr(A), _ptr(B), r, scale, dt,
                             _ptr(Y), _ptr(T_out), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream()))
    return Y


def lq_lora_bwd(dY, X, W0, A, B, scale, T_saved=None, need_dx=True, dA=None, dB=None,
                accumulate=False, ws=None, dX=None, need_grads=True, fused=False):
    _dev(dY, X, A, B, T_saved, dA, dB, dX)
    dt = _dt(dY)
    M = dY.shape[0]
    w = weight_struct(W0, dt)
    r = A.shape[0]
    dev = dY.device
    if dX is None and need_dx:
        dX = torch.empty((M, w.K), dtype=dY.dtype, device=dev)
    if need_grads and dA is None:
        dA = torch.empty((r, w.K), dtype=torch.float32, device=dev)
    if need_grads and dB is None:
        dB = torch.empty((w.N, r), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(lq_workspace_size(LQ_OP_BWD_FUSED if fused else LQ_OP_BWD, M, w.N, w.K, r), dev)
    _check(lib().lq_lora_bwd(_ptr(dY), _ptr(X), M, ctypes.byref(w), _ptr(A), _ptr(B), r, scale, dt,
                             _ptr(T_saved), _ptr(dX), _ptr(dA), _ptr(dB), int(accumulate),
                             _ptr(ws), ws.numel(), _stream()))
    return dX, dA, dB


def lq_lora_bwd_noalloc(dY, X, W0, A, B, scale, dX, dA=None, dB=None, T_saved=None,
                        accumulate=False):
    """lq_lora_bwd with the library's static workspace: the outputs are the
    caller's (dX required; dA and dB both or neither) and nothing is
    allocated."""
    _dev(dY, X, A, B, T_saved, dA, dB, dX)
    dt = _dt(dY)
    w = weight_struct(W0, dt)
    _check(lib().lq_lora_bwd_noalloc(_ptr(dY), _ptr(X), dY.shape[0], ctypes.byref(w), _ptr(A),
                                     _ptr(B), A.shape[0], scale, dt, _ptr(T_saved), _ptr(dX),
                                     _ptr(dA), _ptr(dB), int(accumulate), _stream()))
    return dX, dA, dB


def lq_lora_fwd_dropout(X, W0, A, B, scale, keep, p, T_out=None, ws=None, Y=None, fused=False):
    """Forward with LoRA-input dropout; ``keep`` is the packed uint8 keep mask
    (one bit per element of X, bit j of byte i for element 8 i + j)."""
    _dev(X, A, B, keep, T_out, ws, Y)
    dt = _dt(X)
    M = X.shape[0]
    w = weight_struct(W0, dt)
    r = A.shape[0]
    if keep.dtype != torch.uint8 or keep.numel() * 8 < X.numel():
        raise ValueError("keep must be a uint8 tensor of ceil(M*K/8) bytes")
    if Y is None:
        Y = torch.empty((M, w.N), dtype=X.dtype, device=X.device)
    if ws is None:
        op = LQ_OP_FWD_DROPOUT_FUSED if fused else LQ_OP_FWD_DROPOUT
        ws = _ws(lq_workspace_size(op, M, w.N, w.K, r), X.device)
    _check(lib().lq_lora_fwd_dropout(_ptr(X), M, ctypes.byref(w), _ptr(A), _ptr(B), r, scale,
                                     _ptr(keep), p, dt, _ptr(Y), _ptr(T_out), _ptr(ws), ws.numel(),
                                     _stream()))
    return Y


def lq_lora_bwd_dropout(dY, X, W0, A, B, scale, keep, p, T_saved=None, need_dx=True, dA=None,
                        dB=None, accumulate=False, ws=None, dX=None, need_grads=True,
                        fused=False):
    _dev(dY, X, A, B, keep, T_saved, dA, dB, dX, ws)
    dt = _dt(dY)
    M = dY.shape[0]
    w = weight_struct(W0, dt)
    r = A.shape[0]
    dev = dY.device
    if dX is None and need_dx:
        dX = torch.empty((M, w.K), dtype=dY.dtype, device=dev)
    if need_grads and dA is None:
        dA = torch.empty((r, w.K), dtype=torch.float32, device=dev)
    if need_grads and dB is None:
        dB = torch.empty((w.N, r), dtype=torch.float32, device=dev)
    if ws is None:
        op = LQ_OP_BWD_DROPOUT_FUSED if fused else LQ_OP_BWD_DROPOUT
        ws = _ws(lq_workspace_size(op, M, w.N, w.K, r), dev)
    _check(lib().lq_lora_bwd_dropout(_ptr(dY), _ptr(X), M, ctypes.byref(w), _ptr(A), _ptr(B), r,
                                     scale, _ptr(keep), p, dt, _ptr(T_saved), _ptr(dX), _ptr(dA),
                                     _ptr(dB), int(accumulate), _ptr(ws), ws.numel(), _stream()))
    return dX, dA, dB


def lq_dora_saved_floats(N, r):
    return int(lib().lq_dora_saved_floats(N, r))


def lq_dora_fwd(X, W0, A, B, scale, magnitude, Z_out=None, T_out=None, saved_out=None, ws=None,
                Y=None, fused=False):
    """DoRA forward; returns Y.  Pass Z_out (M x N bf16) to keep Z for lq_dora_bwd, and
    saved_out (lq_dora_saved_floats(N, r) float32; its first N entries are the row norms)
    to hand the weight-side results to it."""
    _dev(X, A, B, magnitude, Z_out, T_out, saved_out, ws, Y)
    dt = _dt(X)
    M = X.shape[0]
    w = weight_struct(W0, dt)
    r = A.shape[0]
    if Y is None:
        Y = torch.empty((M, w.N), dtype=X.dtype, device=X.device)
    if ws is None:
        op = LQ_OP_DORA_FWD_FUSED if fused else LQ_OP_DORA_FWD
        ws = _ws(lq_workspace_size(op, M, w.N, w.K, r), X.device)
    _check(lib().lq_dora_fwd(_ptr(X), M, ctypes.byref(w), _ptr(A), _ptr(B), r, scale,
                             _ptr(magnitude), dt, _ptr(Y), _ptr(Z_out), _ptr(T_out),
                             _ptr(saved_out), _ptr(ws), ws.numel(), _stream()))
    return Y


def lq_dora_bwd(dY, X, W0, A, B, scale, magnitude, Z_saved, T_saved=None, saved=None,
                need_dx=True, dA=None, dB=None, dmag=None, accumulate=False, ws=None, dX=None,
                fused=False):
    _dev(dY, X, A, B, magnitude, Z_saved, T_saved, saved, dA, dB, dmag, ws, dX)
    dt = _dt(dY)
    M = dY.shape[0]
    w = weight_struct(W0, dt)
    r = A.shape[0]
    dev = dY.device
    if dX is None and need_dx:
        dX = torch.empty((M, w.K), dtype=dY.dtype, device=dev)
    if dA is None:
        dA = torch.empty((r, w.K), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((w.N, r), dtype=torch.float32, device=dev)
    if dmag is None:
        dmag = torch.empty(w.N, dtype=torch.float32, device=dev)
    if ws is None:
        op = LQ_OP_DORA_BWD_FUSED if fused else LQ_OP_DORA_BWD
        ws = _ws(lq_workspace_size(op, M, w.N, w.K, r), dev)
    _check(lib().lq_dora_bwd(_ptr(dY), _ptr(X), M, ctypes.byref(w), _ptr(A), _ptr(B), r, scale,
                             _ptr(magnitude), dt, _ptr(Z_saved), _ptr(T_saved), _ptr(saved),
                             _ptr(dX),
                             _ptr(dA), _ptr(dB), _ptr(dmag), int(accumulate), _ptr(ws),
                             ws.numel(), _stream()))
    return dX, dA, dB, dmag


def lq_lora_merge(W0, A, B, scale, dtype=None, out=None):
    _dev(A, B, out)
    dt = _dt(A) if dtype is None else (LQ_F32 if dtype == torch.float32 else LQ_BF16)
    w = weight_struct(W0, dt)
    if out is None:
        out = torch.empty((w.N, w.K), dtype=_torch_dt(dt), device=A.device)
    _check(lib().lq_lora_merge(ctypes.byref(w), _ptr(A), _ptr(B), A.shape[0], scale, dt,
                               _ptr(out), _stream()))
    return out


def lq_lora_fwd_multi(X, W0, A_stack, B_stack, scale, seg_offsets, seg_adapter, ws=None, Y=None,
                      fused=False):
    _dev(X, A_stack, B_stack, seg_offsets, seg_adapter)
    dt = _dt(X)
    T = X.shape[0]
    w = weight_struct(W0, dt)
    n_ad, r = A_stack.shape[0], A_stack.shape[1]
    n_seg = seg_adapter.numel()
    if Y is None:
        Y = torch.empty((T, w.N), dtype=X.dtype, device=X.device)
    if ws is None:
        ws = _ws(lq_workspace_size(LQ_OP_FWD_MULTI_FUSED if fused else LQ_OP_FWD_MULTI, T, w.N,
                                   w.K, r, n_ad), X.device)
    _check(lib().lq_lora_fwd_multi(_ptr(X), T, ctypes.byref(w), _ptr(A_stack), _ptr(B_stack), n_ad,
                                   r, scale, _ptr(seg_offsets), _ptr(seg_adapter), n_seg, dt,
                                   _ptr(Y), _ptr(ws), ws.numel(), _stream()))
    return Y


def lq_lora_fwd_multi_ranks(X, W0, A_cat, B_cat, rank_offsets, scales, seg_offsets, seg_adapter,
                            ws=None, Y=None, fused=False):
    """Adapters of different ranks: A_cat (R x K) and B_cat (the adapters' B
    flattened one after another) on the device; rank_offsets (n+1) and
    scales (n) are host sequences."""
    import numpy as np
    _dev(X, A_cat, B_cat, seg_offsets, seg_adapter)
    dt = _dt(X)
    T = X.shape[0]
    w = weight_struct(W0, dt)
    roff = np.ascontiguousarray(rank_offsets, dtype=np.int32)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    n_ad = sc.size
    R = int(roff[-1])
    if Y is None:
        Y = torch.empty((T, w.N), dtype=X.dtype, device=X.device)
    if ws is None:
        ws = _ws(lq_workspace_size(LQ_OP_FWD_MULTI_FUSED if fused else LQ_OP_FWD_MULTI, T, w.N,
                                   w.K, R, 1), X.device)
    _check(lib().lq_lora_fwd_multi_ranks(_ptr(X), T, ctypes.byref(w), _ptr(A_cat), _ptr(B_cat),
                                         n_ad, roff.ctypes.data_as(ctypes.c_void_p),
                                         sc.ctypes.data_as(ctypes.c_void_p), _ptr(seg_offsets),
                                         _ptr(seg_adapter), seg_adapter.numel(), dt, _ptr(Y),
                                         _ptr(ws), ws.numel(), _stream()))
    return Y


def lq_lora_fwd_decode_layers(X, Ws, As, Bs, scales, T_outs=None, Ys=None):
    """Decode forward of len(Ws) layers that read the same X (M <= 16) in one
    launch; returns the list of Y.  Ws, As, Bs, scales (and T_outs, Ys when
    given, entries may be None) are sequences with one entry per layer."""
    _dev(X, *As, *Bs)
    n = len(Ws)
    M = X.shape[0]
    r = As[0].shape[0]
    dt = _dt(X)
    ws = [weight_struct(w, dt) for w in Ws]
    warr = (LqWeightStruct * n)(*ws)
    if Ys is None:
        Ys = [torch.empty((M, w.N), dtype=X.dtype, device=X.device) for w in ws]
    vp = ctypes.c_void_p * n
    a = vp(*[_ptr(t) for t in As])
    b = vp(*[_ptr(t) for t in Bs])
    y = vp(*[_ptr(t) for t in Ys])
    sc = (ctypes.c_float * n)(*[float(v) for v in scales])
    tp = None if T_outs is None else vp(*[_ptr(t) for t in T_outs])
    _check(lib().lq_lora_fwd_decode_layers(
        _ptr(X), M, n, ctypes.cast(warr, _WP), ctypes.cast(a, _vp), ctypes.cast(b, _vp), r,
        ctypes.cast(sc, _vp), ctypes.cast(y, _vp), None if tp is None else ctypes.cast(tp, _vp),
        _stream()))
    return Ys


def lq_adamw_step(params, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                  grad_scale=1.0):
    """AdamW step t = ``step`` in place on a list of trainable tensors.

    params: sequence of (master, m, v, grad, weight) device tensors; master, m
    and v float32, grad float32 or bf16 (one dtype for the whole list), weight
    a bf16 working copy or None; all of one element count per entry.
    """
    params = list(params)
    if not params:
        return
    arr = (LqAdamwTensor * len(params))()
    gdt = None
    for i, (master, m, v, grad, weight) in enumerate(params):
        _dev(master, m, v, grad, weight)
        for t in (master, m, v):
            if t.dtype != torch.float32:
                raise TypeError("master, m and v must be float32")
        if weight is not None and weight.dtype != torch.bfloat16:
            raise TypeError("the working copy must be bf16")
        n = master.numel()
        if any(t is not None and t.numel() != n for t in (m, v, grad, weight)):
            raise ValueError(f"entry {i}: element counts differ")
        d = _dt(grad)
        if gdt is None:
            gdt = d
        elif d != gdt:
            raise TypeError("all gradients must have one dtype")
        arr[i] = LqAdamwTensor(_ptr(master), _ptr(m), _ptr(v), _ptr(grad), _ptr(weight), n)
    _check(lib().lq_adamw_step(arr, len(params), gdt, lr, beta1, beta2, eps, weight_decay,
                               int(step), grad_scale, _stream()))


def lq_check_segments(offsets, adapter, T_tokens, n_adapters):
    import numpy as np
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    ad = np.ascontiguousarray(adapter, dtype=np.int32)
    return int(lib().lq_check_segments(off.ctypes.data_as(ctypes.c_void_p),
                                       ad.ctypes.data_as(ctypes.c_void_p), ad.size, T_tokens,
                                       n_adapters))


def lq_lora_num_params(N, K, r):
    return int(lib().lq_lora_num_params(N, K, r))


def lq_last_error():
    return lib().lq_last_error().decode()


def lq_timing_enable(on=True):
    _check(lib().lq_timing_enable(int(bool(on))))


def lq_timing_read(name):
    """(total milliseconds, launches) of kernel ``name`` since the last read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().lq_timing_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def lq_debug_set_wait_limit(polls):
    """Bound (in polls) of the in-kernel waits between workgroups: > 0 sets it,
    0 restores the default, < 0 makes every such wait give up at once."""
    _check(lib().lq_debug_set_wait_limit(int(polls)))


def lq_debug_wait_giveups():
    """Waits that gave up on the current device since the last call (synchronises)."""
    n = ctypes.c_int64(0)
    _check(lib().lq_debug_wait_giveups(ctypes.byref(n)))
    return n.value
