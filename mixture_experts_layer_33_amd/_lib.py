"""ctypes view of libmoe.so (include/moe.h).  Loading fails loudly when the
library is missing: there is no fallback path."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

(MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_CAPACITY, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DTYPE,
 MOE_ERR_SCRATCH) = range(8)
MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
OP_ROUTE, OP_DISPATCH, OP_EXPERT_FFN, OP_COMBINE, OP_DECODE, OP_BACKWARD, OP_FORWARD = range(7)

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}


class MoeShape(C.Structure):
    _fields_ = [("tokens", C.c_int64), ("capacity", C.c_int64), ("hidden", C.c_int32),
                ("experts", C.c_int32), ("top_k", C.c_int32), ("ffn", C.c_int32),
                ("shared_ffn", C.c_int32), ("dtype", C.c_int32)]


P = C.c_void_p
I64 = C.c_int64
SZ = C.c_size_t
SHP = C.POINTER(MoeShape)

# name -> argument types (all return int unless listed in _RESTYPE)
SIGNATURES = {
    "moe_route": [SHP, P, P, P, P, P, P, P, SZ, P],
    "moe_dispatch": [SHP, P, P, I64, P, P, P, P, P, P, SZ, P],
    "moe_expert_ffn": [SHP, P, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_expert_ffn_timed": [SHP, P, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P, P],
    "moe_combine": [SHP, P, P, P, P, P],
    "moe_forward": [SHP, P, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, C.c_uint32, P, SZ, P],
    "moe_decode": [SHP, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_decode_noalloc": [SHP, P, P, P, P, P, P, P, P, P, P, P, P, P],
    "moe_backward": [SHP, P, P, P, P, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_workspace_bytes": [SHP, C.c_int],
    "moe_check_shape": [SHP],
    "moe_status_string": [C.c_int],
    "moe_quantize_mx": [P, I64, I64, P, P, P],
    "moe_quantize_mx_t": [P, I64, I64, I64, P, I64, I64, P, P],
    "moe_quantize_mx_both": [P, I64, I64, I64, P, P, P, I64, I64, P, P],
    "moe_backward_mx": [SHP, P, P, P, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
}
_RESTYPE = {"moe_workspace_bytes": SZ, "moe_status_string": C.c_char_p}

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mixture_experts_layer_33_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _RESTYPE.get(name, C.c_int)
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
