"""ctypes view of libzs.so: loads the library and declares every C-ABI symbol.

The library must have been built in-tree (fsdp_sharded_optimizer_flatparameter_amd/libzs.so);
there is no fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzs.so")

ZS_OK = 0
ZS_F32 = 0
ZS_BF16 = 1
ZS_MAX_WORLD = 256
ZS_NOALLOC_MAX_N = 1 << 28
STATUS = {
    0: "ZS_OK", -1: "ZS_ERR_NULL", -2: "ZS_ERR_SIZE", -3: "ZS_ERR_WORLD", -4: "ZS_ERR_RANK",
    -5: "ZS_ERR_DTYPE", -6: "ZS_ERR_HPARAM", -7: "ZS_ERR_SHARD", -8: "ZS_ERR_WORKSPACE",
    -9: "ZS_ERR_LAYOUT", -10: "ZS_ERR_ALIGN", -11: "ZS_ERR_OVERLAP", -100: "ZS_ERR_HIP",
}


class ParamDesc(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("flat_offset", C.c_int64), ("numel", C.c_int64)]


class Dim0Desc(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("flat_offset", C.c_int64), ("numel", C.c_int64),
                ("chunk", C.c_int64), ("local_offset", C.c_int64)]


class AdamWHParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]


# name -> (restype, argtypes), mirroring include/zs.h
_I64P = C.POINTER(C.c_int64)
SIGNATURES = {
    "zs_flat_layout": (C.c_int32, [_I64P, C.c_int32, C.c_int32, C.c_int64, _I64P, _I64P, _I64P, _I64P]),
    "zs_check_layout": (C.c_int32, [C.POINTER(ParamDesc), C.c_int32, C.c_int64, C.c_int32]),
    "zs_pack_shard": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                  C.c_int32, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p]),
    "zs_reduce_grads": (C.c_int32, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32, C.c_int64,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "zs_reduce_grads_noalloc": (C.c_int32, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32, C.c_int64,
                                            C.c_void_p, C.c_void_p, C.c_void_p]),
    "zs_workspace_bytes": (C.c_size_t, [C.c_int64]),
    "zs_adamw_step": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                  C.POINTER(AdamWHParams), C.c_void_p, C.c_void_p, C.c_void_p]),
    "zs_cast_for_gather": (C.c_int32, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "zs_copy_out": (C.c_int32, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int32, C.c_int64,
                                C.c_void_p]),
    "zs_sharded_step": (C.c_int32, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32, C.c_int64,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(AdamWHParams),
                                    C.c_void_p, C.c_void_p, C.c_void_p]),
    "zs_accumulate_grads": (C.c_int32, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32, C.c_int64,
                                        C.c_void_p, C.c_float, C.c_int32, C.c_void_p, C.c_void_p,
                                        C.c_size_t, C.c_void_p]),
    "zs_accumulate_local": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_int32,
                                        C.c_void_p]),
    "zs_clip_coefficient": (C.c_int32, [C.c_void_p, C.c_int32, C.c_double, C.c_void_p, C.c_void_p,
                                        C.c_void_p]),
    "zs_dim0_layout": (C.c_int32, [_I64P, _I64P, C.c_int32, C.c_int32, _I64P, _I64P, _I64P]),
    "zs_check_dim0_layout": (C.c_int32, [C.POINTER(Dim0Desc), C.c_int32, C.c_int32, C.c_int64,
                                         C.c_int64, C.c_int32]),
    "zs_pack_shard_dim0": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "zs_copy_out_dim0": (C.c_int32, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int32, C.c_int32,
                                     C.c_int64, C.c_int64, C.c_void_p]),
    "zs_status_string": (C.c_char_p, [C.c_int32]),
    "zs_version": (C.c_int32, []),
}

_lib = None


def load() -> C.CDLL:
    """Load libzs.so once; raise ImportError (never fall back) when it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m "
                "fsdp_sharded_optimizer_flatparameter_amd.build` (or __graft_entry__.build())")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class ZsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{fn} failed: {self.name}")


class ZsArgumentError(ZsError, ValueError):
    pass


def check(fn: str, status: int) -> None:
    if status == ZS_OK:
        return
    if status == -100:
        raise ZsError(fn, status)
    raise ZsArgumentError(fn, status)
