"""ctypes prototypes of libpkv.so (the C ABI declared in include/pkv.h).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
# device error word bits (include/pkv.h)
PKV_DEVERR_SLOT = 0x1
PKV_DEVERR_BLOCK_ID = 0x2
PKV_DEVERR_CONTEXT_LEN = 0x4
PKV_DEVERR_SEQLENS = 0x8
PKV_DEVERR_WAIT = 0x10
PKV_STATIC_SCRATCH_BYTES = 32 << 20   # fixed device array of the no-allocation entry point

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_F = ctypes.c_float

# name -> (restype, argtypes)
PROTOTYPES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_set_error_word": (ctypes.c_int, [_P]),
    "pkv_get_error_word": (_P, []),
    "pkv_set_wait_limit": (ctypes.c_int, [_U32]),
    "pkv_probe_stream_read": (ctypes.c_int, [_P, _SZ, _P, _I32, _P]),
    "pkv_get_device_info": (ctypes.c_int, [_I32, _P]),
    "pkv_slot_mapping": (ctypes.c_int, [_P, _P, _I32, _P, _I32, _I32, _P]),
    "pkv_kv_store": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I64, _P]),
    "pkv_decode_split_tokens": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "pkv_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_decode_attention": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P, _I32, _P, _I32,
                                                  _I32, _I32, _I32, _I32, _I64, _I32, _F, _I32,
                                                  _P, _SZ, _P]),
    "pkv_decode_attention_partial": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I32, _P, _I32, _I32,
                                                    _I32, _I32, _I32, _I64, _I32, _F, _I32, _P,
                                                    _SZ, _P]),
    "pkv_decode_attention_reduce": (ctypes.c_int, [_P, _I64, _P, _I32, _I32, _I32, _I32, _I32,
                                                   _I32, _I32, _I32, _P, _SZ, _P]),
    "pkv_paged_decode_attention_store": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64,
                                                        _P, _I32, _P, _I32, _I32, _I32, _I32,
                                                        _I32, _I64, _I32, _F, _I32, _P, _SZ,
                                                        _P]),
    "pkv_paged_decode_attention_store_noalloc": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P,
                                                                _P, _I64, _P, _I32, _P, _I32,
                                                                _I32, _I32, _I32, _I32, _I64,
                                                                _I32, _F, _I32, _P]),
    "pkv_decode_attention_partial_store": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _P,
                                                          _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                                          _I64, _I32, _F, _I32, _P, _SZ, _P]),
    "pkv_cascade_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_cascade_decode_attention": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P, _I32, _P, _I32,
                                                    _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32,
                                                    _F, _I32, _P, _SZ, _P]),
    "pkv_varlen_slot_mapping": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _P]),
    "pkv_varlen_split_tokens": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_varlen_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_varlen_paged_attention": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P, _I32, _P, _P,
                                                  _I32, _I32, _I32, _I32, _I32, _I32, _I64, _I32,
                                                  _I32, _F, _I32, _P, _SZ, _P]),
    "pkv_sampler_workspace_bytes": (_SZ, [_I32, _I32]),
    "pkv_sample_next_token": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _P, _P, _I32, _I32, _P,
                                             _SZ, _P]),
    "pkv_sample_next_token_ex": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _I32,
                                                _I32, _P, _P, _P, _P, _SZ, _P]),
}



class DeviceInfo(ctypes.Structure):
    """pkv_device_info (include/pkv.h)."""
    _fields_ = [("name", ctypes.c_char * 256), ("arch", ctypes.c_char * 64),
                ("compute_units", _I32), ("clock_khz", _I32), ("memory_clock_khz", _I32),
                ("memory_bus_width_bits", _I32), ("l2_cache_bytes", _I32),
                ("lds_per_workgroup_bytes", _I32), ("wavefront_size", _I32), ("pad", _I32),
                ("total_memory_bytes", ctypes.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m paged_kv_decode_store_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.pkv_status_string(status).decode()
        detail = L.pkv_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)
