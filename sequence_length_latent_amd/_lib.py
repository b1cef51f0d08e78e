"""ctypes loader for the SFA C ABI (``include/hd_sfa.h``).

Loads the in-tree ``_hd_sfa.so`` and declares every entry point's argument
and return types.  There is no fallback: if the library has not been built
the import of the binding fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_hd_sfa.so")

_i32, _i64, _f32, _vp, _sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t

# name -> (restype, argtypes), in the order of include/hd_sfa.h
SIGNATURES = {
    "hd_status_string": (C.c_char_p, [C.c_int]),
    "hd_abi_version": (C.c_int, []),
    "hd_expand": (C.c_int, [_vp, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "hd_final_stream_rows": (C.c_int, [_vp, _i64, _i32, _i64, _i64, _vp, _vp]),
    "hd_cyclic_replicate": (C.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _vp]),
    "sfa_stream_attn": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32,
                                  _f32, _vp]),
    "sfa_mix_attn": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32,
                               _f32, _vp]),
    "sfa_mix_attn_window": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32,
                                      _f32, _i64, _vp]),
    "sfa_attn_fwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32,
                               _f32, _i32, _vp]),
    "sfa_attn_fwd_window": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32,
                                      _i32, _f32, _i64, _vp]),
    "sfa_attn_split_workspace_size": (_sz, [_i64, _i32, _i64, _i32, _i32, _i32, _i32]),
    "sfa_attn_split": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32,
                                 _f32, _i32, _vp, _sz, _vp]),
    "sfa_attn_bwd_workspace_size": (_sz, [_i64, _i32, _i64, _i32]),
    "sfa_attn_bwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64,
                               _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "sfa_attn_bwd_window": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64,
                                      _i32, _i32, _i32, _f32, _i64, _vp, _sz, _vp]),
    "sfa_decode_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, _i64]),
    "sfa_decode_step": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                  _i64, _i64, _i32, _f32, _vp, _sz, _vp, _vp, _vp]),
    "sfa_decode_step_noalloc": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                          _i32, _i64, _i64, _i32, _f32, _vp, _vp, _vp]),
    "sfa_decode_step_paged": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                        _i32, _i32, _i64, _i32, _i64, _i32, _i64, _f32, _vp, _sz,
                                        _vp, _vp, _vp]),
    "sfa_decode_step_window": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                         _i32, _i64, _i64, _i64, _f32, _vp, _sz, _vp, _vp, _vp]),
}

STATUS = {0: "HD_OK", 1: "HD_ERR_NULL", 2: "HD_ERR_SHAPE", 3: "HD_ERR_UNSUPPORTED",
          4: "HD_ERR_CAPACITY", 5: "HD_ERR_LAUNCH", 6: "HD_ERR_WORKSPACE", 7: "HD_ERR_SCRATCH"}


class HDError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load (once) and return the ctypes library handle."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"SFA HIP library not built: {path} is missing. Build it with "
            "`python -m sequence_length_latent_amd.build` (hipcc, gfx950).")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        text = load().hd_status_string(status).decode()
        raise HDError(fn, status, text)
