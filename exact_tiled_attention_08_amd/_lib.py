"""ctypes loader for libfa.so: prototypes only, no computation.

The library is built in-tree by ``exact_tiled_attention_08_amd.build``.  If it
is missing, every call raises -- there is no fallback path.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, -1, -2, -3, -4
FA_F32, FA_BF16, FA_FP8_E4M3, FA_FP8_E5M2 = 0, 1, 2, 3
FA_DECODE_SPLIT_ALIGN = 128
FA_MAX_SPLITS = 256
FA_NOALLOC_SCRATCH_BYTES = 33554432

_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fa.h
PROTOTYPES = {
    "fa_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _i, _p]),
    "fa_fwd_fp8": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _f, _f, _f, _i, _p]),
    "fa_fwd_varlen": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p]),
    "fa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "fa_decode_splitkv": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _i, _i, _p]),
    "fa_lse_merge": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _p]),
    "fa_decode": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _i, _p, _sz, _i, _p]),
    "fa_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _i, _i, _p]),
    "fa_decode_paged": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _i, _p, _sz, _i, _p]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "fa_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _p, _sz, _i, _p]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_version": (_i, []),
    # measurement aids (include/fa_ceilings.h)
    "fa_ceiling_mfma": (_i, [_p, _p, _i, _i, _p]),
    "fa_ceiling_read": (_i, [_p, _sz, _p, _i, _p]),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} [{status}]")
        self.status = status


def load():
    """Load libfa.so once and attach the prototypes; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_tiled_attention_08_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def check(status):
    if status != FA_OK:
        lib = load()
        raise FAError(lib.fa_status_string(status).decode(), lib.fa_last_error().decode())
