"""ctypes loader for libdta.so (the C ABI declared in include/dta.h)."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdta.so")

DTA_OK = 0
DTA_EINVAL = -1
DTA_EUNSUPPORTED = -2
DTA_EALIGN = -3
DTA_ELAUNCH = -4

# Every symbol include/dta.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "attn_merge": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _P]),
    "attn_fwd_accum": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "attn_merge_into": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "residual_diff": (_I, [_P, _P, _I64, _P, _P, _P]),
    "residual_diff_noalloc": (_I, [_P, _P, _I64, _P, _P]),
    "fbcache_step": (_I, [_P, _P, _I64, _F, _P, _P, _I64, _P, _P, _P, _P]),
    "fp8_quant_per_tensor": (_I, [_P, _I64, _P, _P, _P, _P]),
    "fp8_quant_per_tensor_multi": (_I, [_I, _P, _P, _P, _P, _P, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fp8_quant_rows_pow2": (_I, [_P, _I64, _I, _P, _P, _P]),
    "attn_fwd_fp8_rows": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_fp8_rows_v": (_I, [_P] * 8 + [_I] * 5 + [_F, _P]),
    "seq_concat": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _P]),
    "seq_split": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _P]),
    "head_concat": (_I, [_P, _P, _I, _P, _I, _I, _I, _P]),
    "head_split": (_I, [_P, _P, _I, _P, _I, _I, _I, _P]),
    "dta_ws_bytes": (ctypes.c_size_t, []),
    "dta_status_str": (ctypes.c_char_p, [_I]),
}

_lib = None


class DtaError(RuntimeError):
    """A libdta entry point returned a non-zero status."""

    def __init__(self, fn, status, text):
        super().__init__("%s failed: %s (status %d)" % (fn, text, status))
        self.status = status


def lib():
    """The loaded library; raises if libdta.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libdta.so is not built (%s); run "
                "`python -m diffusion_transformer_attention_flash_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn, status):
    if status != DTA_OK:
        raise DtaError(fn, status, lib().dta_status_str(status).decode())
