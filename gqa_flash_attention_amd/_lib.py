"""ctypes loader for libgqafa.so: argument marshalling only.

The library is built in-tree by gqa_flash_attention_amd/build.py. There is
no fallback path: if the shared library is missing or cannot be loaded,
every call raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# Always the in-tree build (no other library is ever loaded in its place).
LIB_PATH = os.path.join(_HERE, "libgqafa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", -1: "FA_ERR_INVALID_ARG", -2: "FA_ERR_UNSUPPORTED",
                -3: "FA_ERR_WORKSPACE", -4: "FA_ERR_LAUNCH", -5: "FA_ERR_SCRATCH"}
# fa_decode_paged_noalloc's static device buffer (FA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol the C header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "fa_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_decode_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P,
                             _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "fa_prefill_strided": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "fa_decode_paged_strided": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P]),
    "fa_combine_lse": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _P]),
    "fa_decode_paged_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P]),
    "fa_kv_append_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _I, _I, _I, _I, _I, _I, _I, _P]),
    "fa_kv_append": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fa_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_paged_gather": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
}



class ScoreMods(ctypes.Structure):
    """fa_score_mods: logit softcap, ALiBi max_bias, sinks (device fp32 [Hq]),
    additive bf16 mask with its sequence and row strides."""
    _fields_ = [("logit_softcap", ctypes.c_float), ("max_bias", ctypes.c_float),
                ("sinks", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("mask_batch_stride", ctypes.c_int64), ("mask_row_stride", ctypes.c_int64)]


_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libgqafa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with gqa_flash_attention_amd/build.py "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FA_OK:
        msg = load().fa_status_string(status).decode()
        raise FAError(status, msg)
