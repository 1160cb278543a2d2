"""ctypes loader for libflashattn.so (built in-tree by online_softmax_fwd_flash_amd.build).

There is no fallback: if the library is missing or fails to load, every entry point raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FLASHATTN_LIB", os.path.join(_HERE, "libflashattn.so"))

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_F16 = 0, 1, 2
FA_NOALLOC_MAX_DVEC = 4194304    # B * H * T limit of flash_attn_bwd_noalloc (include/flash_attn.h)

EXPORTS = [
    "flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_noalloc", "flash_attn_fwd_ex",
    "flash_attn_bwd_ex",
    "flash_attn_bwd_preprocess", "flash_attn_bwd_dkdv", "flash_attn_bwd_dq",
    "flash_attn_bwd_dq_dvec", "flash_attn_fwd_strided", "flash_attn_bwd_strided",
    "flash_attn_check_layout", "flash_attn_bwd_grad16", "flash_attn_block_class_qk",
    "flash_attn_kv_block_range_qk", "flash_attn_qk_norm_rope",
    "flash_attn_status_string", "flash_attn_block_class", "flash_attn_kv_block_range",
    "flash_attn_default_tiles", "flash_attn_version", "flash_attn_mfma_rate_probe",
]

_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float
_DIMS = [I, I, I, I, I, F, I, I, I, P]          # B T H HKV D scale causal window dtype stream
_DIMS_QK = [I, I, I, I, I, I, F, I, I, I, P]    # B T Tk H HKV D scale causal window dtype stream


class Layout(ctypes.Structure):
    """fa_layout_t: element strides (batch, row, head) of a [B, T, heads, D] view."""
    _fields_ = [("batch", ctypes.c_int64), ("row", ctypes.c_int64), ("head", ctypes.c_int64)]


def _declare(lib):
    sig = {
        "flash_attn_fwd": [P, P, P, P, P] + _DIMS,
        "flash_attn_fwd_ex": [P, P, P, P, P] + _DIMS + [I, I],
        "flash_attn_bwd": [P] * 9 + _DIMS,
        "flash_attn_bwd_noalloc": [P] * 9 + _DIMS,
        "flash_attn_bwd_ex": [P] * 9 + _DIMS + [I, I],
        "flash_attn_bwd_preprocess": [P, P, P, I, I, I, I, I, P],
        "flash_attn_bwd_dkdv": [P] * 8 + _DIMS + [I, I],
        "flash_attn_bwd_dq": [P] * 7 + _DIMS + [I, I],
        "flash_attn_bwd_dq_dvec": [P] * 8 + _DIMS + [I, I],
        "flash_attn_fwd_strided": [P] * 5 + _DIMS_QK + [Layout, Layout],
        "flash_attn_bwd_strided": [P] * 9 + _DIMS_QK + [Layout, Layout],
        "flash_attn_block_class_qk": [I] * 8,
        "flash_attn_qk_norm_rope": [P, ctypes.c_int64, ctypes.c_int64, P, P, ctypes.c_int64, P, P,
                                    I, I, I, I, I, I, I, P],
        "flash_attn_kv_block_range_qk": [I] * 7 + [ctypes.POINTER(I), ctypes.POINTER(I)],
        "flash_attn_check_layout": [Layout, I, I, I, I, I],
        "flash_attn_bwd_grad16": [P] * 9 + _DIMS_QK + [Layout, Layout],
        "flash_attn_block_class": [I, I, I, I, I, I, I, ctypes.POINTER(I)],
        "flash_attn_kv_block_range": [I, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)],
        "flash_attn_default_tiles": [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)],
        "flash_attn_version": [],
        "flash_attn_mfma_rate_probe": [P, P, I, I, P],
        "flash_attn_status_string": [I],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "flash_attn_status_string" else I
    return lib


def lib():
    """The loaded library (raises OSError with a build hint if it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is not built; run `python -m online_softmax_fwd_flash_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(code):
    return lib().flash_attn_status_string(code).decode()
