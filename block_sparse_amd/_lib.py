"""ctypes binding of ``libstarattn.so`` (argument marshalling only).

The functions declared in ``include/star_attn.h`` are exposed with the same
names.  Loading fails loudly when the library has not been built: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# STAR_ATTN_LIB names another build of the library (the host tests load an
# AddressSanitizer build through it)
LIB_PATH = os.environ.get("STAR_ATTN_LIB") or os.path.join(HERE, "libstarattn.so")

STAR_BF16 = 0
STAR_F32 = 1
STAR_MAX_PARTS = 128
STAR_SPLIT_ALIGN = 64
STAR_NOALLOC_SCRATCH_BYTES = 4 << 20
STAR_BLAS_WORKSPACE_BYTES = 64 << 20

STATUS = {
    0: "STAR_OK", -1: "STAR_ERR_NULL", -2: "STAR_ERR_SHAPE", -3: "STAR_ERR_DTYPE",
    -4: "STAR_ERR_ALIGN", -5: "STAR_ERR_UNSUPPORTED", -6: "STAR_ERR_HIP", -7: "STAR_ERR_BLAS",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# every symbol include/star_attn.h declares
EXPORTS = ("star_rope_apply", "star_rope_freqs", "star_kv_append", "star_decode_prepare", "star_phase1_blocklocal",
           "star_phase1_prefix", "star_phase1_rope", "star_gather_rows", "star_stream_read", "star_pulsar_prefix",
           "star_phase2_partial", "star_lse_merge", "star_decode_step",
           "star_decode_step_devpos", "star_decode_step_noalloc",
           "star_context_create", "star_context_destroy", "star_rmsnorm", "star_linear",
           "star_status_string",
           "star_abi_version")


class StarTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("B", ctypes.c_int64), ("H", ctypes.c_int64),
        ("S", ctypes.c_int64), ("D", ctypes.c_int64),
        ("sB", ctypes.c_int64), ("sH", ctypes.c_int64), ("sS", ctypes.c_int64),
    ]


_P = ctypes.POINTER
_T = _P(StarTensor)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double

_SIGS = {
    "star_rope_apply": (ctypes.c_int, [_T, _T, _vp, _i64, _f64, _vp]),
    "star_rope_freqs": (ctypes.c_int, [_i64, _f64, _P(_f64)]),
    "star_kv_append": (ctypes.c_int, [_T, _T, _T, _T, _i64, _i64, _f64, _i32, _vp]),
    "star_decode_prepare": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, _i64, _i64, _f64, _i32, _vp]),
    "star_phase1_blocklocal": (ctypes.c_int, [_T, _T, _T, _i64, _i64, _f32, _T, _vp, _vp, _vp]),
    "star_phase1_rope": (ctypes.c_int, [_T, _T, _T, _i64, _i64, ctypes.c_double, _f32, _T, _vp,
                                        _vp, _vp]),
    "star_phase1_prefix": (ctypes.c_int, [_T, _T, _T, _T, _T, _P(_i64), _P(_i64), _i32, _i64,
                                          _f32, _T, _vp, _vp, _vp]),
    "star_gather_rows": (ctypes.c_int, [_T, _vp, _T, _vp]),
    "star_stream_read": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]),
    "star_pulsar_prefix": (ctypes.c_int, [_P(_i32), _i64, _i64, _i32, _i32, _i32, _P(_i64), _i64,
                                          _P(_i64), _P(_i64), _P(_i64), _i32]),
    "star_phase2_partial": (ctypes.c_int, [_T, _T, _T, _P(_i64), _i32, _i32, _i64, _f32,
                                           _vp, _vp, _vp]),
    "star_lse_merge": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i64, _i64, _i64, _T, _vp, _vp]),
    "star_decode_step": (ctypes.c_int, [_T, _T, _T, _T, _T, _i64, _i64, _f64, _i32, _P(_i64), _i32,
                                        _i32, _f32, _vp, _vp, _T, _vp, _vp]),
    "star_decode_step_devpos": (ctypes.c_int, [_T, _T, _T, _T, _T, _vp, _f64, _i32, _P(_i64),
                                               _i32, _i32, _f32, _vp, _vp, _T, _vp, _vp]),
    "star_decode_step_noalloc": (ctypes.c_int, [_T, _T, _T, _T, _T, _i64, _i64, _f64, _i32,
                                                _P(_i64), _i32, _i32, _f32, _T, _vp, _vp]),
    "star_context_create": (ctypes.c_int, [_P(_vp)]),
    "star_context_destroy": (ctypes.c_int, [_vp]),
    "star_rmsnorm": (ctypes.c_int, [_T, _vp, _f32, _T, _vp]),
    "star_linear": (ctypes.c_int, [_vp, _T, _T, _T, _T, _vp]),
    "star_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "star_abi_version": (ctypes.c_int, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load the shared library (once) and set the ctypes signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m block_sparse_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class StarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')})")


def check(fn: str, status: int):
    if status != 0:
        raise StarError(fn, status)
