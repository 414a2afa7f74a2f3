"""ctypes view of libsa2.so: the C ABI declared in include/sa2.h, nothing more."""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsa2.so"

SA2_OK, SA2_EINVAL, SA2_EUNSUPPORTED, SA2_EDEVICE = 0, 1, 2, 3
SA2_BF16, SA2_F32 = 0, 1
SA2_MASK_NOALLOC_MAX_BYTES = 64 << 20   # include/sa2.h
STATUS_NAMES = {0: "SA2_OK", 1: "SA2_EINVAL", 2: "SA2_EUNSUPPORTED", 3: "SA2_EDEVICE"}


class Sa2Mask(ctypes.Structure):
    """struct sa2_mask (include/sa2.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("bq", ctypes.c_int32), ("bk", ctypes.c_int32), ("Tq", ctypes.c_int32),
        ("Tk", ctypes.c_int32),
        ("bitmap", ctypes.c_void_p), ("row_cnt", ctypes.c_void_p), ("row_idx", ctypes.c_void_p),
        ("col_cnt", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
        ("row_plan", ctypes.c_void_p), ("col_plan", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double
_Z = ctypes.c_size_t
_MP = ctypes.POINTER(Sa2Mask)

SIGNATURES = {
    "sa2_version": ([], ctypes.c_char_p),
    "sa2_last_error": ([], ctypes.c_char_p),
    "sa2_mask_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
    "sa2_mask_plan_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
    "sa2_mask_plans": ([_MP, _P], _I),
    "sa2_build_mask": ([_P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _D, _MP, _P, _Z, _P], _I),
    "sa2_build_mask_noalloc": ([_P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _D, _MP, _P], _I),
    "sa2_fwd_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "sa2_attn_fwd": ([_P, _P, _P, _I, _I, _I, _I, _I, _MP, _P, _P, _P, _Z, _P], _I),
    "sa2_bwd_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "sa2_attn_bwd": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _MP, _P, _P, _P, _P, _Z, _P], _I),
    "sa2_attn_bwd_dq": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _MP, _P, _P, _Z, _P], _I),
    "sa2_attn_bwd_dkdv": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _MP, _P, _P, _P, _Z, _P], _I),
    "sa2_bwd_atomic_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "sa2_attn_bwd_atomic_dq": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _MP, _P, _P, _P, _P,
                                _Z, _P], _I),
    "sa2_distill_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "sa2_distill_loss_grad": ([_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_attention_sa2_amd.build` (there is no fallback path)")
        h = ctypes.CDLL(str(LIB_PATH))
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


class Sa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().sa2_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != SA2_OK:
        raise Sa2Error(fn, status)
