"""ctypes loader for libattn.so (the C ABI of include/attn.h)."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
_lock = threading.Lock()
_lib = None

# ABI symbols and their ctypes signatures (mirrors include/attn.h)
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _vp]),
    "attn_fwd_policy": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _i, _vp]),
    "attn_fwd_default_policy": (_i, [_i, _i, _i, ctypes.POINTER(_f), ctypes.POINTER(_i)]),
    "attn_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _f, _f, _vp]),
    "attn_fwd_rescale_events": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _vp,
                                     _vp]),
    "attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _f,
                      _i, _vp]),
    "attn_bwd_phases": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i,
                             _f, _i, ctypes.c_uint, _vp]),
    "attn_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                              _i, _vp]),
    "attn_noalloc_scratch_bytes": (_sz, []),
    "attn_strerror": (ctypes.c_char_p, [_i]),
    "attn_last_hip_error": (_i, []),
    "attn_version": (_i, []),
}

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_HEAD_DIM",
          4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_SCALE",
          7: "ATTN_ERR_UNSUPPORTED", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_SCRATCH"}


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str, message: str):
        super().__init__("%s: %s (%s)" % (where, message, STATUS.get(code, code)))
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libattn.so once.  PyTorch is imported first so that the library
    binds to the same HIP runtime instance PyTorch uses (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            import torch  # noqa: F401  -- shares its libamdhip64 with the library
            if not os.path.exists(_LIB_PATH):
                raise ImportError(
                    "libattn.so is not built (expected at %s); run "
                    "`python exact_attention_128_amd/build.py` (hipcc, gfx950)" % _LIB_PATH)
            _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path: str):
    """A ctypes handle on a library exporting the C ABI at path, with every
    signature set (also used to open the LDS race-check build,
    libattn_lds_poison.so, beside the product library)."""
    import torch  # noqa: F401  -- shares its libamdhip64 with the library
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def raise_for(rc: int, where: str) -> None:
    if rc == 0:
        return
    lib = load()
    msg = lib.attn_strerror(rc).decode()
    if rc == 8:
        msg += " [hipError %d]" % lib.attn_last_hip_error()
    raise AttnError(rc, where, msg)
