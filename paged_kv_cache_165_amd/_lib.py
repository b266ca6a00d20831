"""ctypes loader for libpa.so, the C-ABI library declared in include/pa.h.

No compute happens here: this module only loads the shared library and
declares the argument types of its exported functions. There is no fallback:
if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_BF16, PA_F16 = 0, 1, 2
PA_OK = 0

# every symbol include/pa.h declares
EXPORTED = (
    "pa_abi_version", "pa_status_string", "pa_last_error", "pa_default_partition_size",
    "pa_decode_workspace_size", "pa_decode", "pa_decode_partitions", "pa_decode_merge",
    "pa_write_cache", "pa_copy_blocks",
)

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_DECODE_ARGS = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                _i, _vp, ctypes.c_size_t, _vp]


class LibraryNotBuilt(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise LibraryNotBuilt(
                f"{path} is missing: build it with `python -m paged_kv_cache_165_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        lib.pa_abi_version.restype = _i
        lib.pa_abi_version.argtypes = []
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [_i]
        lib.pa_last_error.restype = ctypes.c_char_p
        lib.pa_last_error.argtypes = []
        lib.pa_default_partition_size.restype = _i
        lib.pa_default_partition_size.argtypes = []
        lib.pa_decode_workspace_size.restype = ctypes.c_size_t
        lib.pa_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        for name in ("pa_decode", "pa_decode_partitions", "pa_decode_merge"):
            f = getattr(lib, name)
            f.restype = _i
            f.argtypes = _DECODE_ARGS
        lib.pa_write_cache.restype = _i
        lib.pa_write_cache.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
        lib.pa_copy_blocks.restype = _i
        lib.pa_copy_blocks.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
        _lib = lib
        return lib
