"""ctypes loader for libfattn.so with the C prototypes of include/fattn.h."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

c_int, c_float, c_size_t, c_void_p, c_uint64 = (ctypes.c_int, ctypes.c_float, ctypes.c_size_t,
                                                ctypes.c_void_p, ctypes.c_uint64)

# name -> (restype, argtypes), mirroring include/fattn.h
PROTOTYPES = {
    "fattn_fwd": (c_int, [c_void_p] * 5 + [c_int] * 5 + [c_float, c_int, c_void_p]),
    "fattn_fwd_varlen": (c_int, [c_void_p] * 6 + [c_int] * 7 + [c_float, c_int, c_void_p]),
    "fattn_fwd_blocksparse": (c_int, [c_void_p] * 6 + [c_int] * 6 + [c_float, c_int, c_void_p]),
    "fattn_bwd_blocksparse": (c_int, [c_void_p] * 10 + [c_int] * 6
                              + [c_float, c_void_p, c_size_t, c_void_p]),
    "fattn_bwd_workspace_bytes": (c_size_t, [c_int] * 4),
    "fattn_bwd_varlen": (c_int, [c_void_p] * 10 + [c_int] * 7
                         + [c_float, c_void_p, c_size_t, c_void_p]),
    "fattn_bwd": (c_int, [c_void_p] * 9 + [c_int] * 5 + [c_float, c_void_p, c_size_t, c_void_p]),
    "fattn_bwd_noalloc": (c_int, [c_void_p] * 9 + [c_int] * 5 + [c_float, c_void_p]),
    "fattn_fwd_fp8_workspace_bytes": (c_size_t, [c_int] * 4),
    "fattn_fwd_fp8_workspace_layout": (c_int, [c_int] * 4 + [ctypes.POINTER(c_size_t)] * 3),
    "fattn_fwd_fp8": (c_int, [c_void_p] * 5 + [c_int] * 5
                      + [c_float, c_int, c_int, c_uint64, c_void_p, c_size_t, c_void_p]),
    "fattn_fwd_fp8_blocksparse": (c_int, [c_void_p] * 6 + [c_int] * 6
                                  + [c_float, c_int, c_int, c_uint64, c_void_p, c_size_t,
                                     c_void_p]),
    "fattn_fwd_fp8_varlen_workspace_bytes": (c_size_t, [c_int] * 6),
    "fattn_fwd_fp8_varlen": (c_int, [c_void_p] * 6 + [c_int] * 7
                             + [c_float, c_int, c_int, c_uint64, c_void_p, c_size_t, c_void_p]),
    "fattn_fwd_fp8_attend": (c_int, [c_void_p] * 3 + [c_int] * 5
                             + [c_float, c_int, c_int, c_uint64, c_void_p, c_size_t, c_void_p]),
    "fattn_strerror": (ctypes.c_char_p, [c_int]),
    "fattn_last_error": (ctypes.c_char_p, []),
    "fattn_version": (c_int, []),
}


def lib_path():
    return os.environ.get("FATTN_LIB", os.path.join(_HERE, "libfattn.so"))


def lib():
    """Load libfattn.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} not found: build it with `python -m tiled_attention_fattn_amd.build`")
        so = ctypes.CDLL(path)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(so, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = so
    return _LIB


class FattnError(RuntimeError):
    def __init__(self, status):
        self.status = int(status)
        so = lib()
        super().__init__(f"libfattn status {self.status} ({so.fattn_strerror(self.status).decode()}):"
                         f" {so.fattn_last_error().decode()}")
