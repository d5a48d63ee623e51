"""ctypes declarations of libtide.so (include/tide.h).  Loads the library
once; a missing library is an error, never a fallback."""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtide.so")

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_p = ctypes.c_void_p
_pi64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes), in header order
SIGNATURES = {
    "tide_plan_create": (_i32, [_i32, _i32, _pi64, _pi64, _i64, ctypes.POINTER(_p)]),
    "tide_plan_destroy": (None, [_p]),
    "tide_plan_world": (_i32, [_p]),
    "tide_plan_nparams": (_i32, [_p]),
    "tide_plan_shard_numel": (_i64, [_p]),
    "tide_plan_param": (_i32, [_p, _i32, _pi64, _pi64, _pi64]),
    "tide_plan_real": (_i32, [_p, _i32, _i32, _pi64, _pi64]),
    "tide_rs": (_i32, [_p, _i32, _p, _p, _u32, _i32, _p]),
    "tide_ag": (_i32, [_p, _p, _p, _i32, _u32, _i32, _p]),
    "tide_pack": (_i32, [_p, _p, _p, _i32, _u32, _i32, _p]),
    "tide_rs_slots": (_i32, [_p, _i32, _p, _p, _u32, _i32, _p]),
    "tide_rs_noalloc": (_i32, [_p, _i32, _p, _p, _u32, _i32, _p]),
    "tide_last_error": (ctypes.c_char_p, []),
    "tide_status_string": (ctypes.c_char_p, [_i32]),
}

_lib = None


def lib():
    """The loaded libtide.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m parameter_layout_collectives_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
