"""ctypes loader for liblogra.so (the HIP library built by build.py).

The library must exist: there is no fallback of any kind.  Loading it does not
touch the GPU, so CPU-only processes may load it to inspect symbols or drive
argument validation.
"""
import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblogra.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "logra.h")

_lib = None

c_u16p = ctypes.c_void_p
c_vp = ctypes.c_void_p

SIGNATURES = {
    "logra_abi_version": (ctypes.c_int, []),
    "logra_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "logra_regen_A": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                     ctypes.c_int32, ctypes.c_int64, c_vp, c_vp]),
    "logra_sketch_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int32]),
    "logra_sketch_accumulate": (ctypes.c_int, [c_vp, ctypes.c_int64, c_vp, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_int, ctypes.c_int32, c_vp, c_vp,
                                               ctypes.c_size_t, c_vp]),
    "logra_merge": (ctypes.c_int, [c_vp, ctypes.c_int64, c_vp, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_float, c_vp]),
    "logra_sketch_update": (ctypes.c_int, [ctypes.c_int, c_vp, c_vp, c_vp, c_vp, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_int64, c_vp]),
    "logra_kl_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "logra_predicted_kl": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, c_vp, c_vp, c_vp, ctypes.c_size_t,
                                          c_vp]),
    "logra_sketch_shared_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.POINTER(ctypes.c_int64)]),
    "logra_sketch_accumulate_shared": (ctypes.c_int, [c_vp, ctypes.c_int64, ctypes.c_int64,
                                                      ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_uint64, ctypes.c_uint64,
                                                      ctypes.c_int, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.POINTER(c_vp),
                                                      ctypes.POINTER(ctypes.c_int64),
                                                      ctypes.POINTER(ctypes.c_int64),
                                                      ctypes.POINTER(c_vp), c_vp,
                                                      ctypes.c_size_t, c_vp]),
    "logra_sketch_accumulate_noalloc": (ctypes.c_int, [c_vp, ctypes.c_int64, c_vp, ctypes.c_int64,
                                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int32, ctypes.c_uint64,
                                                       ctypes.c_uint64, ctypes.c_int, ctypes.c_int32,
                                                       c_vp, c_vp]),
    "logra_set_kernel_choice": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "logra_kl_sweep_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "logra_predicted_kl_sweep": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_int32, ctypes.c_float, c_vp, c_vp, c_vp,
                                                c_vp, ctypes.c_size_t, c_vp]),
}

MAX_SHARED, MAX_GROUPS, MAX_LAYER_OUT, MAX_MERGE = 4, 4, 8, 8


class SketchGroup(ctypes.Structure):
    """logra_sketch_group of include/logra.h (field for field)."""
    _fields_ = [("X", c_vp), ("ldx", ctypes.c_int64), ("k", ctypes.c_int64),
                ("seed", ctypes.c_uint64), ("stream", ctypes.c_uint64), ("n_out", ctypes.c_int32),
                ("dY", c_vp * MAX_SHARED), ("ldd", ctypes.c_int64 * MAX_SHARED),
                ("d", ctypes.c_int64 * MAX_SHARED), ("S", c_vp * MAX_SHARED)]


class MergeItem(ctypes.Structure):
    """logra_merge_item of include/logra.h (field for field)."""
    _fields_ = [("W", c_vp), ("ldw", ctypes.c_int64), ("S", c_vp), ("d", ctypes.c_int64),
                ("k", ctypes.c_int64), ("seed", ctypes.c_uint64), ("stream", ctypes.c_uint64)]


SIGNATURES.update({
    "logra_sketch_layer_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_int32,
                                                      ctypes.POINTER(SketchGroup)]),
    "logra_sketch_accumulate_layer": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                                                     ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.POINTER(SketchGroup), c_vp,
                                                     ctypes.c_size_t, c_vp]),
    "logra_merge_many": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(MergeItem), ctypes.c_int32,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_float, c_vp]),
    "logra_sketch_p_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "logra_sketch_project_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "logra_sketch_project": (ctypes.c_int, [c_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.c_int, c_vp, ctypes.c_size_t, c_vp,
                                            ctypes.c_size_t, c_vp]),
    "logra_sketch_accumulate_p_ws_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32,
                                                             ctypes.c_int32,
                                                             ctypes.POINTER(ctypes.c_int64)]),
    "logra_sketch_accumulate_p": (ctypes.c_int, [c_vp, ctypes.c_size_t, ctypes.c_int64,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.POINTER(c_vp),
                                                 ctypes.POINTER(ctypes.c_int64),
                                                 ctypes.POINTER(ctypes.c_int64),
                                                 ctypes.POINTER(c_vp), c_vp, ctypes.c_size_t,
                                                 c_vp]),
})

OK, EINVAL, EWORKSPACE, EHIP = 0, -1, -2, -3


class LograError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        super().__init__(f"{name} failed with status {status}: {status_str(status)}")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m rank_gradient_sketching_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status):
    return lib().logra_status_str(int(status)).decode()


def check(status, name):
    if status != OK:
        raise LograError(status, name)


def header_symbols(path=HEADER_PATH):
    """Names of the functions include/logra.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(logra_[a-z_A-Z0-9]+)\s*\(", text)))
