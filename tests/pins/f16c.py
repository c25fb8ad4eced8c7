"""ctypes access to the x86 F16C reference conversions (``f16c_ref.c``)."""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "f16c_ref.c")
_LIB = os.path.join(_HERE, "libf16c_ref.so")
_lib = None


def available() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " f16c" in f.read()
    except OSError:
        return False


def _load():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            tmp = _LIB + ".tmp"
            subprocess.run(["gcc", "-O2", "-mf16c", "-mavx2", "-fPIC", "-shared",
                            "-o", tmp, _SRC], check=True)
            os.replace(tmp, _LIB)
        lib = ctypes.CDLL(_LIB)
        lib.pin_f16c_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        lib.pin_f16c_range.restype = None
        lib.pin_f16c_widen.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        lib.pin_f16c_widen.restype = None
        lib.pin_f16c_count_mismatches.argtypes = [ctypes.c_void_p, ctypes.c_uint64,
                                                  ctypes.c_uint64]
        lib.pin_f16c_count_mismatches.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def range_to_f16(start: int, count: int) -> np.ndarray:
    y = np.empty(count, np.uint16)
    _load().pin_f16c_range(start, count, y.ctypes.data_as(ctypes.c_void_p))
    return y


def count_mismatches(fn_address: int, start: int, count: int) -> int:
    """Patterns in [start, start+count) where the binary32 -> binary16
    function at `fn_address` disagrees with VCVTPS2PH (NaNs by class and
    sign)."""
    return int(_load().pin_f16c_count_mismatches(fn_address, start, count))


def widen(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    _load().pin_f16c_widen(h.ctypes.data_as(ctypes.c_void_p),
                           y.ctypes.data_as(ctypes.c_void_p), h.size)
    return y
