"""CPU oracle for the elementwise operations -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never imports it and shares no code with it.

Each function wraps the plain scalar C loop of the same name in ``oracle.c``
(built by ``oracle/build.py``) and works on numpy arrays:

* ``add_f32(a, b)``            c = a + b, binary32
* ``add_f16(a, b)``            binary16 bits in, binary16 bits out (uint16)
* ``add_bf16(a, b)``           bfloat16 bits in, bfloat16 bits out (uint16)
* ``saxpy_f32(alpha, x, y)``   returns fmaf(alpha, x, y) (y is not modified)
* ``relu_f32(x)``              IEEE maximum(x, +0)
* ``add_relu_f32(a, b)``       maximum(a + b, +0)
* ``saxpy_relu_f32(alpha, x, y)``  maximum(fmaf(alpha, x, y), +0)
* ``bias_relu_f32(x, bias, rows, cols)``  maximum(x[r, c] + bias[c], +0)
* ``saxpy_f16 / saxpy_bf16(alpha, x, y)``  16-bit SAXPY via one binary32 fma
* ``relu_f16 / relu_bf16(x)``  16-bit IEEE maximum(x, +0)
* ``copy_f32(x)``              bitwise copy
* ``gather_f32(x, stride)``    out[i] = x[(stride*i) mod n], bitwise
* ``gather_index(n, stride, i)``  the input index of one gather output
* ``copy2d_f32(base, offset, stride_r, stride_c, rows, cols)``  strided view
  copied to a contiguous array
* ``scale_f32 / scale_f16 / scale_bf16(alpha, x)``  alpha * x
* ``add_scalar_f32 / add_scalar_f16 / add_scalar_bf16(alpha, x)``  x + alpha
* ``sqrt_f32 / sqrt_f16 / sqrt_bf16(x)``  correctly rounded binary32 sqrt
  (16-bit: of the widened value, rounded to the 16-bit format)
* ``abs_f32 / abs_f16 / abs_bf16(x)``  sign bit cleared

plus the scalar conversions and the binary32 ulp distance.  Parity status:
all functions pinned (see ``tests/test_oracle.py``); none unpinned.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    for name in ("oracle_add_f32", "oracle_add_f16", "oracle_add_bf16"):
        getattr(lib, name).argtypes = [vp, vp, vp, sz]
        getattr(lib, name).restype = None
    lib.oracle_saxpy_f32.argtypes = [ctypes.c_float, vp, vp, sz]
    lib.oracle_saxpy_f32.restype = None
    lib.oracle_add_relu_f32.argtypes = [vp, vp, vp, sz]
    lib.oracle_add_relu_f32.restype = None
    lib.oracle_saxpy_relu_f32.argtypes = [ctypes.c_float, vp, vp, sz]
    lib.oracle_saxpy_relu_f32.restype = None
    lib.oracle_bias_relu_f32.argtypes = [vp, vp, vp, sz, sz]
    lib.oracle_bias_relu_f32.restype = None
    for name in ("oracle_saxpy_f16", "oracle_saxpy_bf16"):
        getattr(lib, name).argtypes = [ctypes.c_float, vp, vp, sz]
        getattr(lib, name).restype = None
    for name in ("oracle_relu_f16", "oracle_relu_bf16"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    for name in ("oracle_relu_f32", "oracle_copy_f32",
                 "oracle_f32_to_f16_array", "oracle_f16_to_f32_array",
                 "oracle_f32_to_bf16_array", "oracle_bf16_to_f32_array"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    for name in ("oracle_scale_f32", "oracle_add_scalar_f32", "oracle_scale_f16",
                 "oracle_scale_bf16", "oracle_add_scalar_f16", "oracle_add_scalar_bf16"):
        getattr(lib, name).argtypes = [ctypes.c_float, vp, vp, sz]
        getattr(lib, name).restype = None
    for name in ("oracle_sqrt_f32", "oracle_abs_f32", "oracle_sqrt_f16", "oracle_sqrt_bf16",
                 "oracle_abs_16"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    lib.oracle_copy2d_f32.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, sz, sz]
    lib.oracle_copy2d_f32.restype = None
    lib.oracle_gather_f32.argtypes = [vp, vp, sz, sz]
    lib.oracle_gather_f32.restype = None
    for name in ("oracle_f32_range_to_f16", "oracle_f32_range_to_bf16"):
        getattr(lib, name).argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp]
        getattr(lib, name).restype = None
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_ulp_distance_f32.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.oracle_ulp_distance_f32.restype = ctypes.c_uint64
    lib.oracle_gather_index.argtypes = [sz, sz, sz]
    lib.oracle_gather_index.restype = sz
    lib.oracle_fpenv_ok.argtypes = []
    lib.oracle_fpenv_ok.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(arr):
    return arr.ctypes.data_as(ctypes.c_void_p)


def _as(arr, dtype):
    arr = np.ascontiguousarray(arr)
    if arr.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {arr.dtype}")
    return arr.reshape(-1)


def _check_env(lib):
    if not lib.oracle_fpenv_ok():
        raise RuntimeError("oracle: MXCSR has FTZ/DAZ set or a non-RNE rounding mode")


def fpenv_ok() -> bool:
    """True when the host FP environment is IEEE default (no FTZ/DAZ, RNE)."""
    return bool(_load().oracle_fpenv_ok())


def _binary(name, a, b, dtype):
    lib = _load()
    _check_env(lib)
    a = _as(a, dtype)
    b = _as(b, dtype)
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    c = np.empty_like(a)
    getattr(lib, name)(_ptr(a), _ptr(b), _ptr(c), a.size)
    return c


def add_f32(a, b):
    """c = a + b in binary32."""
    return _binary("oracle_add_f32", a, b, np.float32)


def add_f16(a, b):
    """binary16 add via binary32 then RNE; uint16 bit patterns in and out."""
    return _binary("oracle_add_f16", a, b, np.uint16)


def add_bf16(a, b):
    """bfloat16 add via binary32 then RNE; uint16 bit patterns in and out."""
    return _binary("oracle_add_bf16", a, b, np.uint16)


def saxpy_f32(alpha, x, y):
    """Returns fmaf(alpha, x[i], y[i]) for every i; ``y`` is left unchanged."""
    lib = _load()
    _check_env(lib)
    x = _as(x, np.float32)
    out = np.array(_as(y, np.float32), copy=True)
    if x.shape != out.shape:
        raise ValueError("shape mismatch")
    lib.oracle_saxpy_f32(float(np.float32(alpha)), _ptr(x), _ptr(out), x.size)
    return out


def add_relu_f32(a, b):
    """maximum(a + b, +0), the sum rounded once to binary32."""
    return _binary("oracle_add_relu_f32", a, b, np.float32)


def saxpy_relu_f32(alpha, x, y):
    """maximum(fmaf(alpha, x, y), +0) per element; ``y`` is left unchanged."""
    lib = _load()
    _check_env(lib)
    x = _as(x, np.float32)
    out = np.array(_as(y, np.float32), copy=True)
    if x.shape != out.shape:
        raise ValueError("shape mismatch")
    lib.oracle_saxpy_relu_f32(float(np.float32(alpha)), _ptr(x), _ptr(out), x.size)
    return out


def bias_relu_f32(x, bias, rows, cols):
    """maximum(x[r, c] + bias[c], +0) for a row-major rows x cols x."""
    lib = _load()
    _check_env(lib)
    x = _as(x, np.float32)
    bias = _as(bias, np.float32)
    if x.size != rows * cols or bias.size != cols:
        raise ValueError("shape mismatch")
    y = np.empty_like(x)
    lib.oracle_bias_relu_f32(_ptr(x), _ptr(bias), _ptr(y), int(rows), int(cols))
    return y


def _saxpy16(name, alpha, x, y):
    lib = _load()
    _check_env(lib)
    x = _as(x, np.uint16)
    out = np.array(_as(y, np.uint16), copy=True)
    if x.shape != out.shape:
        raise ValueError("shape mismatch")
    getattr(lib, name)(float(np.float32(alpha)), _ptr(x), _ptr(out), x.size)
    return out


def saxpy_f16(alpha, x, y):
    """rne16(fmaf(alpha, widen(x), widen(y))) on binary16 bit patterns."""
    return _saxpy16("oracle_saxpy_f16", alpha, x, y)


def saxpy_bf16(alpha, x, y):
    """rnebf(fmaf(alpha, widen(x), widen(y))) on bfloat16 bit patterns."""
    return _saxpy16("oracle_saxpy_bf16", alpha, x, y)


def _relu16(name, x):
    lib = _load()
    _check_env(lib)     # the decision compares the widened value with 0 in binary32
    x = _as(x, np.uint16)
    y = np.empty_like(x)
    getattr(lib, name)(_ptr(x), _ptr(y), x.size)
    return y


def relu_f16(x):
    """IEEE maximum(x, +0) on binary16 bit patterns."""
    return _relu16("oracle_relu_f16", x)


def relu_bf16(x):
    """IEEE maximum(x, +0) on bfloat16 bit patterns."""
    return _relu16("oracle_relu_bf16", x)


def relu_f32(x):
    """IEEE 754-2019 maximum(x, +0) per element."""
    lib = _load()
    _check_env(lib)
    x = _as(x, np.float32)
    y = np.empty_like(x)
    lib.oracle_relu_f32(_ptr(x), _ptr(y), x.size)
    return y


def _map(name, dtype, x, alpha=None):
    lib = _load()
    _check_env(lib)
    x = _as(x, dtype)
    y = np.empty_like(x)
    if alpha is None:
        getattr(lib, name)(_ptr(x), _ptr(y), x.size)
    else:
        getattr(lib, name)(float(np.float32(alpha)), _ptr(x), _ptr(y), x.size)
    return y


def scale_f32(alpha, x):
    """alpha * x in binary32."""
    return _map("oracle_scale_f32", np.float32, x, alpha)


def scale_f16(alpha, x):
    """rne16(alpha * widen(x)) on binary16 bit patterns."""
    return _map("oracle_scale_f16", np.uint16, x, alpha)


def scale_bf16(alpha, x):
    """rnebf(alpha * widen(x)) on bfloat16 bit patterns."""
    return _map("oracle_scale_bf16", np.uint16, x, alpha)


def add_scalar_f32(alpha, x):
    """x + alpha in binary32."""
    return _map("oracle_add_scalar_f32", np.float32, x, alpha)


def add_scalar_f16(alpha, x):
    """rne16(widen(x) + alpha) on binary16 bit patterns."""
    return _map("oracle_add_scalar_f16", np.uint16, x, alpha)


def add_scalar_bf16(alpha, x):
    """rnebf(widen(x) + alpha) on bfloat16 bit patterns."""
    return _map("oracle_add_scalar_bf16", np.uint16, x, alpha)


def sqrt_f32(x):
    """Correctly rounded binary32 square root."""
    return _map("oracle_sqrt_f32", np.float32, x)


def sqrt_f16(x):
    """rne16(sqrtf(widen(x))) on binary16 bit patterns."""
    return _map("oracle_sqrt_f16", np.uint16, x)


def sqrt_bf16(x):
    """rnebf(sqrtf(widen(x))) on bfloat16 bit patterns."""
    return _map("oracle_sqrt_bf16", np.uint16, x)


def abs_f32(x):
    """The sign bit cleared, every other bit kept."""
    return _map("oracle_abs_f32", np.float32, x)


def abs_f16(x):
    """Bit 15 cleared (binary16)."""
    return _map("oracle_abs_16", np.uint16, x)


def abs_bf16(x):
    """Bit 15 cleared (bfloat16)."""
    return _map("oracle_abs_16", np.uint16, x)


def copy_f32(x):
    """Bitwise copy."""
    lib = _load()
    x = _as(x, np.float32)
    y = np.empty_like(x)
    lib.oracle_copy_f32(_ptr(x), _ptr(y), x.size)
    return y


def gather_f32(x, stride):
    """out[i] = x[(stride*i) mod n], bitwise; exact index arithmetic."""
    lib = _load()
    x = _as(x, np.float32)
    y = np.empty_like(x)
    if x.size:
        lib.oracle_gather_f32(_ptr(x), _ptr(y), x.size, int(stride))
    return y


def copy2d_f32(base, offset, stride_r, stride_c, rows, cols):
    """out[r, c] = base[offset + r*stride_r + c*stride_c], bitwise, as a
    contiguous rows x cols array (strides in elements, may be negative).
    Every index touched must lie inside `base`."""
    lib = _load()
    base = _as(base, np.float32)
    lo = offset + min(0, (rows - 1) * stride_r) + min(0, (cols - 1) * stride_c)
    hi = offset + max(0, (rows - 1) * stride_r) + max(0, (cols - 1) * stride_c)
    if rows and cols and (lo < 0 or hi >= base.size):
        raise ValueError("view outside the base array")
    out = np.empty(rows * cols, np.float32)
    if rows and cols:
        ptr = base.ctypes.data + 4 * offset
        lib.oracle_copy2d_f32(ctypes.c_void_p(ptr), int(stride_r), int(stride_c), _ptr(out),
                              int(rows), int(cols))
    return out


def gather_index(n, stride, i) -> int:
    """(stride * i) mod n, exact: the input index of gather output i."""
    return int(_load().oracle_gather_index(int(n), int(stride), int(i)))


def f32_to_f16(x):
    lib = _load()
    x = _as(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib.oracle_f32_to_f16_array(_ptr(x), _ptr(y), x.size)
    return y


def f16_to_f32(h):
    lib = _load()
    h = _as(h, np.uint16)
    y = np.empty(h.shape, np.float32)
    lib.oracle_f16_to_f32_array(_ptr(h), _ptr(y), h.size)
    return y


def f32_to_bf16(x):
    lib = _load()
    x = _as(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib.oracle_f32_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(h):
    lib = _load()
    h = _as(h, np.uint16)
    y = np.empty(h.shape, np.float32)
    lib.oracle_bf16_to_f32_array(_ptr(h), _ptr(y), h.size)
    return y


def f32_range_to_f16(start, count):
    """Convert the binary32 bit patterns start..start+count-1 to binary16."""
    lib = _load()
    y = np.empty(count, np.uint16)
    lib.oracle_f32_range_to_f16(start, count, _ptr(y))
    return y


def f32_range_to_bf16(start, count):
    """Convert the binary32 bit patterns start..start+count-1 to bfloat16."""
    lib = _load()
    y = np.empty(count, np.uint16)
    lib.oracle_f32_range_to_bf16(start, count, _ptr(y))
    return y


def ulp_distance_f32(a, b) -> int:
    """|ord(a) - ord(b)| for two binary32 values (not NaN)."""
    return int(_load().oracle_ulp_distance_f32(float(np.float32(a)), float(np.float32(b))))


def library_path() -> str:
    _load()
    return _LIB_PATH
