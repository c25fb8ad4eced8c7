"""Python binding of libew, streaming elementwise kernels for MI355X.

Argument marshalling only: each function below passes device pointers, n and
a HIP stream to the C entry point of the same name in ``libew.so`` (declared
in ``include/ew.h``) and raises ``EwError`` on a non-zero status.  Every
operation runs in the library's HIP kernels; there is no other code path.
If ``libew.so`` has not been built, importing this package raises.

Buffers may be torch tensors (their ``data_ptr()``; pass sliced tensors to
get offset pointers) or plain integers holding device addresses.  ``n``
defaults to the output tensor's ``numel()``; ``stream`` defaults to torch's
current stream on the output's device (an integer ``hipStream_t`` is also
accepted).  Calls are asynchronous, like the C functions.  A tensor argument
must hold elements of the operation's width, be contiguous, hold at least the
n elements the call covers and live on a GPU (a strided view's source: every
element the view touches must lie in its storage); otherwise TypeError or
ValueError is raised before the library is called.  Raw integer addresses are
the caller's responsibility.
"""
import ctypes
import os

__all__ = [
    "EwError", "EwPlan", "OPS", "library_path",
    "ew_add_f32", "ew_add_f16", "ew_add_bf16", "ew_saxpy_f32", "ew_relu_f32",
    "ew_copy_f32", "ew_gather_f32", "ew_gather_walk_f32", "ew_add_relu_f32", "ew_saxpy_relu_f32",
    "ew_bias_relu_f32", "ew_saxpy_f16", "ew_saxpy_bf16", "ew_relu_f16", "ew_relu_bf16",
    "ew_copy2d_f32", "ew_scale_f32", "ew_scale_f16", "ew_scale_bf16", "ew_add_scalar_f32",
    "ew_add_scalar_f16", "ew_add_scalar_bf16", "ew_sqrt_f32", "ew_sqrt_f16", "ew_sqrt_bf16",
    "ew_abs_f32", "ew_abs_f16", "ew_abs_bf16", "ew_status_string", "ew_last_hip_error",
    "ew_abi_version", "ew_set_launch_config", "ew_get_launch_config", "ew_set_launch_row",
    "ew_get_launch_row", "ew_reset_launch_config", "ew_load_launch_table", "ew_make_plan",
    "ew_make_gather_plan", "ew_make_copy2d_plan", "PATHS", "ew_batch", "ew_batch_build",
    "ew_batch_run", "ew_batch_run_static", "BATCH_SCRATCH_BYTES", "EwBatch", "EwBatchItem",
    "EwBatchPlan", "BATCH_MAX",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libew.so")
LAUNCH_TABLE = os.path.join(_PKG, "launch_table.txt")

OPS = ("add_f32", "add_f16", "add_bf16", "saxpy_f32", "relu_f32", "copy_f32", "gather_f32",
       "gather_walk_f32", "add_relu_f32", "saxpy_relu_f32", "bias_relu_f32", "saxpy_f16", "saxpy_bf16",
       "relu_f16", "relu_bf16", "copy2d_f32", "relu_inplace_f32",
       "scale_f32", "scale_f16", "scale_bf16", "add_scalar_f32", "add_scalar_f16",
       "add_scalar_bf16", "sqrt_f32", "sqrt_f16", "sqrt_bf16", "abs_f32", "abs_f16", "abs_bf16")

# The scalar-broadcast maps (alpha, x, y) and the unary maps (x, y).
SCALAR_MAPS = ("scale", "add_scalar")
UNARY_MAPS = ("sqrt", "abs")
MAP_DTYPES = ("f32", "f16", "bf16")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python memory_bound_elementwise_amd/build.py` "
        "or __graft_entry__.build() first")

# torch ships its own HIP runtime under the same soname as ROCm's.  Load it
# first so that libew binds to that one runtime: streams and device pointers
# handed over by torch are only meaningful inside the runtime that made them.
try:
    import torch  # noqa: F401
except ImportError:     # plain C-ABI use without torch: raw pointers only
    torch = None

_lib = ctypes.CDLL(_LIB_PATH)

_vp, _sz, _int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int


class EwPlan(ctypes.Structure):
    """Mirror of ``ew_plan_t``."""
    _fields_ = [
        ("n", _sz), ("head", _sz), ("vectors", _sz), ("tail", _sz), ("tiles", _sz),
        ("vec_elems", _int), ("elem_size", _int), ("in_coaligned", _int * 2),
        ("block", _int), ("blocks_per_cu", _int), ("unroll", _int), ("grid", _int),
        ("segment", _sz), ("reps", _int), ("passes", _int), ("path", _int),
    ]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["in_coaligned"] = tuple(self.in_coaligned)
        return d


class EwBatchItem(ctypes.Structure):
    """Mirror of ``ew_batch_item_t``."""
    _fields_ = [("out", _vp), ("in0", _vp), ("in1", _vp), ("n", _sz)]


class EwBatchPlan(ctypes.Structure):
    """Mirror of ``ew_batch_plan_t``."""
    _fields_ = [("op", ctypes.c_int32), ("block", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("blocks_per_cu", ctypes.c_int32), ("items", ctypes.c_uint64),
                ("tiles", ctypes.c_uint64), ("bytes", ctypes.c_uint64),
                ("total_n", ctypes.c_uint64)]


BATCH_MAX = 96          # EW_BATCH_MAX: items per kernel launch of ew_batch
BATCH_SCRATCH_BYTES = 256 * 1024   # EW_BATCH_SCRATCH_BYTES: largest table of ew_batch_run_static


def _proto(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_c = {
    "ew_add_f32": _proto("ew_add_f32", _int, _vp, _vp, _vp, _sz, _vp),
    "ew_add_f16": _proto("ew_add_f16", _int, _vp, _vp, _vp, _sz, _vp),
    "ew_add_bf16": _proto("ew_add_bf16", _int, _vp, _vp, _vp, _sz, _vp),
    "ew_saxpy_f32": _proto("ew_saxpy_f32", _int, ctypes.c_float, _vp, _vp, _sz, _vp),
    "ew_relu_f32": _proto("ew_relu_f32", _int, _vp, _vp, _sz, _vp),
    "ew_relu_inplace_f32": _proto("ew_relu_inplace_f32", _int, _vp, _sz, _vp),
    "ew_copy_f32": _proto("ew_copy_f32", _int, _vp, _vp, _sz, _vp),
    "ew_gather_f32": _proto("ew_gather_f32", _int, _vp, _vp, _sz, _sz, _vp),
    "ew_gather_walk_f32": _proto("ew_gather_walk_f32", _int, _vp, _vp, _sz, _sz, _vp),
    "ew_add_relu_f32": _proto("ew_add_relu_f32", _int, _vp, _vp, _vp, _sz, _vp),
    "ew_saxpy_relu_f32": _proto("ew_saxpy_relu_f32", _int, ctypes.c_float, _vp, _vp, _sz, _vp),
    "ew_bias_relu_f32": _proto("ew_bias_relu_f32", _int, _vp, _vp, _vp, _sz, _sz, _vp),
    "ew_saxpy_f16": _proto("ew_saxpy_f16", _int, ctypes.c_float, _vp, _vp, _sz, _vp),
    "ew_saxpy_bf16": _proto("ew_saxpy_bf16", _int, ctypes.c_float, _vp, _vp, _sz, _vp),
    "ew_relu_f16": _proto("ew_relu_f16", _int, _vp, _vp, _sz, _vp),
    "ew_relu_bf16": _proto("ew_relu_bf16", _int, _vp, _vp, _sz, _vp),
    "ew_copy2d_f32": _proto("ew_copy2d_f32", _int, _vp, ctypes.c_int64, ctypes.c_int64, _vp,
                            _sz, _sz, _vp),
    **{f"ew_{m}_{d}": _proto(f"ew_{m}_{d}", _int, ctypes.c_float, _vp, _vp, _sz, _vp)
       for m in SCALAR_MAPS for d in MAP_DTYPES},
    **{f"ew_{m}_{d}": _proto(f"ew_{m}_{d}", _int, _vp, _vp, _sz, _vp)
       for m in UNARY_MAPS for d in MAP_DTYPES},
    "ew_batch": _proto("ew_batch", _int, ctypes.c_char_p, ctypes.c_float,
                       ctypes.POINTER(EwBatchItem), _sz, _vp),
    "ew_status_string": _proto("ew_status_string", ctypes.c_char_p, _int),
    "ew_last_hip_error": _proto("ew_last_hip_error", _int),
    "ew_abi_version": _proto("ew_abi_version", _int),
    "ew_batch_build": _proto("ew_batch_build", _int, ctypes.c_char_p,
                             ctypes.POINTER(EwBatchItem), _sz, _vp, _sz,
                             ctypes.POINTER(EwBatchPlan)),
    "ew_batch_run": _proto("ew_batch_run", _int, ctypes.POINTER(EwBatchPlan), ctypes.c_float,
                           _vp, _vp),
    "ew_batch_run_static": _proto("ew_batch_run_static", _int, ctypes.POINTER(EwBatchPlan),
                                  ctypes.c_float, _vp, _vp),
    "ew_set_launch_config": _proto("ew_set_launch_config", _int, ctypes.c_char_p, _int, _int,
                                   _int),
    "ew_get_launch_config": _proto("ew_get_launch_config", _int, ctypes.c_char_p, _sz,
                                   ctypes.POINTER(_int), ctypes.POINTER(_int),
                                   ctypes.POINTER(_int)),
    "ew_set_launch_row": _proto("ew_set_launch_row", _int, ctypes.c_char_p, _sz, _int, _int,
                                _int),
    "ew_get_launch_row": _proto("ew_get_launch_row", _int, ctypes.c_char_p, _sz,
                                ctypes.POINTER(_int), ctypes.POINTER(_int),
                                ctypes.POINTER(_int)),
    "ew_reset_launch_config": _proto("ew_reset_launch_config", None),
    "ew_load_launch_table": _proto("ew_load_launch_table", _int, ctypes.c_char_p),
    "ew_make_plan": _proto("ew_make_plan", _int, ctypes.c_char_p, _vp, _vp, _vp, _sz, _int,
                           ctypes.POINTER(EwPlan)),
    "ew_make_gather_plan": _proto("ew_make_gather_plan", _int, _vp, _vp, _sz, _sz, _int,
                                  ctypes.POINTER(EwPlan)),
    "ew_make_copy2d_plan": _proto("ew_make_copy2d_plan", _int, _vp, ctypes.c_int64,
                                  ctypes.c_int64, _vp, _sz, _sz, _int, ctypes.POINTER(EwPlan)),
}


class EwError(RuntimeError):
    """A libew call returned a non-zero status."""

    def __init__(self, status: int, func: str):
        self.status = status
        self.hip_error = _c["ew_last_hip_error"]() if status == -5 else 0
        msg = _c["ew_status_string"](status).decode()
        if self.hip_error:
            msg += f" (hipError_t {self.hip_error})"
        super().__init__(f"{func}: {msg}")


def _check(status, func):
    if status != 0:
        raise EwError(status, func)


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _buf(x, es, n, role):
    """Device address of one buffer argument.  The C ABI sees only a pointer
    and n, so a tensor is checked here first: elements of the operation's
    width (es bytes), contiguous, at least n elements (a shorter tensor would
    be read or written past its end), on a GPU.  Integers pass unchecked.
    One condition on the fast path (this runs on every call, where the host
    cost of a small launch is a few microseconds)."""
    if x is None or type(x) is int:
        return x
    if x.is_cuda and x.element_size() == es and x.is_contiguous() and x.numel() >= n:
        return x.data_ptr()
    if isinstance(x, int):
        return x
    if x.element_size() != es:
        raise TypeError(f"{role}: {x.dtype} has {x.element_size()}-byte elements, "
                        f"the operation takes {es}-byte elements")
    if not x.is_contiguous():
        raise ValueError(f"{role}: the tensor is not contiguous")
    if x.numel() < n:
        raise ValueError(f"{role}: {x.numel()} elements, the call covers {n}")
    raise ValueError(f"{role}: the tensor is on {x.device}, not on a GPU")


def _numel(x, n):
    if n is not None:
        return int(n)
    if isinstance(x, int):
        raise ValueError("n is required when buffers are raw pointers")
    return x.numel()


# torch's current stream of a device as a raw handle, without building a
# Stream object (which costs about 2 us per call); the public route where the
# internal one is missing.
_raw_current_stream = getattr(getattr(torch, "_C", None), "_cuda_getCurrentRawStream", None)


def _stream(x, stream):
    if stream is None:
        if isinstance(x, int):
            return None
        if _raw_current_stream is not None:
            return _raw_current_stream(x.get_device())
        return torch.cuda.current_stream(x.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ew_add_f32(a, b, c, n=None, stream=None):
    """c = a + b (binary32)."""
    n = _numel(c, n)
    _check(_c["ew_add_f32"](_buf(a, 4, n, "a"), _buf(b, 4, n, "b"), _buf(c, 4, n, "c"), n,
                            _stream(c, stream)), "ew_add_f32")


def ew_add_f16(a, b, c, n=None, stream=None):
    """c = a + b on binary16 data (widen, add in binary32, round RNE)."""
    n = _numel(c, n)
    _check(_c["ew_add_f16"](_buf(a, 2, n, "a"), _buf(b, 2, n, "b"), _buf(c, 2, n, "c"), n,
                            _stream(c, stream)), "ew_add_f16")


def ew_add_bf16(a, b, c, n=None, stream=None):
    """c = a + b on bfloat16 data (widen, add in binary32, round RNE)."""
    n = _numel(c, n)
    _check(_c["ew_add_bf16"](_buf(a, 2, n, "a"), _buf(b, 2, n, "b"), _buf(c, 2, n, "c"), n,
                             _stream(c, stream)), "ew_add_bf16")


def ew_saxpy_f32(alpha, x, y, n=None, stream=None):
    """y = fma(alpha, x, y) in place."""
    n = _numel(y, n)
    _check(_c["ew_saxpy_f32"](float(alpha), _buf(x, 4, n, "x"), _buf(y, 4, n, "y"), n,
                              _stream(y, stream)), "ew_saxpy_f32")


def ew_relu_f32(x, y, n=None, stream=None):
    """y = maximum(x, +0)."""
    n = _numel(y, n)
    _check(_c["ew_relu_f32"](_buf(x, 4, n, "x"), _buf(y, 4, n, "y"), n, _stream(y, stream)),
           "ew_relu_f32")


def ew_relu_inplace_f32(x, n=None, stream=None):
    """x = maximum(x, +0) in place, storing only the 64-byte spans that change."""
    n = _numel(x, n)
    _check(_c["ew_relu_inplace_f32"](_buf(x, 4, n, "x"), n, _stream(x, stream)),
           "ew_relu_inplace_f32")


def ew_copy_f32(src, out, n=None, stream=None):
    """out = src, bitwise."""
    n = _numel(out, n)
    _check(_c["ew_copy_f32"](_buf(src, 4, n, "src"), _buf(out, 4, n, "out"), n,
                             _stream(out, stream)), "ew_copy_f32")


def ew_gather_f32(src, out, stride, n=None, stream=None):
    """out[i] = src[(stride * i) mod n], bitwise."""
    n = _numel(out, n)
    _check(_c["ew_gather_f32"](_buf(src, 4, n, "src"), _buf(out, 4, n, "out"), n, int(stride),
                               _stream(out, stream)), "ew_gather_f32")


def ew_gather_walk_f32(src, out, stride, n=None, stream=None):
    """out[i] = src[(stride * i) mod n], bitwise, one input load per output
    element (the per-output index walk, no reuse)."""
    n = _numel(out, n)
    _check(_c["ew_gather_walk_f32"](_buf(src, 4, n, "src"), _buf(out, 4, n, "out"), n,
                                    int(stride), _stream(out, stream)), "ew_gather_walk_f32")


def ew_add_relu_f32(a, b, c, n=None, stream=None):
    """c = maximum(a + b, +0) in one pass."""
    n = _numel(c, n)
    _check(_c["ew_add_relu_f32"](_buf(a, 4, n, "a"), _buf(b, 4, n, "b"), _buf(c, 4, n, "c"), n,
                                 _stream(c, stream)), "ew_add_relu_f32")


def ew_saxpy_relu_f32(alpha, x, y, n=None, stream=None):
    """y = maximum(fma(alpha, x, y), +0) in place."""
    n = _numel(y, n)
    _check(_c["ew_saxpy_relu_f32"](float(alpha), _buf(x, 4, n, "x"), _buf(y, 4, n, "y"), n,
                                   _stream(y, stream)), "ew_saxpy_relu_f32")


def ew_bias_relu_f32(x, bias, y, rows=None, cols=None, stream=None):
    """y[r, c] = maximum(x[r, c] + bias[c], +0); rows/cols default to y's 2-D shape."""
    if rows is None or cols is None:
        if isinstance(y, int):
            raise ValueError("rows and cols are required when buffers are raw pointers")
        rows, cols = y.shape
    rows, cols = int(rows), int(cols)
    n = rows * cols
    _check(_c["ew_bias_relu_f32"](_buf(x, 4, n, "x"), _buf(bias, 4, cols, "bias"),
                                  _buf(y, 4, n, "y"), rows, cols, _stream(y, stream)),
           "ew_bias_relu_f32")


def ew_saxpy_f16(alpha, x, y, n=None, stream=None):
    """y = rne16(fma(alpha, x, y)) in place on binary16 data."""
    n = _numel(y, n)
    _check(_c["ew_saxpy_f16"](float(alpha), _buf(x, 2, n, "x"), _buf(y, 2, n, "y"), n,
                              _stream(y, stream)), "ew_saxpy_f16")


def ew_saxpy_bf16(alpha, x, y, n=None, stream=None):
    """y = rnebf(fma(alpha, x, y)) in place on bfloat16 data."""
    n = _numel(y, n)
    _check(_c["ew_saxpy_bf16"](float(alpha), _buf(x, 2, n, "x"), _buf(y, 2, n, "y"), n,
                               _stream(y, stream)), "ew_saxpy_bf16")


def ew_relu_f16(x, y, n=None, stream=None):
    """y = maximum(x, +0) on binary16 data."""
    n = _numel(y, n)
    _check(_c["ew_relu_f16"](_buf(x, 2, n, "x"), _buf(y, 2, n, "y"), n, _stream(y, stream)),
           "ew_relu_f16")


def ew_relu_bf16(x, y, n=None, stream=None):
    """y = maximum(x, +0) on bfloat16 data."""
    n = _numel(y, n)
    _check(_c["ew_relu_bf16"](_buf(x, 2, n, "x"), _buf(y, 2, n, "y"), n, _stream(y, stream)),
           "ew_relu_bf16")


def ew_copy2d_f32(src, stride_r, stride_c, out, rows=None, cols=None, stream=None):
    """out[r, c] = src[r*stride_r + c*stride_c] into a contiguous rows x cols
    array; `src` is the address (or tensor) of element (0, 0) of the view.
    rows/cols default to out's 2-D shape."""
    if rows is None or cols is None:
        if isinstance(out, int):
            raise ValueError("rows and cols are required when buffers are raw pointers")
        rows, cols = out.shape
    rows, cols, stride_r, stride_c = int(rows), int(cols), int(stride_r), int(stride_c)
    _check(_c["ew_copy2d_f32"](_view_src(src, stride_r, stride_c, rows, cols), stride_r,
                               stride_c, _buf(out, 4, rows * cols, "out"), rows, cols,
                               _stream(out, stream)), "ew_copy2d_f32")


def _view_src(x, sr, sc, rows, cols):
    """Address of a strided view's element (0, 0).  For a tensor, every
    element the view touches must lie inside the tensor's storage."""
    if isinstance(x, int) or not rows or not cols:
        return _addr(x)
    if x.element_size() != 4:
        raise TypeError(f"src: {x.dtype} has {x.element_size()}-byte elements, the view "
                        "takes 4-byte elements")
    lo = min(0, (rows - 1) * sr) + min(0, (cols - 1) * sc)
    hi = max(0, (rows - 1) * sr) + max(0, (cols - 1) * sc)
    start = x.storage_offset()
    size = x.untyped_storage().nbytes() // 4
    if start + lo < 0 or start + hi >= size:
        raise ValueError(f"src: the view reaches elements {start + lo}..{start + hi} of a "
                         f"storage of {size}")
    if not x.is_cuda:
        raise ValueError(f"src: the tensor is on {x.device}, not on a GPU")
    return x.data_ptr()


def _es(name):
    return 4 if name.endswith("_f32") else 2


def _scalar_map(name, alpha, x, y, n, stream):
    n = _numel(y, n)
    _check(_c[name](float(alpha), _buf(x, _es(name), n, "x"), _buf(y, _es(name), n, "y"), n,
                    _stream(y, stream)), name)


def _unary_map(name, x, y, n, stream):
    n = _numel(y, n)
    _check(_c[name](_buf(x, _es(name), n, "x"), _buf(y, _es(name), n, "y"), n,
                    _stream(y, stream)), name)


def ew_scale_f32(alpha, x, y, n=None, stream=None):
    """y = alpha * x (binary32)."""
    _scalar_map("ew_scale_f32", alpha, x, y, n, stream)


def ew_scale_f16(alpha, x, y, n=None, stream=None):
    """y = rne16(alpha * widen(x)) on binary16 data."""
    _scalar_map("ew_scale_f16", alpha, x, y, n, stream)


def ew_scale_bf16(alpha, x, y, n=None, stream=None):
    """y = rnebf(alpha * widen(x)) on bfloat16 data."""
    _scalar_map("ew_scale_bf16", alpha, x, y, n, stream)


def ew_add_scalar_f32(alpha, x, y, n=None, stream=None):
    """y = x + alpha (binary32)."""
    _scalar_map("ew_add_scalar_f32", alpha, x, y, n, stream)


def ew_add_scalar_f16(alpha, x, y, n=None, stream=None):
    """y = rne16(widen(x) + alpha) on binary16 data."""
    _scalar_map("ew_add_scalar_f16", alpha, x, y, n, stream)


def ew_add_scalar_bf16(alpha, x, y, n=None, stream=None):
    """y = rnebf(widen(x) + alpha) on bfloat16 data."""
    _scalar_map("ew_add_scalar_bf16", alpha, x, y, n, stream)


def ew_sqrt_f32(x, y, n=None, stream=None):
    """y = sqrt(x), correctly rounded binary32."""
    _unary_map("ew_sqrt_f32", x, y, n, stream)


def ew_sqrt_f16(x, y, n=None, stream=None):
    """y = rne16(sqrt(widen(x))) on binary16 data."""
    _unary_map("ew_sqrt_f16", x, y, n, stream)


def ew_sqrt_bf16(x, y, n=None, stream=None):
    """y = rnebf(sqrt(widen(x))) on bfloat16 data."""
    _unary_map("ew_sqrt_bf16", x, y, n, stream)


def ew_abs_f32(x, y, n=None, stream=None):
    """y = |x|: the sign bit cleared."""
    _unary_map("ew_abs_f32", x, y, n, stream)


def ew_abs_f16(x, y, n=None, stream=None):
    """y = |x| on binary16 bit patterns."""
    _unary_map("ew_abs_f16", x, y, n, stream)


def ew_abs_bf16(x, y, n=None, stream=None):
    """y = |x| on bfloat16 bit patterns."""
    _unary_map("ew_abs_bf16", x, y, n, stream)


def _batch_items(op, items):
    """The C item array of a batch (tensors checked), and the first tensor
    given as an output (for the default stream and device)."""
    es = 4 if op.endswith("_f32") else 2
    arr = (EwBatchItem * max(len(items), 1))()
    first = None
    for k, (out, in0, in1, n) in enumerate(items):
        n = _numel(out, n)
        arr[k] = EwBatchItem(
            _buf(out, es, n, f"items[{k}].out"), _buf(in0, es, n, f"items[{k}].in0"),
            _buf(in1, es, n, f"items[{k}].in1") if in1 is not None else None, n)
        if first is None and not isinstance(out, int):
            first = out
    return arr, first


def ew_batch_build(op, items):
    """Validate a batch and build its table image on the host: returns
    (EwBatchPlan, image) with the image as a ctypes array of plan.bytes
    bytes (8-byte aligned).  items as for EwBatch."""
    arr, _ = _batch_items(op, items)
    plan = EwBatchPlan()
    _check(_c["ew_batch_build"](op.encode(), arr, len(items), None, 0, ctypes.byref(plan)),
           "ew_batch_build")
    image = (ctypes.c_uint64 * max(1, plan.bytes // 8))()
    _check(_c["ew_batch_build"](op.encode(), arr, len(items), ctypes.addressof(image),
                                ctypes.sizeof(image), ctypes.byref(plan)), "ew_batch_build")
    return plan, image


def ew_batch_run(plan, alpha, table, stream=None):
    """One launch of a built batch; table: a device tensor (or address)
    holding the image ew_batch_build returned."""
    s = _stream(table, stream) if not isinstance(table, int) else stream
    if s is not None and not isinstance(s, int):
        s = s.cuda_stream
    _check(_c["ew_batch_run"](ctypes.byref(plan), float(alpha), _addr(table), s),
           "ew_batch_run")


def ew_batch_run_static(plan, alpha, image, stream=None):
    """One launch of a built batch whose table the library copies from the
    host image (as ew_batch_build returned it) into its static device array:
    no device memory of the caller's.  Waits for the stream before and after
    the copy; plan.bytes must not exceed BATCH_SCRATCH_BYTES."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    if stream is None and torch is not None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(_c["ew_batch_run_static"](ctypes.byref(plan), float(alpha), ctypes.addressof(image),
                                     stream), "ew_batch_run_static")


class EwBatch:
    """A batched call prepared once.  items: a sequence of (out, in0, in1, n)
    with the single call's pointers (in1 None for one-input operations and
    SAXPY; n None for out's numel()); the tensors must stay alive while the
    batch is used.

    table=True (default): the library builds the item table once
    (ew_batch_build), it is copied to a device tensor on the first output's
    device, and each call -- ``batch(alpha, stream)`` -- is one
    ``ew_batch_run`` launch, however many items.  table=False: each call
    passes the host item array to ``ew_batch`` (one launch per BATCH_MAX
    items; the items are validated on every call)."""

    def __init__(self, op, items, table=True):
        self.op = op
        self._op = op.encode()
        self.count = len(items)
        self._arr, self._first = _batch_items(op, items)
        self.plan = self.table = None
        if table:
            plan, image = ew_batch_build(op, items)
            self.plan = plan
            if plan.tiles:
                if self._first is None:
                    raise ValueError("table=True needs tensor outputs (for the table's device)")
                host = torch.frombuffer(bytearray(image), dtype=torch.uint8)[:plan.bytes]
                self.table = host.to(self._first.device)

    def __call__(self, alpha=0.0, stream=None):
        s = _stream(self._first, stream) if self._first is not None else stream
        if s is not None and not isinstance(s, int):
            s = s.cuda_stream
        if self.plan is not None:
            if self.plan.tiles:
                _check(_c["ew_batch_run"](ctypes.byref(self.plan), float(alpha),
                                          self.table.data_ptr(), s), "ew_batch_run")
            return
        _check(_c["ew_batch"](self._op, float(alpha), self._arr, self.count, s), "ew_batch")


def ew_batch(op, items, alpha=0.0, stream=None):
    """Independent instances of one streaming operation through the host-array
    entry point, in ceil(len(items) / BATCH_MAX) launches (see EwBatch for
    items; EwBatch(op, items) builds a device table once and runs any number
    of items in one launch per call).  stream defaults to torch's current
    stream on the first tensor's device."""
    EwBatch(op, items, table=False)(alpha, stream)


def ew_status_string(status: int) -> str:
    return _c["ew_status_string"](int(status)).decode()


def ew_last_hip_error() -> int:
    return _c["ew_last_hip_error"]()


def ew_abi_version() -> int:
    return _c["ew_abi_version"]()


def ew_set_launch_config(op, block, blocks_per_cu, unroll):
    """One launch configuration for every size of op (replaces its rows)."""
    _check(_c["ew_set_launch_config"](op.encode(), int(block), int(blocks_per_cu), int(unroll)),
           "ew_set_launch_config")


def ew_get_launch_config(op, n):
    """(block, grid, unroll) of the launch the next call of op with n
    elements makes on the current device (16-byte-aligned pointers)."""
    b, g, u = _int(), _int(), _int()
    _check(_c["ew_get_launch_config"](op.encode(), int(n), ctypes.byref(b), ctypes.byref(g),
                                      ctypes.byref(u)), "ew_get_launch_config")
    return b.value, g.value, u.value


def ew_set_launch_row(op, min_n, block, blocks_per_cu, unroll):
    """Set the size-class row of op that applies from min_n elements."""
    _check(_c["ew_set_launch_row"](op.encode(), int(min_n), int(block), int(blocks_per_cu),
                                   int(unroll)), "ew_set_launch_row")


def ew_get_launch_row(op, n):
    """(block, blocks_per_cu, unroll) of the row that applies to n."""
    b, k, u = _int(), _int(), _int()
    _check(_c["ew_get_launch_row"](op.encode(), int(n), ctypes.byref(b), ctypes.byref(k),
                                   ctypes.byref(u)), "ew_get_launch_row")
    return b.value, k.value, u.value


def ew_reset_launch_config():
    _c["ew_reset_launch_config"]()


def ew_load_launch_table(path):
    _check(_c["ew_load_launch_table"](os.fsencode(path)), "ew_load_launch_table")


def ew_make_plan(op, out, in0, in1, n, cu_count) -> EwPlan:
    """Host-side head/body/tail split and launch shape for integer addresses."""
    plan = EwPlan()
    _check(_c["ew_make_plan"](op.encode(), out, in0, in1, int(n), int(cu_count),
                              ctypes.byref(plan)), "ew_make_plan")
    return plan


def ew_make_gather_plan(out, src, n, stride, cu_count) -> EwPlan:
    """The gather's plan (segments and replicas) for integer addresses."""
    plan = EwPlan()
    _check(_c["ew_make_gather_plan"](out, src, int(n), int(stride), int(cu_count),
                                     ctypes.byref(plan)), "ew_make_gather_plan")
    return plan


def ew_make_copy2d_plan(src, stride_r, stride_c, out, rows, cols, cu_count) -> EwPlan:
    """The plan (path and launch) of ew_copy2d_f32 for integer addresses."""
    plan = EwPlan()
    _check(_c["ew_make_copy2d_plan"](src, int(stride_r), int(stride_c), out, int(rows),
                                     int(cols), int(cu_count), ctypes.byref(plan)),
           "ew_make_copy2d_plan")
    return plan


# ew_path_t: the kernel path of a plan
PATHS = ("stream", "copy", "gather_walk", "gather_spans", "gather_passes", "view_rows",
         "view_transpose", "view_generic", "gather_tiles")


def library_path() -> str:
    return _LIB_PATH


if os.path.exists(LAUNCH_TABLE):
    ew_load_launch_table(LAUNCH_TABLE)
