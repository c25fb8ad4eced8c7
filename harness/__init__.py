"""Device plumbing and element comparison shared by bench.py, the GPU tests
and the smoke check: upload a host array at an element offset, download a
result, and compare two results element by element.

Nothing here computes an operation: the results compared come from libew
(the GPU path) and from the oracle (in the tests and the bench's CPU leg).
"""
import numpy as np
import torch

DEV = torch.device("cuda:0")

ELEM = {"add_f32": 4, "add_f16": 2, "add_bf16": 2, "saxpy_f32": 4, "relu_f32": 4,
        "copy_f32": 4, "gather_f32": 4, "gather_walk_f32": 4, "add_relu_f32": 4,
        "saxpy_relu_f32": 4, "bias_relu_f32": 4, "saxpy_f16": 2, "saxpy_bf16": 2, "relu_f16": 2, "relu_bf16": 2,
        "copy2d_f32": 4, "relu_inplace_f32": 4,
        **{f"{m}_{d}": 4 if d == "f32" else 2
           for m in ("scale", "add_scalar", "sqrt", "abs") for d in ("f32", "f16", "bf16")}}
NP_DTYPE = {4: np.float32, 2: np.uint16}
TORCH_DTYPE = {4: torch.float32, 2: torch.int16}


def upload(arr: np.ndarray, off: int = 0, pad: int = 16, device=DEV):
    """Copy arr to the GPU so that the returned view starts `off` elements past
    a fresh allocation.  Returns (view, base); keep `base` alive."""
    es = arr.dtype.itemsize
    host = arr.view(np.int16) if es == 2 else arr
    base = torch.empty(arr.size + off + pad, dtype=TORCH_DTYPE[es], device=device)
    view = base[off:off + arr.size]
    if not (host.flags.writeable and host.flags.c_contiguous):
        host = np.array(host, copy=True, order="C")
    view.copy_(torch.from_numpy(host))
    return view, base


def download(t: torch.Tensor, es: int) -> np.ndarray:
    h = t.cpu().numpy()
    return h.view(NP_DTYPE[es])


def nan_mask(bits: np.ndarray, es: int) -> np.ndarray:
    if es == 4:
        b = bits.view(np.uint32)
        return (b & 0x7FFFFFFF) > 0x7F800000
    return None


def f16_nan(bits):
    return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)


def bf16_nan(bits):
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def mismatches(op: str, got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Indices where got differs from ref: bitwise, except that for the
    arithmetic ops (fused ones included) a NaN matches any NaN (payloads are
    not part of the contract).  Copy, gather, ReLU and abs compare bitwise
    throughout."""
    if op in ("copy_f32", "gather_f32", "gather_walk_f32", "relu_f32", "copy2d_f32",
              "relu_inplace_f32", "abs_f32"):
        g, r = got.view(np.uint32), ref.view(np.uint32)
        return np.nonzero(g != r)[0]
    if op in ("relu_f16", "relu_bf16", "abs_f16", "abs_bf16"):
        return np.nonzero(got.view(np.uint16) != ref.view(np.uint16))[0]
    if op.endswith("_f32"):
        g, r = got.view(np.uint32), ref.view(np.uint32)
        gn = (g & 0x7FFFFFFF) > 0x7F800000
        rn = (r & 0x7FFFFFFF) > 0x7F800000
    else:
        g, r = got.view(np.uint16), ref.view(np.uint16)
        isnan = f16_nan if op.endswith("_f16") else bf16_nan
        gn, rn = isnan(g), isnan(r)
    bad = ((g != r) & ~(gn & rn)) | (gn != rn)
    return np.nonzero(bad)[0]


def ulp_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ord(a) - ord(b)| elementwise for binary32 arrays."""
    def ordv(x):
        u = x.view(np.uint32).astype(np.int64)
        return np.where(u & 0x80000000, -(u & 0x7FFFFFFF), u)
    return np.abs(ordv(a) - ordv(b))
