"""Seeded synthetic inputs for the elementwise workloads.

This module is shared by the tests, the bench and the smoke check.  It holds
only the input recipe -- which distribution, which seed, which size, which
pointer offset -- and none of the arithmetic of the operations themselves.

Recipe (the pages use unseeded ``torch.randn``; every draw here is seeded):

* uniform[-1, 1):  ``u = rng.random(n, dtype=float32)``; ``2*u - 1`` in
  float32.  Every value is a multiple of 2^-23 in [-1, 1); -0.0, subnormals
  and 1.0 cannot occur (both steps are exact in binary32).
* normal(0, 1):    ``rng.standard_normal(n, dtype=float32)``.
* |normal(0, 1)|:  the normal draw with every sign bit cleared (``np.abs``),
  for the in-place ReLU whose input is already non-negative.
* binary16 / bfloat16 inputs "cast from fp32": the float32 draw above cast
  round-to-nearest-even by numpy (``astype(float16)``) or torch CPU
  (``.to(bfloat16)``), kept as uint16 bit patterns.
* The generator is numpy ``Generator(PCG64(seed))``; A is drawn before B from
  one generator.
"""
from dataclasses import dataclass, field
import hashlib

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform_pm1(g: np.random.Generator, n: int) -> np.ndarray:
    """n float32 values uniform on [-1, 1) (multiples of 2^-23)."""
    u = g.random(n, dtype=np.float32)
    u *= np.float32(2.0)
    u -= np.float32(1.0)
    return u


def normal01(g: np.random.Generator, n: int) -> np.ndarray:
    """n float32 standard-normal values."""
    return g.standard_normal(n, dtype=np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 (numpy RNE cast), as uint16 bit patterns."""
    return x.astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (torch CPU RNE cast), as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def sha256(arr: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(arr).view(np.uint8)).hexdigest()


@dataclass(frozen=True)
class Workload:
    """One configuration: operation, size, input recipe, pointer offsets.

    ``offsets`` gives, per buffer role, how many elements past a 256-byte
    aligned allocation the pointer handed to the library starts.
    """
    name: str
    op: str               # a libew operation name (add_f32, saxpy_f32, sqrt_f16, ...)
    n: int
    seed: int
    dist: str             # "uniform" | "normal" | "absnormal"
    offsets: dict = field(default_factory=dict)
    alpha: float = 0.0    # saxpy and the scalar-broadcast maps
    stride: int = 0       # gather only
    cols: int = 0         # bias_relu / copy2d: row length (n = rows * cols)
    view: tuple = ()      # copy2d: (stride_r, stride_c, base elements, offset)
    batch: int = 0        # batched call: n is split into this many equal consecutive items
    description: str = ""


def _w(*args, **kw):
    return Workload(*args, **kw)


# The five configurations (plus the aligned headline add and the contiguous
# copy that the strided gather is compared with).
WORKLOADS = {
    "cfg1_add_f32_2e20": _w(
        "cfg1_add_f32_2e20", "add_f32", 1 << 20, 101, "uniform",
        description="fp32 C=A+B, n=2^20, aligned, A,B uniform[-1,1)"),
    "cfg2_add_f32_2e28p3_offA1": _w(
        "cfg2_add_f32_2e28p3_offA1", "add_f32", (1 << 28) + 3, 102, "uniform",
        offsets={"a": 1},
        description="fp32 C=A+B, n=2^28+3, A offset by one element (4 B), A,B uniform[-1,1)"),
    "cfg3_saxpy_f32_32M": _w(
        "cfg3_saxpy_f32_32M", "saxpy_f32", 1 << 25, 103, "normal", alpha=2.5,
        description="fp32 SAXPY in place y = 2.5*x + y, n=2^25, x,y normal(0,1)"),
    "cfg4a_add_f16_2e28": _w(
        "cfg4a_add_f16_2e28", "add_f16", 1 << 28, 104, "uniform",
        description="fp16 C=A+B, n=2^28, A,B uniform[-1,1) cast RNE from fp32"),
    "cfg4b_add_bf16_2e28": _w(
        "cfg4b_add_bf16_2e28", "add_bf16", 1 << 28, 105, "uniform",
        description="bf16 C=A+B, n=2^28, A,B uniform[-1,1) cast RNE from fp32"),
    "cfg4c_relu_f32_2e28": _w(
        "cfg4c_relu_f32_2e28", "relu_f32", 1 << 28, 106, "normal",
        description="fp32 ReLU y=max(x,0), n=2^28, x normal(0,1), out of place"),
    "cfg5a_copy_f32_2e26": _w(
        "cfg5a_copy_f32_2e26", "copy_f32", 1 << 26, 107, "uniform",
        description="fp32 contiguous copy out[i]=in[i], n=2^26, in uniform[-1,1)"),
    "cfg5b_gather_f32_2e26_s2": _w(
        "cfg5b_gather_f32_2e26_s2", "gather_f32", 1 << 26, 107, "uniform", stride=2,
        description="fp32 strided gather out[i]=in[(2*i) mod n], n=2^26, in uniform[-1,1)"),
    "gather_f32_2e26_s3": _w(
        "gather_f32_2e26_s3", "gather_f32", 1 << 26, 107, "uniform", stride=3,
        description="fp32 strided gather out[i]=in[(3*i) mod n], n=2^26 (gcd 1: a permutation "
                    "read with stride 3)"),
    "gather_f32_2e26_s6": _w(
        "gather_f32_2e26_s6", "gather_f32", 1 << 26, 107, "uniform", stride=6,
        description="fp32 strided gather out[i]=in[(6*i) mod n], n=2^26 (gcd 2: two equal "
                    "halves of three runs each, read with stride 6)"),
    "gather_f32_2e26_s1000": _w(
        "gather_f32_2e26_s1000", "gather_f32", 1 << 26, 107, "uniform", stride=1000,
        description="fp32 strided gather out[i]=in[(1000*i) mod n], n=2^26 (gcd 8: eight equal "
                    "segments of 125 runs, read with stride 1000)"),
    "gather_f32_2e26_s33": _w(
        "gather_f32_2e26_s33", "gather_f32", 1 << 26, 107, "uniform", stride=33,
        description="fp32 strided gather out[i]=in[(33*i) mod n], n=2^26 (gcd 1: 33 runs, read "
                    "with stride 33)"),
    "gather_walk_f32_2e26_s33": _w(
        "gather_walk_f32_2e26_s33", "gather_walk_f32", 1 << 26, 107, "uniform", stride=33,
        description="the same stride-33 gather, one 4-byte load per output (the per-output "
                    "index walk)"),
    "fused_add_relu_f32_2e28": _w(
        "fused_add_relu_f32_2e28", "add_relu_f32", 1 << 28, 108, "normal",
        description="fp32 C=max(A+B,0) in one pass, n=2^28, A,B normal(0,1)"),
    "fused_saxpy_relu_f32_2e28": _w(
        "fused_saxpy_relu_f32_2e28", "saxpy_relu_f32", 1 << 28, 109, "normal", alpha=2.5,
        description="fp32 y=max(2.5*x+y,0) in place, n=2^28, x,y normal(0,1)"),
    "fused_bias_relu_f32_65536x4096": _w(
        "fused_bias_relu_f32_65536x4096", "bias_relu_f32", 1 << 28, 110, "normal", cols=4096,
        description="fp32 y=max(x+bias[col],0), 65536 x 4096 row-major, x,bias normal(0,1)"),
    "saxpy_f16_2e28": _w(
        "saxpy_f16_2e28", "saxpy_f16", 1 << 28, 111, "normal", alpha=2.5,
        description="fp16 SAXPY in place y = 2.5*x + y (fp32 fma, RNE to fp16), n=2^28, "
                    "x,y normal(0,1) cast RNE"),
    "saxpy_bf16_2e28": _w(
        "saxpy_bf16_2e28", "saxpy_bf16", 1 << 28, 112, "normal", alpha=2.5,
        description="bf16 SAXPY in place y = 2.5*x + y (fp32 fma, RNE to bf16), n=2^28, "
                    "x,y normal(0,1) cast RNE"),
    "relu_f16_2e28": _w(
        "relu_f16_2e28", "relu_f16", 1 << 28, 113, "normal",
        description="fp16 ReLU y=max(x,0), n=2^28, x normal(0,1) cast RNE"),
    "relu_bf16_2e28": _w(
        "relu_bf16_2e28", "relu_bf16", 1 << 28, 114, "normal",
        description="bf16 ReLU y=max(x,0), n=2^28, x normal(0,1) cast RNE"),
    "transpose_f32_16384x16384": _w(
        "transpose_f32_16384x16384", "copy2d_f32", 1 << 28, 115, "uniform", cols=16384,
        view=(1, 16384, 1 << 28, 0),
        description="fp32 transposed view copied to contiguous: out[r,c] = in[c*16384 + r], "
                    "16384 x 16384 (LDS-tiled path)"),
    "strided_view_f32_2e26_s2": _w(
        "strided_view_f32_2e26_s2", "copy2d_f32", 1 << 26, 116, "uniform", cols=1 << 26,
        view=(0, 2, 1 << 27, 0),
        description="fp32 1-D strided view x[::2] copied to contiguous, 2^26 outputs from a "
                    "2^27-element array"),
    "strided_view_f32_2e24_s3": _w(
        "strided_view_f32_2e24_s3", "copy2d_f32", 1 << 24, 119, "uniform", cols=1 << 24,
        view=(0, 3, 3 << 24, 0),
        description="fp32 1-D strided view x[::3] copied to contiguous, 2^24 outputs from a "
                    "3*2^24-element array"),
    "strided_view_f32_2e24_s8": _w(
        "strided_view_f32_2e24_s8", "copy2d_f32", 1 << 24, 120, "uniform", cols=1 << 24,
        view=(0, 8, 1 << 27, 0),
        description="fp32 1-D strided view x[::8] copied to contiguous, 2^24 outputs from a "
                    "2^27-element array"),
    "submatrix_f32_16384x16000": _w(
        "submatrix_f32_16384x16000", "copy2d_f32", 16384 * 16000, 117, "uniform", cols=16000,
        view=(16384, 1, 16384 * 16384, 3),
        description="fp32 submatrix view (16384 x 16000 out of 16384-wide rows, starting 3 "
                    "elements in) copied to contiguous"),
    "relu_inplace_f32_2e28": _w(
        "relu_inplace_f32_2e28", "relu_inplace_f32", 1 << 28, 106, "normal",
        description="fp32 ReLU in place x=max(x,0), storing only 64-byte spans that change, "
                    "n=2^28, x normal(0,1) (the ReLU workload's input: signs mixed)"),
    "relu_inplace_f32_2e28_nonneg": _w(
        "relu_inplace_f32_2e28_nonneg", "relu_inplace_f32", 1 << 28, 118, "absnormal",
        description="fp32 ReLU in place, n=2^28, x = |normal(0,1)| (every element already "
                    ">= 0: nothing to store)"),
    "scale_f32_2e28": _w(
        "scale_f32_2e28", "scale_f32", 1 << 28, 121, "normal", alpha=2.5,
        description="fp32 scalar-broadcast multiply y = 2.5*x, n=2^28, x normal(0,1)"),
    "add_scalar_bf16_2e28": _w(
        "add_scalar_bf16_2e28", "add_scalar_bf16", 1 << 28, 122, "normal", alpha=2.5,
        description="bf16 scalar-broadcast add y = x + 2.5 (fp32 add, RNE to bf16), n=2^28, "
                    "x normal(0,1) cast RNE"),
    "sqrt_f32_2e28": _w(
        "sqrt_f32_2e28", "sqrt_f32", 1 << 28, 123, "absnormal",
        description="fp32 square root y = sqrt(x), correctly rounded, n=2^28, x = |normal(0,1)|"),
    "sqrt_f16_2e28": _w(
        "sqrt_f16_2e28", "sqrt_f16", 1 << 28, 124, "absnormal",
        description="fp16 square root y = rne16(sqrt(x)), n=2^28, x = |normal(0,1)| cast RNE"),
    "sqrt_bf16_2e28": _w(
        "sqrt_bf16_2e28", "sqrt_bf16", 1 << 28, 128, "absnormal",
        description="bf16 square root y = rnebf(sqrt(x)), n=2^28, x = |normal(0,1)| cast RNE"),
    "abs_f16_2e28": _w(
        "abs_f16_2e28", "abs_f16", 1 << 28, 125, "normal",
        description="fp16 y = |x| (sign bit cleared), n=2^28, x normal(0,1) cast RNE"),
    "batch_add_f32_64x16384": _w(
        "batch_add_f32_64x16384", "add_f32", 1 << 20, 126, "uniform", batch=64,
        description="fp32 C=A+B on 64 arrays of 16384 elements (2^20 in all, the small "
                    "configuration's bytes) in one batched call, A,B uniform[-1,1)"),
    "batch_add_f32_1024x1024": _w(
        "batch_add_f32_1024x1024", "add_f32", 1 << 20, 127, "uniform", batch=1024,
        description="fp32 C=A+B on 1024 arrays of 1024 elements (2^20 in all) in one batched "
                    "call, A,B uniform[-1,1)"),
    "headline_add_f32_2e28": _w(
        "headline_add_f32_2e28", "add_f32", 1 << 28, 100, "uniform",
        description="fp32 C=A+B, n=2^28, all buffers aligned"),
    # the per-output index walk of the fifth configuration's gather: every
    # output element loads its own input element (the input read twice)
    "gather_walk_f32_2e26_s2": _w(
        "gather_walk_f32_2e26_s2", "gather_walk_f32", 1 << 26, 107, "uniform", stride=2,
        description="fp32 strided gather out[i]=in[(2*i) mod n] as a per-output index walk "
                    "(one 4-byte load per output), n=2^26, in uniform[-1,1)"),
    # the one-read-one-write stream at the headline's size: with the pure
    # read stream (relu_inplace_f32_2e28_nonneg) it brackets what a stream
    # mixing reads and writes attains on the part
    "copy_f32_2e28": _w(
        "copy_f32_2e28", "copy_f32", 1 << 28, 129, "uniform",
        description="fp32 contiguous copy out[i]=in[i], n=2^28, in uniform[-1,1)"),
}

# Number of inputs each operation reads, and its element type.
OP_INPUTS = {
    "add_f32": ("a", "b"), "add_f16": ("a", "b"), "add_bf16": ("a", "b"),
    "saxpy_f32": ("x", "y"), "relu_f32": ("x",), "copy_f32": ("x",),
    "gather_f32": ("x",), "gather_walk_f32": ("x",), "add_relu_f32": ("a", "b"),
    "saxpy_relu_f32": ("x", "y"),
    "bias_relu_f32": ("x", "bias"), "saxpy_f16": ("x", "y"), "saxpy_bf16": ("x", "y"),
    "relu_f16": ("x",), "relu_bf16": ("x",), "copy2d_f32": ("base",),
    "relu_inplace_f32": ("x",),
    **{f"{m}_{d}": ("x",) for m in ("scale", "add_scalar", "sqrt", "abs")
       for d in ("f32", "f16", "bf16")},
}
OP_DTYPE = {
    "add_f32": np.float32, "add_f16": np.uint16, "add_bf16": np.uint16,
    "saxpy_f32": np.float32, "relu_f32": np.float32, "copy_f32": np.float32,
    "gather_f32": np.float32, "gather_walk_f32": np.float32, "add_relu_f32": np.float32,
    "saxpy_relu_f32": np.float32,
    "bias_relu_f32": np.float32, "saxpy_f16": np.uint16, "saxpy_bf16": np.uint16,
    "relu_f16": np.uint16, "relu_bf16": np.uint16, "copy2d_f32": np.float32,
    "relu_inplace_f32": np.float32,
    **{f"{m}_{d}": np.float32 if d == "f32" else np.uint16
       for m in ("scale", "add_scalar", "sqrt", "abs") for d in ("f32", "f16", "bf16")},
}
F16_OPS = ("add_f16", "saxpy_f16", "relu_f16", "scale_f16", "add_scalar_f16", "sqrt_f16",
           "abs_f16")
BF16_OPS = ("add_bf16", "saxpy_bf16", "relu_bf16", "scale_bf16", "add_scalar_bf16",
            "sqrt_bf16", "abs_bf16")


def absnormal(g: np.random.Generator, n: int) -> np.ndarray:
    """|normal(0, 1)|: the normal draw with its sign bit cleared (exact)."""
    return np.abs(normal01(g, n))


_DRAW = {"uniform": uniform_pm1, "normal": normal01, "absnormal": absnormal}


def make_inputs(op: str, n: int, seed: int, dist: str = "uniform", cols: int = 0) -> dict:
    """Draw the inputs of ``op`` (numpy arrays keyed by role) for n elements
    (the bias of bias_relu has `cols` elements)."""
    g = rng(seed)
    draw = _DRAW[dist]
    out = {}
    for role in OP_INPUTS[op]:
        x = draw(g, cols if role == "bias" else n)
        if op in F16_OPS:
            x = to_f16_bits(x)
        elif op in BF16_OPS:
            x = to_bf16_bits(x)
        out[role] = x
    return out


def workload_inputs(w: Workload) -> dict:
    if w.op == "copy2d_f32":      # the base array the view looks into
        return {"base": _DRAW[w.dist](rng(w.seed), w.view[2])}
    return make_inputs(w.op, w.n, w.seed, w.dist, w.cols)
