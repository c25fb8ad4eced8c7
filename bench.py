#!/usr/bin/env python3
"""Achieved HBM bandwidth of the elementwise kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-others] [--others LIST] [--no-cpu-baseline] [--no-context]
                    [--details FILE]

A step is one call of the library on the workload (validation, plan, launch
of the vectorised grid-stride kernel with its scalar head and tail).  The
default workload is the headline: fp32 C = A + B on n = 2^28 elements, every
buffer aligned, A and B uniform on [-1, 1) (seed 100).

Procedure: inputs are generated on the host, copied to the GPU once, and a
parity gate compares one launch with the CPU oracle on every element (a
workload that fails reports no speed).  The oracle runs only inside the CPU
leg (``cpu_baseline_leg``), which also times it.  Then W untimed launches, then K
launches bracketed by HIP events recorded on the stream the kernels run on.
GB/s = algorithmic bytes (read + write, 10^9 bytes per GB) / average launch
time ([HyperAI] Stage 3 benchmark script: bytes = 3 * numel * element size
for the add).

Output, on stdout:
* one JSON line per other workload (``--no-others`` skips them), each
  parity-gated; working sets up to 1 GiB (4 x the 256 MB Infinity Cache) are
  timed cold: back to back over R copies of the workload's buffers, used in
  turn, so that at least 1 GiB of other traffic runs between two uses of one
  copy.  Beside it, ``flushed_per_launch`` gives the median of single
  launches each bracketed by its own events after a 1 GiB fill;
* then the final line, a compact record of the main workload (a few KB):
  metric, value, ``roofline`` -- the dominant kernel's achieved GB/s against
  the 8 TB/s HBM peak, its HBM bytes per launch from the committed rocprofv3
  counter summary (``traffic``, when taken on the current kernel sources and
  launch shape), the committed kernel-trace duration (``profiled``, likewise)
  and ``attainable``: what two library kernels measured in the same run move
  at the same size, the pure read stream (in-place ReLU on non-negative data,
  which stores nothing) and the one-read-one-write copy -- and
  ``cpu_baseline``, the CPU oracle timed on the host on a bounded sample.
``--details FILE`` also writes every record in full, one JSON line each.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "achieved HBM GB/s (read+write bytes/time) and % of MI355X peak, N=2^28"
DEFAULT_WORKLOAD = "headline_add_f32_2e28"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_TRACE_JSON = os.path.join(ROOT, "profiles", "kernel_trace.json")
# The two library streams that bracket a mixed read/write stream's attainable
# rate at the headline's size: a pure read stream and a copy.
ATTAINABLE = {"read": "relu_inplace_f32_2e28_nonneg", "copy": "copy_f32_2e28"}
# The fifth configuration's comparison: the coalesced copy, the library's
# gather and the per-output index walk, all at n = 2^26.
STRIDED = {"copy": "cfg5a_copy_f32_2e26", "gather": "cfg5b_gather_f32_2e26_s2",
           "walk": "gather_walk_f32_2e26_s2"}
FINAL_LINE_MAX_BYTES = 4096

# Algorithmic bytes per element: each input element read once, each output
# element written once.  The gather counts logical bytes (read 4 + write 4).
# The fused chains count what they move: add+ReLU and SAXPY+ReLU 12, bias+ReLU
# 8 (x read, y written) plus the bias row once.
BYTES_PER_ELEM = {"add_f32": 12, "add_f16": 6, "add_bf16": 6, "saxpy_f32": 12,
                  "relu_f32": 8, "copy_f32": 8, "gather_f32": 8, "gather_walk_f32": 8,
                  "add_relu_f32": 12,
                  "saxpy_relu_f32": 12, "bias_relu_f32": 8, "saxpy_f16": 6, "saxpy_bf16": 6,
                  "relu_f16": 4, "relu_bf16": 4, "copy2d_f32": 8, "relu_inplace_f32": 8,
                  # scalar-broadcast and unary maps: one input read, one output written
                  **{f"{m}_{d}": 8 if d == "f32" else 4
                     for m in ("scale", "add_scalar", "sqrt", "abs")
                     for d in ("f32", "f16", "bf16")}}
DTYPE = {"add_f32": "f32", "add_f16": "f16", "add_bf16": "bf16", "saxpy_f32": "f32",
         "relu_f32": "f32", "copy_f32": "f32", "gather_f32": "f32", "gather_walk_f32": "f32",
         "add_relu_f32": "f32",
         "saxpy_relu_f32": "f32", "bias_relu_f32": "f32", "saxpy_f16": "f16",
         "saxpy_bf16": "bf16", "relu_f16": "f16", "relu_bf16": "bf16", "copy2d_f32": "f32",
         "relu_inplace_f32": "f32",
         **{f"{m}_{d}": d for m in ("scale", "add_scalar", "sqrt", "abs")
            for d in ("f32", "f16", "bf16")}}
# The unfused sequence each fused chain replaces, timed beside it.
UNFUSED = {"add_relu_f32": ("add_f32", "relu_f32"), "saxpy_relu_f32": ("saxpy_f32", "relu_f32")}
MALL_BYTES = 256 * 2 ** 20
# Working sets up to 4 x the Infinity Cache are timed cold: back to back, a
# 600 MB stream still found part of its data in the cache (the 10^8 + 1 fp16
# add read 86 % of peak that way, 84 % at 2^28).  Larger working sets are
# timed back to back on one set of buffers.
COLD_MAX_BYTES = 4 * MALL_BYTES
# Cold timing rotates over copies of the buffers so that this much other
# traffic separates two uses of one copy (4 x the Infinity Cache).
COLD_GAP_BYTES = 4 * MALL_BYTES


def rotation_sets(bytes_per_launch: int) -> int:
    """Buffer copies for cold back-to-back timing: with R copies used in
    turn, R - 1 launches of other copies (at least COLD_GAP_BYTES of traffic)
    run between two uses of one copy."""
    return max(2, -(-COLD_GAP_BYTES // bytes_per_launch) + 1)


def algorithmic_bytes(op: str, n: int, cols: int = 0, changed: int = 0) -> int:
    """Read + write bytes of one launch.  The in-place ReLU reads every
    element and writes only the `changed` ones ([PerfNotes] 5.2: an element
    already >= 0 needs no store)."""
    if op == "relu_inplace_f32":
        return 4 * n + 4 * changed
    return BYTES_PER_ELEM[op] * n + (4 * cols if op == "bias_relu_f32" else 0)


def relu_store_counts(x, np):
    """(elements the ReLU changes, 64-byte spans holding one) for a float32
    input whose first element starts a span: an element changes when its
    sign bit is set and it is not a NaN."""
    ch = np.signbit(x) & ~np.isnan(x)
    n = x.size
    pad = (-n) % 16
    spans = np.concatenate([ch, np.zeros(pad, bool)]).reshape(-1, 16).any(axis=1)
    return int(np.count_nonzero(ch)), int(np.count_nonzero(spans))


def kernel_source_hash(op: str = "add_f32", batch: bool = False) -> str:
    """Hash of the kernel sources the workload's kernels are built from."""
    from memory_bound_elementwise_amd import sources
    return sources.source_hash(sources.family(op, batch))


# Operator class of each streaming operation, as rocprofv3 prints the kernel
# instance (template arguments demangled).
OP_CLASS = {"add_f32": "OpAddF32", "add_f16": "OpAddF16", "add_bf16": "OpAddBF16",
            "saxpy_f32": "OpSaxpyF32", "relu_f32": "OpReluF32", "copy_f32": "OpCopyF32",
            "add_relu_f32": "OpAddReluF32", "saxpy_relu_f32": "OpSaxpyReluF32",
            "saxpy_f16": "OpSaxpy16<_Float16>", "saxpy_bf16": "OpSaxpy16<__bf16>",
            "relu_f16": "OpRelu16<_Float16>", "relu_bf16": "OpRelu16<__bf16>",
            "abs_f32": "OpAbs<unsigned int>", "abs_f16": "OpAbs<unsigned short>",
            "abs_bf16": "OpAbs<unsigned short>",
            **{f"{m}_f32": f"OpMapF32<ew::{fn}>" for m, fn in
               (("scale", "FnScale"), ("add_scalar", "FnAddScalar"), ("sqrt", "FnSqrt"))},
            **{f"{m}_{d}": f"OpMap16<{h}, ew::{fn}>" for d, h in
               (("f16", "_Float16"), ("bf16", "__bf16")) for m, fn in
               (("scale", "FnScale"), ("add_scalar", "FnAddScalar"))},
            "sqrt_f16": "OpMap16<_Float16, ew::FnSqrtWidenedF16>",
            "sqrt_bf16": "OpMap16<__bf16, ew::FnSqrtWidenedBF16>"}


def _b(v) -> str:
    return "true" if v else "false"


# What each kernel path of ew_plan_t.path does, for the record.
PATH_TEXT = {
    "stream": "streaming kernel",
    "copy": "copy kernel (stride 1 mod n)",
    "gather_walk": "per-output index walk (one 4-byte load per output element), "
                   "{reps} segment(s)",
    "gather_spans": "contiguous 16-byte loads, even elements kept",
    "gather_passes": "{s} run(s) x {reps} segment(s), input spans staged through LDS",
    "gather_tiles": "{s} run(s) x {reps} segment(s), rows of the stride transposed through "
                    "LDS",
    "view_rows": "rows contiguous",
    "view_transpose": "LDS-tiled transpose (128 x 128 tiles, 1024 threads)",
    "view_generic": "generic (one 4-byte load per element)",
}


def kernel_instance(w, launch: dict, split: dict, plan=None, ew=None, prep=None):
    """The kernel instance one launch of the workload runs (the name
    rocprofv3 reports, without 'void ew::' and the argument list), or None
    where the record does not determine it.  plan: the workload's ew_plan_t
    (its path decides the gather's and the views' kernels)."""
    u = launch.get("unroll")
    if w.batch:
        return f"ew_batch_table_kernel<ew::{OP_CLASS[w.op]}, {u}>"
    if w.op in OP_CLASS:
        co = split.get("in_coaligned", [1, 1])
        return f"ew_stream_kernel<ew::{OP_CLASS[w.op]}, {u}, {_b(co[0])}, {_b(co[1])}>"
    if w.op == "relu_inplace_f32":
        return f"ew_relu_inplace_kernel<{u}>"
    if w.op == "bias_relu_f32":
        co = split.get("in_coaligned", [1, 1])[0]
        vec_bias = w.cols % 4 == 0 and split.get("head", 0) == 0
        return f"ew_bias_relu_kernel<{u}, {_b(co)}, {_b(vec_bias)}>"
    if plan is None or ew is None:
        return None
    path = ew.PATHS[plan.path]
    if path == "copy":
        return f"ew_stream_kernel<ew::OpCopyF32, {u}, {_b(split['in_coaligned'][0])}, true>"
    if path == "gather_walk":
        return f"ew_gather_kernel<{u}>"
    if path == "gather_passes":
        # span S = stride mod n, step G = gcd (runs * segments); a view x[::s]: S = G = s
        if w.op == "copy2d_f32":
            return f"ew_gather_passes_kernel<{w.view[1]}, {w.view[1]}>"
        return f"ew_gather_passes_kernel<{plan.passes * plan.reps}, {plan.reps}>"
    if path == "gather_tiles":
        # whole rows below a stride of 68; else 128 x 128 tiles below 1024
        # rows of A, 256 x 64 ones from there on
        s = w.stride % w.n
        mode = (4 if s % 4 == 0 else 1) if s < 68 else 2 if -(-w.n // s) < 1024 else 3
        return f"ew_gather_tiles_kernel<{mode}>"
    if path == "gather_spans":
        # the input's body start co-aligned: in + 8 * head (two inputs per output)
        src = prep.view_src if w.op == "copy2d_f32" else prep.ptrs[1].data_ptr()
        return f"ew_gather2_kernel<{u}, {_b((src + 8 * plan.head) % 16 == 0)}>"
    if path == "view_transpose":
        return "ew_transpose_kernel"
    if path in ("view_rows", "view_generic"):
        return f"ew_copy2d_kernel<{u}, {_b(path == 'view_rows')}>"
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Prepared:
    """Device buffers of one workload and a launcher bound to a stream."""

    def __init__(self, w, torch, np, ew, synth, stream, inp=None):
        from harness import upload
        self.w = w
        self.inp = synth.workload_inputs(w) if inp is None else inp
        self.keep = []
        offs = w.offsets
        s = stream.cuda_stream
        self.stream = s
        self.unfused = None
        self.unfused_label = None   # what `unfused` runs, when not the op's UNFUSED pair
        self.pre = None          # run before every timed launch (in-place ReLU: restore x)
        self.torch_context = None  # (label, launcher) of PyTorch's kernel for the same op
        self.changed = 0
        self.batch_plan = self.host_form = None
        if w.op == "relu_inplace_f32":
            x, kx = upload(self.inp["x"], offs.get("x", 0))
            pristine = x.clone()
            self.keep += [kx, pristine]
            self.launch = lambda: ew.ew_relu_inplace_f32(x, stream=s)
            # the same in-place ReLU storing every element, for comparison
            self.unfused = lambda: ew.ew_relu_f32(x, x, stream=s)
            self.changed, self.spans_changed = relu_store_counts(self.inp["x"], np)
            # restore x before every timed launch -- unless no element
            # changes, when every launch does the same work on the same data
            self.pre = (lambda: x.copy_(pristine)) if self.changed else None
            self.out, self.ptrs = x, (x, x, None)
        elif w.op == "copy2d_f32":
            sr, sc, _, offset = w.view
            base, kb = upload(self.inp["base"], 0)
            out, ko = upload(np.zeros(w.n, np.float32), 0)
            self.keep += [kb, ko]
            rows = w.n // w.cols
            src = base.data_ptr() + 4 * offset
            self.launch = lambda: ew.ew_copy2d_f32(src, sr, sc, out, rows, w.cols, stream=s)
            self.view_src = src
            self.out, self.ptrs = out, (out, base, None)
        elif w.op == "bias_relu_f32":
            x, kx = upload(self.inp["x"], offs.get("x", 0))
            bias, kb = upload(self.inp["bias"], 0)
            y, ky = upload(np.zeros(w.n, np.float32), offs.get("y", 0))
            self.keep += [kx, kb, ky]
            rows = w.n // w.cols
            self.launch = lambda: ew.ew_bias_relu_f32(x, bias, y, rows, w.cols, stream=s)
            self.out, self.ptrs = y, (y, x, None)
        elif w.batch:
            # consecutive equal items of three arrays: the batched call's result
            # over all items is the single operation's result over the arrays
            a, ka = upload(self.inp["a"], offs.get("a", 0))
            b, kb = upload(self.inp["b"], offs.get("b", 0))
            c, kc = upload(np.zeros(w.n, self.inp["a"].dtype), offs.get("c", 0))
            self.keep += [ka, kb, kc]
            m = w.n // w.batch
            parts = [(c[k * m:(k + 1) * m], a[k * m:(k + 1) * m], b[k * m:(k + 1) * m])
                     for k in range(w.batch)]
            # the device item table: one launch for all items
            batch = ew.EwBatch(w.op, [(o, x, y, m) for o, x, y in parts])
            self.batch_plan = batch.plan
            self.launch = lambda: batch(stream=s)
            # the host-array form: one launch per BATCH_MAX items
            host_form = ew.EwBatch(w.op, [(o, x, y, m) for o, x, y in parts], table=False)
            self.host_form = lambda: host_form(stream=s)
            fn = getattr(ew, "ew_" + w.op)

            def separate():
                for o, x, y in parts:
                    fn(x, y, o, stream=s)
            self.unfused = separate
            self.unfused_label = [f"{w.batch} x ew_{w.op}, one launch each"]
            la, lb, lc = ([p[i] for p in parts] for i in (1, 2, 0))

            def t_foreach():
                with torch.cuda.stream(stream):
                    torch._foreach_add(la, lb)
            self.torch_context = ("torch._foreach_add(a_list, b_list) (allocates its outputs)",
                                  t_foreach)
            self.out, self.ptrs = c, (c, a, b)
        elif w.op in ("add_f32", "add_f16", "add_bf16", "add_relu_f32"):
            a, ka = upload(self.inp["a"], offs.get("a", 0))
            b, kb = upload(self.inp["b"], offs.get("b", 0))
            c, kc = upload(np.zeros(w.n, self.inp["a"].dtype), offs.get("c", 0))
            self.keep += [ka, kb, kc]
            fn = getattr(ew, "ew_" + w.op)
            self.launch = lambda: fn(a, b, c, stream=s)
            self.out, self.ptrs = c, (c, a, b)
            tdt = {"add_f32": torch.float32, "add_f16": torch.float16,
                   "add_bf16": torch.bfloat16}.get(w.op)
            if tdt is not None:
                ta, tb, tc = (t.view(tdt) for t in (a, b, c))

                def t_add():
                    with torch.cuda.stream(stream):
                        torch.add(ta, tb, out=tc)
                self.torch_context = ("torch.add(a, b, out=c)", t_add)
            if w.op == "add_relu_f32":
                def unfused():
                    ew.ew_add_f32(a, b, c, stream=s)
                    ew.ew_relu_f32(c, c, stream=s)
                self.unfused = unfused
        elif w.op in ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16"):
            x, kx = upload(self.inp["x"], offs.get("x", 0))
            y, ky = upload(self.inp["y"], offs.get("y", 0))
            self.keep += [kx, ky]
            fn = getattr(ew, "ew_" + w.op)
            self.launch = lambda: fn(w.alpha, x, y, stream=s)
            self.out, self.ptrs = y, (y, x, y)
            if w.op == "saxpy_f32":
                def t_saxpy():
                    with torch.cuda.stream(stream):
                        y.add_(x, alpha=w.alpha)
                self.torch_context = ("y.add_(x, alpha=2.5)", t_saxpy)
            if w.op == "saxpy_relu_f32":
                def unfused():
                    ew.ew_saxpy_f32(w.alpha, x, y, stream=s)
                    ew.ew_relu_f32(y, y, stream=s)
                self.unfused = unfused
        else:
            x, kx = upload(self.inp["x"], offs.get("x", 0))
            y, ky = upload(np.zeros(w.n, self.inp["x"].dtype), offs.get("y", 0))
            self.keep += [kx, ky]
            if w.op in ("relu_f32", "relu_f16", "relu_bf16"):
                fn = getattr(ew, "ew_" + w.op)
                self.launch = lambda: fn(x, y, stream=s)
                if w.op == "relu_f32":
                    def t_relu():
                        with torch.cuda.stream(stream):
                            torch.relu(x)
                    self.torch_context = ("torch.relu(x)", t_relu)
            elif w.op == "copy_f32":
                self.launch = lambda: ew.ew_copy_f32(x, y, stream=s)

                def t_copy():
                    with torch.cuda.stream(stream):
                        y.copy_(x)
                self.torch_context = ("y.copy_(x)", t_copy)
            elif w.op.rsplit("_", 1)[0] in ew.SCALAR_MAPS + ew.UNARY_MAPS:
                self._map(w, torch, ew, x, y, stream)
            elif w.op == "gather_walk_f32":
                self.launch = lambda: ew.ew_gather_walk_f32(x, y, w.stride, stream=s)
            else:
                self.launch = lambda: ew.ew_gather_f32(x, y, w.stride, stream=s)
            self.out, self.ptrs = y, (y, x, None)

    def _map(self, w, torch, ew, x, y, stream):
        """Launcher of a scalar-broadcast or unary map, and PyTorch's kernel for
        the same map on the same buffers (viewed in the op's dtype)."""
        s = stream.cuda_stream
        kind, dt = w.op.rsplit("_", 1)
        fn = getattr(ew, "ew_" + w.op)
        if kind in ew.SCALAR_MAPS:
            self.launch = lambda: fn(w.alpha, x, y, stream=s)
        else:
            self.launch = lambda: fn(x, y, stream=s)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
        tx, ty = x.view(tdt), y.view(tdt)
        label, tfn = {
            "scale": ("torch.mul(x, alpha, out=y)", lambda: torch.mul(tx, w.alpha, out=ty)),
            "add_scalar": ("torch.add(x, alpha, out=y)", lambda: torch.add(tx, w.alpha, out=ty)),
            "sqrt": ("torch.sqrt(x, out=y)", lambda: torch.sqrt(tx, out=ty)),
            "abs": ("torch.abs(x, out=y)", lambda: torch.abs(tx, out=ty)),
        }[kind]

        def t_map():
            with torch.cuda.stream(stream):
                tfn()
        self.torch_context = (label, t_map)

    def plan(self, ew, cus):
        out, in0, in1 = self.ptrs
        if self.w.op == "gather_f32":
            return ew.ew_make_gather_plan(out.data_ptr(), in0.data_ptr(), self.w.n,
                                          self.w.stride, cus)
        if self.w.op == "copy2d_f32":
            sr, sc = self.w.view[0], self.w.view[1]
            return ew.ew_make_copy2d_plan(self.view_src, sr, sc, out.data_ptr(),
                                          self.w.n // self.w.cols, self.w.cols, cus)
        return ew.ew_make_plan(self.w.op, out.data_ptr(), in0.data_ptr(),
                               in1.data_ptr() if in1 is not None else 0, self.w.n, cus)

    def result(self, torch):
        """One launch on fresh buffers; returns the output copied to the host."""
        from harness import ELEM, download
        self.launch()
        torch.cuda.synchronize()
        return download(self.out, ELEM[self.w.op])


LAST_DIST = {}     # p10 / p90 of the last per-launch (flushed) timing, in ms


def time_launches(torch, launch, stream, steps, warmup, flush=None, pre=None):
    """Average launch time in ms.  Without flush: `steps` back-to-back
    launches between two events on `stream`.  With flush: each launch is
    bracketed by its own events after a cache-flush write (and after pre(),
    which restores an in-place input), median."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            if pre is not None:
                pre()
            launch()
    torch.cuda.synchronize()
    if flush is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    evs = []
    with torch.cuda.stream(stream):
        for _ in range(steps):
            if pre is not None:
                pre()
            flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            evs.append((a, b))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    LAST_DIST["p10"] = ts[len(ts) // 10]
    LAST_DIST["p90"] = ts[(9 * len(ts)) // 10]
    return ts[len(ts) // 2]


def time_rotated(torch, launches, stream, steps, warmup):
    """Mean time per launch in ms of `steps` back-to-back launches between
    two events on `stream`, launch i calling launches[i mod R]: each copy's
    data has left the caches by the time it is used again, and no per-launch
    event or flush sits between the launches."""
    r = len(launches)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 2 * r)):
            launches[i % r]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        launches[i % r]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


GRAPH_LAUNCHES = 100
GRAPH_MAX_N = 1 << 22


def time_graph(torch, launch, stream, steps):
    """Mean time per launch, in ms, of GRAPH_LAUNCHES launches captured into
    one HIP graph and replayed back to back on `stream` (the launch-bound
    regime of small arrays: the graph removes the per-call host work and most
    of the gap between dependent launches)."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(GRAPH_LAUNCHES):
            launch()
    replays = max(1, steps // GRAPH_LAUNCHES) * 4
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * GRAPH_LAUNCHES)
    del g
    return ms


def cpu_baseline_leg(w, inp, got, target_s):
    """The CPU leg: the only place bench.py runs the oracle.

    1. One oracle pass over the whole workload; its output is the reference
       for the parity gate (every element of the GPU result `got`).
    2. The oracle timed as it stands (scalar C loop, one thread) on a bounded
       sample: the first m elements of the same inputs, repeated until about
       target_s seconds (target_s <= 0: the full pass of step 1 is the sample).
    Returns (number of mismatching elements, cpu_baseline record)."""
    import oracle
    import synth
    from harness import mismatches

    def run(d):
        if w.op in ("add_f32", "add_f16", "add_bf16", "add_relu_f32"):
            return getattr(oracle, w.op)(d["a"], d["b"])
        if w.op in ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16"):
            return getattr(oracle, w.op)(w.alpha, d["x"], d["y"])
        if w.op == "bias_relu_f32":
            return oracle.bias_relu_f32(d["x"], d["bias"], d["x"].size // w.cols, w.cols)
        if w.op == "copy2d_f32":       # always the full view (see below)
            sr, sc, _, offset = w.view
            return oracle.copy2d_f32(d["base"], offset, sr, sc, w.n // w.cols, w.cols)
        if w.op in ("gather_f32", "gather_walk_f32"):    # one definition, two kernels
            return oracle.gather_f32(d["x"], w.stride)
        if w.op == "relu_inplace_f32":     # same result as the out-of-place ReLU
            return oracle.relu_f32(d["x"])
        if w.op.rsplit("_", 1)[0] in ("scale", "add_scalar"):
            return getattr(oracle, w.op)(w.alpha, d["x"])
        return getattr(oracle, w.op)(d["x"])

    def changed(d):
        if w.op != "relu_inplace_f32":
            return 0
        import numpy as np
        return relu_store_counts(d["x"], np)[0]

    t0 = time.perf_counter()
    ref = run(inp)
    full_s = time.perf_counter() - t0
    bad = int(mismatches(w.op, got, ref).size)
    del ref
    if target_s <= 0 or w.op == "copy2d_f32":
        gbs = algorithmic_bytes(w.op, w.n, w.cols if w.op == "bias_relu_f32" else 0,
                                changed(inp)) / full_s / 1e9
        sample = f"one full pass over all {w.n} elements ({full_s:.2f} s)"
    else:
        m = min(w.n, 1 << 26)
        small = synth.make_inputs(w.op, m, w.seed, w.dist, w.cols)
        run(small)                                   # warm-up, first touch
        reps, t0 = 0, time.perf_counter()
        while True:
            run(small)
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s or reps >= 1000:
                break
        gbs = algorithmic_bytes(w.op, m, 0, changed(small)) / (el / reps) / 1e9
        sample = (f"{w.op} on the first {m} elements of the workload's inputs, {reps} passes "
                  f"in {el:.1f} s")
    rec = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": sample + " (scalar C loop, one thread)", "cpu": _cpu_model()}
    if target_s > 0 and w.op not in ("copy2d_f32", "gather_f32", "gather_walk_f32"):
        rec["all_cores"] = _all_cores(w, run, changed, small, m, target_s / 2)
    return bad, rec


def _all_cores(w, run, changed, small, m, target_s):
    """The same oracle loop, unchanged, on static contiguous chunks of the
    sample, one chunk per core of this process's affinity set, run from a
    thread pool (the C call releases the GIL).  Context for the one-thread
    figure; the outputs are discarded."""
    from concurrent.futures import ThreadPoolExecutor
    cores = len(os.sched_getaffinity(0))
    unit = w.cols if w.op == "bias_relu_f32" else 16
    step = -(-m // cores)
    step = -(-step // unit) * unit
    parts = []
    for lo in range(0, m, step):
        hi = min(m, lo + step)
        parts.append({k: (v if k == "bias" else v[lo:hi]) for k, v in small.items()})
    with ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(run, parts))                       # warm-up, first touch
        reps, t0 = 0, time.perf_counter()
        while True:
            list(ex.map(run, parts))
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s or reps >= 1000:
                break
    gbs = algorithmic_bytes(w.op, m, 0, changed(small)) / (el / reps) / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": len(parts),
            "sample": f"the same {m} elements in {len(parts)} contiguous chunks, one thread "
                      f"each, {reps} passes in {el:.1f} s"}


def _clocks(props):
    """Current clocks of the device torch uses, read from the amdgpu driver's
    DPM tables in sysfs (the level marked "*"), or None if they are not
    readable.  Plain file reads: no child process is started from this
    GPU-initialised process."""
    try:
        addr = "%04x:%02x:%02x.0" % (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
    except (AttributeError, TypeError):
        return None
    base = os.path.join("/sys/bus/pci/devices", addr)
    out = {}
    for name in ("sclk", "mclk", "fclk", "socclk"):
        try:
            with open(os.path.join(base, "pp_dpm_" + name)) as f:
                for line in f:
                    line = line.strip()
                    if line.endswith("*") and ":" in line:
                        out[name] = line.split(":", 1)[1].rstrip("*").strip()
        except OSError:
            continue
    return out or None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _committed(path, workload, src_hash, launch_desc):
    """The record of `workload` in a committed profile index, if it was taken
    on the given kernel source hash and launch shape; else None."""
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get("workloads", {}).get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != src_hash:
        return None
    if rec.get("launch") != launch_desc:
        return None
    return rec


def traffic_for(workload: str, launch_desc: dict, src_hash: str = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources and launch shape; else None."""
    rec = _committed(TRAFFIC_JSON, workload, src_hash or kernel_source_hash(), launch_desc)
    return rec.get("hbm_bytes_per_launch") if rec else None


def profiled_for(workload: str, launch_desc: dict, src_hash: str = None):
    """The committed rocprofv3 kernel-trace record of the workload's kernel
    (average and median duration per dispatch), if it was taken on the current
    kernel sources and launch shape; else None."""
    return _committed(KERNEL_TRACE_JSON, workload, src_hash or kernel_source_hash(),
                      launch_desc)


def measure(w, torch, np, ew, synth, stream, steps, warmup, cus, flush_buf, cpu_target_s,
            check=True, context=True):
    """Parity gate, then the timing of the workload's launch; with context,
    also the comparisons beside it (per-launch flushed timing, warm timing,
    PyTorch's kernel, graph replay, unfused or separate calls)."""
    prep = Prepared(w, torch, np, ew, synth, stream)
    plan = prep.plan(ew, cus)
    launch_desc = {"block": plan.block, "grid": plan.grid, "unroll": plan.unroll}
    if w.batch:
        # one launch for the whole call: the table's row for the total n
        bp = prep.batch_plan
        launch_desc = {"block": bp.block, "grid": min(bp.blocks_per_cu * cus, bp.tiles),
                       "unroll": bp.unroll, "items": bp.items, "tiles": bp.tiles,
                       "table_bytes": bp.bytes, "launches": 1,
                       "path": "batched: device item table, one kernel for every item"}
        steps = min(steps, 200)
    if not w.batch and w.op in ("gather_f32", "gather_walk_f32", "copy2d_f32"):
        launch_desc["path"] = PATH_TEXT[ew.PATHS[plan.path]].format(s=plan.passes,
                                                                   reps=plan.reps)
    res = {"workload": w.name, "op": w.op, "n": w.n, "launch": launch_desc,
           "split": {"head": plan.head, "vectors": plan.vectors, "tail": plan.tail,
                     "in_coaligned": list(plan.in_coaligned)}}
    res["kernel"] = kernel_instance(w, launch_desc, res["split"], plan, ew, prep)
    res["source_sha256_16"] = kernel_source_hash(w.op, bool(w.batch))
    if w.batch:
        res["split"] = {"items": w.batch, "elements_per_item": w.n // w.batch,
                        "note": "consecutive slices of three arrays, every item 16-byte aligned"}
    got = prep.result(torch)
    if check:
        bad, cpu = cpu_baseline_leg(w, prep.inp, got, cpu_target_s)
        res.update({"parity": "PASS" if bad == 0 else "FAIL", "mismatches": bad,
                    "cpu_baseline": cpu})
    else:
        bad = 0
        res["parity"] = "not checked (--no-cpu-baseline)"
    del got
    if bad:
        return res, prep, None
    if prep.changed:
        res["changed"] = prep.changed
    nbytes = algorithmic_bytes(w.op, w.n, w.cols if w.op == "bias_relu_f32" else 0,
                               prep.changed)
    footprint = nbytes if w.op != "gather_f32" else 8 * w.n
    # an in-place input must be restored before every launch, so it is
    # always timed launch by launch, restore and flush outside the events
    cold = footprint <= COLD_MAX_BYTES or prep.pre is not None
    flush = (lambda: flush_buf.fill_(1)) if cold else None
    sets = [prep]
    if cold and prep.pre is None:
        # cold, back to back: R copies of the buffers (same inputs, same
        # offsets, so the same plan) used in turn
        sets += [Prepared(w, torch, np, ew, synth, stream, inp=prep.inp)
                 for _ in range(rotation_sets(footprint) - 1)]
        ms = time_rotated(torch, [p.launch for p in sets], stream, steps, warmup)
        timing = (f"cold: back to back over {len(sets)} copies of the buffers used in turn "
                  f"(>= 1 GiB of other traffic between two uses of one copy), mean")
    if cold and prep.pre is None and context:
        fl_ms = time_launches(torch, prep.launch, stream, steps, warmup, flush=flush)
        res["flushed_per_launch"] = {
            "ms": round(fl_ms, 5), "gbs": round(nbytes / (fl_ms / 1e3) / 1e9, 1),
            "p10_ms": round(LAST_DIST["p10"], 5), "p90_ms": round(LAST_DIST["p90"], 5),
            "timing": "each launch between its own events after a 1 GiB fill, median "
                      "(includes the per-launch event gap and the fill's write-back)"}
    elif not (cold and prep.pre is None):
        ms = time_launches(torch, prep.launch, stream, steps, warmup, flush=flush, pre=prep.pre)
        timing = ("cold (1 GiB flush before each launch), median" if cold else
                  "back-to-back, mean")
        if cold:
            res["p10_ms"], res["p90_ms"] = round(LAST_DIST["p10"], 5), round(LAST_DIST["p90"], 5)
    gbs = nbytes / (ms / 1e3) / 1e9
    res.update({"ms": round(ms, 5), "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_GBS, 4),
                "timing": timing, "algorithmic_bytes": nbytes})
    traffic = traffic_for(w.name, launch_desc, res["source_sha256_16"])
    if traffic is not None:
        res["traffic_bytes"] = traffic
        res["traffic_ratio"] = round(traffic / nbytes, 4)
    if not context:
        res["context"] = "skipped (--no-context)"
        del sets[1:]
        return res, prep, ms
    ctx = prep.torch_context
    if ctx is not None:
        if len(sets) > 1:
            t_ms = time_rotated(torch, [p.torch_context[1] for p in sets], stream, steps, warmup)
        else:
            t_ms = time_launches(torch, ctx[1], stream, steps, warmup, flush=flush)
        res["torch_context"] = {"op": ctx[0], "ms": round(t_ms, 5),
                                "gbs": round(nbytes / (t_ms / 1e3) / 1e9, 1),
                                "note": "PyTorch's own kernel on the same buffers, same timing; "
                                        "context, not a target"}
    if cold and prep.pre is None:
        warm_ms = time_launches(torch, prep.launch, stream, steps, 2)
        res["warm_gbs"] = round(nbytes / (warm_ms / 1e3) / 1e9, 1)
    if w.n <= GRAPH_MAX_N and prep.pre is None:
        eager_ms = warm_ms if cold else ms
        g_ms = time_graph(torch, prep.launch, stream, steps)
        res["graph"] = {"launches_per_graph": GRAPH_LAUNCHES, "us_per_launch": round(g_ms * 1e3, 3),
                        "gbs": round(nbytes / (g_ms / 1e3) / 1e9, 1),
                        "eager_us_per_launch": round(eager_ms * 1e3, 3),
                        "timing": "warm: back-to-back replays of one captured graph"}
    if w.op == "relu_inplace_f32":
        all_ms = time_launches(torch, prep.unfused, stream, steps, warmup, flush=flush,
                               pre=prep.pre)
        n_spans = -(-w.n // 16)
        span_bytes = 4 * w.n + 64 * prep.spans_changed
        res["stores"] = {"elements_changed": prep.changed,
                         "spans_64B_changed_frac": round(prep.spans_changed / n_spans, 4),
                         "span_bytes_per_launch": span_bytes,
                         "span_gbs": round(span_bytes / (ms / 1e3) / 1e9, 1)}
        res["vs_storing_every_element"] = {"op": "ew_relu_f32(x, x)", "ms": round(all_ms, 5),
                                           "speedup": round(all_ms / ms, 3)}
    elif prep.unfused is not None:
        if len(sets) > 1:
            un_ms = time_rotated(torch, [p.unfused for p in sets], stream, steps, warmup)
        else:
            un_ms = time_launches(torch, prep.unfused, stream, steps, warmup, flush=flush)
        if prep.unfused_label is not None:
            res["separate_calls"] = {"ops": prep.unfused_label, "ms": round(un_ms, 5),
                                     "gbs": round(nbytes / (un_ms / 1e3) / 1e9, 1),
                                     "speedup_of_batch": round(un_ms / ms, 3)}
            if prep.host_form is not None:
                hf_ms = (time_rotated(torch, [p.host_form for p in sets], stream, steps, warmup)
                         if len(sets) > 1 else
                         time_launches(torch, prep.host_form, stream, steps, warmup, flush=flush))
                res["host_array_form"] = {
                    "op": f"ew_batch: the item array in the kernel arguments, "
                          f"{-(-w.batch // ew.BATCH_MAX)} launches", "ms": round(hf_ms, 5),
                    "gbs": round(nbytes / (hf_ms / 1e3) / 1e9, 1),
                    "speedup_of_table": round(hf_ms / ms, 3)}
        else:
            res["unfused"] = {"ops": list(UNFUSED[w.op]), "ms": round(un_ms, 5),
                              "speedup_of_fused": round(un_ms / ms, 3)}
    del sets[1:]
    return res, prep, ms


# The roofline curve: each op of the five configurations, its config's input
# distribution, N = 2^20 .. 2^28 and one odd N per decade; seed 200 + log2 N
# (300 + floor(log2 N) for the odd sizes).
SWEEP_OPS = (("add_f32", "uniform"), ("add_f16", "uniform"), ("add_bf16", "uniform"),
             ("saxpy_f32", "normal"), ("relu_f32", "normal"), ("copy_f32", "uniform"),
             ("gather_f32", "uniform"))
SWEEP_SIZES = [1 << k for k in range(20, 29)] + [10 ** 6 + 1, 10 ** 7 + 1, 10 ** 8 + 1]


def run_sweep(torch, np, ew, synth, stream, cus, flush_buf, out_path=None):
    """One JSON line per (op, N): parity against the oracle on every element
    (the CPU leg, one full pass), then the timing of measure().  With
    out_path, each record is also appended to that JSONL file as soon as it
    is measured, and points already recorded there with parity PASS are
    skipped (an interrupted sweep resumes where it stopped)."""
    import math
    rc = 0
    done = set()
    if out_path and os.path.exists(out_path):
        with open(out_path) as f:
            for line in f:
                try:
                    r = json.loads(line)
                except ValueError:
                    continue
                if r.get("parity") == "PASS":
                    done.add((r["op"], r["n"]))
    for op, dist in SWEEP_OPS:
        for n in sorted(SWEEP_SIZES):
            if (op, n) in done:
                log(f"sweep {op} n={n}: already recorded")
                continue
            lg = math.floor(math.log2(n))
            seed = 200 + lg if n == 1 << lg else 300 + lg
            w = synth.Workload(f"sweep_{op}_{n}", op, n, seed, dist,
                               alpha=2.5 if op == "saxpy_f32" else 0.0,
                               stride=2 if op == "gather_f32" else 0,
                               description=f"{op}, n={n}, {dist}, seed {seed}")
            log(f"sweep {op} n={n}")
            steps = 200 if n >= (1 << 25) else 1000
            res, prep, _ = measure(w, torch, np, ew, synth, stream, steps, 10, cus, flush_buf,
                                   0.0)
            del prep
            torch.cuda.empty_cache()
            res.pop("cpu_baseline", None)
            res.pop("split", None)
            print(json.dumps(res), flush=True)
            if out_path:
                with open(out_path, "a") as f:
                    f.write(json.dumps(res) + "\n")
            if res["parity"] != "PASS":
                rc = 1
    return rc


# The stride curve: the gather and the per-output walk at n = 2^26 (the fifth
# configuration's size and input) for every stride 1..32 and a few beyond.
STRIDE_SWEEP = list(range(1, 33)) + [33, 48, 63, 64, 100, 127, 128, 129, 255, 257, 1000, 1024,
                                      4097, 65537, (1 << 19) + 1, (1 << 26) - 1]


def run_stride_sweep(torch, np, ew, synth, stream, cus, flush_buf, out_path=None):
    """One JSON line per (op, stride): parity against the oracle on every
    element, then the timing of measure(); resumable like run_sweep."""
    rc = 0
    done = set()
    if out_path and os.path.exists(out_path):
        with open(out_path) as f:
            for line in f:
                try:
                    r = json.loads(line)
                except ValueError:
                    continue
                if r.get("parity") == "PASS":
                    done.add((r["op"], r["stride"]))
    n = 1 << 26
    for op in ("gather_f32", "gather_walk_f32"):
        for stride in STRIDE_SWEEP:
            if (op, stride) in done:
                log(f"stride sweep {op} s={stride}: already recorded")
                continue
            w = synth.Workload(f"stride_{op}_{stride}", op, n, 107, "uniform", stride=stride,
                               description=f"{op}, n=2^26, stride {stride}, seed 107")
            log(f"stride sweep {op} s={stride}")
            res, prep, _ = measure(w, torch, np, ew, synth, stream, 100, 5, cus, flush_buf, 0.0,
                                   context=False)
            del prep
            torch.cuda.empty_cache()
            res.pop("cpu_baseline", None)
            res.pop("split", None)
            res["stride"] = stride
            print(json.dumps(res), flush=True)
            if out_path:
                with open(out_path, "a") as f:
                    f.write(json.dumps(res) + "\n")
            if res["parity"] != "PASS":
                rc = 1
    return rc


def _ratio(a, b):
    return round(a / b, 4) if a and b else None


def attainable(by: dict, value):
    """The pure read stream and the copy, measured in this run at the
    headline's size: what the part attains for the two ends of a streaming
    mix (no write; one write per read) -- the ceiling a two-read-one-write
    stream is judged against.  None without those records."""
    rd, cp = by.get(ATTAINABLE["read"]), by.get(ATTAINABLE["copy"])
    if not (rd and cp and rd.get("gbs") and cp.get("gbs")):
        return None
    return {"read_stream_gbs": rd["gbs"], "copy_gbs": cp["gbs"],
            "value_over_copy": _ratio(value, cp["gbs"]),
            "value_over_read_stream": _ratio(value, rd["gbs"]),
            "read_stream": f"{rd['workload']} ({rd.get('kernel')}, stores nothing)",
            "copy": f"{cp['workload']} ({cp.get('kernel')})"}


def strided_over_coalesced(by: dict):
    """[PerfNotes] 3.2-3.3's experiment at n = 2^26: the strided gather
    out[i] = in[(2i) mod n] against the coalesced copy, for the per-output
    index walk (the page's kernel) and the library's gather."""
    cp = by.get(STRIDED["copy"])
    if not (cp and cp.get("gbs")):
        return None
    out = {"copy_gbs": cp["gbs"]}
    for key in ("walk", "gather"):
        r = by.get(STRIDED[key])
        if r and r.get("gbs"):
            out[key] = {"gbs": r["gbs"], "over_copy": _ratio(r["gbs"], cp["gbs"]),
                        "traffic_ratio": r.get("traffic_ratio"), "kernel": r.get("kernel")}
    out["bytes"] = "logical: 8 per output element for all three"
    return out


def final_line(args, w, res, others, env):
    """The last stdout line: the main workload's record, compact (the
    other workloads are printed before it, one line each)."""
    gbs = res.get("gbs")
    line = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.get("ms"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[w.op], "data": f"synthetic (seeded {w.dist}, seed {w.seed})",
        "config": {"workload": w.description, "name": w.name, "op": w.op, "n": w.n,
                   "launch": res["launch"], "global_batch": w.n, "parallelism": "single GPU"},
        "parity": res["parity"], "mismatches": res.get("mismatches"),
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2) if gbs else None,
        "timing": res.get("timing"),
    }
    if gbs:
        alg = res["algorithmic_bytes"]
        prof = profiled_for(w.name, res["launch"], res["source_sha256_16"])
        by = {r["workload"]: r for r in others}
        line["roofline"] = {
            "bound": "hbm", "achieved": gbs, "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_GBS, 4), "traffic": res.get("traffic_bytes"),
            "traffic_ratio": res.get("traffic_ratio"), "kernel": res.get("kernel"),
            "algorithmic_bytes_per_launch": alg,
            "avg_launch_us": round(res["ms"] * 1e3, 3),
            "profiled": ({"avg_us": round(prof["avg_ns"] / 1e3, 3),
                          "median_us": round(prof["median_ns"] / 1e3, 3),
                          "gbs_at_avg": round(alg / prof["avg_ns"], 1),
                          "frac_at_avg": round(alg / prof["avg_ns"] / PEAK_GBS, 4),
                          "summary": "profiles/" + prof["summary"]} if prof else None),
            "attainable": attainable(by, gbs),
        }
        so = strided_over_coalesced(by)
        if so:
            line["strided_over_coalesced"] = so
    if "cpu_baseline" in res:
        cb = dict(res["cpu_baseline"])
        allc = cb.pop("all_cores", None)
        line["cpu_baseline"] = cb
        if allc:
            line["cpu_baseline_all_cores"] = {"value": allc["value"], "unit": allc["unit"],
                                              "cores": allc["cores"]}
    if "torch_context" in res:
        line["torch_context_gbs"] = res["torch_context"]["gbs"]
    if "graph" in res:        # small workloads: launches replayed from a captured graph
        line["graph_gbs"] = res["graph"]["gbs"]
    if others:
        line["others"] = {"workloads": len(others),
                          "parity_pass": sum(r.get("parity") == "PASS" for r in others),
                          "not_passing": [r["workload"] for r in others
                                          if r.get("parity") not in ("PASS", None)
                                          and not r.get("parity", "").startswith("not checked")],
                          "where": "the JSON lines above this one"}
    line["env"] = env
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-others", action="store_true", help="skip the other configurations")
    ap.add_argument("--others", help="comma-separated: run only these other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="time only the workload's own launch: no flushed, warm, PyTorch, "
                         "graph, unfused or separate-call figures (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--details", help="also write every record in full to this file, one JSON "
                                      "line each (the main workload's last)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: each op of the five configurations over "
                         "N = 2^20 .. 2^28 plus odd N, one parity-gated JSON line per point")
    ap.add_argument("--stride-sweep", action="store_true",
                    help="instead of the bench line: the gather and the per-output walk at "
                         "n = 2^26 for strides 1..32 and a few beyond, one parity-gated JSON "
                         "line per point")
    ap.add_argument("--sweep-out", help="with --sweep or --stride-sweep: append each point to this JSONL file "
                                        "and skip points it already holds with parity PASS")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs each operation on one GPU; runs on more than one "
              "GPU are not part of it (--gpus must be 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import memory_bound_elementwise_amd as ew
    from memory_bound_elementwise_amd import sources
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev_props = torch.cuda.get_device_properties(0)
    cus = dev_props.multi_processor_count
    stream = torch.cuda.Stream()          # default priority
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB

    if args.sweep:
        return run_sweep(torch, np, ew, synth, stream, cus, flush_buf, args.sweep_out)
    if args.stride_sweep:
        return run_stride_sweep(torch, np, ew, synth, stream, cus, flush_buf, args.sweep_out)

    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.description}")
    input_sha = {k: synth.sha256(v)[:16] for k, v in synth.workload_inputs(w).items()}
    res, prep, ms = measure(w, torch, np, ew, synth, stream, args.steps, args.warmup, cus,
                            flush_buf, args.cpu_seconds, check=not args.no_cpu_baseline,
                            context=not args.no_context)
    log(f"parity {res['parity']}; {res.get('gbs')} GB/s")
    del prep
    torch.cuda.empty_cache()
    details = open(args.details, "w") if args.details else None

    others = []
    only = set(args.others.split(",")) if args.others else None
    if only and not only <= set(synth.WORKLOADS):
        print(f"bench.py: unknown workloads {sorted(only - set(synth.WORKLOADS))}",
              file=sys.stderr)
        return 2
    if not args.no_others:
        for name, ow in synth.WORKLOADS.items():
            if name == w.name or (only and name not in only):
                continue
            log(f"other config {name}")
            steps = 200 if ow.n >= (1 << 25) else 1000
            try:
                r, p, _ = measure(ow, torch, np, ew, synth, stream, steps, 10, cus, flush_buf,
                                  0.0, check=not args.no_cpu_baseline,
                                  context=not args.no_context)
                del p
            except Exception as exc:
                # recorded, and nothing more is launched (the error may have left the
                # device unusable); the final line below still prints
                r = {"workload": name, "op": ow.op, "n": ow.n,
                     "error": f"{type(exc).__name__}: {exc}"}
                others.append(r)
                print(json.dumps(r), flush=True)
                log(f"other config {name} failed, remaining configs skipped: {exc}")
                break
            others.append(r)
            print(json.dumps(r), flush=True)
            if details:
                details.write(json.dumps(r) + "\n")
            torch.cuda.empty_cache()

    env = {"device": torch.cuda.get_device_name(0),
           "arch": getattr(dev_props, "gcnArchName", None), "cus": cus,
           "clocks": _clocks(dev_props), "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None), "numpy": np.__version__,
           "kernel_source_sha256_16": res["source_sha256_16"],
           "sources_sha256_16": sources.all_hashes(), "input_sha256": input_sha}
    line = final_line(args, w, res, others, env)
    if details:
        details.write(json.dumps({**res, "env": env}) + "\n")
        details.close()
    text = json.dumps(line, separators=(",", ":"))
    if len(text) > FINAL_LINE_MAX_BYTES:      # never let the record outgrow the reader
        for k in ("strided_over_coalesced", "cpu_baseline_all_cores", "others", "env"):
            line.pop(k, None)
            text = json.dumps(line, separators=(",", ":"))
            if len(text) <= FINAL_LINE_MAX_BYTES:
                break
    print(text, flush=True)
    return 1 if res["parity"] == "FAIL" else 0


if __name__ == "__main__":
    sys.exit(main())
