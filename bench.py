#!/usr/bin/env python3
"""Achieved HBM bandwidth of the elementwise kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-others] [--no-cpu-baseline]

A step is one call of the library on the workload (validation, plan, launch
of the vectorised grid-stride kernel with its scalar head and tail).  The
default workload is fp32 C = A + B on n = 2^28 + 3 elements with A one
element (4 bytes) past an aligned allocation.

Procedure: inputs are generated on the host, copied to the GPU once, and a
parity gate compares one launch with the CPU oracle on every element (a
workload that fails reports no speed).  The oracle runs only inside the CPU
leg (``cpu_baseline_leg``), which also times it.  Then W untimed launches, then K
launches bracketed by HIP events recorded on the stream the kernels run on.
GB/s = algorithmic bytes (read + write, 10^9 bytes per GB) / average launch
time.  Prints one JSON line.

Also reported, in the same line:
* ``roofline``: the dominant kernel's achieved GB/s against the 8 TB/s HBM
  peak, and (``traffic``) the HBM bytes per launch measured by rocprofv3
  counters when a summary for the current kernel source is in
  ``profiles/traffic.json`` (else null);
* ``cpu_baseline``: the CPU oracle timed on the host on a bounded sample;
* ``other_configs``: the remaining workloads (each parity-gated); working
  sets up to 1 GiB (4 x the 256 MB Infinity Cache) are timed cold: back to
  back over R copies of the workload's buffers, used in turn, so that at
  least 1 GiB of other traffic runs between two uses of one copy.  Beside it,
  ``flushed_per_launch`` gives the median of single launches each bracketed
  by its own events after a 1 GiB fill.
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
DEFAULT_WORKLOAD = "cfg2_add_f32_2e28p3_offA1"
KERNEL_SRC = os.path.join(ROOT, "memory_bound_elementwise_amd", "csrc", "ew_kernels.hip")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

# Algorithmic bytes per element: each input element read once, each output
# element written once.  The gather counts logical bytes (read 4 + write 4).
# The fused chains count what they move: add+ReLU and SAXPY+ReLU 12, bias+ReLU
# 8 (x read, y written) plus the bias row once.
BYTES_PER_ELEM = {"add_f32": 12, "add_f16": 6, "add_bf16": 6, "saxpy_f32": 12,
                  "relu_f32": 8, "copy_f32": 8, "gather_f32": 8, "add_relu_f32": 12,
                  "saxpy_relu_f32": 12, "bias_relu_f32": 8, "saxpy_f16": 6, "saxpy_bf16": 6,
                  "relu_f16": 4, "relu_bf16": 4, "copy2d_f32": 8, "relu_inplace_f32": 8,
                  # scalar-broadcast and unary maps: one input read, one output written
                  **{f"{m}_{d}": 8 if d == "f32" else 4
                     for m in ("scale", "add_scalar", "sqrt", "abs")
                     for d in ("f32", "f16", "bf16")}}
DTYPE = {"add_f32": "f32", "add_f16": "f16", "add_bf16": "bf16", "saxpy_f32": "f32",
         "relu_f32": "f32", "copy_f32": "f32", "gather_f32": "f32", "add_relu_f32": "f32",
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


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Prepared:
    """Device buffers of one workload and a launcher bound to a stream."""

    def __init__(self, w, torch, np, ew, synth, stream, inp=None):
        from tests.gpu_util import upload
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
        if w.op == "relu_inplace_f32":
            x, kx = upload(self.inp["x"], offs.get("x", 0))
            pristine = x.clone()
            self.keep += [kx, pristine]
            self.launch = lambda: ew.ew_relu_inplace_f32(x, stream=s)
            self.pre = lambda: x.copy_(pristine)
            # the same in-place ReLU storing every element, for comparison
            self.unfused = lambda: ew.ew_relu_f32(x, x, stream=s)
            self.changed, self.spans_changed = relu_store_counts(self.inp["x"], np)
            self.out, self.ptrs = x, (x, x, None)
        elif w.op == "copy2d_f32":
            sr, sc, _, offset = w.view
            base, kb = upload(self.inp["base"], 0)
            out, ko = upload(np.zeros(w.n, np.float32), 0)
            self.keep += [kb, ko]
            rows = w.n // w.cols
            src = base.data_ptr() + 4 * offset
            self.launch = lambda: ew.ew_copy2d_f32(src, sr, sc, out, rows, w.cols, stream=s)
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
            batch = ew.EwBatch(w.op, [(o, x, y, m) for o, x, y in parts])
            self.launch = lambda: batch(stream=s)
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
        return ew.ew_make_plan(self.w.op, out.data_ptr(), in0.data_ptr(),
                               in1.data_ptr() if in1 is not None else 0, self.w.n, cus)

    def result(self, torch):
        """One launch on fresh buffers; returns the output copied to the host."""
        from tests.gpu_util import ELEM, download
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
    from tests.gpu_util import mismatches

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
        if w.op == "gather_f32":
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
    if target_s > 0 and w.op not in ("copy2d_f32", "gather_f32"):
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


def traffic_for(workload: str, launch_desc: dict):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source and launch shape; else None."""
    try:
        with open(TRAFFIC_JSON) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get("workloads", {}).get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if rec.get("launch") != launch_desc:
        return None
    return rec.get("hbm_bytes_per_launch")


def measure(w, torch, np, ew, synth, stream, steps, warmup, cus, flush_buf, cpu_target_s,
            check=True):
    prep = Prepared(w, torch, np, ew, synth, stream)
    plan = prep.plan(ew, cus)
    launch_desc = {"block": plan.block, "grid": plan.grid, "unroll": plan.unroll}
    if w.batch:
        # one launch shape for the whole call: the table's row for the total n
        block, bpc, unroll = ew.ew_get_launch_config(w.op, w.n)
        m = w.n // w.batch
        vec = 16 // (4 if w.op.endswith("_f32") else 2)
        tiles = max(1, -(-(m // vec) // (block * min(unroll, 4))))     # per item
        launch_desc = {"block": block, "unroll": min(unroll, 4), "items": w.batch,
                       "items_per_launch": ew.BATCH_MAX,
                       "launches": -(-w.batch // ew.BATCH_MAX),
                       "grid_per_launch": min(bpc * cus, tiles * min(w.batch, ew.BATCH_MAX)),
                       "path": "batched: items' tiles numbered consecutively, one kernel"}
        steps = min(steps, 200)
    if w.op == "gather_f32":
        launch_desc["path"] = ("copy kernel" if w.stride % w.n == 1 else
                               f"{plan.passes} passes, input staged through LDS"
                               if plan.passes > 1 else
                               "contiguous 16-byte loads, even elements kept" if
                               (plan.reps == 2 and w.stride % w.n == 2) else
                               f"per-output index walk, {plan.reps} segment(s)")
    if w.op == "copy2d_f32":
        sr, sc = w.view[0], w.view[1]
        launch_desc["path"] = ("contiguous 16-byte loads, even elements kept (stride-2 gather "
                               "kernel)" if (w.n == w.cols and sc == 2) else
                               f"span read contiguously through LDS, one element in {sc} kept"
                               if (w.n == w.cols and 3 <= sc <= 8) else
                               "rows contiguous" if sc == 1 else
                               "LDS-tiled transpose (128 x 128 tiles, 1024 threads)" if sr == 1 else
                               "generic (one 4-byte load per element)")
    res = {"workload": w.name, "op": w.op, "n": w.n, "launch": launch_desc,
           "split": {"head": plan.head, "vectors": plan.vectors, "tail": plan.tail,
                     "in_coaligned": list(plan.in_coaligned)}}
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
        fl_ms = time_launches(torch, prep.launch, stream, steps, warmup, flush=flush)
        timing = (f"cold: back to back over {len(sets)} copies of the buffers used in turn "
                  f"(>= 1 GiB of other traffic between two uses of one copy), mean")
        res["flushed_per_launch"] = {
            "ms": round(fl_ms, 5), "gbs": round(nbytes / (fl_ms / 1e3) / 1e9, 1),
            "p10_ms": round(LAST_DIST["p10"], 5), "p90_ms": round(LAST_DIST["p90"], 5),
            "timing": "each launch between its own events after a 1 GiB fill, median "
                      "(includes the per-launch event gap and the fill's write-back)"}
    else:
        ms = time_launches(torch, prep.launch, stream, steps, warmup, flush=flush, pre=prep.pre)
        timing = ("cold (1 GiB flush before each launch), median" if cold else
                  "back-to-back, mean")
        if cold:
            res["p10_ms"], res["p90_ms"] = round(LAST_DIST["p10"], 5), round(LAST_DIST["p90"], 5)
    gbs = nbytes / (ms / 1e3) / 1e9
    res.update({"ms": round(ms, 5), "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_GBS, 4),
                "timing": timing})
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-others", action="store_true", help="skip the other configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: each op of the five configurations over "
                         "N = 2^20 .. 2^28 plus odd N, one parity-gated JSON line per point")
    ap.add_argument("--sweep-out", help="with --sweep: append each point to this JSONL file "
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

    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.description}")
    input_sha = {k: synth.sha256(v)[:16] for k, v in synth.workload_inputs(w).items()}
    res, prep, ms = measure(w, torch, np, ew, synth, stream, args.steps, args.warmup, cus,
                            flush_buf, args.cpu_seconds, check=not args.no_cpu_baseline)
    log(f"parity {res['parity']}; {res.get('gbs')} GB/s")

    line = {
        "metric": "achieved HBM GB/s (read+write bytes/time) and % of MI355X peak, N=2^28",
        "value": res.get("gbs"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.get("ms"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[w.op],
        "data": "synthetic (seeded: " + w.dist + ")",
        "config": {"workload": w.description, "name": w.name, "op": w.op, "n": w.n,
                   "offsets_elems": w.offsets, "launch": res["launch"], "split": res["split"],
                   "global_batch": w.n, "parallelism": "single GPU"},
        "parity": res["parity"],
        "pct_of_peak": round(100 * res["gbs"] / PEAK_GBS, 2) if res.get("gbs") else None,
    }
    for k in ("p10_ms", "p90_ms", "timing", "warm_gbs", "flushed_per_launch", "torch_context",
              "graph", "unfused", "separate_calls"):
        if k in res:
            line[k] = res[k]
    if ms is not None:
        traffic = traffic_for(w.name, res["launch"])
        line["roofline"] = {"bound": "hbm", "achieved": res["gbs"], "peak": PEAK_GBS,
                            "unit": "GB/s", "frac": round(res["gbs"] / PEAK_GBS, 4),
                            "traffic": traffic,
                            "kernel": f"ew_stream_kernel<{w.op}, U={res['launch']['unroll']}>",
                            "algorithmic_bytes_per_launch": algorithmic_bytes(
                                w.op, w.n, w.cols if w.op == "bias_relu_f32" else 0,
                                res.get("changed", 0)),
                            "avg_launch_ms": res["ms"]}
    del prep
    torch.cuda.empty_cache()

    if "cpu_baseline" in res:
        line["cpu_baseline"] = res.pop("cpu_baseline")
        if "all_cores" in line["cpu_baseline"]:
            line["cpu_baseline_all_cores"] = line["cpu_baseline"].pop("all_cores")

    if not args.no_others:
        others = []
        for name, ow in synth.WORKLOADS.items():
            if name == w.name:
                continue
            log(f"other config {name}")
            steps = 200 if ow.n >= (1 << 25) else 1000
            try:
                r, p, _ = measure(ow, torch, np, ew, synth, stream, steps, 10, cus, flush_buf,
                                  0.0, check=not args.no_cpu_baseline)
                del p
            except Exception as exc:
                # recorded, and nothing more is launched (the error may have left the
                # device unusable); the headline line below still prints
                others.append({"workload": name, "op": ow.op, "n": ow.n,
                               "error": f"{type(exc).__name__}: {exc}"})
                log(f"other config {name} failed, remaining configs skipped: {exc}")
                break
            others.append(r)
            torch.cuda.empty_cache()
        line["other_configs"] = others
        if any("error" in r for r in others):
            line["other_configs_incomplete"] = True
        by = {r["workload"]: r for r in others + [res]}
        sg, cg = by.get("cfg5b_gather_f32_2e26_s2"), by.get("cfg5a_copy_f32_2e26")
        if sg and cg and sg.get("gbs") and cg.get("gbs"):
            # the fifth configuration's comparison: strided gather vs coalesced copy
            line["strided_over_coalesced"] = {
                "gather_s2_gbs": sg["gbs"], "copy_gbs": cg["gbs"],
                "ratio": round(sg["gbs"] / cg["gbs"], 4),
                "traffic_note": "logical bytes for both; the gather reads each input line once"}

    line["env"] = {"device": torch.cuda.get_device_name(0),
                   "arch": getattr(dev_props, "gcnArchName", None), "cus": cus,
                   "hbm_bytes": dev_props.total_memory, "clocks": _clocks(dev_props),
                   "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                   "numpy": np.__version__, "kernel_source_sha256_16": kernel_source_hash(),
                   "input_sha256": input_sha}
    print(json.dumps(line), flush=True)
    return 1 if res["parity"] == "FAIL" else 0


if __name__ == "__main__":
    sys.exit(main())
