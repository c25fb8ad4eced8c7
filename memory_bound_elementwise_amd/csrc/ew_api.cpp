// ew_api.cpp -- host side of libew: argument validation, the head/body/tail
// plan, the launch-configuration table and the exported C ABI (include/ew.h).
//
// Validation runs before any HIP call, so every argument error is reported
// the same way on a machine without a GPU.

#include "ew.h"
#include "ew_batch_args.h"
#include "ew_gather_args.h"
#include "ew_internal.h"
#include "ew_view_args.h"

#include <algorithm>
#include <climits>
#include <atomic>
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

namespace ew {
namespace {

constexpr int kAbiVersion = 14;
static_assert(kBatchScratchBytes == EW_BATCH_SCRATCH_BYTES, "one scratch size for both sides");

struct OpInfo {
    const char *name;
    int elem_size;
    int inputs;          // 1 or 2
    bool alias_ok;       // output may be exactly an input
    int align;           // the planned head aligns the output body to this many bytes
};

constexpr OpInfo kOps[kOpCount] = {
    {"add_f32", 4, 2, true, 16},
    {"add_f16", 2, 2, true, 16},
    {"add_bf16", 2, 2, true, 16},
    {"saxpy_f32", 4, 2, true, 16},
    {"relu_f32", 4, 1, true, 16},
    {"copy_f32", 4, 1, true, 16},
    {"gather_f32", 4, 1, false, 16},
    {"add_relu_f32", 4, 2, true, 16},
    {"saxpy_relu_f32", 4, 2, true, 16},
    {"bias_relu_f32", 4, 1, true, 16},
    {"saxpy_f16", 2, 2, true, 16},
    {"saxpy_bf16", 2, 2, true, 16},
    {"relu_f16", 2, 1, true, 16},
    {"relu_bf16", 2, 1, true, 16},
    {"copy2d_f32", 4, 1, false, 16},
    {"relu_inplace_f32", 4, 1, true, 64},
    {"scale_f32", 4, 1, true, 16},
    {"scale_f16", 2, 1, true, 16},
    {"scale_bf16", 2, 1, true, 16},
    {"add_scalar_f32", 4, 1, true, 16},
    {"add_scalar_f16", 2, 1, true, 16},
    {"add_scalar_bf16", 2, 1, true, 16},
    {"sqrt_f32", 4, 1, true, 16},
    {"sqrt_f16", 2, 1, true, 16},
    {"sqrt_bf16", 2, 1, true, 16},
    {"abs_f32", 4, 1, true, 16},
    {"abs_f16", 2, 1, true, 16},
    {"abs_bf16", 2, 1, true, 16},
    {"gather_walk_f32", 4, 1, false, 16},
};

int op_from_name(const char *name)
{
    if (!name) return -1;
    for (int i = 0; i < kOpCount; ++i)
        if (std::strcmp(kOps[i].name, name) == 0) return i;
    return -1;
}

// ---------------------------------------------------------------------------
// Launch-configuration table
// ---------------------------------------------------------------------------

struct Row {
    size_t min_n;
    int block;
    int blocks_per_cu;
    int unroll;
};

// Compiled-in defaults: the table written by tune.py on MI355X (256 CUs,
// 8 TB/s HBM3E); a row covers n >= min_n up to the next row.  blocks_per_cu
// 1024 means one block per tile at every size used in practice.  The
// two-input operations have a third, mid-size row (2^22 <= n < 2^25) from a
// sweep timed cold, where 512-thread tiles of two vectors per lane beat the
// large shapes by 2-14 %; the 16-bit one-input operations likewise take
// 512-thread tiles from 2^22 to 2^26 (3-19 %).  The gather's rows apply to the length of the
// segment its kernel computes (n / 2 for stride 2 and even n): 512-thread
// tiles from 2^21, the large row from 2^25.
struct DefaultRow {
    int op;
    Row row;
};
constexpr DefaultRow kDefaults[] = {
    {kOpAddF32, {0, 512, 1, 2}},
    {kOpAddF32, {size_t(1) << 22, 512, 1024, 2}},
    {kOpAddF32, {size_t(1) << 25, 1024, 1024, 1}},
    {kOpAddF16, {0, 128, 2, 2}},
    {kOpAddF16, {size_t(1) << 22, 512, 1024, 2}},
    {kOpAddF16, {size_t(1) << 25, 128, 1024, 1}},
    {kOpAddBF16, {0, 256, 2, 2}},
    {kOpAddBF16, {size_t(1) << 22, 512, 1024, 2}},
    {kOpAddBF16, {size_t(1) << 25, 128, 1024, 1}},
    {kOpSaxpyF32, {0, 512, 1, 1}},
    {kOpSaxpyF32, {size_t(1) << 22, 512, 1024, 2}},
    {kOpSaxpyF32, {size_t(1) << 25, 1024, 1024, 1}},
    {kOpReluF32, {0, 512, 8, 1}},
    {kOpReluF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpCopyF32, {0, 256, 8, 1}},
    {kOpCopyF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpGatherF32, {0, 128, 4, 1}},
    {kOpGatherF32, {size_t(1) << 21, 512, 1024, 1}},
    {kOpGatherF32, {size_t(1) << 25, 128, 1024, 1}},
    {kOpAddReluF32, {0, 512, 1024, 2}},
    {kOpAddReluF32, {size_t(1) << 22, 512, 1024, 2}},
    {kOpAddReluF32, {size_t(1) << 25, 1024, 1024, 1}},
    {kOpSaxpyReluF32, {0, 512, 4, 2}},
    {kOpSaxpyReluF32, {size_t(1) << 22, 512, 1024, 2}},
    {kOpSaxpyReluF32, {size_t(1) << 25, 1024, 1024, 1}},
    {kOpBiasReluF32, {0, 1024, 1024, 1}},
    {kOpBiasReluF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpSaxpyF16, {0, 256, 1024, 4}},
    {kOpSaxpyF16, {size_t(1) << 22, 512, 1024, 2}},
    {kOpSaxpyF16, {size_t(1) << 25, 128, 1024, 1}},
    {kOpSaxpyBF16, {0, 128, 2, 2}},
    {kOpSaxpyBF16, {size_t(1) << 22, 512, 1024, 2}},
    {kOpSaxpyBF16, {size_t(1) << 25, 128, 1024, 1}},
    {kOpReluF16, {0, 1024, 8, 1}},
    {kOpReluF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpReluF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpReluBF16, {0, 128, 4, 2}},
    {kOpReluBF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpReluBF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpCopy2dF32, {0, 256, 2, 2}},
    {kOpCopy2dF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpReluInplaceF32, {0, 1024, 1, 4}},
    {kOpReluInplaceF32, {size_t(1) << 22, 512, 1024, 1}},
    {kOpScaleF32, {0, 256, 8, 1}},
    {kOpScaleF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpScaleF16, {0, 1024, 8, 1}},
    {kOpScaleF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpScaleF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpScaleBF16, {0, 1024, 8, 1}},
    {kOpScaleBF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpScaleBF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpAddScalarF32, {0, 256, 8, 1}},
    {kOpAddScalarF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpAddScalarF16, {0, 1024, 8, 1}},
    {kOpAddScalarF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpAddScalarF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpAddScalarBF16, {0, 1024, 8, 1}},
    {kOpAddScalarBF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpAddScalarBF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpSqrtF32, {0, 256, 8, 1}},
    {kOpSqrtF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpSqrtF16, {0, 1024, 8, 1}},
    {kOpSqrtF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpSqrtF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpSqrtBF16, {0, 1024, 8, 1}},
    {kOpSqrtBF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpSqrtBF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpAbsF32, {0, 256, 8, 1}},
    {kOpAbsF32, {size_t(1) << 22, 256, 1024, 1}},
    {kOpAbsF16, {0, 1024, 8, 1}},
    {kOpAbsF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpAbsF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpAbsBF16, {0, 1024, 8, 1}},
    {kOpAbsBF16, {size_t(1) << 22, 512, 1024, 1}},
    {kOpAbsBF16, {size_t(1) << 26, 128, 1024, 1}},
    {kOpGatherWalkF32, {0, 128, 4, 1}},
    {kOpGatherWalkF32, {size_t(1) << 21, 512, 1024, 1}},
    {kOpGatherWalkF32, {size_t(1) << 25, 128, 1024, 1}},
};

constexpr int kMaxRows = 16;

// Fixed capacity, so that no table operation allocates (or can throw).
struct Rows {
    Row row[kMaxRows];
    int count = 0;
    Row *begin() { return row; }
    Row *end() { return row + count; }
};

struct Table {
    std::mutex mu;
    bool loaded = false;
    Rows rows[kOpCount];
};

Table &table()
{
    static Table t;
    return t;
}

void reset_locked(Table &t)
{
    for (auto &r : t.rows) r.count = 0;
    for (const auto &d : kDefaults) {
        Rows &r = t.rows[d.op];
        if (r.count < kMaxRows) r.row[r.count++] = d.row;
    }
    t.loaded = true;
}

void ensure_loaded_locked(Table &t)
{
    if (!t.loaded) reset_locked(t);
}

bool valid_row(int block, int bpc, int unroll)
{
    if (block < 64 || block > 1024 || block % 64 != 0) return false;
    if (bpc < 1 || bpc > 1024) return false;
    return unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8;
}

ew_status_t set_row(int op, size_t min_n, int block, int bpc, int unroll)
{
    if (op < 0 || !valid_row(block, bpc, unroll)) return EW_ERR_INVALID_ARG;
    Table &t = table();
    std::lock_guard<std::mutex> g(t.mu);
    ensure_loaded_locked(t);
    auto &rows = t.rows[op];
    for (auto &r : rows) {
        if (r.min_n == min_n) {
            r = Row{min_n, block, bpc, unroll};
            return EW_OK;
        }
    }
    if (rows.count >= kMaxRows) return EW_ERR_INVALID_ARG;
    int pos = 0;
    while (pos < rows.count && rows.row[pos].min_n < min_n) ++pos;
    for (int k = rows.count; k > pos; --k) rows.row[k] = rows.row[k - 1];
    rows.row[pos] = Row{min_n, block, bpc, unroll};
    ++rows.count;
    return EW_OK;
}

Row get_row(int op, size_t n)
{
    Table &t = table();
    std::lock_guard<std::mutex> g(t.mu);
    ensure_loaded_locked(t);
    Row best{0, 256, 8, 1};
    bool found = false;
    for (const auto &r : t.rows[op]) {
        if (r.min_n <= n && (!found || r.min_n >= best.min_n)) {
            best = r;
            found = true;
        }
    }
    return best;
}

// ---------------------------------------------------------------------------
// Devices
// ---------------------------------------------------------------------------

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<bool> g_device_seen{false};

// Current device and its compute-unit count, or an error status.
ew_status_t current_device(int *cu_count)
{
    hipError_t e;
    if (!g_device_seen.load(std::memory_order_acquire)) {
        int count = 0;
        e = hipGetDeviceCount(&count);
        if (e != hipSuccess || count <= 0) {
            (void)hipGetLastError();  // do not leave our probe's error behind
            return EW_ERR_NO_DEVICE;
        }
        g_device_seen.store(true, std::memory_order_release);
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return EW_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return EW_ERR_NO_DEVICE;
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cus <= 0) {
            g_last_hip_error = (int)e;
            return EW_ERR_HIP;
        }
        g_cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    *cu_count = cus;
    return EW_OK;
}

// ---------------------------------------------------------------------------
// Validation and planning
// ---------------------------------------------------------------------------

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool ranges_intersect(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks shared by every operation.  ins[k] may be nullptr only when the op
// has fewer inputs.
ew_status_t validate(int op, const void *out, const void *in0, const void *in1, size_t n)
{
    const OpInfo &info = kOps[op];
    if (!out || !in0 || (info.inputs == 2 && !in1)) return EW_ERR_INVALID_ARG;
    const size_t es = (size_t)info.elem_size;
    if (n > SIZE_MAX / es) return EW_ERR_INVALID_ARG;
    const size_t bytes = n * es;
    // Element indices and the gather's index sums stay below 2^62.
    if (n >= (size_t(1) << 62)) return EW_ERR_INVALID_ARG;
    const void *ptrs[3] = {out, in0, info.inputs == 2 ? in1 : nullptr};
    for (const void *p : ptrs) {
        if (!p) continue;
        const uintptr_t u = reinterpret_cast<uintptr_t>(p);
        if (u > UINTPTR_MAX - bytes) return EW_ERR_INVALID_ARG;
    }
    for (const void *p : ptrs) {
        if (p && reinterpret_cast<uintptr_t>(p) % es != 0) return EW_ERR_MISALIGNED;
    }
    const Range ro{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + bytes};
    for (int k = 1; k <= info.inputs; ++k) {
        const Range ri{reinterpret_cast<uintptr_t>(ptrs[k]),
                       reinterpret_cast<uintptr_t>(ptrs[k]) + bytes};
        if (!ranges_intersect(ro, ri)) continue;
        if (info.alias_ok && ro.lo == ri.lo) continue;  // exact alias
        return EW_ERR_OVERLAP;
    }
    return EW_OK;
}

struct Plan {
    size_t head, vectors, tail, tiles;
    bool co[2];
    Launch launch;
    int blocks_per_cu;
};

// The split and the launch shape (arguments already validated, n > 0).
Plan make_plan(int op, const void *out, const void *in0, const void *in1, size_t n, int cu_count)
{
    const OpInfo &info = kOps[op];
    const size_t es = (size_t)info.elem_size;
    const size_t vec = 16 / es;
    Plan p{};
    const uintptr_t o = reinterpret_cast<uintptr_t>(out);
    const size_t al = (size_t)info.align;
    size_t head = ((al - (o % al)) % al) / es;
    if (head > n) head = n;
    p.head = head;
    p.vectors = (n - head) / vec;
    p.tail = n - head - p.vectors * vec;
    const void *ins[2] = {in0, info.inputs == 2 ? in1 : nullptr};
    for (int k = 0; k < 2; ++k) {
        p.co[k] = true;
        if (op != kOpGatherF32 && op != kOpGatherWalkF32 && ins[k])
            p.co[k] = (reinterpret_cast<uintptr_t>(ins[k]) + head * es) % 16 == 0;
    }
    const Row r = get_row(op, n);
    const size_t tile_vecs = (size_t)r.block * (size_t)r.unroll;
    p.tiles = (p.vectors + tile_vecs - 1) / tile_vecs;
    size_t grid = (size_t)r.blocks_per_cu * (size_t)(cu_count > 0 ? cu_count : 1);
    if (grid > p.tiles) grid = p.tiles;
    if (grid == 0) grid = 1;  // head/tail lanes still need one block
    p.launch = Launch{r.block, (int)grid, r.unroll};
    p.blocks_per_cu = r.blocks_per_cu;
    return p;
}

ew_status_t fail_hip(hipError_t e)
{
    g_last_hip_error = (int)e;
    return EW_ERR_HIP;
}

// EW_LOG set to anything but "" or "0": every launch prints its plan to
// stderr (read once per process).
bool log_enabled()
{
    static const bool on = [] {
        const char *v = std::getenv("EW_LOG");
        return v != nullptr && *v != '\0' && std::strcmp(v, "0") != 0;
    }();
    return on;
}

void log_launch(const char *op, size_t n, uint64_t head, uint64_t vectors, uint64_t tail,
                const Launch &l, const char *path)
{
    if (!log_enabled()) return;
    std::fprintf(stderr,
                 "[ew] %s n=%zu head=%llu vectors=%llu tail=%llu grid=%d block=%d unroll=%d "
                 "path=%s\n",
                 op, n, (unsigned long long)head, (unsigned long long)vectors,
                 (unsigned long long)tail, l.grid, l.block, l.unroll, path);
}

ew_status_t run_stream(int op, const void *out, const void *in0, const void *in1, size_t n,
                       float alpha, hipStream_t stream)
{
    if (n == 0) return EW_OK;
    ew_status_t st = validate(op, out, in0, in1, n);
    if (st != EW_OK) return st;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    const Plan p = make_plan(op, out, in0, in1, n, cus);
    StreamArgs a{};
    a.in0 = in0;
    a.in1 = kOps[op].inputs == 2 ? in1 : nullptr;
    a.out = const_cast<void *>(out);
    a.head = p.head;
    a.vectors = p.vectors;
    a.tail = p.tail;
    a.tiles = p.tiles;
    a.alpha = alpha;
    log_launch(kOps[op].name, n, p.head, p.vectors, p.tail, p.launch,
               p.co[0] && p.co[1] ? "stream, inputs co-aligned" : "stream, an input misaligned");
    const hipError_t e = launch_stream(static_cast<OpId>(op), a, p.co[0], p.co[1], p.launch, stream);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

// Operations the batched entry point runs: every one-pass streaming
// operation of ew_stream_kernel.
bool batchable(int op)
{
    switch (op) {
    case kOpGatherF32:
    case kOpGatherWalkF32:
    case kOpBiasReluF32:
    case kOpCopy2dF32:
    case kOpReluInplaceF32: return false;
    default: return op >= 0 && op < kOpCount;
    }
}

// Operations whose single call passes y as both the second input and the
// output (y <- f(x, y) in place).
bool in_place_second(int op)
{
    return op == kOpSaxpyF32 || op == kOpSaxpyReluF32 || op == kOpSaxpyF16 ||
           op == kOpSaxpyBF16;
}

// Items of one batched call must not race: an item's output range may not
// intersect any range (input or output) of another item.  Outputs and
// inputs are each ordered by start -- already in order for the usual list of
// consecutive arrays, then without sorting -- the outputs must be disjoint,
// and one merge pass compares every input with the outputs that start
// before it ends.
ew_status_t batch_overlap(int op, const ew_batch_item_t *items, size_t count)
{
    struct R {
        uintptr_t lo, hi;
        size_t item;
    };
    const auto by_lo = [](const R &x, const R &y) { return x.lo < y.lo; };
    const size_t es = (size_t)kOps[op].elem_size;
    const bool two = kOps[op].inputs == 2 && !in_place_second(op);
    std::vector<R> w, r;
    w.reserve(count);
    r.reserve(two ? 2 * count : count);
    for (size_t i = 0; i < count; ++i) {
        const ew_batch_item_t &it = items[i];
        if (it.n == 0) continue;
        const uintptr_t bytes = (uintptr_t)(it.n * es);
        const uintptr_t o = reinterpret_cast<uintptr_t>(it.out);
        w.push_back(R{o, o + bytes, i});
        const uintptr_t a = reinterpret_cast<uintptr_t>(it.in0);
        r.push_back(R{a, a + bytes, i});
        if (two) {
            const uintptr_t b = reinterpret_cast<uintptr_t>(it.in1);
            r.push_back(R{b, b + bytes, i});
        }
    }
    if (!std::is_sorted(w.begin(), w.end(), by_lo)) std::sort(w.begin(), w.end(), by_lo);
    if (!std::is_sorted(r.begin(), r.end(), by_lo)) std::sort(r.begin(), r.end(), by_lo);
    for (size_t k = 1; k < w.size(); ++k)
        if (w[k - 1].hi > w[k].lo) return EW_ERR_OVERLAP;
    size_t j = 0;                                   // first output that may still meet an input
    for (const R &in : r) {
        while (j < w.size() && w[j].hi <= in.lo) ++j;   // ends before this (and every later) input
        for (size_t k = j; k < w.size() && w[k].lo < in.hi; ++k)
            if (w[k].item != in.item) return EW_ERR_OVERLAP;
    }
    return EW_OK;
}

// (a * b) mod m without overflow (host: 128-bit arithmetic).
uint64_t mulmod_host(uint64_t a, uint64_t b, uint64_t m)
{
    return (uint64_t)(((unsigned __int128)a * (unsigned __int128)b) % (unsigned __int128)m);
}

// a^-1 mod m for gcd(a, m) == 1 and m >= 2 (extended Euclid).
uint64_t modinv_host(uint64_t a, uint64_t m)
{
    __int128 r0 = m, r1 = a % m, t0 = 0, t1 = 1;
    while (r1 != 0) {
        const __int128 q = r0 / r1;
        const __int128 r2 = r0 - q * r1, t2 = t0 - q * t1;
        r0 = r1; r1 = r2; t0 = t1; t1 = t2;
    }
    if (t0 < 0) t0 += m;
    return (uint64_t)t0;
}

// The gather's plan.  With g = gcd(stride mod n, n), output i and output
// i + n/g read the same input element ((stride * n/g) mod n == 0), so the
// output is g copies of its first n/g elements, and the kernels compute one
// segment and store each value g times: every input line is then fetched
// once instead of g times.  Strides 2..32: the pass decomposition (see
// GatherArgs).  Larger strides with at least 128 rows of `stride` elements,
// g < 32, s' = s/g below 2^32 and s' * n/g below 2^64: the tiled
// transposition.  Otherwise the per-output walk, over one segment when n/g
// is a multiple of 4 (every copy then has the same 16-byte alignment) and
// 2 <= g <= 8 or n/g >= kGatherLongSegment, else over all n.
//
// walk: the per-output index walk whatever the stride (no pass decomposition
// and no replicated segments: every output element loads its own input
// element), with the launch rows of gather_walk_f32.
void gather_plan(const float *in, float *out, size_t n, size_t stride, int cus, GatherArgs *g,
                 Launch *l, int *blocks_per_cu = nullptr, bool walk = false)
{
    const uint64_t s = stride % n;
    const uint64_t gcd = std::gcd(s, (uint64_t)n);  // gcd(0, n) == n
    // stride 2 with two segments whose length is a multiple of 4: the
    // stride-2 kernel (contiguous loads, no LDS) below
    const bool spans2 = s == 2 && gcd == 2 && (n / 2) % 4 == 0;
    if (!walk && s >= 2 && s <= (uint64_t)kMaxPasses && !spans2) {
        // Pass decomposition of one of the g = gcd(s, n) equal segments of
        // n' = n/g outputs, with s' = s/g coprime with n': pass k
        // (floor(s'*i/n') == k) starts at i_k = ceil(k*n'/s') and reads
        // in[s*m + g*r_k], r_k = s'*i_k - k*n'; the r_k are distinct.
        const uint64_t sp = s / gcd, np = n / gcd;
        *g = GatherArgs{};
        g->in = reinterpret_cast<const uint32_t *>(in);
        g->out = reinterpret_cast<uint32_t *>(out);
        g->n = n;
        g->stride = s;
        g->passes = (int)s;
        g->skip = (int)gcd;
        for (uint64_t k = 0; k < sp; ++k) {
            const unsigned __int128 kn = (unsigned __int128)k * np;
            const uint64_t ik = (uint64_t)((kn + sp - 1) / sp);
            const uint64_t r = (uint64_t)((unsigned __int128)sp * ik - kn);
            g->dest[r] = ik;
        }
        g->seg = np;
        g->reps = gcd;
        g->vectors = ((np + sp - 1) / sp + 3) / 4;
        // fixed block shape (one group per thread); the table's
        // blocks_per_cu still caps the grid
        const Row r = get_row(kOpGatherF32, n);
        const uint64_t tile = (uint64_t)gather_passes_threads();
        g->tiles = (g->vectors + tile - 1) / tile;
        uint64_t grid = (uint64_t)r.blocks_per_cu * (uint64_t)(cus > 0 ? cus : 1);
        if (grid > g->tiles) grid = g->tiles;
        if (grid == 0) grid = 1;
        *l = Launch{gather_passes_threads(), (int)grid, 1};
        if (blocks_per_cu) *blocks_per_cu = r.blocks_per_cu;
        return;
    }
    if (!walk && s > (uint64_t)kMaxPasses) {
        // Tiled transposition of A[m][c] = in[s*m + c]: column c = g*r is
        // the pass k = (-r * inv) mod s' of a segment (see GatherArgs).
        const uint64_t sp = s / gcd, np = n / gcd;
        const uint64_t rows = (n - 1) / s + 1;
        if (sp >= 2 && gcd < 32 && rows >= 128 && sp < ((uint64_t)1 << 32) &&
            (unsigned __int128)sp * np <= (unsigned __int128)UINT64_MAX) {
            *g = GatherArgs{};
            g->in = reinterpret_cast<const uint32_t *>(in);
            g->out = reinterpret_cast<uint32_t *>(out);
            g->n = n;
            g->stride = s;
            g->seg = np;
            g->reps = gcd;
            g->sp = sp;
            g->inv = modinv_host(np % sp, sp);
            const bool narrow = s < kGatherNarrowStrides;
            const int wide = rows < kGatherTallRows ? 2 : 3;
            g->tile_mode = narrow ? (s % 4 == 0 ? 4 : 1) : wide;
            const uint32_t cols = narrow ? (uint32_t)s : kGatherWideCols[wide - 2];
            g->tile_rows = narrow ? (uint32_t)(kGatherTileWords / s) & ~3u : kGatherWideRows[wide - 2];
            g->tiles_m = (rows + g->tile_rows - 1) / g->tile_rows;
            g->tiles = g->tiles_m * ((s + cols - 1) / cols);
            g->vectors = (np + 3) / 4;
            // one block per tile, the grid capped at the table's blocks per
            // CU for this size (beyond it blocks stride over the tiles)
            const Row r = get_row(kOpGatherF32, n);
            const uint64_t cap = (uint64_t)r.blocks_per_cu * (uint64_t)(cus > 0 ? cus : 1);
            const uint64_t grid = g->tiles < cap ? g->tiles : cap;
            *l = Launch{gather_tiles_threads(), (int)grid, 1};
            if (blocks_per_cu) *blocks_per_cu = r.blocks_per_cu;
            return;
        }
    }
    // one segment stored g times when every copy has the same 16-byte
    // alignment, for g up to 8 or, beyond, segments long enough to spread
    // over the GPU (each lane then stores its vector g times)
    uint64_t reps = 1, seg = n;
    if (!walk && gcd >= 2 && (n / gcd) % 4 == 0 &&
        (gcd <= 8 || n / gcd >= kGatherLongSegment)) {
        reps = gcd;
        seg = n / gcd;
    }
    const Plan p = make_plan(walk ? kOpGatherWalkF32 : kOpGatherF32, out, in, nullptr, seg, cus);
    *g = GatherArgs{};
    g->in = reinterpret_cast<const uint32_t *>(in);
    g->out = reinterpret_cast<uint32_t *>(out);
    g->n = n;
    g->stride = s;
    g->seg = seg;
    g->reps = reps;
    g->head = p.head;
    g->vectors = p.vectors;
    g->tail = p.tail;
    g->tiles = p.tiles;
    const uint64_t nthr = (uint64_t)p.launch.block;
    g->step_vec = mulmod_host(s, (4 * nthr) % n, n);
    const uint64_t tile_elems = (4 * nthr * (uint64_t)p.launch.unroll) % n;
    g->step_tile = mulmod_host(mulmod_host(s, tile_elems, n), (uint64_t)p.launch.grid % n, n);
    g->wide = (s != 0 && (n - 1) > UINT64_MAX / s) ? 1 : 0;
    *l = p.launch;
    if (blocks_per_cu) *blocks_per_cu = p.blocks_per_cu;
}

}  // namespace
}  // namespace ew

using namespace ew;

extern "C" {

ew_status_t ew_add_f32(const float *a, const float *b, float *c, size_t n, hipStream_t s)
{
    return run_stream(kOpAddF32, c, a, b, n, 0.0f, s);
}

ew_status_t ew_add_f16(const uint16_t *a, const uint16_t *b, uint16_t *c, size_t n, hipStream_t s)
{
    return run_stream(kOpAddF16, c, a, b, n, 0.0f, s);
}

ew_status_t ew_add_bf16(const uint16_t *a, const uint16_t *b, uint16_t *c, size_t n,
                        hipStream_t s)
{
    return run_stream(kOpAddBF16, c, a, b, n, 0.0f, s);
}

ew_status_t ew_saxpy_f32(float alpha, const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSaxpyF32, y, x, y, n, alpha, s);
}

ew_status_t ew_relu_f32(const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpReluF32, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_copy_f32(const float *in, float *out, size_t n, hipStream_t s)
{
    if (n == 0) return EW_OK;
    ew_status_t st = validate(kOpCopyF32, out, in, nullptr, n);
    if (st != EW_OK) return st;
    if (static_cast<const void *>(in) == static_cast<const void *>(out)) return EW_OK;
    return run_stream(kOpCopyF32, out, in, nullptr, n, 0.0f, s);
}

ew_status_t ew_gather_f32(const float *in, float *out, size_t n, size_t stride, hipStream_t s)
{
    if (n == 0) return EW_OK;
    if (stride == 0) return EW_ERR_INVALID_ARG;
    ew_status_t st = validate(kOpGatherF32, out, in, nullptr, n);
    if (st != EW_OK) return st;
    if (n == 1 || stride % n == 1) {
        // out[i] = in[i mod n] = in[i]: the contiguous copy
        return run_stream(kOpCopyF32, out, in, nullptr, n, 0.0f, s);
    }
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    GatherArgs g{};
    Launch l{};
    gather_plan(in, out, n, stride, cus, &g, &l);
    log_launch("gather_f32", n, g.head, g.vectors, g.tail, l,
               g.passes ? "passes" : g.tile_mode ? "tiles" : g.reps > 1 ? "replicated segments"
                                                              : "index walk");
    const hipError_t e = launch_gather(g, l, s);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

ew_status_t ew_gather_walk_f32(const float *in, float *out, size_t n, size_t stride,
                               hipStream_t s)
{
    if (n == 0) return EW_OK;
    if (stride == 0) return EW_ERR_INVALID_ARG;
    ew_status_t st = validate(kOpGatherWalkF32, out, in, nullptr, n);
    if (st != EW_OK) return st;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    GatherArgs g{};
    Launch l{};
    gather_plan(in, out, n, stride, cus, &g, &l, nullptr, true);
    log_launch("gather_walk_f32", n, g.head, g.vectors, g.tail, l, "index walk");
    const hipError_t e = launch_gather(g, l, s);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

ew_status_t ew_add_relu_f32(const float *a, const float *b, float *c, size_t n, hipStream_t s)
{
    return run_stream(kOpAddReluF32, c, a, b, n, 0.0f, s);
}

ew_status_t ew_saxpy_relu_f32(float alpha, const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSaxpyReluF32, y, x, y, n, alpha, s);
}

ew_status_t ew_saxpy_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSaxpyF16, y, x, y, n, alpha, s);
}

ew_status_t ew_saxpy_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSaxpyBF16, y, x, y, n, alpha, s);
}

ew_status_t ew_relu_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpReluF16, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_relu_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpReluBF16, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_scale_f32(float alpha, const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpScaleF32, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_scale_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpScaleF16, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_scale_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpScaleBF16, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_add_scalar_f32(float alpha, const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpAddScalarF32, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_add_scalar_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                              hipStream_t s)
{
    return run_stream(kOpAddScalarF16, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_add_scalar_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                               hipStream_t s)
{
    return run_stream(kOpAddScalarBF16, y, x, nullptr, n, alpha, s);
}

ew_status_t ew_sqrt_f32(const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSqrtF32, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_sqrt_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSqrtF16, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_sqrt_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpSqrtBF16, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_abs_f32(const float *x, float *y, size_t n, hipStream_t s)
{
    return run_stream(kOpAbsF32, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_abs_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpAbsF16, y, x, nullptr, n, 0.0f, s);
}

ew_status_t ew_abs_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t s)
{
    return run_stream(kOpAbsBF16, y, x, nullptr, n, 0.0f, s);
}

}  // extern "C"

namespace ew {
namespace {

// Validation shared by the batched entry points: every item (n > 0) as its
// single call, the sum of n below 2^62, and no output range intersecting a
// range of another item.  *total = the sum of n.
ew_status_t batch_validate(int op, const ew_batch_item_t *items, size_t count, size_t *total)
{
    size_t sum = 0;
    for (size_t i = 0; i < count; ++i) {
        const ew_batch_item_t &it = items[i];
        if (it.n == 0) continue;
        const void *in1 = in_place_second(op) ? it.out : it.in1;
        const ew_status_t st = validate(op, it.out, it.in0, in1, it.n);
        if (st != EW_OK) return st;
        if (it.n > (size_t(1) << 62) - sum) return EW_ERR_INVALID_ARG;
        sum += it.n;
    }
    ew_status_t st;
    try {
        st = batch_overlap(op, items, count);
    } catch (...) {      // no exception crosses the C ABI (the check's vectors: 3 x count)
        return EW_ERR_INVALID_ARG;
    }
    *total = sum;
    return st;
}

// The launch shape of a batched call: the table's row for the total element
// count (unroll at most 4), with the tile shrunk -- unroll first, then the
// block, down to 64 threads -- while half of it still covers the items' mean
// vector count (a tile longer than an item leaves its lanes idle).  A shrunk
// tile takes one block per tile (blocks_per_cu raised so that the grid
// covers the tiles).
Row batch_row(int op, const ew_batch_item_t *items, size_t count, size_t total)
{
    Row r = get_row(op, total);
    if (r.unroll > 4) r.unroll = 4;
    const uint64_t vec = 16 / (uint64_t)kOps[op].elem_size;
    uint64_t live = 0, vectors = 0;
    for (size_t i = 0; i < count; ++i) {
        if (items[i].n == 0) continue;
        ++live;
        vectors += items[i].n / vec;
    }
    if (live == 0) return r;
    const uint64_t mean = (vectors + live - 1) / live;
    bool shrunk = false;
    while (r.unroll > 1 && (uint64_t)r.block * (uint64_t)r.unroll / 2 >= mean) {
        r.unroll /= 2;
        shrunk = true;
    }
    while (r.block > 64 && (uint64_t)r.block / 2 >= mean) {
        r.block /= 2;
        shrunk = true;
    }
    if (shrunk) r.blocks_per_cu = 1024;
    return r;
}

// Tiles of one item (n > 0) under tiles of tile_vecs vectors: the single
// call's vector count decides them (the kernel recomputes the split from the
// same pointer and n); at least one, for the scalar head and tail.
uint64_t item_tiles(int op, const ew_batch_item_t &it, uint64_t tile_vecs)
{
    const size_t es = (size_t)kOps[op].elem_size;
    const uintptr_t o = reinterpret_cast<uintptr_t>(it.out);
    size_t head = ((16 - (o % 16)) % 16) / es;
    if (head > it.n) head = it.n;
    const uint64_t vectors = (it.n - head) / (16 / es);
    const uint64_t tiles = (vectors + tile_vecs - 1) / tile_vecs;
    return tiles ? tiles : 1;
}

// Bytes of a table image with `items` records and `tiles` tile entries
// (8-byte multiple), or 0 if that does not fit in size_t.
size_t table_image_bytes(uint64_t items, uint64_t tiles)
{
    const uint64_t rec = (uint64_t)sizeof(BatchTableItem);
    if (items > (SIZE_MAX / 2) / rec) return 0;
    const uint64_t head = items * rec;
    if (tiles > (SIZE_MAX / 2 - head) / 4) return 0;
    return (size_t)((head + 4 * tiles + 7) & ~uint64_t(7));
}

}  // namespace
}  // namespace ew

extern "C" {

ew_status_t ew_batch(const char *op_name, float alpha, const ew_batch_item_t *items,
                     size_t count, hipStream_t s)
{
    const int op = op_from_name(op_name);
    if (op < 0 || !batchable(op)) return EW_ERR_INVALID_ARG;
    if (count == 0) return EW_OK;
    if (!items) return EW_ERR_INVALID_ARG;
    size_t total = 0;
    ew_status_t st = batch_validate(op, items, count, &total);
    if (st != EW_OK) return st;
    if (total == 0) return EW_OK;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    // One launch shape for the whole call.
    const Row r = batch_row(op, items, count, total);
    const uint64_t tile_vecs = (uint64_t)r.block * (uint64_t)r.unroll;
    BatchArgs a{};
    a.alpha = alpha;
    size_t i = 0;
    while (i < count) {
        a.count = 0;
        a.tiles = 0;
        for (; i < count && a.count < (uint32_t)kBatchMax; ++i) {
            const ew_batch_item_t &it = items[i];
            if (it.n == 0) continue;
            const void *in1 = kOps[op].inputs == 2 ? (in_place_second(op) ? it.out : it.in1)
                                                   : nullptr;
            a.item[a.count] = BatchItem{it.in0, in1, it.out, (uint64_t)it.n};
            a.tiles += item_tiles(op, it, tile_vecs);
            a.tile_end[a.count] = a.tiles;
            ++a.count;
        }
        if (a.count == 0) break;
        uint64_t grid = (uint64_t)r.blocks_per_cu * (uint64_t)(cus > 0 ? cus : 1);
        if (grid > a.tiles) grid = a.tiles;
        const Launch l{r.block, (int)grid, r.unroll};
        log_launch(kOps[op].name, (size_t)a.count, 0, a.tiles, 0, l,
                   "batch (n = items, vectors = tiles)");
        const hipError_t e = launch_batch(static_cast<OpId>(op), a, l, s);
        if (e != hipSuccess) return fail_hip(e);
    }
    return EW_OK;
}

ew_status_t ew_batch_build(const char *op_name, const ew_batch_item_t *items, size_t count,
                           void *table, size_t table_bytes, ew_batch_plan_t *plan)
{
    if (!plan) return EW_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof *plan);
    const int op = op_from_name(op_name);
    if (op < 0 || !batchable(op)) return EW_ERR_INVALID_ARG;
    if (count > 0 && !items) return EW_ERR_INVALID_ARG;
    size_t total = 0;
    ew_status_t st = batch_validate(op, items, count, &total);
    if (st != EW_OK) return st;
    const Row r = batch_row(op, items, count, total);
    const uint64_t tile_vecs = (uint64_t)r.block * (uint64_t)r.unroll;
    uint64_t live = 0, tiles = 0;
    for (size_t i = 0; i < count; ++i) {
        if (items[i].n == 0) continue;
        ++live;
        tiles += item_tiles(op, items[i], tile_vecs);
    }
    if (live > UINT32_MAX) return EW_ERR_INVALID_ARG;   // item indices are 32-bit
    const size_t bytes = table_image_bytes(live, tiles);
    if (live > 0 && bytes == 0) return EW_ERR_INVALID_ARG;
    plan->op = op;
    plan->block = r.block;
    plan->unroll = r.unroll;
    plan->blocks_per_cu = r.blocks_per_cu;
    plan->items = live;
    plan->tiles = tiles;
    plan->bytes = bytes;
    plan->total_n = total;
    if (!table) return EW_OK;                           // size query
    if (table_bytes < bytes) return EW_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(table) % 8 != 0) return EW_ERR_MISALIGNED;
    BatchTableItem *rec = static_cast<BatchTableItem *>(table);
    uint32_t *tile_item = reinterpret_cast<uint32_t *>(static_cast<char *>(table) +
                                                       live * sizeof(BatchTableItem));
    uint64_t k = 0, t = 0;
    for (size_t i = 0; i < count; ++i) {
        const ew_batch_item_t &it = items[i];
        if (it.n == 0) continue;
        const void *in1 = kOps[op].inputs == 2 ? (in_place_second(op) ? it.out : it.in1)
                                               : nullptr;
        const uint64_t nt = item_tiles(op, it, tile_vecs);
        rec[k] = BatchTableItem{it.in0, in1, it.out, (uint64_t)it.n, t};
        for (uint64_t q = 0; q < nt; ++q) tile_item[t + q] = (uint32_t)k;
        t += nt;
        ++k;
    }
    // the padding word, if any, is defined too
    const size_t used = live * sizeof(BatchTableItem) + 4 * tiles;
    if (bytes > used) std::memset(static_cast<char *>(table) + used, 0, bytes - used);
    return EW_OK;
}

}  // extern "C"

namespace ew {
namespace {

// A built plan's fields, checked for consistency (plan->tiles > 0).
bool plan_consistent(const ew_batch_plan_t *plan)
{
    const int op = plan->op;
    return op >= 0 && op < kOpCount && batchable(op) &&
           valid_row(plan->block, plan->blocks_per_cu, plan->unroll) && plan->unroll <= 4 &&
           plan->items > 0 && plan->items <= UINT32_MAX && plan->tiles >= plan->items &&
           plan->bytes == table_image_bytes(plan->items, plan->tiles);
}

// One launch of the table kernel over a table image at device address
// `table` (plan checked, device known).
ew_status_t launch_table(const ew_batch_plan_t *plan, float alpha, const void *table, int cus,
                         hipStream_t s, const char *path)
{
    const int op = plan->op;
    uint64_t grid = (uint64_t)plan->blocks_per_cu * (uint64_t)cus;
    if (grid > plan->tiles) grid = plan->tiles;
    const Launch l{plan->block, (int)grid, plan->unroll};
    BatchTableArgs a{};
    a.item = static_cast<const BatchTableItem *>(table);
    a.tile_item = reinterpret_cast<const uint32_t *>(static_cast<const char *>(table) +
                                                     plan->items * sizeof(BatchTableItem));
    a.tiles = plan->tiles;
    a.alpha = alpha;
    log_launch(kOps[op].name, (size_t)plan->items, 0, plan->tiles, 0, l, path);
    const hipError_t e = launch_batch_table(static_cast<OpId>(op), a, l, s);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

}  // namespace
}  // namespace ew

extern "C" {

ew_status_t ew_batch_run(const ew_batch_plan_t *plan, float alpha, const void *table,
                         hipStream_t s)
{
    if (!plan) return EW_ERR_INVALID_ARG;
    if (plan->tiles == 0) return EW_OK;
    if (!table) return EW_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(table) % 8 != 0) return EW_ERR_MISALIGNED;
    if (!plan_consistent(plan)) return EW_ERR_INVALID_ARG;
    int cus = 0;
    const ew_status_t st = current_device(&cus);
    if (st != EW_OK) return st;
    return launch_table(plan, alpha, table, cus, s, "batch table (n = items, vectors = tiles)");
}

ew_status_t ew_batch_run_static(const ew_batch_plan_t *plan, float alpha, const void *table_host,
                                hipStream_t s)
{
    if (!plan) return EW_ERR_INVALID_ARG;
    if (plan->tiles == 0) return EW_OK;
    if (!table_host) return EW_ERR_INVALID_ARG;
    if (!plan_consistent(plan)) return EW_ERR_INVALID_ARG;
    if (plan->bytes > kBatchScratchBytes) return EW_ERR_TOO_LARGE;
    int cus = 0;
    ew_status_t st = current_device(&cus);
    if (st != EW_OK) return st;
    void *table = nullptr;
    hipError_t e = batch_scratch(&table);
    if (e != hipSuccess) return fail_hip(e);
    // The array still holds the table of the previous call on this device,
    // which a kernel on this stream may still be reading: wait for the
    // stream, copy, and wait for the copy, so that the caller may reuse its
    // image once the call returns.
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail_hip(e);
    e = hipMemcpyAsync(table, table_host, plan->bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail_hip(e);
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail_hip(e);
    return launch_table(plan, alpha, table, cus, s,
                        "batch table in static scratch (n = items, vectors = tiles)");
}

ew_status_t ew_relu_inplace_f32(float *x, size_t n, hipStream_t s)
{
    if (n == 0) return EW_OK;
    ew_status_t st = validate(kOpReluInplaceF32, x, x, nullptr, n);
    if (st != EW_OK) return st;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    const Plan p = make_plan(kOpReluInplaceF32, x, x, nullptr, n, cus);
    StreamArgs a{};
    a.in0 = x;
    a.out = x;
    a.head = p.head;
    a.vectors = p.vectors;
    a.tail = p.tail;
    a.tiles = p.tiles;
    log_launch("relu_inplace_f32", n, p.head, p.vectors, p.tail, p.launch, "64-byte spans");
    const hipError_t e = launch_relu_inplace(a, p.launch, s);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

}  // extern "C"

namespace ew {
namespace {

// Argument checks of a strided view copy (rows, cols > 0), before any HIP
// call.
ew_status_t copy2d_check(const float *in, int64_t stride_r, int64_t stride_c, const float *out,
                         size_t rows, size_t cols)
{
    if (!in || !out || rows > SIZE_MAX / cols) return EW_ERR_INVALID_ARG;
    const size_t n = rows * cols;
    if (n >= (size_t(1) << 62) || n > SIZE_MAX / 4) return EW_ERR_INVALID_ARG;
    // Element offsets touched in the input: [lo, hi], exact in 128 bits.
    const __int128 er = (__int128)(rows - 1) * stride_r, ec = (__int128)(cols - 1) * stride_c;
    const __int128 lo = (er < 0 ? er : 0) + (ec < 0 ? ec : 0);
    const __int128 hi = (er > 0 ? er : 0) + (ec > 0 ? ec : 0);
    const __int128 ip = (__int128)reinterpret_cast<uintptr_t>(in);
    const __int128 in_lo = ip + 4 * lo, in_hi = ip + 4 * (hi + 1);   // byte range [in_lo, in_hi)
    if (in_lo < 0 || in_hi > (__int128)UINTPTR_MAX) return EW_ERR_INVALID_ARG;
    const uintptr_t op = reinterpret_cast<uintptr_t>(out);
    if (op > UINTPTR_MAX - n * 4) return EW_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(in) % 4 != 0 || op % 4 != 0) return EW_ERR_MISALIGNED;
    if (in_lo < (__int128)op + (__int128)(n * 4) && (__int128)op < in_hi) return EW_ERR_OVERLAP;
    return EW_OK;
}

// The launch of a strided view copy: its path, kernel arguments and shape.
struct Copy2dPlan {
    int path;            // an ew_path_t
    Launch launch;       // as launched (a kernel with a fixed block reports that block)
    int blocks_per_cu;
    Copy2dArgs a;        // EW_PATH_VIEW_*
    GatherArgs g;        // EW_PATH_GATHER_SPANS / EW_PATH_GATHER_PASSES
};

// Path: a 1-D view with stride 2 (x[::2]) reads contiguous 16-byte spans and
// keeps the even elements (the stride-2 gather kernel, one segment, no wrap);
// a 1-D view with stride 3..32 keeps one element in s of contiguously read
// spans (the pass kernel's residue-0 run); rows contiguous; a transposed view
// (tiles through LDS); generic.  Arguments already checked.
Copy2dPlan copy2d_plan(const float *in, int64_t stride_r, int64_t stride_c, float *out,
                       size_t rows, size_t cols, int cus)
{
    const size_t n = rows * cols;
    const Plan p = make_plan(kOpCopy2dF32, out, out, nullptr, n, cus);
    Copy2dPlan c{};
    c.blocks_per_cu = p.blocks_per_cu;
    Copy2dArgs &a = c.a;
    a.in = reinterpret_cast<const uint32_t *>(in);
    a.out = reinterpret_cast<uint32_t *>(out);
    a.sr = stride_r;
    a.sc = stride_c;
    a.rows = rows;
    a.cols = cols;
    a.head = p.head;
    a.vectors = p.vectors;
    a.tail = p.tail;
    a.tiles = p.tiles;
    const uint64_t sv = 4 * (uint64_t)p.launch.block;
    const unsigned __int128 st_t = (unsigned __int128)sv * (uint64_t)p.launch.unroll *
                                   (uint64_t)p.launch.grid;
    a.step_vec_r = sv / cols;
    a.step_vec_c = sv % cols;
    a.step_tile_r = (uint64_t)(st_t / cols);
    a.step_tile_c = (uint64_t)(st_t % cols);
    if (rows == 1 && stride_c == 2) {
        GatherArgs &g = c.g;
        g.in = a.in;
        g.out = a.out;
        g.n = 2 * n;
        g.stride = 2;
        g.seg = n;
        g.reps = 1;
        const Plan pg = make_plan(kOpGatherF32, out, in, nullptr, n, cus);
        // The kernel reads 16 bytes per output pair (input elements 2i ..
        // 2i + 3); the view ends at element 2(n - 1), so the body must stop
        // one output early (head + 4 * vectors <= n - 1) and the scalar tail,
        // which reads only in[2e], finishes the rest (1 to 4 elements).
        g.head = pg.head;
        g.vectors = n - 1 >= pg.head ? (n - 1 - pg.head) / 4 : 0;
        g.tail = n - g.head - 4 * g.vectors;
        const uint64_t tile_vecs = (uint64_t)pg.launch.block * (uint64_t)pg.launch.unroll;
        g.tiles = (g.vectors + tile_vecs - 1) / tile_vecs;
        c.launch = pg.launch;
        c.blocks_per_cu = pg.blocks_per_cu;
        const uint64_t cap = (uint64_t)pg.blocks_per_cu * (uint64_t)cus;
        c.launch.grid = (int)(g.tiles == 0 ? 1 : (g.tiles < cap ? g.tiles : cap));
        c.path = EW_PATH_GATHER_SPANS;
        return c;
    }
    if (rows == 1 && stride_c >= 3 && stride_c <= kMaxPasses) {
        // x[::s]: each wave reads its 1 KiB * s input span contiguously and
        // keeps every s-th element.  n (the kernel's input length) is the
        // view's extent.
        GatherArgs &g = c.g;
        g.in = a.in;
        g.out = a.out;
        g.stride = (uint64_t)stride_c;
        g.n = (uint64_t)stride_c * (n - 1) + 1;
        g.passes = (int)stride_c;
        g.skip = (int)stride_c;
        g.dest[0] = 0;
        g.seg = n;
        g.reps = 1;
        g.vectors = (n + 3) / 4;
        const uint64_t tile = (uint64_t)gather_passes_threads();
        g.tiles = (g.vectors + tile - 1) / tile;
        const uint64_t cap = (uint64_t)p.blocks_per_cu * (uint64_t)cus;
        c.launch = Launch{gather_passes_threads(), (int)(g.tiles < cap ? g.tiles : cap), 1};
        if (c.launch.grid == 0) c.launch.grid = 1;
        c.path = EW_PATH_GATHER_PASSES;
        return c;
    }
    c.launch = p.launch;
    c.path = EW_PATH_VIEW_GENERIC;
    if (stride_c == 1) {
        c.path = EW_PATH_VIEW_ROWS;
    } else if (stride_r == 1 && rows >= 2 && cols >= 2) {
        c.path = EW_PATH_VIEW_TRANSPOSE;
        // 128 x 128 tiles of 1024 threads; the grid is capped at
        // blocks_per_cu blocks per CU (the table's row for this size), beyond
        // which blocks stride
        const uint64_t tiles = ((rows + 127) / 128) * ((cols + 127) / 128);
        const uint64_t cap = (uint64_t)cus * (uint64_t)p.blocks_per_cu;
        c.launch.grid = (int)(tiles < cap ? tiles : cap);
        c.launch.block = transpose_threads();
        c.launch.unroll = 1;
    }
    return c;
}

}  // namespace
}  // namespace ew

extern "C" {

ew_status_t ew_copy2d_f32(const float *in, int64_t stride_r, int64_t stride_c, float *out,
                          size_t rows, size_t cols, hipStream_t s)
{
    if (rows == 0 || cols == 0) return EW_OK;
    ew_status_t st = copy2d_check(in, stride_r, stride_c, out, rows, cols);
    if (st != EW_OK) return st;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    const Copy2dPlan c = copy2d_plan(in, stride_r, stride_c, out, rows, cols, cus);
    const size_t n = rows * cols;
    hipError_t e;
    switch (c.path) {
    case EW_PATH_GATHER_SPANS:
        log_launch("copy2d_f32", n, c.g.head, c.g.vectors, c.g.tail, c.launch, "view x[::2]");
        e = launch_gather(c.g, c.launch, s);
        break;
    case EW_PATH_GATHER_PASSES:
        log_launch("copy2d_f32", n, 0, c.g.vectors, 0, c.launch, "view x[::s], s = 3..32");
        e = launch_gather(c.g, c.launch, s);
        break;
    default: {
        const int mode = c.path == EW_PATH_VIEW_ROWS ? 1 : c.path == EW_PATH_VIEW_TRANSPOSE ? 2 : 0;
        log_launch("copy2d_f32", n, c.a.head, c.a.vectors, c.a.tail, c.launch,
                   mode == 1 ? "rows contiguous" : mode == 2 ? "transpose tiles" : "generic");
        e = launch_copy2d(c.a, mode, c.launch, s);
    }
    }
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

ew_status_t ew_make_copy2d_plan(const void *in, int64_t stride_r, int64_t stride_c,
                                const void *out, size_t rows, size_t cols, int cu_count,
                                ew_plan_t *plan)
{
    if (!plan || cu_count <= 0) return EW_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof *plan);
    plan->vec_elems = 4;
    plan->elem_size = 4;
    plan->in_coaligned[0] = plan->in_coaligned[1] = 1;
    plan->reps = 1;
    plan->passes = 1;
    if (rows == 0 || cols == 0) return EW_OK;
    const float *inf = static_cast<const float *>(in);
    float *outf = static_cast<float *>(const_cast<void *>(out));
    const ew_status_t st = copy2d_check(inf, stride_r, stride_c, outf, rows, cols);
    if (st != EW_OK) return st;
    const Copy2dPlan c = copy2d_plan(inf, stride_r, stride_c, outf, rows, cols, cu_count);
    const bool gather = c.path == EW_PATH_GATHER_SPANS || c.path == EW_PATH_GATHER_PASSES;
    plan->n = rows * cols;
    plan->head = gather ? c.g.head : c.a.head;
    plan->vectors = gather ? c.g.vectors : c.a.vectors;
    plan->tail = gather ? c.g.tail : c.a.tail;
    plan->tiles = gather ? c.g.tiles : c.a.tiles;
    if (c.path == EW_PATH_VIEW_TRANSPOSE) plan->tiles = ((rows + 127) / 128) * ((cols + 127) / 128);
    plan->block = c.launch.block;
    plan->grid = c.launch.grid;
    plan->unroll = c.launch.unroll;
    plan->blocks_per_cu = c.blocks_per_cu;
    plan->segment = plan->n;
    plan->path = c.path;
    return EW_OK;
}

ew_status_t ew_bias_relu_f32(const float *x, const float *bias, float *y, size_t rows,
                             size_t cols, hipStream_t s)
{
    if (rows == 0 || cols == 0) return EW_OK;
    if (!bias || rows > SIZE_MAX / cols) return EW_ERR_INVALID_ARG;
    const size_t n = rows * cols;
    ew_status_t st = validate(kOpBiasReluF32, y, x, nullptr, n);
    if (st != EW_OK) return st;
    const uintptr_t bp = reinterpret_cast<uintptr_t>(bias);
    if (cols > SIZE_MAX / 4 || bp > UINTPTR_MAX - cols * 4) return EW_ERR_INVALID_ARG;
    if (bp % 4 != 0) return EW_ERR_MISALIGNED;
    const uintptr_t yp = reinterpret_cast<uintptr_t>(y);
    if (bp < yp + n * 4 && yp < bp + cols * 4) return EW_ERR_OVERLAP;
    int cus = 0;
    st = current_device(&cus);
    if (st != EW_OK) return st;
    const Plan p = make_plan(kOpBiasReluF32, y, x, nullptr, n, cus);
    BiasArgs a{};
    a.x = x;
    a.bias = bias;
    a.y = y;
    a.cols = cols;
    a.head = p.head;
    a.vectors = p.vectors;
    a.tail = p.tail;
    a.tiles = p.tiles;
    const uint64_t nthr = (uint64_t)p.launch.block;
    a.step_vec = (4 * nthr) % cols;
    a.step_tile = mulmod_host((4 * nthr * (uint64_t)p.launch.unroll) % cols,
                              (uint64_t)p.launch.grid % cols, cols);
    log_launch("bias_relu_f32", n, p.head, p.vectors, p.tail, p.launch, "bias row broadcast");
    const hipError_t e = launch_bias_relu(a, p.co[0], p.launch, s);
    return e == hipSuccess ? EW_OK : fail_hip(e);
}

static_assert(sizeof(ew_status_t) == sizeof(int), "the status enum is an int in C");

const char *ew_status_string(ew_status_t status)
{
    // A C caller may pass any int.  In C++ a value outside the enumerators'
    // range read as the enum type is undefined, so the bytes are read as int.
    int v;
    std::memcpy(&v, &status, sizeof v);
    switch (v) {
    case EW_OK: return "EW_OK";
    case EW_ERR_INVALID_ARG: return "EW_ERR_INVALID_ARG: null pointer, invalid size, stride or op";
    case EW_ERR_MISALIGNED: return "EW_ERR_MISALIGNED: pointer not aligned to its element size";
    case EW_ERR_OVERLAP: return "EW_ERR_OVERLAP: output partially overlaps an input";
    case EW_ERR_NO_DEVICE: return "EW_ERR_NO_DEVICE: no usable HIP device";
    case EW_ERR_HIP: return "EW_ERR_HIP: HIP runtime error (see ew_last_hip_error)";
    case EW_ERR_TOO_LARGE:
        return "EW_ERR_TOO_LARGE: the batch table exceeds the static scratch "
               "(EW_BATCH_SCRATCH_BYTES)";
    }
    return "EW_ERR_UNKNOWN";
}

int ew_last_hip_error(void) { return g_last_hip_error; }

int ew_abi_version(void) { return kAbiVersion; }

ew_status_t ew_set_launch_config(const char *op, int block, int blocks_per_cu, int unroll)
{
    const int id = op_from_name(op);
    if (id < 0 || !valid_row(block, blocks_per_cu, unroll)) return EW_ERR_INVALID_ARG;
    Table &t = table();
    std::lock_guard<std::mutex> g(t.mu);
    ensure_loaded_locked(t);
    Rows &rows = t.rows[id];
    rows.count = 1;
    rows.row[0] = Row{0, block, blocks_per_cu, unroll};
    return EW_OK;
}

ew_status_t ew_get_launch_config(const char *op, size_t n, int *block, int *grid, int *unroll)
{
    const int id = op_from_name(op);
    if (id < 0 || !block || !grid || !unroll) return EW_ERR_INVALID_ARG;
    int cus = 0;
    const ew_status_t st = current_device(&cus);
    if (st != EW_OK) return st;
    // the plan of a call whose pointers are all 256-byte aligned (what a
    // device allocation returns): no head, so only n decides the grid
    const Row r = get_row(id, n);
    const size_t es = (size_t)kOps[id].elem_size;
    const size_t tile_vecs = (size_t)r.block * (size_t)r.unroll;
    const size_t tiles = (n / (16 / es) + tile_vecs - 1) / tile_vecs;
    size_t g = (size_t)r.blocks_per_cu * (size_t)cus;
    if (g > tiles) g = tiles;
    if (g == 0 && n > 0) g = 1;  // a head or tail still needs one block
    *block = r.block;
    *grid = (int)g;
    *unroll = r.unroll;
    return EW_OK;
}

ew_status_t ew_set_launch_row(const char *op, size_t min_n, int block, int blocks_per_cu,
                              int unroll)
{
    return set_row(op_from_name(op), min_n, block, blocks_per_cu, unroll);
}

ew_status_t ew_get_launch_row(const char *op, size_t n, int *block, int *blocks_per_cu,
                              int *unroll)
{
    const int id = op_from_name(op);
    if (id < 0 || !block || !blocks_per_cu || !unroll) return EW_ERR_INVALID_ARG;
    const Row r = get_row(id, n);
    *block = r.block;
    *blocks_per_cu = r.blocks_per_cu;
    *unroll = r.unroll;
    return EW_OK;
}

void ew_reset_launch_config(void)
{
    Table &t = table();
    std::lock_guard<std::mutex> g(t.mu);
    reset_locked(t);
}

ew_status_t ew_load_launch_table(const char *path)
{
    if (!path) return EW_ERR_INVALID_ARG;
    FILE *f = std::fopen(path, "r");
    if (!f) return EW_ERR_INVALID_ARG;
    char line[512];
    ew_status_t st = EW_OK;
    while (std::fgets(line, sizeof line, f)) {
        char *hash = std::strchr(line, '#');
        if (hash) *hash = '\0';
        char name[64];
        unsigned long long min_n = 0;
        int block = 0, bpc = 0, unroll = 0;
        char extra[2];
        const int got = std::sscanf(line, "%63s %llu %d %d %d %1s", name, &min_n, &block, &bpc,
                                    &unroll, extra);
        if (got <= 0) continue;  // blank or comment-only line
        if (got != 5) {
            st = EW_ERR_INVALID_ARG;
            break;
        }
        st = set_row(op_from_name(name), (size_t)min_n, block, bpc, unroll);
        if (st != EW_OK) break;
    }
    std::fclose(f);
    return st;
}

ew_status_t ew_make_plan(const char *op, const void *out, const void *in0, const void *in1,
                         size_t n, int cu_count, ew_plan_t *plan)
{
    const int id = op_from_name(op);
    if (id < 0 || !plan || cu_count <= 0) return EW_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof *plan);
    if (n != 0) {
        const ew_status_t st = validate(id, out, in0, in1, n);
        if (st != EW_OK) return st;
    }
    const OpInfo &info = kOps[id];
    plan->n = n;
    plan->elem_size = info.elem_size;
    plan->vec_elems = 16 / info.elem_size;
    plan->in_coaligned[0] = plan->in_coaligned[1] = 1;
    plan->reps = 1;
    plan->passes = 1;
    const Row r = get_row(id, n);
    plan->block = r.block;
    plan->blocks_per_cu = r.blocks_per_cu;
    plan->unroll = r.unroll;
    if (n == 0) return EW_OK;
    // one table read for everything reported (another thread may be
    // rewriting the table)
    const Plan p = make_plan(id, out, in0, in1, n, cu_count);
    plan->block = p.launch.block;
    plan->blocks_per_cu = p.blocks_per_cu;
    plan->unroll = p.launch.unroll;
    plan->head = p.head;
    plan->vectors = p.vectors;
    plan->tail = p.tail;
    plan->tiles = p.tiles;
    plan->in_coaligned[0] = p.co[0] ? 1 : 0;
    plan->in_coaligned[1] = p.co[1] ? 1 : 0;
    plan->grid = p.launch.grid;
    plan->segment = n;
    plan->reps = 1;
    plan->passes = 1;
    plan->path = id == kOpGatherWalkF32 ? EW_PATH_GATHER_WALK : EW_PATH_STREAM;
    return EW_OK;
}

ew_status_t ew_make_gather_plan(const void *out, const void *in, size_t n, size_t stride,
                                int cu_count, ew_plan_t *plan)
{
    if (!plan || cu_count <= 0) return EW_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof *plan);
    if (n == 0) return EW_OK;
    if (stride == 0) return EW_ERR_INVALID_ARG;
    const ew_status_t st = validate(kOpGatherF32, out, in, nullptr, n);
    if (st != EW_OK) return st;
    if (n == 1 || stride % n == 1) {
        // out[i] = in[i mod n] = in[i]: ew_gather_f32 runs the contiguous copy
        const ew_status_t sc = ew_make_plan("copy_f32", out, in, nullptr, n, cu_count, plan);
        plan->path = EW_PATH_COPY;
        return sc;
    }
    GatherArgs g{};
    Launch l{};
    int bpc = 0;
    gather_plan(static_cast<const float *>(in), static_cast<float *>(const_cast<void *>(out)), n,
                stride, cu_count, &g, &l, &bpc);
    plan->path = g.passes ? EW_PATH_GATHER_PASSES
                 : g.tile_mode ? EW_PATH_GATHER_TILES
                 : (g.stride == 2 && g.reps == 2) ? EW_PATH_GATHER_SPANS
                 : EW_PATH_GATHER_WALK;
    plan->n = n;
    plan->head = g.head;
    plan->vectors = g.vectors;
    plan->tail = g.tail;
    plan->tiles = g.tiles;
    plan->vec_elems = 4;
    plan->elem_size = 4;
    plan->in_coaligned[0] = plan->in_coaligned[1] = 1;
    plan->block = l.block;
    plan->blocks_per_cu = bpc;
    plan->unroll = l.unroll;
    plan->grid = l.grid;
    plan->segment = g.seg;
    plan->reps = (int)g.reps;
    // runs per segment (the tiled path's s' is clamped to INT_MAX)
    plan->passes = g.passes     ? g.passes / g.skip
                   : g.tile_mode ? (int)std::min<uint64_t>(g.sp, (uint64_t)INT_MAX)
                                 : 1;
    return EW_OK;
}

}  // extern "C"
