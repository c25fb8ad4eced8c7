// ew_batch.hip -- batched streaming calls for CDNA4 (gfx950): many small
// arrays of one operation in one kernel launch.

#include "ew_device.h"
#include "ew_batch_args.h"

#include <mutex>

namespace ew {

// ---------------------------------------------------------------------------
// Batched streaming: independent operand sets of one operation, one launch
// ---------------------------------------------------------------------------

// One tile of one batch item: the body of ew_stream_kernel for local tile lt.
template <class Op, int U, bool Co0, bool Co1>
__device__ __forceinline__ void batch_tile(const char *in0, const char *in1, char *out,
                                           uint64_t vectors, uint64_t lt, uint32_t tid,
                                           uint64_t nthr, float alpha)
{
    using E = typename Op::Elem;
    constexpr uint64_t kElem = sizeof(E);
    constexpr bool kTwo = Op::kInputs == 2;
    const uint64_t tile_vecs = nthr * U;
    const uint64_t v0 = lt * tile_vecs + tid;
    char *tile = out + lt * tile_vecs * 16;
    const uint32_t tile_bytes = (uint32_t)(tile_vecs * 16);
    if (v0 + (U - 1) * nthr < vectors) {
        u32x4 x[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = load16<Co0, kElem>(in0 + (v0 + u * nthr) * 16);
        if constexpr (kTwo) {
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = load16<Co1, kElem>(in1 + (v0 + u * nthr) * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 b = kTwo ? y[u] : u32x4{0, 0, 0, 0};
            if constexpr (kTwo)
                store16(out + (v0 + u * nthr) * 16, Op::vec(x[u], b, alpha));
            else
                store16_device(tile, tile_bytes, (uint32_t)((tid + u * nthr) * 16),
                               Op::vec(x[u], b, alpha));
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t v = v0 + u * nthr;
            if (v < vectors) {
                const u32x4 a = load16<Co0, kElem>(in0 + v * 16);
                const u32x4 b = kTwo ? load16<Co1, kElem>(in1 + v * 16) : u32x4{0, 0, 0, 0};
                if constexpr (kTwo)
                    store16(out + v * 16, Op::vec(a, b, alpha));
                else
                    store16_device(tile, tile_bytes, (uint32_t)((tid + u * nthr) * 16),
                                   Op::vec(a, b, alpha));
            }
        }
    }
}

// One tile of one item of a batched call: the item's split is recomputed from
// its pointers and n exactly as the host plans a single call (the head
// aligns the output to 16 bytes), the item's first tile (lt == 0) also does
// the scalar head and tail, and the tile's vectors stream with the item's
// own alignment path.  Block-uniform arguments.
template <class Op, int U>
__device__ __forceinline__ void batch_item_tile(const void *in0v, const void *in1v, void *outv,
                                                uint64_t n, uint64_t lt, float alpha)
{
    using E = typename Op::Elem;
    constexpr uint64_t kVec = 16 / sizeof(E);
    constexpr bool kTwo = Op::kInputs == 2;
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    uint64_t head = ((16u - (reinterpret_cast<uintptr_t>(outv) & 15u)) & 15u) / sizeof(E);
    if (head > n) head = n;
    const uint64_t vectors = (n - head) / kVec;
    const uint64_t tail = n - head - vectors * kVec;
    if (lt == 0 && tid < head + tail) {
        const uint64_t e = tid < head ? (uint64_t)tid : head + vectors * kVec + (tid - head);
        const E a = static_cast<const E *>(in0v)[e];
        const E b = kTwo ? static_cast<const E *>(in1v)[e] : E(0);
        static_cast<E *>(outv)[e] = Op::one(a, b, alpha);
    }
    const char *in0 = static_cast<const char *>(in0v) + head * sizeof(E);
    const char *in1 = kTwo ? static_cast<const char *>(in1v) + head * sizeof(E) : nullptr;
    char *out = static_cast<char *>(outv) + head * sizeof(E);
    const bool co0 = (reinterpret_cast<uintptr_t>(in0) & 15u) == 0;
    const bool co1 = !kTwo || (reinterpret_cast<uintptr_t>(in1) & 15u) == 0;
    if constexpr (kTwo) {
        if (co0 && co1) batch_tile<Op, U, true, true>(in0, in1, out, vectors, lt, tid, nthr, alpha);
        else if (co0) batch_tile<Op, U, true, false>(in0, in1, out, vectors, lt, tid, nthr, alpha);
        else if (co1) batch_tile<Op, U, false, true>(in0, in1, out, vectors, lt, tid, nthr, alpha);
        else batch_tile<Op, U, false, false>(in0, in1, out, vectors, lt, tid, nthr, alpha);
    } else {
        if (co0) batch_tile<Op, U, true, true>(in0, in1, out, vectors, lt, tid, nthr, alpha);
        else batch_tile<Op, U, false, true>(in0, in1, out, vectors, lt, tid, nthr, alpha);
    }
}

// Many small arrays cost one launch each through the single-array entry
// points, and below about 2^21 elements the launch, not HBM, sets the time
// ([HyperAI] Stage 3: the smallest size runs at the same few microseconds in
// every version).  Here the tiles of all items are numbered consecutively and
// walked with a grid stride; a block finds the item that owns its tile by a
// binary search over tile_end (block-uniform, kernel-argument loads) and
// runs batch_item_tile.  At most kBatchMax items travel in the kernel
// arguments.
template <class Op, int U>
__global__ void __launch_bounds__(1024) ew_batch_kernel(BatchArgs args)
{
    for (uint64_t t = blockIdx.x; t < args.tiles; t += gridDim.x) {
        uint32_t lo = 0, hi = args.count - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) / 2;
            if (args.tile_end[mid] > t) hi = mid;
            else lo = mid + 1;
        }
        const BatchItem &it = args.item[lo];
        const uint64_t lt = t - (lo ? args.tile_end[lo - 1] : 0);
        batch_item_tile<Op, U>(it.in0, it.in1, it.out, it.n, lt, args.alpha);
    }
}

// A pointer read from memory is generic to the compiler (it could address
// LDS or scratch), so accesses through it would be flat instructions.  The
// item table holds global-memory pointers by contract; this re-types one as
// global, so that the accesses after inlining are global (and buffer)
// instructions like those of the single-call kernels.
template <typename T>
__device__ __forceinline__ T *as_global(T *p)
{
    typedef __attribute__((address_space(1))) T *GlobalPtr;
    return (T *)(GlobalPtr)(uintptr_t)p;
}

// The same work with the item table in device memory, so that one launch
// runs any number of items: the table (built on the host by the library,
// placed in device memory by the caller) holds every item with its first
// global tile and, per tile, the index of the item that owns it.  A block
// reads its tile's item index and the item's record with two dependent
// block-uniform loads (read-only, not aliased: scalar loads), no search.
template <class Op, int U>
__global__ void __launch_bounds__(1024)
    ew_batch_table_kernel(const BatchTableItem *__restrict__ item,
                          const uint32_t *__restrict__ tile_item, uint64_t tiles, float alpha)
{
    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const BatchTableItem &it = item[tile_item[t]];
        batch_item_tile<Op, U>(as_global(it.in0), as_global(it.in1), as_global(it.out), it.n,
                               t - it.first_tile, alpha);
    }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

namespace {

template <class Op>
hipError_t launch_batch_op(const BatchArgs &args, const Launch &l, hipStream_t s)
{
    BatchArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    switch (l.unroll) {
    case 1: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 1>); break;
    case 2: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 2>); break;
    case 4: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 4>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}

template <class Op>
hipError_t launch_batch_table_op(const BatchTableArgs &args, const Launch &l, hipStream_t s)
{
    const BatchTableItem *item = args.item;
    const uint32_t *tile_item = args.tile_item;
    uint64_t tiles = args.tiles;
    float alpha = args.alpha;
    void *kargs[] = {&item, &tile_item, &tiles, &alpha};
    const void *fn = nullptr;
    switch (l.unroll) {
    case 1: fn = reinterpret_cast<const void *>(&ew_batch_table_kernel<Op, 1>); break;
    case 2: fn = reinterpret_cast<const void *>(&ew_batch_table_kernel<Op, 2>); break;
    case 4: fn = reinterpret_cast<const void *>(&ew_batch_table_kernel<Op, 4>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}

// The operator class of each batchable operation, handed to F as a type.
template <template <class> class F, class... A>
hipError_t by_op(OpId op, A &&...a)
{
    switch (op) {
    case kOpAddF32: return F<OpAddF32>::run(a...);
    case kOpAddF16: return F<OpAddF16>::run(a...);
    case kOpAddBF16: return F<OpAddBF16>::run(a...);
    case kOpSaxpyF32: return F<OpSaxpyF32>::run(a...);
    case kOpReluF32: return F<OpReluF32>::run(a...);
    case kOpCopyF32: return F<OpCopyF32>::run(a...);
    case kOpAddReluF32: return F<OpAddReluF32>::run(a...);
    case kOpSaxpyReluF32: return F<OpSaxpyReluF32>::run(a...);
    case kOpSaxpyF16: return F<OpSaxpyF16>::run(a...);
    case kOpSaxpyBF16: return F<OpSaxpyBF16>::run(a...);
    case kOpReluF16: return F<OpReluF16>::run(a...);
    case kOpReluBF16: return F<OpReluBF16>::run(a...);
    case kOpScaleF32: return F<OpScaleF32>::run(a...);
    case kOpScaleF16: return F<OpScaleF16>::run(a...);
    case kOpScaleBF16: return F<OpScaleBF16>::run(a...);
    case kOpAddScalarF32: return F<OpAddScalarF32>::run(a...);
    case kOpAddScalarF16: return F<OpAddScalarF16>::run(a...);
    case kOpAddScalarBF16: return F<OpAddScalarBF16>::run(a...);
    case kOpSqrtF32: return F<OpSqrtF32>::run(a...);
    case kOpSqrtF16: return F<OpSqrtF16>::run(a...);
    case kOpSqrtBF16: return F<OpSqrtBF16>::run(a...);
    case kOpAbsF32: return F<OpAbsF32>::run(a...);
    // binary16 and bfloat16 share the sign bit's position: one kernel
    case kOpAbsF16:
    case kOpAbsBF16: return F<OpAbs16>::run(a...);
    default: return hipErrorInvalidValue;
    }
}

template <class Op>
struct ArgsLauncher {
    static hipError_t run(const BatchArgs &args, const Launch &l, hipStream_t s)
    {
        return launch_batch_op<Op>(args, l, s);
    }
};

template <class Op>
struct TableLauncher {
    static hipError_t run(const BatchTableArgs &args, const Launch &l, hipStream_t s)
    {
        return launch_batch_table_op<Op>(args, l, s);
    }
};

}  // namespace

// The batch table of ew_batch_run_static, for callers that cannot allocate:
// one copy per GPU for the life of the process.  Host code never passes this
// name to a kernel or a copy (on the host it names a stand-in, not device
// memory); it uses the address batch_scratch() returns for the current device.
static __device__ __align__(256) unsigned char scratch[kBatchScratchBytes];

hipError_t batch_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_batch(OpId op, const BatchArgs &args, const Launch &l, hipStream_t s)
{
    return by_op<ArgsLauncher>(op, args, l, s);
}

hipError_t launch_batch_table(OpId op, const BatchTableArgs &args, const Launch &l,
                              hipStream_t s)
{
    return by_op<TableLauncher>(op, args, l, s);
}

}  // namespace ew
