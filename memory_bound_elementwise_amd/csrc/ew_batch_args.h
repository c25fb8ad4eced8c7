// ew_batch_args.h -- the batched calls' arguments and launchers, shared by
// the host API (ew_api.cpp) and ew_batch.hip.  Not installed; not part of the
// C ABI.
#pragma once

#include "ew_internal.h"

namespace ew {

// A batched call: up to kBatchMax independent operand sets of one streaming
// operation in one launch.  Item k owns the global tiles [tile_end[k - 1],
// tile_end[k]) -- at least one, so that its scalar head and tail have a block.
// Each block recomputes its item's head / vectors / tail split and input
// alignment from the pointers and n, exactly as the host plans a single
// call, so an item travels as four words.  The whole struct is the kernel
// argument (3856 bytes, under the 4 KiB kernel-argument limit).
constexpr int kBatchMax = 96;
struct BatchItem {
    const void *in0;
    const void *in1;     // nullptr for one-input operations
    void *out;
    uint64_t n;
};
struct BatchArgs {
    uint64_t tiles;      // tiles of all items together
    uint32_t count;      // items in this launch, 1..kBatchMax
    float alpha;         // saxpy, scale and add-scalar only
    uint64_t tile_end[kBatchMax];
    BatchItem item[kBatchMax];
};
static_assert(sizeof(BatchArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// A batched call whose item table lives in device memory (any number of
// items per launch).  Table image, 8-byte aligned: `count` BatchTableItem
// records, then one uint32_t per global tile naming the item that owns it.
// Item k owns the tiles [first_tile, first_tile + its tile count), at least
// one per item so that its scalar head and tail have a block.
struct BatchTableItem {
    const void *in0;
    const void *in1;     // nullptr for one-input operations
    void *out;
    uint64_t n;
    uint64_t first_tile;
};
static_assert(sizeof(BatchTableItem) == 40, "table record layout");
struct BatchTableArgs {
    const BatchTableItem *item;
    const uint32_t *tile_item;
    uint64_t tiles;      // tiles of all items together
    float alpha;         // saxpy, scale and add-scalar only
};

// Launch one batched streaming kernel (block and unroll from `launch`; the
// unroll must be 1, 2 or 4).
hipError_t launch_batch(OpId op, const BatchArgs &args, const Launch &launch,
                        hipStream_t stream);

// Launch one batched kernel reading its item table from device memory
// (unroll 1, 2 or 4).
hipError_t launch_batch_table(OpId op, const BatchTableArgs &args, const Launch &launch,
                              hipStream_t stream);

// Size of the library's static device array that holds a batch table for
// the entry point that allocates nothing (ew_batch_run_static).
constexpr uint64_t kBatchScratchBytes = 256 * 1024;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t batch_scratch(void **ptr);

}  // namespace ew
