// Schedule format shared by the host planner, the launcher and the gfx950 kernels.
//
// A plan is a list of forward work items.  An item is one run of KV blocks
// (a chunk of a prefix-tree node or of one query's private tail) together
// with the queries that attend over it.  Items of several queries read each
// shared block once for all of them (PAT review, memory-centric prefix-aware
// packing, Fig 5(d) caption).  An item runs for every KV head: as one task per
// KV head (MFMA items) or one task per group of four KV heads (VALU items).
// Tasks wait in per-XCD work queues, longest first, and persistent workgroups
// pull them.  MFMA and VALU tasks share one launch, so the MFMA work of packed
// groups overlaps the bandwidth-bound streaming of private tails.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvattn.h"

namespace kvattn {

constexpr int kBlock = 16;              // tokens per KV block
constexpr int kValuMaxRows = 8;         // rows per KV head the VALU path holds
constexpr int kWaves = 4;               // waves per forward workgroup (both paths)
constexpr int kMfmaMaxRows = 128;       // rows per MFMA item: 4 waves x 32 rows
constexpr int kMfmaTileTokens = 32;     // KV tokens per LDS stage
constexpr int kMfmaStages = 4;          // LDS stages of the MFMA pipeline (3 tiles in flight)
constexpr int kMaxItemBlocks = 512;     // KV blocks per item (8192 tokens)
constexpr int kMaxGroup = 64;           // q heads per KV head supported
constexpr int kQueues = 8;              // work queues, one per XCD of an MI355X
constexpr int kCounters = 16;           // per launch: kQueues cursors, one finished count, spare
constexpr uint32_t kBlobMagic = 0x4B564154u;  // "KVAT"
constexpr uint32_t kBlobVersion = 2;

// Device view of one item; identical layout to kvattn_item_info.
struct Item {
    int32_t kind;       // KVATTN_VARIANT_VALU / _MFMA
    int32_t tile;       // VALU: rows template (1,2,4,8); MFMA: 16-row tiles per wave (1 or 2)
    int32_t pos_begin;  // logical block position where the range starts
    int32_t n_tokens;   // tokens in the range
    int32_t q_begin;    // first Entry
    int32_t n_q;        // entries
    int32_t blk_begin;  // first block id
    int32_t n_rows;     // n_q * G
};
static_assert(sizeof(Item) == sizeof(kvattn_item_info), "item layout");

struct Entry {
    int32_t query;      // b
    int32_t dest;       // -1 direct; else partial slot of q head h = dest + h
    int32_t limit;      // tokens [0, limit) of the range are attended by this query
    int32_t pad;
};
static_assert(sizeof(Entry) == sizeof(kvattn_item_query), "entry layout");

// A forward task: one item for KV head `head` (MFMA) or for KV heads
// [head, head + 4) (VALU).
struct Task {
    int32_t item;
    int32_t head;
};

// Header at offset 0 of the device workspace.  Offsets are in bytes from the
// workspace base and 256-byte aligned.
struct BlobHeader {
    uint32_t magic, version;
    int32_t n_items, n_entries, n_block_ids, n_merge_q, n_slots, head_dim;
    int32_t n_tasks, n_launches, pad0, pad1;
    uint64_t off_items, off_entries, off_block_ids, off_merge_query, off_merge_ptr, off_merge_dest, off_zero;
    uint64_t off_tasks;       // Task [n_tasks], grouped by launch, then queue, longest first
    uint64_t off_queue_ptr;   // int32 [n_launches][kQueues + 1]: task ranges of each queue
    uint64_t off_counters;    // int32 [n_launches][kCounters]: zero at upload, zero after every launch
    uint64_t blob_bytes;      // bytes copied by kvattn_plan_upload
    uint64_t off_part_ml;     // float2 [n_slots]: (m in log2 units, l)
    uint64_t off_part_acc;    // float [n_slots][head_dim]
    uint64_t total_bytes;     // workspace bytes
};

// One forward launch: persistent workgroups draining its queues of MFMA and
// VALU tasks.  A plan needs more than one only when its VALU items use
// several row templates or its MFMA items several row tilings.
struct Launch {
    int valu_rows;     // VALU row template (1, 2, 4, 8)
    int mfma_tiles;    // MFMA 16-row tiles per wave (1, 2)
    int index;         // queue set
    int n_tasks;
    int task_base;     // first task of the launch
};

// Pointers the kernels take, resolved from the bound workspace.
struct DevPlan {
    const Item* items;
    const Entry* entries;
    const int32_t* block_ids;
    const Task* tasks;
    const int32_t* queue_ptr;   // this launch's kQueues + 1 offsets into tasks
    int32_t* counters;          // this launch's kCounters counters
    const int32_t* merge_query;
    const int32_t* merge_ptr;
    const int32_t* merge_dest;
    const uint16_t* zero;       // >= 256 zero bytes: source for token slots outside a range
    float* part_ml;
    float* part_acc;
};

struct Dims {
    int num_q_heads, num_kv_heads, head_dim, group;
    float scale_log2;         // softmax scale * log2(e): scores are kept in log2 units
};

// Kernel launchers (kvattn_kernels.hip).  Return hipSuccess or the launch error.
int launch_forward(const DevPlan& p, const Dims& d, int valu_rows, int mfma_tiles, int n_tasks,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream);
int launch_merge(const DevPlan& p, const Dims& d, int q_count, float* out, void* stream);

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace kvattn
