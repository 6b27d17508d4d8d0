// Schedule format shared by the host planner, the launcher and the gfx950 kernels.
//
// A plan is a list of forward work items.  An item is one run of KV blocks
// (a chunk of a prefix-tree node or of one query's private tail) together
// with the queries that attend over it; it runs once per KV head.  Items of
// several queries read each shared block once for all of them (PAT review,
// memory-centric prefix-aware packing, Fig 5(d) caption).
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvattn.h"

namespace kvattn {

constexpr int kBlock = 16;              // tokens per KV block
constexpr int kValuMaxRows = 8;         // rows per KV head the VALU kernel holds
constexpr int kMfmaRowsPerWave = 32;    // two 16-row MFMA tiles per wave
constexpr int kMfmaMaxWaves = 8;        // 256 rows per workgroup
constexpr int kMfmaTileTokens = 32;     // KV tokens per LDS stage
constexpr int kMaxItemBlocks = 512;     // KV blocks per item (8192 tokens)
constexpr int kMaxGroup = 64;           // q heads per KV head supported
constexpr uint32_t kBlobMagic = 0x4B564154u;  // "KVAT"
constexpr uint32_t kBlobVersion = 1;

// Device view of one item; identical layout to kvattn_item_info.
struct Item {
    int32_t kind;       // KVATTN_VARIANT_VALU / _MFMA
    int32_t tile;       // VALU: rows template (1,2,4,8); MFMA: waves per workgroup
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

// Header at offset 0 of the device workspace.  Offsets are in bytes from the
// workspace base and 256-byte aligned.
struct BlobHeader {
    uint32_t magic, version;
    int32_t n_items, n_entries, n_block_ids, n_merge_q, n_slots, head_dim;
    uint64_t off_items, off_entries, off_block_ids, off_merge_query, off_merge_ptr, off_merge_dest, off_zero;
    uint64_t blob_bytes;      // bytes copied by kvattn_plan_upload
    uint64_t off_part_ml;     // float2 [n_slots]: (m in log2 units, l)
    uint64_t off_part_acc;    // float [n_slots][head_dim]
    uint64_t total_bytes;     // workspace bytes
};

// One kernel launch of kvattn_forward / kvattn_merge.
struct Launch {
    int kind;          // 0 VALU forward, 1 MFMA forward, 2 merge
    int tile;          // VALU rows / MFMA waves
    int item_begin;    // first item (forward) or merge query (merge)
    int item_count;
};

// Pointers the kernels take, resolved from the bound workspace.
struct DevPlan {
    const Item* items;
    const Entry* entries;
    const int32_t* block_ids;
    const int32_t* merge_query;
    const int32_t* merge_ptr;
    const int32_t* merge_dest;
    const uint16_t* zero;     // >= 256 zero bytes: source for token slots outside a range
    float* part_ml;
    float* part_acc;
};

struct Dims {
    int num_q_heads, num_kv_heads, head_dim, group;
    float scale_log2;         // softmax scale * log2(e): scores are kept in log2 units
};

// Kernel launchers (kvattn_kernels.hip).  Return hipSuccess or the launch error.
int launch_forward_valu(const DevPlan& p, const Dims& d, int rows, int item_begin, int item_count,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream);
int launch_forward_mfma(const DevPlan& p, const Dims& d, int waves, int item_begin, int item_count,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream);
int launch_merge(const DevPlan& p, const Dims& d, int q_begin, int q_count, float* out, void* stream);

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace kvattn
