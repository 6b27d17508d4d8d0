// Schedule format shared by the host planner, the launcher and the gfx950 kernels.
//
// A plan is a list of forward work items.  An item is one run of KV blocks
// (a chunk of a prefix-tree node or of one query's private tail) together
// with the queries that attend over it.  Items of several queries read each
// shared block once for all of them (PAT review, memory-centric prefix-aware
// packing, Fig 5(d) caption).  An item runs for every KV head: as one task per
// KV head (MFMA items) or one task per group of four KV heads (VALU items).
// Each persistent workgroup runs one static task list built by the planner
// (longest first over the workgroups): its MFMA tasks, then its VALU tasks as
// continuous per-wave streams.  MFMA and VALU tasks share one launch, so the
// MFMA work of packed groups overlaps the bandwidth-bound streaming of
// private tails.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvattn.h"

namespace kvattn {

constexpr int kBlock = 16;              // tokens per KV block
constexpr int kValuMaxRows = 8;         // rows per KV head the VALU path holds (D = 64)
// At D = 128 eight rows do not fit the VALU path's register budget next to
// its load ring; wider groups go to the MFMA path there.
constexpr int valu_max_rows(int D) { return D == 128 ? 4 : kValuMaxRows; }
constexpr int kWaves = 4;               // waves per forward workgroup (both paths)
constexpr int kMfmaMaxRows = 128;       // rows per MFMA item: 4 waves x 32 rows
constexpr int kMfmaTileTokens = 32;     // KV tokens per LDS stage
constexpr int kMfmaStages = 4;          // LDS stages of the MFMA pipeline (3 tiles in flight)
constexpr int kMaxItemBlocks = 512;     // KV blocks per VALU item (8192 tokens): descriptors share the VALU LDS window
constexpr int kMfmaMaxItemBlocks = 1408;  // KV blocks per MFMA item (22528 tokens): two descriptors beside the 64 KB
                                          // of MFMA stages keep a workgroup within 80 KB of LDS (two per CU)
constexpr int kMaxGroup = 64;           // q heads per KV head supported
constexpr int kXcds = 8;                // XCDs of an MI355X (L2 domains)
constexpr uint32_t kBlobMagic = 0x4B564154u;  // "KVAT"
constexpr uint32_t kBlobVersion = 9;

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
// [head, head + 4) (VALU).  Host-side schedule; the device reads descriptors.
struct Task {
    int32_t item;
    int32_t head;
};

// Task descriptor (device, int32 words, 16-byte aligned): a kDescHeader-word
// header, n_q entries of 4 words (query, dest, limit, merge record index of the
// query, or -1 for a row written directly), then the item's block ids, padded
// to a multiple of 4 words.
enum : int {
    kDescKind = 0,        // KVATTN_VARIANT_VALU / _MFMA
    kDescTile = 1,        // VALU rows template; MFMA 16-row tiles per wave
    kDescHead = 2,        // first KV head
    kDescTokens = 3,      // tokens of the range (with a folded leaf)
    kDescNq = 4,          // entries
    kDescRows = 5,        // n_q * G
    kDescBlocks = 6,      // ceil(tokens / 16)
    kDescLimAll = 7,      // min limit over the entries: tokens every row attends
    kDescWords = 8,       // words of this descriptor
    kDescNextWords = 9,   // words of the next descriptor of the same static list, 0 if last
    kDescHeader = 16
};
constexpr int kMaxItemQueries = kMfmaMaxRows;   // rows per item >= queries per item
constexpr int kDescMaxWords = kDescHeader + 4 * kMaxItemQueries + kMfmaMaxItemBlocks;
inline int32_t desc_words(int n_q, int nblk) { return kDescHeader + 4 * n_q + ((nblk + 3) & ~3); }

// LDS window of the VALU phase: the MFMA stages (kMfmaStages x 2 x 32 tokens x
// D bf16 = 512 D bytes) are reused for the list's VALU descriptors and, per
// wave, four q slots of R rows x D bf16.  Returns the descriptor words that fit.
constexpr int valu_window_words(int D, int R) { return (512 * D - kWaves * 4 * R * D * 2) / 4; }

// Header at offset 0 of the device workspace.  Offsets are in bytes from the
// workspace base and 256-byte aligned.
struct BlobHeader {
    uint32_t magic, version;
    int32_t n_desc_words, n_merge_q, n_slots, head_dim;
    int32_t n_tasks, n_launches, n_lists, pad0;
    uint64_t off_desc;        // int32 [n_desc_words]: task descriptors
    uint64_t off_list_ptr;    // int32 [n_launches][n_lists][3]: word offsets (MFMA begin, VALU begin, end) per list
    uint64_t off_merge_rec;   // int32 [n_merge_q][4]: (query, first slot, partials, 0); partial k at first + k Hq
    uint64_t off_claim;       // int32: list claim counter, zero between launches
    uint64_t off_arrive;      // int32 [n_merge_q][Hkv]: fused-merge arrival counters, zero between launches
    uint64_t blob_bytes;      // bytes copied by kvattn_plan_upload
    uint64_t off_part_ml;     // float2 [n_slots]: (m in log2 units, l)
    uint64_t off_part_acc;    // float [n_slots][head_dim]
    uint64_t total_bytes;     // workspace bytes
};

// One forward launch: persistent workgroups, each running static list
// blockIdx.x, then lists claimed at run time (MFMA tasks, then VALU tasks as
// per-wave streams).  A plan needs more than
// one only when its VALU items use several row templates or its MFMA items
// several row tilings.
struct Launch {
    int valu_rows;     // VALU row template (1, 2, 4, 8)
    int mfma_tiles;    // MFMA 16-row tiles per wave (1, 2)
    int index;         // list set
    int n_tasks;
    int task_base;     // first task of the launch in the host schedule
    int side;          // multi-stream plans: 1 for the MFMA launches (side stream); also the claim counter
};

// Merge record of one query whose rows have several partials: partial k of
// q head h sits in slot first + k * Hq + h.  In new-token plans every query
// has one (count may be 0 or 1) and new_slot = block * 16 + slot of its new
// token's paged position; otherwise new_slot is 0.
struct alignas(16) MergeRec {
    int32_t query, first, count, new_slot;
};
constexpr int32_t kMaxNewTokenBlock = 1 << 27;   // block * 16 + slot fits int32

// Inputs of the fused KV append (kvattn_decode_append).
struct NewTokens {
    const uint16_t* q;          // bf16 [B][Hq][D]
    const uint16_t* k_new;      // bf16 [B][Hkv][D]
    const uint16_t* v_new;
    uint16_t* k_cache;          // bf16 [blocks][Hkv][16][D]
    uint16_t* v_cache;
};

// Pointers the kernels take, resolved from the bound workspace.
struct DevPlan {
    const int32_t* desc;
    const int32_t* list_ptr;    // this launch's n_lists x 3 word offsets into desc
    int32_t n_lists;
    const MergeRec* merge_rec;  // per merged query
    int32_t* claim;             // list claim counter (zero between launches)
    float* part_ml;
    float* part_acc;
    // Fused merge (plans with fused_merge): arrival counter of each (merge record,
    // KV head), zero between launches; NULL when a merge launch follows the forward.
    int32_t* arrive;
    uint32_t part_ml_bytes;     // bytes of part_ml and part_acc (< 4 GiB when fused)
    uint32_t part_acc_bytes;
    // 1 when both partial arrays fit 32-bit byte offsets (always when fused): the
    // kernels then store partials written through the L2 (sc1); 0: plain stores
    int32_t part_wt;
    // 1 when some task of the plan runs on the VALU_SPLIT tile; 0: the forward
    // skips the second pass over each list's VALU descriptors
    int32_t has_split;
};

struct Dims {
    int num_q_heads, num_kv_heads, head_dim, group;
    float scale_log2;         // softmax scale * log2(e): scores are kept in log2 units
};

// Kernel launchers (kvattn_kernels.hip).  Return hipSuccess or the launch error.
int launch_forward(const DevPlan& p, const Dims& d, int valu_rows, int mfma_tiles, int n_tasks,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream);
int launch_merge(const DevPlan& p, const Dims& d, int q_count, float* out, void* stream);
int launch_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, int grid,
                      int depth, int threads, void* stream);
int launch_merge_append(const DevPlan& p, const Dims& d, int q_count, const NewTokens& nt, float* out, void* stream);

// kvattn_decode_noalloc: bytes of the static per-device scratch that holds a
// plan's workspace (schedule blob + partial triples), and devices supported.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
// Device address of this device's scratch (hipGetSymbolAddress, looked up once
// per device); returns hipSuccess or the lookup's error.
int scratch_device_pointer(void** ptr);

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace kvattn
