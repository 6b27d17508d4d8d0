// Host-side plan object and error helpers (no HIP dependency).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kvattn_internal.h"

struct kvattn_plan_s {
    kvattn_shape shape{};
    kvattn_plan_options opts{};
    float scale = 0.f;                      // effective softmax scale
    std::vector<kvattn::Item> items;
    std::vector<kvattn::Entry> entries;
    std::vector<int32_t> block_ids;
    std::vector<int32_t> merge_query, merge_ptr, merge_dest;   // host copy (export)
    std::vector<int32_t> merge_rec;                            // device: (b, slot base, partials, new-token slot) per merged query
    std::vector<int32_t> rec_of_query;                         // [B] index of the query's merge record, -1 if none
    bool fused_merge = false;                                  // the forward launch merges (no merge launch)
    bool has_split = false;                                    // some task runs on the VALU_SPLIT tile
    int32_t n_slots = 0;
    std::vector<kvattn::Task> tasks;
    std::vector<int32_t> list_ptr;          // [launch][n_lists + 1] task ranges of the static lists
    std::vector<int32_t> desc;              // device task descriptors
    std::vector<int32_t> task_desc;         // [tasks] word offset of each task's descriptor in desc
    std::vector<int32_t> desc_list_ptr;     // [launch][n_lists][3] (MFMA begin, VALU begin, end) in words
    int32_t n_lists = 0;                    // static task lists per launch (one per persistent workgroup)
    std::vector<kvattn::Launch> forward_launches;
    std::vector<unsigned char> blob;        // serialised schedule: header + arrays + zero region
    kvattn::BlobHeader header{};
    kvattn_stats stats{};
    // incremental updates (kvattn_plan_update)
    std::vector<int32_t> tables;            // [B][max_blocks] block tables of the last plan or update
    std::vector<int32_t> lens;              // [B] their sequence lengths
    std::vector<int32_t> entry_item;        // [entries] item of each entry
    std::vector<int32_t> tail_entry;        // [B] entry holding each query's last token
    std::vector<int32_t> reads;             // new-token plans: [num_physical_blocks] most tokens a cached part reads
    void* fork_event = nullptr;             // multi-stream decode: hipEvent_t pair, created on first use
    void* join_event = nullptr;
    // hipEvent_t recorded on the upload stream right after the last upload's
    // copy, and the runtime's function that waits for it.  The copy reads the
    // host blob asynchronously, so kvattn_plan_update and kvattn_plan_destroy
    // wait for it before they change or free the blob.  Both are set by the
    // runtime (this header has no HIP dependency); a plan never uploaded has none.
    void* upload_event = nullptr;
    void (*upload_wait)(void* event) = nullptr;
    void* dev_ws = nullptr;                 // bound device workspace (caller-owned)
    size_t dev_bytes = 0;
    // Distinct for every plan and every state of a plan (kvattn_plan and each
    // kvattn_plan_update draw a new one): kvattn_decode_noalloc copies the blob
    // into its device's static scratch only when the scratch holds another one.
    uint64_t generation = 0;
};

namespace kvattn {
kvattn_status set_error(kvattn_status s, const std::string& msg);
void clear_error();
uint64_t next_generation();   // process-wide counter, starts at 1
}  // namespace kvattn
