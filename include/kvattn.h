/*
 * kvattn -- prefix-aware paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * Computes, for a batch of single-token decode queries, out = softmax(q K^T / sqrt(d)) V
 * over a paged bf16 KV cache whose blocks are shared by requests along a
 * prefix tree (PAT review, "core formula" section: decode attention with Q a
 * single token and K, V the accumulated cache).  Execution follows the
 * pack-forward-merge scheme of the PAT review ("pack-forward-merge paradigm"):
 *   pack    -- host: group the queries that share a run of KV blocks so the run
 *              is fetched from HBM once (memory-centric prefix-aware packing,
 *              Fig 5(d) caption; profit-model heuristic packing; tree-structure
 *              block table, Fig 7 caption);
 *   forward -- device: split-KV multi-tile kernels, tile variant chosen per
 *              work item at plan time (multi-tile kernel, runtime tile
 *              selector, long-KV splitting);
 *   merge   -- device: combine the per-item partial (m, l, acc) triples of each
 *              query row by the online-softmax rule (online-softmax merge).
 *
 * Conventions for every entry point:
 *   - Plain C ABI; no exception crosses it.  Every call returns a kvattn_status;
 *     on failure kvattn_last_error() gives a thread-local detail string.
 *   - Host pointers are read during the call only, except where stated.
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates device memory (no hipMalloc, no hipFree).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Device work is enqueued asynchronously on `stream`; faults inside a
 *     kernel surface at the caller's next synchronisation.
 *
 * Layouts (all row-major, C order):
 *   block_tables int32 [num_queries][max_blocks_per_seq]  physical block of each
 *                logical 16-token block; entries at j >= ceil(seq_len/16) are ignored
 *   seq_lens     int32 [num_queries]  tokens each query attends over, the current
 *                token included (short-term-memory concept page, autoregressive
 *                KV-cache step: K_t, V_t are appended before attending)
 *   q            bf16  [num_queries][num_q_heads][head_dim]
 *   k_cache, v_cache bf16 [num_physical_blocks][num_kv_heads][block_size][head_dim]
 *                (paged cache: concept page, PagedAttention section).  Token t of
 *                query b is slot t % 16 of block block_tables[b][t / 16].  Slots a
 *                block does not hold are never read into the result (they may be NaN).
 *   out          fp32  [num_queries][num_q_heads][head_dim]
 *   GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVATTN_OK = 0,
    KVATTN_EINVAL = 1,        /* bad argument: NULL, shape, block id, length, tree     */
    KVATTN_EUNSUPPORTED = 2,  /* valid but not built: head_dim not 64/128, block_size != 16,
                                 more than 64 q heads per KV head                        */
    KVATTN_ENOMEM = 3,        /* host allocation failed                                  */
    KVATTN_EWORKSPACE = 4,    /* device workspace too small, misaligned or not bound    */
    KVATTN_EHIP = 5,          /* a HIP runtime call (copy, launch) failed               */
    KVATTN_ESTATE = 6         /* call order: decode before upload                       */
} kvattn_status;

typedef struct kvattn_plan_s* kvattn_plan_t; /* opaque; host memory owned by the library */

typedef struct {
    int32_t num_queries;          /* B  >= 1                                  */
    int32_t num_q_heads;          /* Hq >= 1                                  */
    int32_t num_kv_heads;         /* Hkv >= 1, Hq % Hkv == 0                  */
    int32_t head_dim;             /* D: 64 or 128                            */
    int32_t block_size;           /* tokens per KV block: 16                 */
    int32_t max_blocks_per_seq;   /* row stride of block_tables              */
    int32_t num_physical_blocks;  /* blocks in each of k_cache, v_cache      */
} kvattn_shape;

/*
 * Optional explicit prefix tree (PAT review, Fig 7(b) caption: the pack
 * scheduler works on a tree-structured block table).  Node n covers logical
 * block positions [block_begin[n], block_end[n]) of every query whose path
 * passes through it; a root has parent -1 and block_begin 0; a child starts
 * where its parent ends; query b's path ends at node query_leaf[b] with
 * block_end == ceil(seq_len[b] / 16).  All queries passing through a node must
 * hold the same physical blocks with the same token counts over its range.
 * kvattn_plan checks all of this and returns KVATTN_EINVAL otherwise.  Pass
 * NULL to let the planner derive the (maximal) tree from the block tables.
 * Arrays are read during the kvattn_plan call only.
 */
typedef struct {
    int32_t num_nodes;
    const int32_t* parent;        /* [num_nodes]                        */
    const int32_t* block_begin;   /* [num_nodes]                        */
    const int32_t* block_end;     /* [num_nodes]                        */
    const int32_t* query_leaf;    /* [num_queries]                      */
} kvattn_prefix_tree;

enum { KVATTN_PACK_AUTO = 0, KVATTN_PACK_QUERY = 1, KVATTN_PACK_FULL = 2 };
enum { KVATTN_VARIANT_AUTO = -1, KVATTN_VARIANT_VALU = 0, KVATTN_VARIANT_MFMA = 1, KVATTN_VARIANT_VALU_SPLIT = 2 };

/*
 * Plan options.  kvattn_plan_options_default() fills the defaults.
 *   scale          softmax scale; 0 selects 1/sqrt(head_dim) (core formula).
 *   pack_mode      AUTO: pack a shared node when the profit model says the
 *                  HBM bytes saved outweigh the partial-result traffic and lost
 *                  parallelism (profit-model heuristic packing, which weighs
 *                  prefix length against query count); QUERY: one query per work
 *                  item, shared blocks re-read (query-centric packing, Fig 5(b));
 *                  FULL: pack every node shared by >= 2 queries (memory-centric
 *                  packing, Fig 5(d)).
 *   scheme         0 auto, 1 = packing scheme 1 only (leaves always split off their
 *                  parent, Fig 7(c)), 2 = also allow scheme 2 (one short leaf folded
 *                  into its parent's item, Fig 7(d)).
 *   force_variant  -1 auto; KVATTN_VARIANT_VALU / _MFMA / _VALU_SPLIT force one
 *                  forward tile for every item (for tests).  VALU handles at most 8
 *                  rows per KV head at head_dim 64 and 4 at head_dim 128 (wider packs
 *                  are split into several items; a wider GQA group is EUNSUPPORTED).
 *                  The two VALU tiles differ in how a workgroup's four waves share an
 *                  item: VALU gives each wave one KV head of the item's range (four
 *                  heads per task); VALU_SPLIT gives the four waves a quarter each of
 *                  one KV head's range and combines their partial results in LDS
 *                  (one task per head), so a range is read four-wide without being
 *                  cut into partials across workgroups.  VALU_SPLIT needs at least 4
 *                  blocks (64 tokens) per range; shorter ranges keep the VALU tile.
 *                  AUTO picks the tile per item by its KV length (runtime tile
 *                  selector): MFMA for packed groups, VALU for single queries and
 *                  small packs, and -- for batches too small to fill the GPU, where
 *                  one launch without partials beats cutting ranges and merging --
 *                  VALU_SPLIT for every range of 4 or more blocks.
 *   split_tokens   0 auto; otherwise the KV chunk length of split items, rounded
 *                  up to a multiple of 16 (long-KV splitting).
 *   num_cus        compute units the split model balances over; 0 means 256
 *                  (a whole MI355X).  The plan makes 2 * num_cus static lists,
 *                  two workgroups per CU; set it to the device's CU count when
 *                  the GPU is partitioned or smaller.  Lists beyond what the
 *                  device holds at once are claimed at run time (correct, but
 *                  slower than a matching count).
 *   new_token      0: seq_lens count tokens already in the cache (kvattn_decode).
 *                  1: the last token of each query, position seq_len - 1, comes
 *                  with the call as k_new / v_new (kvattn_decode_append), which
 *                  writes it into its paged slot and attends to it; the plan
 *                  covers the first seq_len - 1 tokens, read from the cache
 *                  (short-term-memory page, technical principles, the KV cache
 *                  in autoregressive generation: a step appends its token's K
 *                  and V, then attends to all of them).  The new token's slot
 *                  must belong to its query alone: no other query reads it
 *                  (copy-on-write paging), else kvattn_plan returns EINVAL.
 *   multi_stream   0: MFMA and VALU tasks share each forward launch.  1: each
 *                  launch is split into an MFMA-only launch and a VALU-only
 *                  launch with lists of their own (the PAT review's multi-stream
 *                  forward: kernel variants on separate streams, implementation
 *                  details); kvattn_decode_streams runs the MFMA launches on a
 *                  side stream beside the VALU ones.  kvattn_decode runs all
 *                  launches in turn on one stream.
 *   fused_merge    -1 auto (0: measured faster on every workload), 0 or 1: with
 *                  1, the forward launch also merges: the
 *                  task that completes the last partial triple of a (query, KV
 *                  head) combines that query's partials for the head's q heads
 *                  with the same online-softmax rule and writes out, and no merge
 *                  launch follows (PAT review, merge stage).  Partials are
 *                  written and read with agent-scope coherent accesses, and a
 *                  per-(query, KV head) arrival counter in the workspace tells
 *                  which task is last; it returns to zero within the launch.  0
 *                  keeps the separate merge launch.  Plans with new_token or
 *                  multi_stream always use the merge launch.  kvattn_forward of
 *                  a fused plan therefore writes every output row, and
 *                  kvattn_merge recomputes the merged rows identically.
 */
typedef struct {
    float scale;
    int32_t pack_mode;
    int32_t scheme;
    int32_t force_variant;
    int32_t split_tokens;
    int32_t num_cus;
    int32_t new_token;
    int32_t multi_stream;
    int32_t fused_merge;
} kvattn_plan_options;

/* Statistics of a plan (bytes are per decode call, all KV heads). */
typedef struct {
    int64_t unique_kv_bytes;         /* distinct (physical block) tokens x 2 x Hkv x D x 2 B     */
    int64_t planned_kv_bytes;        /* KV bytes the forward items read (>= unique)              */
    int64_t query_centric_kv_bytes;  /* sum over queries of seq_len x 2 x Hkv x D x 2 B          */
    int64_t partial_bytes;           /* partial triples written by forward and read by merge     */
    int32_t num_nodes;               /* prefix-tree nodes                                       */
    int32_t num_packed_nodes;        /* nodes read once for all their queries                   */
    int32_t num_items;               /* forward work items (each runs for every KV head)        */
    int32_t num_items_valu;
    int32_t num_items_mfma;
    int32_t num_folded_leaves;       /* leaves folded into a parent item (scheme 2)            */
    int32_t num_partial_slots;       /* (query, q head) partial triples                         */
    int32_t num_merge_rows;          /* (query, q head) rows the merge kernel combines          */
    int32_t num_direct_rows;         /* rows written by exactly one forward item                */
    int32_t num_launches;            /* kernel launches per kvattn_decode                       */
    int32_t split_tokens;            /* longest chunk of a split KV range (0: nothing split)     */
    int32_t update_path;             /* last kvattn_plan / _update: 0 full plan, 1 descriptors
                                        patched in place, 2 lists re-serialized, 3 update fell
                                        back to a full plan                                      */
    double plan_seconds;             /* host wall time of kvattn_plan                            */
    uint64_t blob_bytes;             /* schedule bytes uploaded by kvattn_plan_upload            */
    uint64_t workspace_bytes;        /* = kvattn_plan_device_bytes                               */
    int32_t num_items_valu_split;    /* items on the VALU_SPLIT tile (counted in num_items_valu) */
    int32_t one_launch;              /* 1: a small batch's forward planned as one launch without packs
                                        or cuts (no partials and no merge launch, except that
                                        new-token plans merge every row)                          */
} kvattn_stats;

/* One forward work item, as exported for inspection and coverage checks. */
typedef struct {
    int32_t kind;        /* KVATTN_VARIANT_VALU, _MFMA or _VALU_SPLIT                          */
    int32_t tile;        /* VALU tiles: rows per KV head (1,2,4,8); MFMA: 16-row tiles per wave (1,2) */
    int32_t pos_begin;   /* first logical block position of the item's KV range               */
    int32_t n_tokens;    /* tokens in the item's KV range                                     */
    int32_t q_begin;     /* first entry in entries[]                                          */
    int32_t n_q;         /* queries in the item                                               */
    int32_t blk_begin;   /* first entry in block_ids[]; the range has ceil(n_tokens/16) blocks */
    int32_t n_rows;      /* n_q x (Hq / Hkv) query rows per KV head                           */
} kvattn_item_info;

typedef struct {
    int32_t query;       /* b                                                                  */
    int32_t dest;        /* -1: the item writes out[b] directly; else partial slot of q head h
                            is dest + h                                                          */
    int32_t limit;       /* query b attends to tokens [0, limit) of the item's range            */
    int32_t pad;
} kvattn_item_query;

/* Host views of a plan's schedule; pointers stay valid until kvattn_plan_destroy. */
typedef struct {
    int32_t num_items;
    const kvattn_item_info* items;
    int32_t num_entries;
    const kvattn_item_query* entries;
    int32_t num_block_ids;
    const int32_t* block_ids;
    int32_t num_merge_queries;
    const int32_t* merge_query;   /* [num_merge_queries] b                                 */
    const int32_t* merge_ptr;     /* [num_merge_queries + 1] CSR offsets into merge_dest  */
    const int32_t* merge_dest;    /* partial slot bases of the query's items              */
    int32_t num_partial_slots;
    int32_t head_dim;
    int32_t num_tasks;
    const int32_t* tasks;         /* [num_tasks][2]: (item, first KV head); MFMA and VALU_SPLIT
                                     items run one task per KV head, a VALU item one per 4
                                     consecutive KV heads */
    /* The task descriptors as uploaded to the device.  A descriptor is a run of
     * int32 words: a 16-word header (kind, tile, first KV head, tokens, entries
     * n_q, rows, blocks nb, min limit, words of this descriptor, words of the
     * next MFMA descriptor of the same list or 0, then 6 zero words), n_q
     * entries of 4 words (query, dest, limit, index of the query's merge record
     * or -1 when dest is -1), nb block ids, zero padding to
     * a multiple of 4 words.  List l of launch L (one per persistent
     * workgroup) holds its MFMA descriptors in words [lp[0], lp[1]) and its
     * VALU descriptors in [lp[1], lp[2]), lp = list_ptr + 3 (L num_lists + l). */
    int32_t num_launches;
    int32_t num_lists;
    int32_t num_desc_words;
    const int32_t* desc;
    const int32_t* list_ptr;      /* [num_launches][num_lists][3]              */
    const int32_t* merge_rec;     /* [num_merge_queries][4] as uploaded: b, first partial slot,
                                     partial count, and in new-token plans block * 16 + slot
                                     of the query's new token (else 0)                        */
} kvattn_export;

/* Fill *opts with the defaults (AUTO packing, scheme auto, auto variant and split). */
void kvattn_plan_options_default(kvattn_plan_options* opts);

/*
 * Build a decode plan on the host (no HIP call; usable without a GPU): the
 * pack stage of the PAT review's pack-forward-merge paradigm (method overview;
 * pack scheduler workflow over a tree-structured block table, Fig 7 caption;
 * memory-centric prefix-aware packing, Fig 5(d) caption; profit-model
 * heuristic weighing prefix length against query count, implementation
 * details of the pack scheduler), plus the forward stage's schedule (long-KV
 * splitting and the runtime tile selector of the multi-tile kernel).
 * Steps: derive or check the prefix tree, decide packs with the profit model,
 * split long KV ranges, pick a kernel variant and KV tile per item, order items
 * longest first, build the merge map, serialise the schedule.
 *   shape, block_tables, seq_lens: required; layouts above.
 *   tree: optional (NULL derives it); opts: optional (NULL = defaults).
 *   *out receives a plan owned by the caller until kvattn_plan_destroy.
 * Errors: EINVAL (NULL pointer, B/H/D <= 0, Hq % Hkv, seq_len outside
 * [1, max_blocks*16], block id outside [0, num_physical_blocks), bad tree or
 * option; with new_token: two queries' new tokens in one block, or a query
 * reading another's new-token slot), EUNSUPPORTED (head_dim not 64/128,
 * block_size != 16, Hq/Hkv > 64, num_queries * Hq * head_dim >= 2^31, more
 * than 2^31 - 1 partial slots; with new_token, a new-token block id >= 2^27),
 * ENOMEM.  Reentrant; plans are independent.  With new_token, a tree (if
 * given) describes the cached part, the first seq_len - 1 tokens of each query;
 * a query with seq_len 1 has no cached part and query_leaf -1.
 */
kvattn_status kvattn_plan(const kvattn_shape* shape, const int32_t* block_tables, const int32_t* seq_lens,
                          const kvattn_prefix_tree* tree, const kvattn_plan_options* opts, kvattn_plan_t* out);

/*
 * Bring a plan to the next decode step in place (PAT review, overhead
 * analysis, Fig 16: the pack scheduler's cost next to decoding).  block_tables
 * and seq_lens describe the same queries (same shape) one or more steps later:
 * each seq_len is at least the plan's, and the blocks the plan's lengths cover
 * are unchanged.  When every query's new tokens extend the item that holds its
 * last token -- its own private item, or a shared item whose end queries all
 * grow alike into the same new blocks (a session's shared KV growing) -- only
 * those items, their queries' limits and their descriptors change: nothing is
 * re-planned, and the item-to-list schedule is kept.  Otherwise (a length
 * shrinks, a block changes, a new private run starts, an item would exceed its
 * block cap) the plan is rebuilt from scratch with its options, the tree derived.
 * stats.update_path tells which happened.  The device copy of the schedule is
 * stale afterwards: kvattn_plan_upload again before the next kvattn_decode (its
 * size, kvattn_plan_device_bytes, changes only on a rebuild).  If the plan was
 * uploaded, the call first waits (host) for that upload's copy to finish.
 * New-token plans (options.new_token) take seq_lens with each query's new
 * token, as kvattn_plan does: the cached parts are extended, each merge record
 * gets its query's new slot, and the slot-ownership rule is checked again.
 * Errors: EINVAL (NULL, seq_len or block id out of range, a new-token slot
 * that another query reads or shares; the plan is then unchanged), ENOMEM.
 */
kvattn_status kvattn_plan_update(kvattn_plan_t plan, const int32_t* block_tables, const int32_t* seq_lens);

/*
 * Multi-token queries (stateful-streaming digest, method breakdown: a query of
 * |q| tokens against a session's cached KV, prefix-aware grouped prefill).
 * Query b brings q_lens[b] >= 1 new tokens: the last q_lens[b] of its
 * seq_lens[b] tokens, their K/V already in the cache.  New token i of query b
 * (0-based) attends causally to the first seq_lens[b] - q_lens[b] + i + 1
 * tokens.  This writes one single-token row per new token, in query order:
 * out_block_tables [sum q_lens][max_blocks_per_seq] (the query's table, -1
 * past the row's blocks) and out_seq_lens [sum q_lens] (caller-allocated).
 * A plan over these rows (num_queries = sum q_lens) packs the tokens of a query
 * like the queries of a shared prefix, so their KV is fetched once; q and out
 * then hold [sum q_lens][Hq][D] in the same row order.
 * Errors: EINVAL (NULL, q_lens[b] outside [1, seq_lens[b]], seq_lens[b] outside
 * [1, max_blocks_per_seq * 16]).
 */
kvattn_status kvattn_expand_query_tokens(const kvattn_shape* shape, const int32_t* block_tables,
                                         const int32_t* seq_lens, const int32_t* q_lens,
                                         int32_t* out_block_tables, int32_t* out_seq_lens);

/* Device workspace bytes the plan needs: schedule blob + partial triples (256-B aligned). */
kvattn_status kvattn_plan_device_bytes(kvattn_plan_t plan, size_t* bytes);

/*
 * Copy the plan's schedule into the caller's device workspace (one async
 * host-to-device copy on `stream`) and bind the workspace to the plan.
 * dev_workspace must be 256-byte aligned and at least kvattn_plan_device_bytes.
 * The copy reads the plan's host blob asynchronously; the plan records an
 * event (created on the first upload) right after it, and kvattn_plan_update
 * and kvattn_plan_destroy wait on the host for that event before they change
 * or free the blob.  So update -> upload -> decode steps may follow each other
 * without host synchronisation: each update blocks only until the previous
 * upload's copy, queued on its stream, has run.  The upload must not be
 * captured into a graph (a replay would read the blob as it is then): on a
 * capturing stream it returns EINVAL.  Binding again replaces the binding.
 * Errors: EINVAL (NULL, capturing stream), EWORKSPACE (too small /
 * misaligned), EHIP.
 */
kvattn_status kvattn_plan_upload(kvattn_plan_t plan, void* dev_workspace, size_t bytes, void* stream);

/*
 * One decode-attention call, out = softmax(q K^T / sqrt(d)) V per (query, q
 * head) over the query's paged KV (PAT review, core formula): the forward
 * stage (split-KV multi-tile kernels over every planned item, each shared
 * block read once for all the queries packed on it; PAT review, forward
 * stage), then the merge stage over rows that have several partial triples
 * (online-softmax combination of (m, l, acc); PAT review, merge stage).
 * q, k_cache,
 * v_cache, out: device pointers, layouts above, matching the plan's shape.
 * The bound workspace holds the partial triples, so at most one decode per
 * workspace may be in flight.  One plan serves any number of calls (e.g. every
 * layer of a decode step) with different q / caches of the same shape.
 * Partial triples are stored written through the L2 while the partial arrays
 * fit 32-bit byte offsets, with plain stores beyond; the environment variable
 * KVATTN_PLAIN_PARTIALS=1 selects the plain stores at any size (for tests;
 * plans with a fused merge always write through).
 * Errors: EINVAL (NULL, plan made with new_token: use kvattn_decode_append),
 * ESTATE (no workspace bound), EHIP (launch failed).
 */
kvattn_status kvattn_decode(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                            float* out, void* stream);

/*
 * One decode step with the KV append fused in (short-term-memory page,
 * technical principles, the KV cache in autoregressive generation: append the
 * step's K and V to the cache, then attend over all cached tokens).  The plan
 * must have been made with options.new_token = 1.  k_new, v_new: device bf16
 * [B][Hkv][D], the K and V of each query's newest token (position
 * seq_len[b] - 1).  The forward kernels read the first seq_len[b] - 1 tokens
 * from the cache; the merge kernel scores the new token against q, folds it
 * into each row's online softmax as one more partial, and copies k_new / v_new
 * (bit-exact) into slot (seq_len[b] - 1) % 16 of block
 * block_tables[b][(seq_len[b] - 1) / 16] of k_cache / v_cache.  No kernel of
 * the call reads that slot, so out equals attention over the cache after the
 * append.  Two launches, as kvattn_decode; every row goes through the merge.
 * Calling it again with the same inputs rewrites the same bytes.
 * Errors: EINVAL (NULL or misaligned pointer, plan made without new_token),
 * ESTATE (no workspace bound), EHIP (launch failed).
 */
kvattn_status kvattn_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, kvattn_plan_t plan, float* out, void* stream);

/*
 * kvattn_decode with the PAT review's multi-stream forward (implementation
 * details: variants launched on separate streams so their kernels overlap).
 * For plans made with options.multi_stream = 1: the MFMA-only launches go on
 * side_stream, the VALU-only launches on stream; side_stream first waits for
 * the work already on stream, and stream waits for side_stream before the
 * merge launch, so the call is ordered on `stream` like kvattn_decode.  The
 * plan owns two HIP events for the fork and join (created on first use,
 * destroyed with the plan): calls with one plan must not overlap.  Works under
 * stream capture (the side stream joins the capture).
 * Errors: EINVAL (NULL or misaligned pointer, plan made without multi_stream,
 * side_stream equal to stream), ESTATE (no workspace bound), EHIP.
 */
kvattn_status kvattn_decode_streams(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                                    float* out, void* stream, void* side_stream);

/*
 * kvattn_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * plan, same kernels and same result as kvattn_decode, but the workspace
 * (schedule blob + partial triples) is a static device array of the library,
 * 64 MiB per device, that every GPU the library runs on holds from the first
 * call on it until the process ends; no kvattn_plan_upload or caller workspace
 * is needed.  The call copies the plan's schedule into the array only when the
 * array holds another plan's (or another state's: each kvattn_plan_update makes
 * a new one), so repeated calls with one plan (every layer of a decode step)
 * copy nothing; that copy reads the plan's host blob like kvattn_plan_upload
 * and is ordered against kvattn_plan_update / destroy the same way.  A copy
 * cannot be captured: under stream capture the plan must already be staged by
 * an earlier call on the device.  The array keeps the last call's contents
 * (the claim counter returns to zero at the end of every launch), and all
 * calls on one GPU share it: calls that overlap on one GPU (other streams,
 * other threads) race and give wrong results.  Nothing is allocated: no
 * hipMalloc, hipFree or allocating library call (the first call with a plan
 * that was never uploaded creates its host-side upload event).
 * Errors: EINVAL (NULL, plan made with new_token, capture with the plan not
 * staged), EWORKSPACE (the plan's kvattn_plan_device_bytes exceed 64 MiB:
 * use kvattn_decode), EHIP.
 */
kvattn_status kvattn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                                    float* out, void* stream);

/* The forward stage of kvattn_decode alone (PAT review, forward stage). */
kvattn_status kvattn_forward(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                             float* out, void* stream);

/* The merge stage of kvattn_decode alone (PAT review, merge stage); reads the
 * partial triples the last kvattn_forward on this workspace wrote.  EINVAL for
 * a plan made with new_token (its merge needs the new token's inputs). */
kvattn_status kvattn_merge(kvattn_plan_t plan, float* out, void* stream);

/*
 * Measurement helper, not part of the attention path.  One launch of `grid`
 * workgroups of `threads` threads (256, 512 or 1024) that reads a_bytes of a
 * then b_bytes of b (device buffers, 16-byte aligned, sizes multiples of 16),
 * each workgroup one contiguous share with `loads_in_flight` (2, 4 or 8)
 * 16-byte loads per lane in flight, and writes one word per thread into sink
 * (device, >= grid * threads * 4 bytes).  It times what the memory system
 * delivers for a plain streaming read of the same bytes, e.g. the K and V
 * pools a decode reads, beside the decode's own rate.
 * Errors: EINVAL (NULL, misaligned, sink too small, grid < 1, other depths or
 * sizes), EHIP.
 */
kvattn_status kvattn_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, void* sink,
                                size_t sink_bytes, int32_t grid, int32_t loads_in_flight, int32_t threads,
                                void* stream);

/* Plan statistics (host only). */
kvattn_status kvattn_plan_stats(kvattn_plan_t plan, kvattn_stats* stats);

/* Host views of the schedule, for coverage checks and inspection. */
kvattn_status kvattn_plan_export(kvattn_plan_t plan, kvattn_export* out);

/* Free a plan (NULL is a no-op).  Waits (host) for the plan's last upload copy, if
 * one is pending; does not touch the bound device workspace. */
void kvattn_plan_destroy(kvattn_plan_t plan);

/* Static name of a status code. */
const char* kvattn_status_string(kvattn_status status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* kvattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
