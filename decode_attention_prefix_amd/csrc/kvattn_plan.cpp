// Host pack scheduler: prefix tree -> packs -> split items -> schedule blob.
//
// Follows the pack stage of the PAT review ("pack-forward-merge paradigm",
// pack scheduler workflow of Fig 7, key implementation details of the pack
// scheduler): queries sharing a prefix are grouped into one work item so each
// shared KV block is fetched once; a profit model that weighs prefix length
// against query count decides which shared nodes are packed; packing scheme 1
// splits leaves off their parent's item, scheme 2 folds a specific leaf into
// it; long KV ranges are split so unequal lengths leave no bubbles; each item
// gets a kernel variant chosen by its row count (multi-tile kernel, runtime
// tile selector).  Nothing here calls HIP, so plans can be built and checked
// on a host without a GPU.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <new>
#include <numeric>
#include <queue>
#include <set>
#include <string>
#include <vector>

#include "kvattn_plan.hpp"

namespace kvattn {

static thread_local std::string g_last_error;

kvattn_status set_error(kvattn_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}
void clear_error() { g_last_error.clear(); }

uint64_t next_generation() {
    static std::atomic<uint64_t> counter{0};
    return ++counter;
}

namespace {

struct Node {
    int parent = -1;
    int pos_begin = 0, pos_end = 0;     // logical block positions
    int64_t tokens = 0;
    std::vector<int> queries;           // ascending
    std::vector<int> children;
    bool packed = false;
    int fold_child = -1;                // scheme 2: leaf folded into this node's item
};

struct Batch {
    int B, mb;
    const int32_t* bt;
    const int32_t* sl;
    std::vector<int> nb;                // blocks per query
    int valid(int b, int j) const {
        int n = nb[b];
        return j < n - 1 ? kBlock : sl[b] - kBlock * (n - 1);
    }
    uint64_t key(int b, int j) const {
        return (uint64_t(uint32_t(bt[size_t(b) * mb + j])) << 5) | uint64_t(valid(b, j));
    }
    int32_t id(int b, int j) const { return bt[size_t(b) * mb + j]; }
};

// Lengths within [1, max_blocks * 16] and block ids of every used block within
// [0, num_physical_blocks).
kvattn_status check_tables(const kvattn_shape& s, const int32_t* block_tables, const int32_t* seq_lens) {
    for (int b = 0; b < s.num_queries; ++b) {
        const int T = seq_lens[b];
        if (T < 1 || int64_t(T) > int64_t(s.max_blocks_per_seq) * kBlock)
            return set_error(KVATTN_EINVAL, "seq_lens[" + std::to_string(b) + "] = " + std::to_string(T) +
                                                " outside [1, max_blocks_per_seq * 16]");
        const int nb = (T + kBlock - 1) / kBlock;
        for (int j = 0; j < nb; ++j) {
            const int32_t id = block_tables[size_t(b) * s.max_blocks_per_seq + j];
            if (id < 0 || id >= s.num_physical_blocks)
                return set_error(KVATTN_EINVAL, "block_tables[" + std::to_string(b) + "][" + std::to_string(j) +
                                                    "] = " + std::to_string(id) + " outside [0, num_physical_blocks)");
        }
    }
    return KVATTN_OK;
}

// Per physical block, the most tokens any query's first lens[b] tokens read from it.
std::vector<int32_t> block_reads(const kvattn_shape& s, const int32_t* block_tables, const int32_t* lens) {
    std::vector<int32_t> r(size_t(s.num_physical_blocks), 0);
    for (int b = 0; b < s.num_queries; ++b) {
        const int T = lens[b];
        for (int j = 0; j * kBlock < T; ++j) {
            int32_t& x = r[size_t(block_tables[size_t(b) * s.max_blocks_per_seq + j])];
            x = std::max(x, int32_t(std::min(kBlock, T - j * kBlock)));
        }
    }
    return r;
}

// New-token plans: query b's new token goes to position cached[b], slot
// cached[b] % 16 of block block_tables[b][cached[b] / 16] (ids range-checked by
// the caller).  Its slot must be the query's alone: no two queries' new tokens
// in one block (one slot: two writers; two slots: the later one's cached part
// reads the earlier one's new slot), and no cached read covering a new slot
// (reads_of(id) = most tokens any cached part reads from block id).  Writes
// block * 16 + slot per query into code.
template <typename Reads>
kvattn_status check_new_slots(const kvattn_shape& s, const int32_t* block_tables, const int32_t* cached,
                              Reads reads_of, std::vector<int32_t>& code) {
    const int B = s.num_queries;
    std::vector<std::pair<int32_t, int>> owner(static_cast<size_t>(B));
    code.resize(size_t(B));
    for (int b = 0; b < B; ++b) {
        const int32_t id = block_tables[size_t(b) * s.max_blocks_per_seq + cached[b] / kBlock];
        if (id >= kMaxNewTokenBlock)
            return set_error(KVATTN_EUNSUPPORTED, "new token of query " + std::to_string(b) + " in block " +
                                                      std::to_string(id) + " >= 2^27");
        const int slot = cached[b] % kBlock;
        if (reads_of(id) > slot)
            return set_error(KVATTN_EINVAL, "new token slot " + std::to_string(slot) + " of block " + std::to_string(id) +
                                                " (query " + std::to_string(b) + ") is read by a cached part");
        owner[size_t(b)] = {id, b};
        code[size_t(b)] = id * kBlock + slot;
    }
    std::sort(owner.begin(), owner.end());
    for (int b = 1; b < B; ++b)
        if (owner[size_t(b)].first == owner[size_t(b) - 1].first)
            return set_error(KVATTN_EINVAL, "queries " + std::to_string(owner[size_t(b) - 1].second) + " and " +
                                                std::to_string(owner[size_t(b)].second) + " put their new tokens in block " +
                                                std::to_string(owner[size_t(b)].first));
    return KVATTN_OK;
}

// Maximal tree: a node is a maximal run of positions over which one fixed set
// of queries holds the same (physical block, token count) keys.
void derive_tree(const Batch& bt, std::vector<Node>& nodes, std::vector<int>& leaf) {
    std::vector<int> stack;
    auto make_children = [&](std::vector<int>& qs, int pos, int parent) {
        std::vector<std::pair<uint64_t, int>> kq;
        kq.reserve(qs.size());
        for (int q : qs) kq.emplace_back(bt.key(q, pos), q);
        std::sort(kq.begin(), kq.end());
        size_t i = 0;
        std::vector<int> created;
        while (i < kq.size()) {
            size_t j = i;
            while (j < kq.size() && kq[j].first == kq[i].first) ++j;
            Node n;
            n.parent = parent;
            n.pos_begin = pos;
            for (size_t t = i; t < j; ++t) n.queries.push_back(kq[t].second);
            std::sort(n.queries.begin(), n.queries.end());
            nodes.push_back(std::move(n));
            created.push_back(int(nodes.size()) - 1);
            i = j;
        }
        if (parent >= 0)
            for (int c : created) nodes[parent].children.push_back(c);
        for (auto it = created.rbegin(); it != created.rend(); ++it) stack.push_back(*it);
    };
    std::vector<int> all;               // queries with a cached part
    for (int b = 0; b < bt.B; ++b)
        if (bt.nb[b] > 0) all.push_back(b);
    if (!all.empty()) make_children(all, 0, -1);
    while (!stack.empty()) {
        int n = stack.back();
        stack.pop_back();
        const std::vector<int> qs = nodes[n].queries;
        int min_nb = bt.nb[qs[0]];
        for (int q : qs) min_nb = std::min(min_nb, bt.nb[q]);
        int p = nodes[n].pos_begin + 1;
        while (p < min_nb) {
            uint64_t k0 = bt.key(qs[0], p);
            bool same = true;
            for (size_t i = 1; i < qs.size() && same; ++i) same = bt.key(qs[i], p) == k0;
            if (!same) break;
            ++p;
        }
        nodes[n].pos_end = p;
        nodes[n].tokens = int64_t(kBlock) * (p - nodes[n].pos_begin - 1) + bt.valid(qs[0], p - 1);
        std::vector<int> rest;
        for (int q : qs) {
            if (bt.nb[q] == p)
                leaf[q] = n;
            else
                rest.push_back(q);
        }
        if (!rest.empty()) make_children(rest, p, n);
    }
}

// Check a caller-supplied tree against the block tables and adopt it.
kvattn_status adopt_tree(const Batch& bt, const kvattn_prefix_tree& t, std::vector<Node>& nodes,
                         std::vector<int>& leaf) {
    const int N = t.num_nodes;
    if (N < 1 || !t.parent || !t.block_begin || !t.block_end || !t.query_leaf)
        return set_error(KVATTN_EINVAL, "prefix tree: num_nodes < 1 or NULL array");
    nodes.assign(N, Node());
    for (int n = 0; n < N; ++n) {
        int p = t.parent[n], b0 = t.block_begin[n], b1 = t.block_end[n];
        if (p < -1 || p >= N || p == n) return set_error(KVATTN_EINVAL, "prefix tree: bad parent of node " + std::to_string(n));
        if (b0 < 0 || b1 <= b0 || b1 > bt.mb)
            return set_error(KVATTN_EINVAL, "prefix tree: bad block range of node " + std::to_string(n));
        if (p == -1 && b0 != 0) return set_error(KVATTN_EINVAL, "prefix tree: root must start at block 0");
        if (p >= 0 && b0 != t.block_end[p])
            return set_error(KVATTN_EINVAL, "prefix tree: node " + std::to_string(n) + " does not start where its parent ends");
        nodes[n].parent = p;
        nodes[n].pos_begin = b0;
        nodes[n].pos_end = b1;
    }
    // depth bound rules out cycles
    for (int n = 0; n < N; ++n) {
        int x = n, steps = 0;
        while (x != -1) {
            x = nodes[x].parent;
            if (++steps > N) return set_error(KVATTN_EINVAL, "prefix tree: cycle");
        }
    }
    for (int b = 0; b < bt.B; ++b) {
        int lf = t.query_leaf[b];
        if (bt.nb[b] == 0 && lf == -1) continue;   // no cached part (new-token plans)
        if (lf < 0 || lf >= N) return set_error(KVATTN_EINVAL, "prefix tree: bad leaf of query " + std::to_string(b));
        if (nodes[lf].pos_end != bt.nb[b])
            return set_error(KVATTN_EINVAL, "prefix tree: leaf of query " + std::to_string(b) + " does not end at its last block");
        leaf[b] = lf;
        for (int x = lf; x != -1; x = nodes[x].parent) nodes[x].queries.push_back(b);
    }
    for (int n = 0; n < N; ++n) {
        Node& nd = nodes[n];
        std::sort(nd.queries.begin(), nd.queries.end());
        if (nd.parent >= 0) nodes[nd.parent].children.push_back(n);
        if (nd.queries.empty()) continue;
        for (int j = nd.pos_begin; j < nd.pos_end; ++j) {
            uint64_t k0 = bt.key(nd.queries[0], j);
            for (int q : nd.queries)
                if (bt.key(q, j) != k0)
                    return set_error(KVATTN_EINVAL, "prefix tree: queries of node " + std::to_string(n) +
                                                        " differ at block position " + std::to_string(j));
        }
        nd.tokens = int64_t(kBlock) * (nd.pos_end - nd.pos_begin - 1) + bt.valid(nd.queries[0], nd.pos_end - 1);
    }
    return KVATTN_OK;
}

// A run of KV positions read by a fixed set of queries.
struct Unit {
    std::vector<int> queries;
    int ref_query;              // block table row that supplies the ids
    int pos_begin, pos_end;
    int64_t tokens;
    int fold_query = -1;        // scheme 2: this query also reads the leaf range below
    int fold_pos_end = 0;
    int64_t fold_tokens = 0;
};

struct Proto {                  // item before ordering
    Item it;
    double cost;
    std::vector<Entry> entries;
    std::vector<int32_t> blocks;
};

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

int64_t ceil16(int64_t x) { return (x + kBlock - 1) / kBlock * kBlock; }

// Item size caps: a chunk plus a folded leaf stays within kMaxItemBlocks
// (VALU) or kMfmaMaxItemBlocks (MFMA) blocks.
constexpr int64_t kFoldCapTokens = 256;
constexpr int64_t kChunkCapTokens = int64_t(kMaxItemBlocks) * kBlock - kFoldCapTokens;
constexpr int64_t kMfmaChunkCapTokens = int64_t(kMfmaMaxItemBlocks) * kBlock - kFoldCapTokens;

// Task costs, in units of one wave streaming one KV head-token with every CU
// busy (about 0.18 us on MI355X: 512 bytes at 1/2048 of the HBM bandwidth).
// An MFMA workgroup streams one KV head at four to five times a VALU wave's
// rate (measured on MI355X: ~45 ns against ~180-280 ns per head-token under
// load) after a pipeline fill of ~7 us; wider row groups add matrix work per
// token.  A VALU task adds a small boundary cost to its wave streams
// (epilogue, q rows); a fit of per-task traces (workgroup end times against
// blocks and tasks per list) put it near 1.5 block-times, and 24 units beat 8
// on the Llama-3-8B-shaped layer (49.1 against 49.8 us per call, two rounds;
// the other workloads within noise), while a larger MFMA task cost (100) was
// slower on both shared workloads.  With the task end's cross-lane reductions
// done by lane swaps instead of LDS permutes, 20 measured 43.4-44.0 against
// 44.0-44.5 us per call there (four rounds, two boxes; 12, 16 and 28 no better,
// the two-level tree and the no-sharing batch within noise).
constexpr double kMfmaTokenCost = 0.2;
constexpr double kMfmaTaskCost = 40.0;
constexpr double kValuTaskCost = 20.0;
// Partial triples are written into a saturated HBM read stream; on MI355X a
// VALU wave's small partial stores cost about twenty read bytes per byte
// (measured), which is why the VALU work is cut at most once per stripe.  An
// MFMA task writes its partials as one burst of up to 128 rows, which costs
// far less per byte.
constexpr double kPartialWriteCostMfma = 2.0;
// Relative streaming rate of the lists with an odd index, for launches whose
// lists hold at least kOddRateMinLoad units (32 blocks per wave); shorter
// lists keep 1.0, since a block is already ~10 % of them.  Lists w and w + 8
// share an XCD (and its L2); which XCD is up to the dispatcher, and per-task
// traces (the XCC_ID register, eager and graph launches, two GPUs) put
// workgroup w of the forward launch on XCC (w + 7) mod 8, so the odd lists run
// on the even-numbered XCCs.  The same traces show the odd-numbered XCCs
// streaming 8-12 % slower while every workgroup streams.  Measured with
// back-to-back calls: 1.1 took the no-sharing batch from 1506.1 to
// 1462.8-1468.9 us and the two-level tree from 232.6-233.2 to 228.8-229.5 us
// per call on two boxes (1.05 and 1.2 in between; 0.9, i.e. more work on the
// slower XCCs, cost 2.8 % and 2.5 %), while the Llama-3-8B-shaped layer,
// whose lists hold ~11 blocks, lost 2 % (hence the threshold).  MFMA-only
// launches take their rates through chunk lengths (kMfmaOddXcdRate,
// kMfmaSecondSlotRate below).  The rate is tied to that placement: on a GPU
// that placed workgroups otherwise the balance would be worse, the results
// the same.
constexpr double kOddXcdRate = 1.1;
constexpr double kOddRateMinLoad = 512.0;
// Relative streaming rate of the second workgroup of each CU (lists n_lists/2
// and up run on the same CUs as lists 0 and up, dispatched after them).
// Per-task traces show it 11-15 % slower per block for the whole launch.  A 0.9
// fill measured, over two boxes and two rounds each, 47.35-47.55 against
// 48.1-48.26 us per call on the Llama-3-8B-shaped layer and 231.0 against
// 233.4 us on the two-level tree; the no-sharing batch and the streaming
// sessions within noise (0.85: no better).
constexpr double kSecondSlotRate = 0.9;
// The same for the chunk classes of MFMA-only launches (four classes: XCD
// parity x workgroup slot, each chunk as long as its class's rate), where the
// second slot lags more: its chunks end ~5 % after the first slot's at 0.9.
// On the streaming sessions: equal chunks 1506-1510 us per call, parity
// classes at 1.1 1490-1503 us, four classes with 0.9 1476-1488 us, with 0.85
// 1461.7-1470.7 us (four rounds; 0.8: 1496-1502 us).
constexpr double kMfmaSecondSlotRate = 0.85;
// And the odd-list rate of those chunk classes (used only where the launch's
// odd-list rate applies): 1.15 measured 1467.9-1471.9 against 1475.7-1477.8 us
// per call (four rounds, 0.85 second slot) and 1476-1483 against 1483-1488 us
// with a 0.9 second slot.
constexpr double kMfmaOddXcdRate = 1.15;
// A list that runs MFMA tasks starts its VALU stream late and from cold: the
// descriptor window, the q rows and the first blocks each take a round trip
// under full load (per-task traces on MI355X: a 16-token VALU remainder after
// a C2 prefix task ended ~8 us after it).  A stripe with MFMA load is filled
// only above that load plus this start cost, so no such list gets a remainder
// too small to pay for its start.
constexpr double kValuRestartCost = 40.0;
// The VALU_SPLIT tile gives each of a workgroup's four waves at least one block
// of the range.
constexpr int kSplitMinBlocks = kWaves;
// Fixed cost of the merge launch and the launch gap before it, in block-times of
// one wave on an otherwise idle GPU (a wave streams a block in ~0.6 us there,
// two in flight; the merge launch of a small batch measured ~6 us).
constexpr double kMergeLaunchBlocks = 10.0;

// Append the descriptor of task t (see kDesc*) to P.desc; returns its words.
int32_t put_desc(kvattn_plan_s& P, const Task& t) {
    const Item& it = P.items[size_t(t.item)];
    const int nblk = (it.n_tokens + kBlock - 1) / kBlock;
    const int32_t words = desc_words(it.n_q, nblk);
    const size_t at = P.desc.size();
    P.desc.resize(at + size_t(words), 0);
    int32_t* d = P.desc.data() + at;
    int32_t lim_all = it.n_tokens;
    for (int e = 0; e < it.n_q; ++e) lim_all = std::min(lim_all, P.entries[size_t(it.q_begin + e)].limit);
    d[kDescKind] = it.kind;
    d[kDescTile] = it.tile;
    d[kDescHead] = t.head;
    d[kDescTokens] = it.n_tokens;
    d[kDescNq] = it.n_q;
    d[kDescRows] = it.n_rows;
    d[kDescBlocks] = nblk;
    d[kDescLimAll] = lim_all;
    d[kDescWords] = words;
    for (int e = 0; e < it.n_q; ++e) {
        const Entry& en = P.entries[size_t(it.q_begin + e)];
        d[kDescHeader + 4 * e + 0] = en.query;
        d[kDescHeader + 4 * e + 1] = en.dest;
        d[kDescHeader + 4 * e + 2] = en.limit;
        d[kDescHeader + 4 * e + 3] = en.dest >= 0 ? P.rec_of_query[size_t(en.query)] : -1;
    }
    int32_t* blk = d + kDescHeader + 4 * it.n_q;
    for (int j = 0; j < nblk; ++j) blk[j] = P.block_ids[size_t(it.blk_begin + j)];
    return words;
}

// Task descriptors of every launch, from the lists in P.tasks / P.list_ptr.
// Everything a task reads before its KV stream sits in one contiguous record:
// a 16-word header, the entries, the block ids.  A list's MFMA records lie back
// to back (each header gives the next one's size), so a workgroup finds the next
// record right after the current one and copies it into LDS while the current
// task streams; its VALU records follow and are copied into LDS in one piece.
// Returns false if a list's VALU records overflow the launch's LDS window.
bool serialize_lists(kvattn_plan_s& P) {
    const int n_lists = P.n_lists;
    const int D = P.shape.head_dim;
    P.desc.clear();
    P.desc_list_ptr.assign(P.forward_launches.size() * size_t(n_lists) * 3, 0);
    P.task_desc.assign(P.tasks.size(), 0);
    for (const Launch& Lr : P.forward_launches) {
        const int32_t window = valu_window_words(D, Lr.valu_rows);
        for (int w = 0; w < n_lists; ++w) {
            const int t0 = Lr.task_base + P.list_ptr[size_t(Lr.index) * (n_lists + 1) + w];
            const int t1 = Lr.task_base + P.list_ptr[size_t(Lr.index) * (n_lists + 1) + w + 1];
            int32_t* lp = P.desc_list_ptr.data() + (size_t(Lr.index) * n_lists + w) * 3;
            lp[0] = int32_t(P.desc.size());
            size_t prev = SIZE_MAX;
            int t = t0;
            for (; t < t1 && P.items[size_t(P.tasks[size_t(t)].item)].kind == KVATTN_VARIANT_MFMA; ++t) {
                const size_t at = P.desc.size();
                P.task_desc[size_t(t)] = int32_t(at);
                const int32_t words = put_desc(P, P.tasks[size_t(t)]);
                if (prev != SIZE_MAX) P.desc[prev + kDescNextWords] = words;
                prev = at;
            }
            lp[1] = int32_t(P.desc.size());
            for (; t < t1; ++t) {
                P.task_desc[size_t(t)] = int32_t(P.desc.size());
                put_desc(P, P.tasks[size_t(t)]);
            }
            lp[2] = int32_t(P.desc.size());
            if (lp[2] - lp[1] > window) return false;
        }
    }
    return true;
}

// Header and arrays of the device blob (the part kvattn_plan_upload copies);
// the partial triples follow it in the workspace.
void serialize_blob(kvattn_plan_s& P) {
    P.has_split = false;
    for (const Item& it : P.items) P.has_split |= it.kind == KVATTN_VARIANT_VALU_SPLIT;
    BlobHeader& h = P.header;
    std::memset(&h, 0, sizeof(h));
    h.magic = kBlobMagic;
    h.version = kBlobVersion;
    h.n_desc_words = int32_t(P.desc.size());
    h.n_merge_q = int32_t(P.merge_query.size());
    h.n_slots = P.n_slots;
    h.head_dim = P.shape.head_dim;
    h.n_tasks = int32_t(P.tasks.size());
    h.n_launches = int32_t(P.forward_launches.size());
    h.n_lists = P.n_lists;
    uint64_t off = align256(sizeof(BlobHeader));
    h.off_desc = off;         off = align256(off + P.desc.size() * 4);
    h.off_list_ptr = off;     off = align256(off + P.desc_list_ptr.size() * 4);
    h.off_merge_rec = off;    off = align256(off + P.merge_rec.size() * 4);
    h.off_claim = off;        off = align256(off + 2 * 4);   // one counter per stream
    h.off_arrive = off;
    if (P.fused_merge) off = align256(off + uint64_t(P.merge_query.size()) * uint64_t(P.shape.num_kv_heads) * 4);
    h.blob_bytes = off;
    h.off_part_ml = off;      off = align256(off + uint64_t(P.n_slots) * 8);
    h.off_part_acc = off;     off = align256(off + uint64_t(P.n_slots) * uint64_t(P.shape.head_dim) * 4);
    h.total_bytes = off;
    P.blob.assign(h.blob_bytes, 0);
    std::memcpy(P.blob.data(), &h, sizeof(h));
    auto put = [&](uint64_t at, const void* src, size_t n) {
        if (n) std::memcpy(P.blob.data() + at, src, n);
    };
    put(h.off_desc, P.desc.data(), P.desc.size() * 4);
    put(h.off_list_ptr, P.desc_list_ptr.data(), P.desc_list_ptr.size() * 4);
    put(h.off_merge_rec, P.merge_rec.data(), P.merge_rec.size() * 4);
}

}  // namespace

kvattn_status build_plan(const kvattn_shape& s, const int32_t* block_tables, const int32_t* seq_lens,
                         const kvattn_prefix_tree* tree, const kvattn_plan_options& o, kvattn_plan_s& P) {
    const auto t0 = std::chrono::steady_clock::now();
    const int B = s.num_queries, Hq = s.num_q_heads, Hkv = s.num_kv_heads, D = s.head_dim;
    const int G = Hq / Hkv;
    if (kvattn_status vs = check_tables(s, block_tables, seq_lens); vs != KVATTN_OK) return vs;
    // New-token plans cover each query's cached part, its first seq_len - 1
    // tokens; the last one comes with the call and joins in the merge.
    std::vector<int32_t> cached;
    std::vector<int32_t> new_slot;
    if (o.new_token) {
        cached.resize(size_t(B));
        for (int b = 0; b < B; ++b) cached[size_t(b)] = seq_lens[b] - 1;
        seq_lens = cached.data();
        P.reads = block_reads(s, block_tables, seq_lens);
        kvattn_status ns = check_new_slots(s, block_tables, seq_lens, [&](int32_t id) { return P.reads[size_t(id)]; },
                                           new_slot);
        if (ns != KVATTN_OK) return ns;
    }
    Batch bt{B, s.max_blocks_per_seq, block_tables, seq_lens, std::vector<int>(B)};
    for (int b = 0; b < B; ++b) bt.nb[b] = (seq_lens[b] + kBlock - 1) / kBlock;

    // ---- prefix tree ---------------------------------------------------------
    std::vector<Node> nodes;
    std::vector<int> leaf(B, -1);
    if (tree) {
        kvattn_status st = adopt_tree(bt, *tree, nodes, leaf);
        if (st != KVATTN_OK) return st;
    } else {
        derive_tree(bt, nodes, leaf);
    }

    const int64_t bpt = int64_t(2) * Hkv * D * 2;          // K+V bytes per token, all KV heads
    const int64_t partial_row_bytes = int64_t(D + 2) * 4;   // one (m, l, acc) triple
    const int num_cus = o.num_cus > 0 ? o.num_cus : 256;

    // ---- one launch for batches too small to fill the GPU (runtime tile selector) ----
    // Cutting ranges across workgroups spreads a decode over the GPU but adds
    // partials and a merge launch.  A batch whose (query, KV head) blocks, read
    // as they are, do not even give every wave one block leaves most of the GPU
    // idle either way; when each query's range, read four-wide by the
    // VALU_SPLIT tile, then finishes sooner than the usual plan's share plus the
    // merge launch's fixed cost, the plan reads each query's own range once per
    // KV head, in one launch, with no packs, cuts or partials.  Times are in
    // block-times of one wave.  New-token plans take the same decision for their
    // forward; their merge launch (which adds the new tokens) follows either way,
    // and on such batches the usual plan's many small pieces cost about a launch
    // more than its model time (measured on MI355X: the tiny batch's fused append
    // takes 9.3 us with this forward against 13.0 us with the usual one).
    bool one_launch = false;
    if (o.pack_mode == KVATTN_PACK_AUTO && o.force_variant == KVATTN_VARIANT_AUTO && o.split_tokens == 0 &&
        !o.multi_stream && G <= valu_max_rows(D)) {
        const double waves = double(num_cus) * 2.0 * kWaves;
        double t_one = 0.0, all = 0.0;
        int max_nb = 0;
        for (int b = 0; b < B; ++b) {
            const int nb = bt.nb[b];
            max_nb = std::max(max_nb, nb);
            t_one = std::max(t_one, nb >= kSplitMinBlocks ? std::ceil(nb / double(kWaves)) : double(nb));
            all += double(nb) * Hkv;
        }
        double uniq_tok = 0.0;
        for (int32_t v : block_reads(s, block_tables, seq_lens)) uniq_tok += v;
        const double t_two = std::ceil(uniq_tok / kBlock * Hkv / waves) + kMergeLaunchBlocks;
        one_launch = all <= waves && max_nb <= kMaxItemBlocks && t_one <= t_two;
    }

    // ---- pack decision (profit model) -----------------------------------------
    int packed_nodes = 0;
    for (Node& n : nodes) {
        const int64_t k = int64_t(n.queries.size());
        if (k < 2 || o.pack_mode == KVATTN_PACK_QUERY || one_launch) continue;
        if (o.pack_mode == KVATTN_PACK_FULL) {
            n.packed = true;
        } else {
            // bytes saved by reading the node once instead of k times, against the
            // partial triples the pack adds (written by forward, read by merge) for
            // every (query, q head) and every ~2K-token chunk of the node.
            const double saved = double(k - 1) * double(n.tokens) * double(bpt);
            const double chunks = 1.0 + double(n.tokens) / 2048.0;
            const double extra = 2.0 * double(k) * Hq * double(partial_row_bytes) * chunks;
            n.packed = saved > extra;
        }
        packed_nodes += n.packed;
    }

    // ---- scheme 2: fold one short singleton leaf into its packed parent ------
    int folded = 0;
    if (o.scheme != 1) {
        // a folded leaf rides on the parent's last chunk; the cap keeps an item
        // within the item block caps together with the chunk caps below
        const int64_t fold_max = o.scheme == 2 ? kFoldCapTokens : 128;
        for (size_t ni = 0; ni < nodes.size(); ++ni) {
            Node& n = nodes[ni];
            if (!n.packed) continue;
            int best = -1;
            for (int c : n.children) {
                const Node& cn = nodes[c];
                if (cn.queries.size() != 1 || !cn.children.empty() || cn.tokens > fold_max) continue;
                if (leaf[cn.queries[0]] != c) continue;
                if (best < 0 || cn.tokens < nodes[best].tokens ||
                    (cn.tokens == nodes[best].tokens && cn.queries[0] < nodes[best].queries[0]))
                    best = c;
            }
            if (best >= 0) {
                n.fold_child = best;
                ++folded;
            }
        }
    }

    // ---- units: packed nodes, then each query's private runs -------------------
    std::vector<Unit> units;
    std::vector<char> folded_leaf(nodes.size(), 0);
    for (size_t ni = 0; ni < nodes.size(); ++ni) {
        const Node& n = nodes[ni];
        if (!n.packed) continue;
        Unit u;
        u.queries = n.queries;
        u.ref_query = n.queries[0];
        u.pos_begin = n.pos_begin;
        u.pos_end = n.pos_end;
        u.tokens = n.tokens;
        if (n.fold_child >= 0) {
            const Node& c = nodes[n.fold_child];
            u.fold_query = c.queries[0];
            u.fold_pos_end = c.pos_end;
            u.fold_tokens = c.tokens;
            folded_leaf[n.fold_child] = 1;
        }
        units.push_back(std::move(u));
    }
    {
        std::vector<int> path;
        for (int b = 0; b < B; ++b) {
            path.clear();
            for (int x = leaf[b]; x != -1; x = nodes[x].parent) path.push_back(x);
            std::reverse(path.begin(), path.end());
            int run_begin = -1, run_end = -1;
            auto flush = [&]() {
                if (run_begin < 0) return;
                Unit u;
                u.queries = {b};
                u.ref_query = b;
                u.pos_begin = run_begin;
                u.pos_end = run_end;
                u.tokens = int64_t(kBlock) * (run_end - run_begin - 1) + bt.valid(b, run_end - 1);
                units.push_back(std::move(u));
                run_begin = -1;
            };
            for (int x : path) {
                const Node& n = nodes[x];
                if (n.packed || folded_leaf[x]) {
                    flush();
                    continue;
                }
                if (run_begin < 0) run_begin = n.pos_begin;
                run_end = n.pos_end;
            }
            flush();
        }
    }

    // ---- row groups and kernel variant (runtime tile selector) -------------------
    // VALU: at most 8 rows per KV head; MFMA: at most 128 rows (4 waves x 32),
    // 16 rows per wave when the group fits 64 rows.  Wider packs are split into
    // row groups that read the same KV range (in the same XCD's L2).
    struct Group {
        int unit;
        std::vector<int> queries;
        int kind, tile, rows;
        double w;                // cost per token and KV head relative to streaming it from HBM
    };
    // VALU groups read ranges of kSplitMinBlocks or more blocks with the VALU_SPLIT
    // tile when it is forced or in a one-launch plan; shorter ones keep the VALU tile.
    const bool split_tiles = one_launch || o.force_variant == KVATTN_VARIANT_VALU_SPLIT;
    std::vector<Group> groups;
    for (size_t ui = 0; ui < units.size(); ++ui) {
        const Unit& u = units[ui];
        const int R = int(u.queries.size()) * G;
        int kind;
        if (o.force_variant == KVATTN_VARIANT_VALU || o.force_variant == KVATTN_VARIANT_VALU_SPLIT) {
            if (G > valu_max_rows(D))
                return set_error(KVATTN_EUNSUPPORTED, "VALU forward holds at most " + std::to_string(valu_max_rows(D)) +
                                                          " rows per KV head at this head_dim");
            kind = KVATTN_VARIANT_VALU;
        } else if (o.force_variant == KVATTN_VARIANT_MFMA) {
            kind = KVATTN_VARIANT_MFMA;
        } else {
            kind = (R <= valu_max_rows(D)) ? KVATTN_VARIANT_VALU : KVATTN_VARIANT_MFMA;
        }
        const int max_rows = kind == KVATTN_VARIANT_VALU ? valu_max_rows(D) : kMfmaMaxRows;
        const int qpg = std::max(1, max_rows / G);
        const int n = int(u.queries.size());
        const int ng = (n + qpg - 1) / qpg;
        for (int gi = 0; gi < ng; ++gi) {
            Group g;
            g.unit = int(ui);
            const int lo = int(int64_t(n) * gi / ng), hi = int(int64_t(n) * (gi + 1) / ng);
            g.queries.assign(u.queries.begin() + lo, u.queries.begin() + hi);
            g.kind = kind;
            g.rows = int(g.queries.size()) * G;
            if (kind == KVATTN_VARIANT_VALU) {
                g.tile = next_pow2(g.rows);
                g.w = 1.0;
            } else {
                g.tile = g.rows <= 64 ? 1 : 2;
                g.w = kMfmaTokenCost * (1.0 + std::max(0, g.rows - 64) / 256.0);
            }
            groups.push_back(std::move(g));
        }
    }

    // ---- forward launches ----------------------------------------------------------------
    // One launch runs VALU and MFMA tasks side by side.  Launch i takes the
    // i-th largest VALU row template and the i-th largest MFMA tiling, so a
    // plan needs max(#templates, #tilings) launches -- normally one.
    std::vector<int> vt, mt;
    for (const Group& g : groups) {
        std::vector<int>& v = g.kind == KVATTN_VARIANT_MFMA ? mt : vt;
        if (std::find(v.begin(), v.end(), g.tile) == v.end()) v.push_back(g.tile);
    }
    std::sort(vt.begin(), vt.end(), std::greater<int>());
    std::sort(mt.begin(), mt.end(), std::greater<int>());
    // VALU groups share the largest row template: a second launch (its gap,
    // ramp and tail, ~5 us) costs more than the idle rows of the smaller groups,
    // whose streams are bandwidth-bound anyway
    if (vt.size() > 1 && vt.size() > mt.size()) {
        for (Group& g : groups)
            if (g.kind == KVATTN_VARIANT_VALU) g.tile = vt[0];
        vt.resize(1);
    }
    const int n_launch = int(std::max(vt.size(), mt.size()));
    auto launch_of = [&](const Group& g) {
        const std::vector<int>& v = g.kind == KVATTN_VARIANT_MFMA ? mt : vt;
        return int(std::find(v.begin(), v.end(), g.tile) - v.begin());
    };

    // ---- schedule: MFMA tasks placed longest first, VALU work cut to fill -------------------
    // Time unit: one wave streaming one KV head-token with every CU busy.  Each
    // launch has n_lists static lists, one per persistent workgroup.
    //  * MFMA items (packed groups) run one task per KV head on a whole
    //    workgroup.  Their chunk length is chosen from a few candidates; for
    //    each, the tasks are placed longest first on the least-loaded list (an
    //    MFMA task of KV head g prefers a list w = g mod 8 (mod 8) -- workgroups
    //    w and w + 8 run on one XCD -- so the row groups and chunks reading one
    //    head's shared range meet in one L2).
    //  * VALU items run one task per four KV heads, one wave per head, as part
    //    of continuous per-wave streams.  The lists are taken in groups of
    //    ceil(Hkv / 4) lists on one XCD ("stripes", all KV heads of an item);
    //    the VALU token stream of the launch (every VALU range in order) is cut
    //    into pieces that fill every stripe up to one common level above its
    //    MFMA load.  The stripes then end together, and at most one cut per
    //    stripe adds partial triples.
    //  The candidate with the lowest makespan plus partial-write cost wins.
    //  Forced split lengths (tests) cut every range uniformly instead and place
    //  VALU items on the least-loaded stripe.
    const int n_lists = num_cus * 2;
    const int quads = (Hkv + kWaves - 1) / kWaves;
    const int n_stripes = std::max(1, n_lists / quads);
    // A stripe's lists sit on one XCD (workgroups w and w + 8 share one):
    // members w, w + 8, ... when the lists split evenly, so they stream at one rate.
    const bool xcd_stripes = n_lists % (kXcds * quads) == 0;
    auto stripe_list = [&](int s, int q) {
        return xcd_stripes ? (s / kXcds) * kXcds * quads + s % kXcds + kXcds * q : s * quads + q;
    };
    // relative streaming rate of list w (XCD parity and workgroup slot); the
    // odd-list rate is set per launch
    double odd_rate = 1.0;
    // odd lists run on the faster (even-numbered) XCCs; second-slot lists share CUs with the first slot's
    auto list_rate = [&](int w) { return ((w % kXcds) % 2 ? odd_rate : 1.0) * (w >= n_lists / 2 ? kSecondSlotRate : 1.0); };
    auto stripe_rate = [&](int s) { return list_rate(stripe_list(s, 0)); };
    const double pu_mfma = (kPartialWriteCostMfma + 1.0) * double(partial_row_bytes) / double(2 * D * 2);
    auto mfma_cost = [&](const Group& g, int64_t tok) { return double(tok) * g.w + kMfmaTaskCost; };
    auto unit_tokens = [&](const Group& g) { return units[g.unit].tokens; };

    struct Piece {                      // a chunk of one group's range, before it becomes an item
        int group;
        int64_t tok0, ntok;             // range within the group's unit (ntok excludes a folded leaf)
        bool last;
        int stripe = -1;                // VALU: stripe; MFMA: -1
        std::vector<int> head_list;     // MFMA: list of each KV head's task; one-launch VALU plans: list of
                                        // each task (per KV head, or per four heads on the VALU tile)
        bool split = false;             // VALU piece on the VALU_SPLIT tile
    };
    std::vector<Piece> pieces;
    int64_t C = 0;                      // longest chunk of a split range (statistics)

    for (int L = 0; L < n_launch; ++L) {
        std::vector<int> mg, vg;
        for (size_t gi = 0; gi < groups.size(); ++gi) {
            if (launch_of(groups[gi]) != L) continue;
            (groups[gi].kind == KVATTN_VARIANT_MFMA ? mg : vg).push_back(int(gi));
        }
        double w_valu = 0.0, w_mfma = 0.0;
        for (int gi : vg) w_valu += double(unit_tokens(groups[gi])) * quads;
        for (int gi : mg) w_mfma += double(unit_tokens(groups[gi])) * groups[gi].w * Hkv;
        const double mean0 = std::max(64.0, (w_valu + w_mfma) / n_lists);
        odd_rate = mean0 >= kOddRateMinLoad ? kOddXcdRate : 1.0;

        // chunks of MFMA group g at a target task cost `target`
        auto mfma_chunks = [&](const Group& g, double target) {
            int64_t chunk;
            if (o.split_tokens > 0) {
                chunk = std::min<int64_t>(ceil16(o.split_tokens), kMfmaChunkCapTokens);
            } else {
                chunk = ceil16(int64_t(std::ceil((target - kMfmaTaskCost) / g.w)));
                chunk = std::min<int64_t>(std::max<int64_t>(chunk, 128), kMfmaChunkCapTokens);
            }
            return (unit_tokens(g) + chunk - 1) / chunk;
        };
        // MFMA chunking and placement for a target task cost `target`
        struct MfmaPlan {
            std::vector<Piece> pieces;
            std::vector<double> load;
            double extra = 0.0;
        };
        // Rate classes of MFMA chunks.  An MFMA-only launch has no VALU work to
        // fill by rate, and a group's chunk serves all its KV heads at once, so
        // the rates enter through chunk lengths: with ncls = 2 a group's chunks
        // alternate between even and odd lists (XCD parity), with ncls = 4 also between
        // first- and second-slot lists, each as long as its class's rate.
        auto class_rate = [&](int cls) {
            return (cls & 1 ? kMfmaOddXcdRate : 1.0) * (cls >> 1 ? kMfmaSecondSlotRate : 1.0);
        };
        // chunk lengths of group g at `target` (ncls 1: equal chunks)
        auto chunk_lens = [&](const Group& g, double target, int ncls) {
            const int64_t tokens = unit_tokens(g);
            const int64_t nch = mfma_chunks(g, target);
            std::vector<int64_t> lens;
            if (ncls == 1) {
                const int64_t len = ceil16((tokens + nch - 1) / nch);
                for (int64_t t0 = 0; t0 < tokens; t0 += len) lens.push_back(std::min(len, tokens - t0));
                return lens;
            }
            double sum = 0.0;
            for (int64_t c = 0; c < nch; ++c) sum += class_rate(int(c % ncls));
            int64_t t0 = 0;
            for (int64_t c = 0; c < nch && t0 < tokens; ++c) {
                const int64_t len = c == nch - 1 ? tokens - t0
                                                 : ceil16(int64_t(std::ceil(double(tokens) * class_rate(int(c % ncls)) / sum)));
                lens.push_back(std::min(len, tokens - t0));
                t0 += lens.back();
            }
            return lens;
        };
        auto place_mfma = [&](double target, int ncls) {
            MfmaPlan mp;
            mp.load.assign(size_t(n_lists), 0.0);
            struct T {
                int piece, head;
                double cost;
                int cls;   // rate class of the task's list (ncls > 1); else -1
            };
            std::vector<T> tasks;
            for (int gi : mg) {
                const Group& g = groups[size_t(gi)];
                const int64_t tokens = unit_tokens(g);
                const std::vector<int64_t> lens = chunk_lens(g, target, ncls);
                mp.extra += double(lens.size() - 1) * g.rows * Hkv * pu_mfma;
                int64_t tok0 = 0;
                for (size_t c = 0; c < lens.size(); ++c) {
                    Piece pc;
                    pc.group = gi;
                    pc.tok0 = tok0;
                    pc.ntok = lens[c];
                    pc.last = tok0 + pc.ntok == tokens;
                    pc.head_list.assign(size_t(Hkv), 0);
                    const int64_t with_fold = pc.ntok + (pc.last ? units[g.unit].fold_tokens : 0);
                    for (int h = 0; h < Hkv; ++h)
                        tasks.push_back({int(mp.pieces.size()), h, mfma_cost(g, with_fold), ncls > 1 ? int(c % size_t(ncls)) : -1});
                    tok0 += pc.ntok;
                    mp.pieces.push_back(std::move(pc));
                }
            }
            std::stable_sort(tasks.begin(), tasks.end(), [](const T& a, const T& b) { return a.cost > b.cost; });
            // one min-heap of (load, list) per XCD and workgroup slot; the least-loaded
            // list overall is the least of the heap minima
            using LE = std::pair<double, int>;
            using Heap = std::priority_queue<LE, std::vector<LE>, std::greater<LE>>;
            // keys are times: a list's load divided by its rate
            std::vector<Heap> heap_xs(2 * kXcds);
            auto hidx = [&](int w) { return w % kXcds + (w >= n_lists / 2 ? kXcds : 0); };
            for (int w = 0; w < n_lists; ++w) heap_xs[size_t(hidx(w))].push({0.0, w});
            auto allowed = [&](const T& t, int h) {
                if (t.cls < 0) return true;
                if ((h % kXcds) % 2 != (t.cls & 1)) return false;
                return ncls < 4 || (h >= kXcds) == ((t.cls >> 1) != 0);
            };
            for (const T& t : tasks) {
                int hb = -1;
                for (int h = 0; h < 2 * kXcds; ++h)
                    if (allowed(t, h) && !heap_xs[size_t(h)].empty() &&
                        (hb < 0 || heap_xs[size_t(h)].top() < heap_xs[size_t(hb)].top()))
                        hb = h;
                // preferred: a list of the XCD of the task's KV head (of the class's parity)
                const int xp = t.cls < 0 ? t.head % kXcds : ((t.head % kXcds) & ~1) | (t.cls & 1);
                int hp = -1;
                for (int h : {xp, xp + kXcds})
                    if (allowed(t, h) && !heap_xs[size_t(h)].empty() &&
                        (hp < 0 || heap_xs[size_t(h)].top() < heap_xs[size_t(hp)].top()))
                        hp = h;
                int h = hb;
                if (hp >= 0 && heap_xs[size_t(hp)].top().first <= heap_xs[size_t(hb)].top().first + 0.25 * t.cost) h = hp;
                const int w = heap_xs[size_t(h)].top().second;
                heap_xs[size_t(h)].pop();
                mp.pieces[size_t(t.piece)].head_list[size_t(t.head)] = w;
                mp.load[size_t(w)] += t.cost;
                heap_xs[size_t(h)].push({mp.load[size_t(w)] / list_rate(w), w});
            }
            return mp;
        };
        // the stripes' common fill level for the VALU work above their MFMA loads
        auto stripe_base = [&](const std::vector<double>& load) {
            std::vector<double> base(size_t(n_stripes), 0.0);
            // multi-stream plans run the MFMA lists in a launch of their own, beside the VALU one
            if (o.multi_stream) return base;
            for (int s = 0; s < n_stripes; ++s) {
                for (int q = 0; q < quads; ++q) base[size_t(s)] = std::max(base[size_t(s)], load[size_t(stripe_list(s, q))]);
                if (base[size_t(s)] > 0.0) base[size_t(s)] += kValuRestartCost;
            }
            return base;
        };
        // the level at which the stripes, each filled from its base, hold `work`
        auto fill_level = [&](const std::vector<double>& base, double work) {
            double lo = *std::min_element(base.begin(), base.end());
            double hi = 0.0, rmin = 1.0;
            for (int s = 0; s < n_stripes; ++s) {
                hi = std::max(hi, base[size_t(s)] / stripe_rate(s));
                rmin = std::min(rmin, stripe_rate(s));
            }
            hi += work / (n_stripes * rmin) + 1.0;   // every stripe then holds >= work / n_stripes
            for (int it = 0; it < 60; ++it) {
                const double mid = 0.5 * (lo + hi);
                double cap = 0.0;
                for (int s = 0; s < n_stripes; ++s) cap += std::max(0.0, mid * stripe_rate(s) - base[size_t(s)]);
                (cap >= work ? hi : lo) = mid;
            }
            return hi;
        };
        const double valu_work = w_valu / quads + kValuTaskCost * double(vg.size() + size_t(n_stripes));

        MfmaPlan best;
        bool have = false;
        double best_score = 0.0;
        std::vector<double> targets{mean0};
        if (!mg.empty() && o.split_tokens <= 0) {
            targets.push_back(2.0 * mean0);
            for (int i = 1; i <= 24; ++i) targets.push_back(mean0 * std::pow(2.0, -i / 4.0));
            // task costs at which the MFMA work makes whole numbers of tasks per list
            for (int k = 1; k <= 8; ++k)
                targets.push_back((w_mfma + double(k) * n_lists * kMfmaTaskCost) / (double(k) * n_lists));
        }
        std::set<std::vector<int64_t>> tried;   // chunk counts per group already placed
        for (double target : targets) {
            std::vector<int64_t> key;
            int64_t n_tasks = 0;
            for (int gi : mg) {
                key.push_back(mfma_chunks(groups[size_t(gi)], target));
                n_tasks += key.back() * Hkv;
            }
            // more than 16 MFMA tasks per list never pays for its partials
            if (have && n_tasks > 16 * int64_t(n_lists)) continue;
            if (!tried.insert(key).second) continue;
            // rate-class chunking (MFMA-only launches): 2 classes with an odd-list
            // rate, 4 with a second-slot rate too; every group's chunk count a
            // multiple of the class count, no chunk over the cap
            std::vector<int> classes{1};
            for (int ncls : {2, 4}) {
                bool ok = vg.empty() && odd_rate != 1.0 && (ncls == 2 || kMfmaSecondSlotRate != 1.0) && o.split_tokens <= 0 &&
                          n_lists % (2 * kXcds) == 0;
                for (int gi : mg) {
                    const Group& g = groups[size_t(gi)];
                    const int64_t nch = mfma_chunks(g, target);
                    if (!ok || nch < ncls || nch % ncls != 0) { ok = false; break; }
                    for (int64_t l : chunk_lens(g, target, ncls)) ok = ok && l <= kMfmaChunkCapTokens;
                }
                if (ok) classes.push_back(ncls);
            }
            for (int ncls : classes) {
                MfmaPlan mp = place_mfma(target, ncls);
                const std::vector<double> base = stripe_base(mp.load);
                double makespan = 0.0;
                for (int w = 0; w < n_lists; ++w) makespan = std::max(makespan, mp.load[size_t(w)] / list_rate(w));
                if (!vg.empty()) makespan = std::max(makespan, fill_level(base, valu_work));
                const double score = makespan + mp.extra / (double(n_lists) * kWaves);
                if (!have || score < best_score * 0.995) {
                    best = std::move(mp);
                    best_score = score;
                    have = true;
                }
            }
        }
        for (const Piece& pc : best.pieces) C = std::max(C, pc.ntok < unit_tokens(groups[size_t(pc.group)]) ? pc.ntok : 0);
        const std::vector<double> base = stripe_base(best.load);

        // VALU pieces
        auto split_piece = [&](int64_t ntok) { return split_tiles && (ntok + kBlock - 1) / kBlock >= kSplitMinBlocks; };
        if (one_launch) {
            // Each range whole (up to the item cap); its tasks -- one per KV head on the
            // VALU_SPLIT tile, one per four heads on the VALU tile -- placed longest
            // first on the least-loaded list, in block-times of one wave.  A task of KV
            // head (or head quad) k prefers a list w = k (mod 8), one XCD, so the queries that
            // share a range read its blocks through one L2: they run at the same time,
            // and the L2 fetches each block from HBM once for all of them.
            struct T {
                size_t piece;
                int slot;
                double cost;
            };
            std::vector<T> tl;
            const size_t first_piece = best.pieces.size();
            for (int gi : vg) {
                const int64_t tokens = unit_tokens(groups[size_t(gi)]);
                const int64_t nch = (tokens + kChunkCapTokens - 1) / kChunkCapTokens;
                const int64_t len = ceil16((tokens + nch - 1) / nch);
                for (int64_t c = 0; c < nch; ++c) {
                    const int64_t tok0 = c * len;
                    if (tok0 >= tokens) break;
                    Piece pc;
                    pc.group = gi;
                    pc.tok0 = tok0;
                    pc.ntok = std::min(len, tokens - tok0);
                    pc.last = tok0 + pc.ntok == tokens;
                    pc.split = split_piece(pc.ntok);
                    if (pc.ntok < tokens) C = std::max(C, pc.ntok);
                    const double nb = double((pc.ntok + kBlock - 1) / kBlock);
                    const int n_t = pc.split ? Hkv : quads;
                    pc.head_list.assign(size_t(n_t), 0);
                    for (int k = 0; k < n_t; ++k)
                        tl.push_back({best.pieces.size(), k, pc.split ? std::ceil(nb / kWaves) : nb});
                    best.pieces.push_back(std::move(pc));
                }
            }
            std::stable_sort(tl.begin(), tl.end(), [](const T& a, const T& b) { return a.cost > b.cost; });
            using LE = std::pair<double, int>;
            using Heap = std::priority_queue<LE, std::vector<LE>, std::greater<LE>>;
            std::vector<Heap> heap_x(kXcds);   // keys are times: load / rate
            std::vector<double> lload(static_cast<size_t>(n_lists), 0.0);
            for (int w = 0; w < n_lists; ++w) heap_x[size_t(w % kXcds)].push({0.0, w});
            for (const T& t : tl) {
                int xb = -1;
                for (int x = 0; x < kXcds; ++x)
                    if (!heap_x[size_t(x)].empty() && (xb < 0 || heap_x[size_t(x)].top() < heap_x[size_t(xb)].top())) xb = x;
                const int xp = t.slot % kXcds;
                int x = xb;
                if (!heap_x[size_t(xp)].empty() && heap_x[size_t(xp)].top().first <= heap_x[size_t(xb)].top().first + 0.25 * t.cost)
                    x = xp;
                const int w = heap_x[size_t(x)].top().second;
                heap_x[size_t(x)].pop();
                best.pieces[t.piece].head_list[size_t(t.slot)] = w;
                lload[size_t(w)] += t.cost + kValuTaskCost / kBlock;
                heap_x[size_t(x)].push({lload[size_t(w)] / list_rate(w), w});
            }
            (void)first_piece;
        } else if (o.split_tokens > 0) {
            const int64_t chunk = std::min<int64_t>(ceil16(o.split_tokens), kChunkCapTokens);
            std::vector<double> sload = base;
            for (int gi : vg) {
                const int64_t tokens = unit_tokens(groups[size_t(gi)]);
                const int64_t nch = (tokens + chunk - 1) / chunk;
                const int64_t len = ceil16((tokens + nch - 1) / nch);
                for (int64_t c = 0; c < nch; ++c) {
                    const int64_t tok0 = c * len;
                    if (tok0 >= tokens) break;
                    Piece pc;
                    pc.group = gi;
                    pc.tok0 = tok0;
                    pc.ntok = std::min(len, tokens - tok0);
                    pc.last = tok0 + pc.ntok == tokens;
                    pc.split = split_piece(pc.ntok);
                    pc.stripe = int(std::min_element(sload.begin(), sload.end()) - sload.begin());
                    sload[size_t(pc.stripe)] += double(pc.ntok) + kValuTaskCost;
                    if (pc.ntok < tokens) C = std::max(C, pc.ntok);
                    best.pieces.push_back(std::move(pc));
                }
            }
        } else if (!vg.empty()) {
            // Greedy pass: stripes in order, each filled up to `level` with whole
            // blocks.  Returns the work left over for the last stripe past level.
            auto fill = [&](double level, std::vector<Piece>* out) {
                int s = 0;
                double room = level * stripe_rate(0) - base[0];
                double over = 0.0;
                for (int gi : vg) {
                    const int64_t tokens = unit_tokens(groups[size_t(gi)]);
                    int64_t t0 = 0;
                    while (t0 < tokens) {
                        // move on when the stripe cannot take one more block
                        while (s < n_stripes - 1 && room < kValuTaskCost + kBlock) {
                            ++s;
                            room = level * stripe_rate(s) - base[size_t(s)];
                        }
                        int64_t take = tokens - t0;
                        if (s < n_stripes - 1) {
                            const int64_t fit = int64_t(std::floor((room - kValuTaskCost) / kBlock)) * kBlock;
                            take = std::min(take, std::max<int64_t>(fit, kBlock));
                        }
                        take = std::min<int64_t>(take, kChunkCapTokens);
                        if (out) {
                            Piece pc;
                            pc.group = gi;
                            pc.tok0 = t0;
                            pc.ntok = take;
                            pc.last = t0 + take == tokens;
                            pc.split = split_piece(take);
                            pc.stripe = s;
                            if (take < tokens) C = std::max(C, take);
                            out->push_back(std::move(pc));
                        }
                        room -= double(take) + kValuTaskCost;
                        t0 += take;
                    }
                }
                if (room < 0) over = -room;
                return over;
            };
            // lowest level at which the last stripe ends within one block of it
            double lo = fill_level(base, valu_work), hi = lo;
            while (fill(hi, nullptr) > kBlock + kValuTaskCost) hi += std::max(1.0, hi - lo) + kBlock;
            for (int it = 0; it < 40 && hi - lo > 0.5; ++it) {
                const double mid = 0.5 * (lo + hi);
                (fill(mid, nullptr) > kBlock + kValuTaskCost ? lo : hi) = mid;
            }
            fill(hi, &best.pieces);
        }
        for (Piece& pc : best.pieces) pieces.push_back(std::move(pc));
    }

    // ---- items ----------------------------------------------------------------------
    std::vector<Proto> protos;
    std::vector<const Piece*> proto_piece;
    for (const Piece& pc : pieces) {
        const Group& g = groups[size_t(pc.group)];
        const Unit& u = units[g.unit];
        const bool has_fold = u.fold_query >= 0 &&
                              std::find(g.queries.begin(), g.queries.end(), u.fold_query) != g.queries.end();
        Proto p;
        p.it.kind = g.kind == KVATTN_VARIANT_VALU && pc.split ? KVATTN_VARIANT_VALU_SPLIT : g.kind;
        p.it.tile = g.tile;
        p.it.pos_begin = u.pos_begin + int(pc.tok0 / kBlock);
        const int nblk = int((pc.ntok + kBlock - 1) / kBlock);
        for (int j = 0; j < nblk; ++j) p.blocks.push_back(bt.id(u.ref_query, p.it.pos_begin + j));
        int64_t item_tokens = pc.ntok;
        for (int q : g.queries) {
            Entry e{q, -1, int32_t(pc.ntok), 0};
            if (has_fold && pc.last && q == u.fold_query) e.limit = int32_t(pc.ntok + u.fold_tokens);
            p.entries.push_back(e);
        }
        if (has_fold && pc.last) {
            for (int j = u.pos_end; j < u.fold_pos_end; ++j) p.blocks.push_back(bt.id(u.fold_query, j));
            item_tokens = pc.ntok + u.fold_tokens;
        }
        if ((item_tokens + kBlock - 1) / kBlock > (g.kind == KVATTN_VARIANT_MFMA ? kMfmaMaxItemBlocks : kMaxItemBlocks))
            return set_error(KVATTN_EINVAL, "internal: item exceeds the per-item block cap");
        p.it.n_tokens = int32_t(item_tokens);
        p.it.n_q = int32_t(g.queries.size());
        p.it.n_rows = g.rows;
        p.cost = g.kind == KVATTN_VARIANT_MFMA ? mfma_cost(g, item_tokens) : double(item_tokens) + kValuTaskCost;
        protos.push_back(std::move(p));
        proto_piece.push_back(&pc);
    }
    auto proto_launch = [&](size_t i) { return launch_of(groups[size_t(proto_piece[i]->group)]); };

    // ---- item order: by launch, MFMA before VALU; MFMA longest first, VALU in stream order
    std::vector<int> order(protos.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        const int la = proto_launch(size_t(a)), lb = proto_launch(size_t(b));
        if (la != lb) return la < lb;
        const bool ma = protos[size_t(a)].it.kind == KVATTN_VARIANT_MFMA, mb = protos[size_t(b)].it.kind == KVATTN_VARIANT_MFMA;
        if (ma != mb) return ma;
        return ma && protos[size_t(a)].cost > protos[size_t(b)].cost;
    });

    // ---- destinations and merge map ----------------------------------------------------
    std::vector<int> count(B, 0);
    for (const Proto& p : protos)
        for (const Entry& e : p.entries) count[e.query]++;
    P.items.clear();
    P.entries.clear();
    P.block_ids.clear();
    // A query's partials take consecutive slot blocks (partial k of query b at
    // base_b + k Hq), so the merge finds them from (base, count) alone.
    std::vector<std::vector<int32_t>> dests(B);
    std::vector<int32_t> slot_base(B, -1);
    std::vector<int> item_proto;
    int32_t slots_used = 0;
    // rows with one partial write out directly, unless the new token joins them in the merge
    const int min_merged = o.new_token ? 1 : 2;
    int64_t slots_wide = 0;
    for (int b = 0; b < B; ++b)
        if (count[b] >= min_merged) slots_wide += int64_t(count[b]) * Hq;
    if (slots_wide > std::numeric_limits<int32_t>::max())
        return set_error(KVATTN_EUNSUPPORTED, "more than 2^31 - 1 partial slots: split the batch");
    for (int b = 0; b < B; ++b)
        if (count[b] >= min_merged) {
            slot_base[b] = slots_used;
            slots_used += count[b] * Hq;
        }
    for (int idx : order) {
        Proto& p = protos[size_t(idx)];
        p.it.q_begin = int32_t(P.entries.size());
        p.it.blk_begin = int32_t(P.block_ids.size());
        for (Entry e : p.entries) {
            if (count[e.query] >= min_merged) {
                e.dest = slot_base[e.query] + int32_t(dests[e.query].size()) * Hq;
                dests[e.query].push_back(e.dest);
            }
            P.entries.push_back(e);
        }
        P.block_ids.insert(P.block_ids.end(), p.blocks.begin(), p.blocks.end());
        P.items.push_back(p.it);
        item_proto.push_back(idx);
    }
    P.n_slots = slots_used;
    P.merge_query.clear();
    P.merge_dest.clear();
    P.merge_ptr.assign(1, 0);
    P.merge_rec.clear();
    P.rec_of_query.assign(size_t(B), -1);
    int direct_rows = 0;
    for (int b = 0; b < B; ++b) {
        if (count[b] < min_merged && !o.new_token) {
            direct_rows += Hq;
            continue;
        }
        P.merge_rec.insert(P.merge_rec.end(), {b, std::max(slot_base[b], 0), count[b], o.new_token ? new_slot[size_t(b)] : 0});
        P.rec_of_query[size_t(b)] = int32_t(P.merge_query.size());
        P.merge_query.push_back(b);
        P.merge_dest.insert(P.merge_dest.end(), dests[b].begin(), dests[b].end());
        P.merge_ptr.push_back(int32_t(P.merge_dest.size()));
    }

    // ---- fused merge: the forward's last task of each (query, KV head) merges ----------------
    // Not with a new token (its merge also scores the token and writes the cache)
    // or with concurrent multi-stream launches; the kernels address the partials
    // with 32-bit byte offsets.
    {
        bool split_items = false;   // VALU_SPLIT tasks count no arrivals
        for (const Item& it : P.items) split_items |= it.kind == KVATTN_VARIANT_VALU_SPLIT;
        const bool eligible = !o.new_token && !o.multi_stream && !P.merge_query.empty() && !split_items &&
                              uint64_t(slots_used) * uint64_t(D) * 4 < (uint64_t(1) << 32);
        // measured on MI355X: merging in the forward is slower on every workload here
        // (the last arrivers' merges lengthen the tail by more than a merge launch
        // costs), so AUTO keeps the merge launch
        P.fused_merge = eligible && o.fused_merge == 1;
    }

    // ---- tasks: one static list per persistent workgroup -------------------------------------------
    // A list runs its MFMA tasks (longest first), then its VALU tasks as
    // continuous per-wave streams (in stream order), whose descriptors must fit
    // the LDS window.
    P.tasks.clear();
    // Multi-stream plans split every launch into an MFMA-only launch (side
    // stream) and a VALU-only launch, each with its own list set.
    const int sets_per_launch = o.multi_stream ? 2 : 1;
    P.list_ptr.assign(size_t(n_launch) * sets_per_launch * (n_lists + 1), 0);
    P.forward_launches.clear();
    P.n_lists = n_lists;
    for (int L = 0; L < n_launch; ++L) {
        const int launch_valu_rows = L < int(vt.size()) ? vt[size_t(L)] : 1;
        const int32_t window = valu_window_words(D, launch_valu_rows);
        std::vector<std::vector<Task>> mlist(static_cast<size_t>(n_lists)), vlist(static_cast<size_t>(n_lists));
        std::vector<int32_t> vwords(static_cast<size_t>(n_lists), 0);
        for (size_t i = 0; i < P.items.size(); ++i) {
            const int pi = item_proto[i];
            if (proto_launch(size_t(pi)) != L) continue;
            const Piece& pc = *proto_piece[size_t(pi)];
            const Item& it = P.items[i];
            if (it.kind == KVATTN_VARIANT_MFMA) {
                for (int h = 0; h < Hkv; ++h) mlist[size_t(pc.head_list[size_t(h)])].push_back({int32_t(i), h});
            } else {
                // VALU tile: one task per four KV heads; VALU_SPLIT: one task per KV head
                const bool split = it.kind == KVATTN_VARIANT_VALU_SPLIT;
                const int32_t words = desc_words(it.n_q, (it.n_tokens + kBlock - 1) / kBlock);
                for (int q = 0; q < (split ? Hkv : quads); ++q) {
                    int w = pc.head_list.empty() ? stripe_list(pc.stripe, split ? q / kWaves : q) : pc.head_list[size_t(q)];
                    if (vwords[size_t(w)] + words > window) {
                        // the stripe's window is full: the least-filled list with room takes it
                        int best_w = -1;
                        for (int x = 0; x < n_lists; ++x)
                            if (vwords[size_t(x)] + words <= window && (best_w < 0 || vwords[size_t(x)] < vwords[size_t(best_w)]))
                                best_w = x;
                        if (best_w < 0) return set_error(KVATTN_EINVAL, "internal: VALU task descriptors exceed the LDS windows");
                        w = best_w;
                    }
                    vlist[size_t(w)].push_back({int32_t(i), split ? q : q * kWaves});
                    vwords[size_t(w)] += words;
                }
            }
        }
        for (int part = 0; part < sets_per_launch; ++part) {
            // part 0 of a multi-stream plan holds the MFMA tasks, part 1 the VALU tasks
            const bool take_m = !o.multi_stream || part == 0, take_v = !o.multi_stream || part == 1;
            size_t n_part = 0;
            for (int w = 0; w < n_lists; ++w)
                n_part += (take_m ? mlist[size_t(w)].size() : 0) + (take_v ? vlist[size_t(w)].size() : 0);
            if (o.multi_stream && n_part == 0) continue;   // an empty part is not launched
            const int set = int(P.forward_launches.size());   // list sets stay contiguous
            const int base = int(P.tasks.size());
            for (int w = 0; w < n_lists; ++w) {
                P.list_ptr[size_t(set) * (n_lists + 1) + w] = int32_t(P.tasks.size()) - base;
                if (take_m)
                    for (const Task& t : mlist[size_t(w)]) P.tasks.push_back(t);
                if (take_v)
                    for (const Task& t : vlist[size_t(w)]) P.tasks.push_back(t);
            }
            P.list_ptr[size_t(set) * (n_lists + 1) + n_lists] = int32_t(P.tasks.size()) - base;
            Launch Lr;
            // a kind without tasks in this launch takes the smallest instantiation
            Lr.valu_rows = launch_valu_rows;
            Lr.mfma_tiles = L < int(mt.size()) ? mt[size_t(L)] : 1;
            Lr.index = set;
            Lr.n_tasks = int(P.tasks.size()) - base;
            Lr.task_base = base;
            Lr.side = o.multi_stream && part == 0 ? 1 : 0;
            P.forward_launches.push_back(Lr);
        }
    }
    if (!serialize_lists(P)) return set_error(KVATTN_EINVAL, "internal: VALU task descriptors exceed the LDS window");

    // ---- blob ------------------------------------------------------------------------------------
    P.n_slots = slots_used;
    serialize_blob(P);
    const BlobHeader& h = P.header;

    // ---- statistics ------------------------------------------------------------------------------
    kvattn_stats& st = P.stats;
    std::memset(&st, 0, sizeof(st));
    {
        int64_t qc = 0;
        for (int b = 0; b < B; ++b) qc += seq_lens[b];
        const std::vector<int32_t> maxv = o.new_token ? P.reads : block_reads(s, block_tables, seq_lens);
        int64_t uniq = 0;
        for (int32_t v : maxv) uniq += v;
        st.unique_kv_bytes = uniq * bpt;
        st.query_centric_kv_bytes = qc * bpt;
    }
    int64_t planned = 0;
    for (const Item& it : P.items) {
        planned += it.n_tokens;
        if (it.kind == KVATTN_VARIANT_MFMA)
            st.num_items_mfma++;
        else
            st.num_items_valu++;
        if (it.kind == KVATTN_VARIANT_VALU_SPLIT) st.num_items_valu_split++;
    }
    st.planned_kv_bytes = planned * bpt;
    st.partial_bytes = int64_t(slots_used) * partial_row_bytes * 2;
    st.num_nodes = int32_t(nodes.size());
    st.num_packed_nodes = packed_nodes;
    st.num_items = int32_t(P.items.size());
    st.num_folded_leaves = folded;
    st.num_partial_slots = slots_used;
    st.num_merge_rows = int32_t(P.merge_query.size()) * Hq;
    st.num_direct_rows = direct_rows;
    st.num_launches = int32_t(P.forward_launches.size() + (P.merge_query.empty() || P.fused_merge ? 0 : 1));
    st.split_tokens = int32_t(C);
    st.one_launch = one_launch ? 1 : 0;
    st.blob_bytes = h.blob_bytes;
    st.workspace_bytes = h.total_bytes;
    st.plan_seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();

    // ---- state for incremental updates --------------------------------------------------------
    P.tables.assign(block_tables, block_tables + size_t(B) * s.max_blocks_per_seq);
    P.lens.assign(seq_lens, seq_lens + B);
    P.entry_item.assign(P.entries.size(), 0);
    P.tail_entry.assign(size_t(B), -1);
    for (size_t i = 0; i < P.items.size(); ++i) {
        const Item& it = P.items[i];
        for (int e = it.q_begin; e < it.q_begin + it.n_q; ++e) {
            P.entry_item[size_t(e)] = int32_t(i);
            const Entry& en = P.entries[size_t(e)];
            if (int64_t(it.pos_begin) * kBlock + en.limit == seq_lens[en.query]) P.tail_entry[size_t(en.query)] = e;
        }
    }
    return KVATTN_OK;
}

// Extend the plan in place to longer sequences (PAT review, overhead analysis,
// Fig 16: the pack scheduler's cost must stay negligible next to decoding).
// A decode step appends tokens to each query; when every query's old blocks are
// unchanged and its new tokens extend the item that holds its last token --
// its own private item, or a shared item all of whose end queries grow alike
// into the same new blocks -- only those items, their entries' limits and
// their descriptors change: no tree, pack, split or list work.  Returns 1 when
// the descriptors were patched in place, 2 when their sizes changed and the
// lists were re-serialized, 0 (plan unchanged) when the step does not fit, -1
// (plan unchanged) when a new block id is out of range, -2 (plan unchanged, err
// set) when a new-token plan's new token would land in a slot that is not its
// query's alone.  Lengths are checked by the caller (for new-token plans they
// are the cached parts); old blocks are compared with the plan's, new ones
// range-checked.  New-token plans also move every merge record's new-token
// slot, in the host copy and in the blob.
int extend_plan(kvattn_plan_s& P, const int32_t* block_tables, const int32_t* seq_lens, kvattn_status& err) {
    const kvattn_shape& s = P.shape;
    const int B = s.num_queries, MB = s.max_blocks_per_seq;
    if (P.lens.size() != size_t(B) || P.tail_entry.size() != size_t(B)) return 0;
    // the blocks the old lengths cover are unchanged
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < P.lens[size_t(b)]) return 0;
        const int nb = (P.lens[size_t(b)] + kBlock - 1) / kBlock;
        const int32_t* a = block_tables + size_t(b) * MB;
        const int32_t* o = P.tables.data() + size_t(b) * MB;
        if (std::memcmp(a, o, size_t(nb) * 4) != 0) return 0;
        for (int j = nb; j < (seq_lens[b] + kBlock - 1) / kBlock; ++j)
            if (a[j] < 0 || a[j] >= s.num_physical_blocks) return -1;
    }
    // growth per item: the entries that grow are exactly those ending with the item
    struct Grow {
        int item, delta, growing, query;
    };
    std::vector<Grow> grow;
    std::vector<int> slot(P.items.size(), -1);
    for (int b = 0; b < B; ++b) {
        const int d = seq_lens[b] - P.lens[size_t(b)];
        if (d == 0) continue;
        const int e = P.tail_entry[size_t(b)];
        if (e < 0) return 0;
        const int i = P.entry_item[size_t(e)];
        const Item& it = P.items[size_t(i)];
        if (P.entries[size_t(e)].limit != it.n_tokens) return 0;
        if (slot[size_t(i)] < 0) {
            slot[size_t(i)] = int(grow.size());
            grow.push_back({i, d, 0, b});
        }
        Grow& g = grow[size_t(slot[size_t(i)])];
        if (g.delta != d) return 0;
        g.growing++;
    }
    // (new-token plans go on: the new tokens' slots move even when nothing grows)
    if (grow.empty() && !P.opts.new_token) return 1;
    int64_t uniq_add = 0, qc_add = 0;
    for (int b = 0; b < B; ++b) qc_add += seq_lens[b] - P.lens[size_t(b)];
    bool resize = false;
    std::vector<std::vector<int32_t>> new_ids(grow.size());
    for (size_t k = 0; k < grow.size(); ++k) {
        const Grow& g = grow[k];
        const Item& it = P.items[size_t(g.item)];
        int at_end = 0;
        for (int e = it.q_begin; e < it.q_begin + it.n_q; ++e) at_end += P.entries[size_t(e)].limit == it.n_tokens;
        if (at_end != g.growing) return 0;
        const int nt = it.n_tokens + g.delta;
        const int nb0 = (it.n_tokens + kBlock - 1) / kBlock, nb1 = (nt + kBlock - 1) / kBlock;
        if (nb1 > (it.kind == KVATTN_VARIANT_MFMA ? kMfmaMaxItemBlocks : kMaxItemBlocks)) return 0;
        if (it.pos_begin + nb1 > MB) return 0;
        // the new blocks, alike for every growing query
        for (int j = nb0; j < nb1; ++j) new_ids[k].push_back(block_tables[size_t(g.query) * MB + it.pos_begin + j]);
        for (int e = it.q_begin; e < it.q_begin + it.n_q; ++e) {
            const int q = P.entries[size_t(e)].query;
            if (P.entries[size_t(e)].limit != it.n_tokens || q == g.query) continue;
            for (int j = nb0; j < nb1; ++j)
                if (block_tables[size_t(q) * MB + it.pos_begin + j] != new_ids[k][size_t(j - nb0)]) return 0;
        }
        resize |= desc_words(it.n_q, nb1) != desc_words(it.n_q, nb0);
    }
    // unique tokens: the valid-token count each touched physical block gains
    std::vector<std::pair<int32_t, int>> touched;   // (block id, valid tokens after the step), sorted
    {
        for (int b = 0; b < B; ++b) {
            const int T0 = P.lens[size_t(b)], T1 = seq_lens[b];
            if (T1 == T0) continue;
            for (int j = (T0 - 1) / kBlock; j < (T1 + kBlock - 1) / kBlock; ++j)
                touched.emplace_back(block_tables[size_t(b) * MB + j], std::min(kBlock, T1 - j * kBlock));
        }
        std::sort(touched.begin(), touched.end());
        for (size_t x = 0; x < touched.size(); ++x) {
            if (x + 1 < touched.size() && touched[x + 1].first == touched[x].first) continue;   // keep the largest
            const int32_t id = touched[x].first;
            // tokens the block held before: the largest old valid count among the queries that hold it
            int before = 0;
            for (int b = 0; b < B; ++b) {
                const int T0 = P.lens[size_t(b)];
                const int j = (T0 - 1) / kBlock;
                if (P.tables[size_t(b) * MB + j] == id) before = std::max(before, T0 - j * kBlock);
            }
            uniq_add += touched[x].second - before;
        }
    }
    // new-token plans: the new tokens' slots, checked against the reads after the step
    std::vector<int32_t> new_slot;
    if (P.opts.new_token) {
        auto reads_of = [&](int32_t id) {
            int32_t r = P.reads[size_t(id)];
            auto it = std::upper_bound(touched.begin(), touched.end(), std::make_pair(id, std::numeric_limits<int>::max()));
            if (it != touched.begin() && std::prev(it)->first == id) r = std::max(r, int32_t(std::prev(it)->second));
            return r;
        };
        err = check_new_slots(s, block_tables, seq_lens, reads_of, new_slot);
        if (err != KVATTN_OK) return -2;
    }
    // apply: items, entries, block ids
    std::vector<int32_t> old_ids;
    std::vector<Item> old_items;
    std::vector<Entry> old_entries;
    if (resize) {
        old_ids = P.block_ids;
        old_items = P.items;
        old_entries = P.entries;
    }
    bool new_blocks = false;
    for (size_t k = 0; k < grow.size(); ++k) {
        Item& it = P.items[size_t(grow[k].item)];
        for (int e = it.q_begin; e < it.q_begin + it.n_q; ++e)
            if (P.entries[size_t(e)].limit == it.n_tokens) P.entries[size_t(e)].limit += grow[k].delta;
        it.n_tokens += grow[k].delta;
        new_blocks |= !new_ids[k].empty();
    }
    if (new_blocks) {
        std::vector<int32_t> ids;
        ids.reserve(P.block_ids.size() + 64);
        for (size_t i = 0; i < P.items.size(); ++i) {
            Item& it = P.items[i];
            const int nb = (it.n_tokens + kBlock - 1) / kBlock;
            const int32_t begin = int32_t(ids.size());
            const int have = slot[i] >= 0 ? nb - int(new_ids[size_t(slot[i])].size()) : nb;
            ids.insert(ids.end(), P.block_ids.begin() + it.blk_begin, P.block_ids.begin() + it.blk_begin + have);
            if (slot[i] >= 0) ids.insert(ids.end(), new_ids[size_t(slot[i])].begin(), new_ids[size_t(slot[i])].end());
            it.blk_begin = begin;
        }
        P.block_ids.swap(ids);
    }
    // descriptors
    int path = 1;
    if (!resize) {
        // same record sizes: rewrite the header words, the limits and the new
        // block ids of the grown items' records, here and in the blob
        int32_t* blob_desc = reinterpret_cast<int32_t*>(P.blob.data() + P.header.off_desc);
        for (size_t t = 0; t < P.tasks.size(); ++t) {
            const int i = P.tasks[t].item;
            if (slot[size_t(i)] < 0) continue;
            const Item& it = P.items[size_t(i)];
            const std::vector<int32_t>& add = new_ids[size_t(slot[size_t(i)])];
            const int nb = (it.n_tokens + kBlock - 1) / kBlock;
            const size_t off = size_t(P.task_desc[t]);
            int32_t* d = P.desc.data() + off;
            int32_t* bd = blob_desc + off;
            int32_t lim_all = it.n_tokens;
            for (int e = 0; e < it.n_q; ++e) {
                const int32_t lim = P.entries[size_t(it.q_begin + e)].limit;
                d[kDescHeader + 4 * e + 2] = bd[kDescHeader + 4 * e + 2] = lim;
                lim_all = std::min(lim_all, lim);
            }
            d[kDescTokens] = bd[kDescTokens] = it.n_tokens;
            d[kDescBlocks] = bd[kDescBlocks] = nb;
            d[kDescLimAll] = bd[kDescLimAll] = lim_all;
            const int nb0 = nb - int(add.size());
            for (size_t j = 0; j < add.size(); ++j)
                d[kDescHeader + 4 * it.n_q + nb0 + int(j)] = bd[kDescHeader + 4 * it.n_q + nb0 + int(j)] = add[j];
        }
    } else {
        if (!serialize_lists(P)) {
            // a VALU window overflows: leave the plan as it was
            P.block_ids.swap(old_ids);
            P.items.swap(old_items);
            P.entries.swap(old_entries);
            if (!serialize_lists(P)) return 0;
            serialize_blob(P);
            return 0;
        }
        serialize_blob(P);
        path = 2;
    }
    // state and statistics (the old blocks are unchanged: copy the new ones)
    for (int b = 0; b < B; ++b) {
        const int T0 = P.lens[size_t(b)], T1 = seq_lens[b];
        if (T1 == T0) continue;
        const size_t row = size_t(b) * MB;
        std::copy(block_tables + row + (T0 - 1) / kBlock, block_tables + row + (T1 + kBlock - 1) / kBlock,
                  P.tables.begin() + std::ptrdiff_t(row + (T0 - 1) / kBlock));
        P.lens[size_t(b)] = T1;
    }
    if (P.opts.new_token) {
        for (const auto& t : touched) P.reads[size_t(t.first)] = std::max(P.reads[size_t(t.first)], int32_t(t.second));
        int32_t* blob_rec = reinterpret_cast<int32_t*>(P.blob.data() + P.header.off_merge_rec);
        for (size_t r = 0; r < P.merge_rec.size() / 4; ++r)
            P.merge_rec[4 * r + 3] = blob_rec[4 * r + 3] = new_slot[size_t(P.merge_rec[4 * r])];
    }
    const int64_t bpt = int64_t(2) * s.num_kv_heads * s.head_dim * 2;
    P.stats.unique_kv_bytes += uniq_add * bpt;
    P.stats.query_centric_kv_bytes += qc_add * bpt;
    int64_t planned = 0;
    for (const Item& it : P.items) planned += it.n_tokens;
    P.stats.planned_kv_bytes = planned * bpt;
    P.stats.blob_bytes = P.header.blob_bytes;
    P.stats.workspace_bytes = P.header.total_bytes;
    return path;
}

}  // namespace kvattn

// ============================================================================
// C ABI: host-only entry points
// ============================================================================
extern "C" {

void kvattn_plan_options_default(kvattn_plan_options* o) {
    if (!o) return;
    o->scale = 0.f;
    o->pack_mode = KVATTN_PACK_AUTO;
    o->scheme = 0;
    o->force_variant = KVATTN_VARIANT_AUTO;
    o->split_tokens = 0;
    o->num_cus = 0;
    o->new_token = 0;
    o->multi_stream = 0;
    o->fused_merge = -1;
}

kvattn_status kvattn_plan(const kvattn_shape* shape, const int32_t* block_tables, const int32_t* seq_lens,
                          const kvattn_prefix_tree* tree, const kvattn_plan_options* opts, kvattn_plan_t* out) {
    using namespace kvattn;
    clear_error();
    if (!out) return set_error(KVATTN_EINVAL, "out is NULL");
    *out = nullptr;
    if (!shape || !block_tables || !seq_lens) return set_error(KVATTN_EINVAL, "shape, block_tables or seq_lens is NULL");
    const kvattn_shape& s = *shape;
    if (s.num_queries < 1 || s.num_q_heads < 1 || s.num_kv_heads < 1 || s.head_dim < 1 || s.max_blocks_per_seq < 1 ||
        s.num_physical_blocks < 1)
        return set_error(KVATTN_EINVAL, "shape fields must be >= 1");
    if (s.num_q_heads % s.num_kv_heads != 0) return set_error(KVATTN_EINVAL, "num_q_heads % num_kv_heads != 0");
    if (s.block_size != kBlock) return set_error(KVATTN_EUNSUPPORTED, "block_size must be 16");
    if (s.head_dim != 64 && s.head_dim != 128) return set_error(KVATTN_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (s.num_q_heads / s.num_kv_heads > kMaxGroup)
        return set_error(KVATTN_EUNSUPPORTED, "more than 64 q heads per KV head");
    // the kernels index q (and out) rows with 32-bit element offsets
    if (int64_t(s.num_queries) * s.num_q_heads * s.head_dim >= (int64_t(1) << 31))
        return set_error(KVATTN_EUNSUPPORTED, "num_queries * num_q_heads * head_dim must stay below 2^31");
    kvattn_plan_options o;
    kvattn_plan_options_default(&o);
    if (opts) o = *opts;
    if (o.pack_mode < 0 || o.pack_mode > 2 || o.scheme < 0 || o.scheme > 2 || o.force_variant < -1 ||
        o.force_variant > 2 || o.split_tokens < 0 || o.num_cus < 0 || !(o.scale >= 0.f) || std::isinf(o.scale) ||
        o.new_token < 0 || o.new_token > 1 || o.multi_stream < 0 || o.multi_stream > 1 || o.fused_merge < -1 ||
        o.fused_merge > 1)
        return set_error(KVATTN_EINVAL, "bad option value");
    kvattn_plan_s* P = new (std::nothrow) kvattn_plan_s();
    if (!P) return set_error(KVATTN_ENOMEM, "plan allocation failed");
    P->shape = s;
    P->opts = o;
    P->scale = o.scale > 0.f ? o.scale : float(1.0 / std::sqrt(double(s.head_dim)));
    kvattn_status st;
    try {
        st = build_plan(s, block_tables, seq_lens, tree, o, *P);
    } catch (const std::bad_alloc&) {
        st = set_error(KVATTN_ENOMEM, "host allocation failed while planning");
    }
    if (st != KVATTN_OK) {
        delete P;
        return st;
    }
    P->generation = next_generation();
    if (std::getenv("KVATTN_LOG")) {
        const kvattn_stats& x = P->stats;
        std::fprintf(stderr,
                     "kvattn_plan: nodes %d packed %d folded %d items %d (valu %d mfma %d) split %d slots %d "
                     "merge_rows %d unique %.3f MB planned %.3f MB partial %.3f MB plan %.3f ms\n",
                     x.num_nodes, x.num_packed_nodes, x.num_folded_leaves, x.num_items, x.num_items_valu,
                     x.num_items_mfma, x.split_tokens, x.num_partial_slots, x.num_merge_rows,
                     x.unique_kv_bytes / 1e6, x.planned_kv_bytes / 1e6, x.partial_bytes / 1e6, x.plan_seconds * 1e3);
    }
    *out = P;
    return KVATTN_OK;
}

kvattn_status kvattn_plan_update(kvattn_plan_t plan, const int32_t* block_tables, const int32_t* seq_lens) {
    using namespace kvattn;
    clear_error();
    if (!plan || !block_tables || !seq_lens) return set_error(KVATTN_EINVAL, "plan, block_tables or seq_lens is NULL");
    // an upload still in flight reads the blob this call changes or frees
    if (plan->upload_event && plan->upload_wait) plan->upload_wait(plan->upload_event);
    const auto t0 = std::chrono::steady_clock::now();
    const kvattn_shape& s = plan->shape;
    for (int b = 0; b < s.num_queries; ++b)
        if (seq_lens[b] < 1 || int64_t(seq_lens[b]) > int64_t(s.max_blocks_per_seq) * kBlock)
            return set_error(KVATTN_EINVAL, "seq_lens[" + std::to_string(b) + "] = " + std::to_string(seq_lens[b]) +
                                                " outside [1, max_blocks_per_seq * 16]");
    // new-token plans extend over the cached parts; their new tokens' blocks are range-checked here
    const int32_t* lens = seq_lens;
    std::vector<int32_t> cached;
    if (plan->opts.new_token) {
        cached.resize(size_t(s.num_queries));
        for (int b = 0; b < s.num_queries; ++b) {
            cached[size_t(b)] = seq_lens[b] - 1;
            const int32_t id = block_tables[size_t(b) * s.max_blocks_per_seq + cached[size_t(b)] / kBlock];
            if (id < 0 || id >= s.num_physical_blocks) return check_tables(s, block_tables, seq_lens);
        }
        lens = cached.data();
    }
    int path = 0;
    try {
        kvattn_status err = KVATTN_OK;
        path = extend_plan(*plan, block_tables, lens, err);
        if (path == -2) return err;                                       // new-token slot conflict
        if (path < 0) return check_tables(s, block_tables, seq_lens);   // names the bad block id
        if (path == 0) {
            // the step does not extend the plan's items: plan from scratch
            kvattn_plan_t fresh = nullptr;
            const kvattn_status st = kvattn_plan(&s, block_tables, seq_lens, nullptr, &plan->opts, &fresh);
            if (st != KVATTN_OK) return st;
            // the plan keeps its events (owned by the runtime) across the rebuild
            void* fork_event = plan->fork_event;
            void* join_event = plan->join_event;
            void* upload_event = plan->upload_event;
            void (*upload_wait)(void*) = plan->upload_wait;
            *plan = std::move(*fresh);
            plan->fork_event = fork_event;
            plan->join_event = join_event;
            plan->upload_event = upload_event;
            plan->upload_wait = upload_wait;
            delete fresh;
            path = 3;
        }
    } catch (const std::bad_alloc&) {
        return set_error(KVATTN_ENOMEM, "host allocation failed while updating the plan");
    }
    // the device copy of the schedule is stale until the next upload
    plan->dev_ws = nullptr;
    plan->dev_bytes = 0;
    plan->generation = next_generation();
    plan->stats.update_path = path;
    plan->stats.plan_seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    return KVATTN_OK;
}

kvattn_status kvattn_expand_query_tokens(const kvattn_shape* shape, const int32_t* block_tables,
                                         const int32_t* seq_lens, const int32_t* q_lens,
                                         int32_t* out_block_tables, int32_t* out_seq_lens) {
    using namespace kvattn;
    clear_error();
    if (!shape || !block_tables || !seq_lens || !q_lens || !out_block_tables || !out_seq_lens)
        return set_error(KVATTN_EINVAL, "NULL argument");
    const int B = shape->num_queries, MB = shape->max_blocks_per_seq;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 1 || int64_t(seq_lens[b]) > int64_t(MB) * kBlock)
            return set_error(KVATTN_EINVAL, "seq_lens[" + std::to_string(b) + "] outside [1, max_blocks_per_seq * 16]");
        if (q_lens[b] < 1 || q_lens[b] > seq_lens[b])
            return set_error(KVATTN_EINVAL, "q_lens[" + std::to_string(b) + "] outside [1, seq_lens[b]]");
    }
    size_t row = 0;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < q_lens[b]; ++i, ++row) {
            const int T = seq_lens[b] - q_lens[b] + i + 1;
            const int nb = (T + kBlock - 1) / kBlock;
            int32_t* dst = out_block_tables + row * size_t(MB);
            std::copy(block_tables + size_t(b) * MB, block_tables + size_t(b) * MB + nb, dst);
            std::fill(dst + nb, dst + MB, -1);
            out_seq_lens[row] = T;
        }
    }
    return KVATTN_OK;
}

kvattn_status kvattn_plan_device_bytes(kvattn_plan_t plan, size_t* bytes) {
    using namespace kvattn;
    clear_error();
    if (!plan || !bytes) return set_error(KVATTN_EINVAL, "plan or bytes is NULL");
    *bytes = size_t(plan->header.total_bytes);
    return KVATTN_OK;
}

kvattn_status kvattn_plan_stats(kvattn_plan_t plan, kvattn_stats* stats) {
    using namespace kvattn;
    clear_error();
    if (!plan || !stats) return set_error(KVATTN_EINVAL, "plan or stats is NULL");
    *stats = plan->stats;
    return KVATTN_OK;
}

kvattn_status kvattn_plan_export(kvattn_plan_t plan, kvattn_export* out) {
    using namespace kvattn;
    clear_error();
    if (!plan || !out) return set_error(KVATTN_EINVAL, "plan or out is NULL");
    out->num_items = int32_t(plan->items.size());
    out->items = reinterpret_cast<const kvattn_item_info*>(plan->items.data());
    out->num_entries = int32_t(plan->entries.size());
    out->entries = reinterpret_cast<const kvattn_item_query*>(plan->entries.data());
    out->num_block_ids = int32_t(plan->block_ids.size());
    out->block_ids = plan->block_ids.data();
    out->num_merge_queries = int32_t(plan->merge_query.size());
    out->merge_query = plan->merge_query.data();
    out->merge_ptr = plan->merge_ptr.data();
    out->merge_dest = plan->merge_dest.data();
    out->num_partial_slots = plan->n_slots;
    out->head_dim = plan->shape.head_dim;
    out->num_tasks = int32_t(plan->tasks.size());
    out->tasks = reinterpret_cast<const int32_t*>(plan->tasks.data());
    out->num_launches = int32_t(plan->forward_launches.size());
    out->num_lists = plan->n_lists;
    out->num_desc_words = int32_t(plan->desc.size());
    out->desc = plan->desc.data();
    out->list_ptr = plan->desc_list_ptr.data();
    out->merge_rec = plan->merge_rec.data();
    return KVATTN_OK;
}


const char* kvattn_status_string(kvattn_status s) {
    switch (s) {
        case KVATTN_OK: return "KVATTN_OK";
        case KVATTN_EINVAL: return "KVATTN_EINVAL";
        case KVATTN_EUNSUPPORTED: return "KVATTN_EUNSUPPORTED";
        case KVATTN_ENOMEM: return "KVATTN_ENOMEM";
        case KVATTN_EWORKSPACE: return "KVATTN_EWORKSPACE";
        case KVATTN_EHIP: return "KVATTN_EHIP";
        case KVATTN_ESTATE: return "KVATTN_ESTATE";
    }
    return "KVATTN_UNKNOWN";
}

const char* kvattn_last_error(void) { return kvattn::g_last_error.c_str(); }

}  // extern "C"
