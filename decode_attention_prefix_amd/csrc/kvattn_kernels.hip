// gfx950 (MI355X) kernels of the forward and merge stages.
//
// Forward (PAT review, forward stage: multi-tile kernels picked per work item,
// long KV split into chunks, no execution bubbles): one persistent launch;
// workgroup w runs task list w the planner built for it (and claims lists
// past the grid at run time).  A task is
// one item (a run of paged KV blocks and the query rows attending to it) on
// one KV head (MFMA path) or four KV heads (VALU path); it yields either final
// output rows or partial triples (m, l, acc), m in log2 units.
//   * MFMA path -- packed groups (up to 128 rows per KV head): S^T = K Q^T and
//                  O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, K/V tiles staged
//                  in LDS by buffer->LDS DMA, three tiles in flight, V^T read
//                  by transposing LDS reads.
//   * VALU path -- at most 4 (D = 128) or 8 (D = 64) rows per KV head: a
//                  query's GQA group or a few queries of a small pack.
//                  Bandwidth bound: q K^T with v_dot2_f32_bf16, p V with fp32
//                  FMAs, 16-byte coalesced loads into a register ring that
//                  runs across the list's tasks, 8-lane DPP reductions.
// Merge (PAT review, merge stage: online-softmax combination of the per-
// workgroup partial results of a query): one wave per 256 output floats of a
// query, single pass over its partials (consecutive slot blocks).  Its
// fused-append form also scores each query's new token and writes the token's
// K/V into its paged slot (short-term-memory page: the decode step appends
// K_t, V_t, then attends).
// A measurement helper, a plain streaming read of two buffers, sits before
// the launchers; it is not part of the attention path.
//
// Scores are kept in log2 units (q.k * scale * log2 e) so every exponential is
// a single v_exp_f32.  The running max is refreshed lazily: a row is rescaled
// only when a new score exceeds the reference by more than kRescaleLog2, so
// exponentials stay below 2^kRescaleLog2 and the result is unchanged.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kvattn_internal.h"

namespace kvattn {

// Per-task trace (a diagnostic build only: compiled with -DKVATTN_TASK_TRACE,
// see build.py; the library itself has none of it).  Each workgroup slot of the
// forward launch owns kTraceEvents records of 4 words in a caller buffer set
// with kvattn_trace_set: (type | XCC id << 8, s_memrealtime low word (100 MHz),
// HW_ID register, extra).  Types: 0 list start (extra: list), 1 MFMA task start
// (tokens | rows << 20), 2 MFMA task end, 3 VALU window ready (words), 4 a
// wave's VALU stream end (at record 40 + wave; extra: its blocks), 5 VALU end.
// Records past kTraceEvents are dropped; each launch overwrites its slots.
#ifdef KVATTN_TASK_TRACE
__device__ uint32_t* g_trace;
#endif

namespace {
#ifdef KVATTN_TASK_TRACE
constexpr int kTraceEvents = 64;
__device__ __forceinline__ void trace_ev(int slot_wg, int idx, uint32_t type, uint32_t extra) {
    if (!g_trace || idx >= kTraceEvents) return;
    uint32_t* e = g_trace + (size_t(slot_wg) * kTraceEvents + idx) * 4;
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
    *reinterpret_cast<uint4*>(e) = make_uint4(type | (xcc << 8), uint32_t(t), hw, extra);
}
#define KV_TRACE(...) trace_ev(__VA_ARGS__)
#define KV_TRACE_ON 1
#else
#define KV_TRACE(...) ((void)0)
#define KV_TRACE_ON 0
#endif

constexpr float kRescaleLog2 = 8.0f;
// VALU load ring depth in 16-token blocks.  Two (one block in flight while
// one is processed) already saturates HBM with 2048 streaming waves; deeper
// rings only lengthen the request queues (measured on MI355X: depth 2 beat 3
// and 4 on every workload).
constexpr int kValuRing = 2;
constexpr float kNegSentinel = -1.0e30f;   // "no score yet"; finite so m - m stays 0

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): reads past the resource's size return zero.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 8 consecutive lanes of an aligned octet: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], then row_half_mirror (lane i <-> 7 - i).
__device__ __forceinline__ float octet_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x;
}

// Cross-lane exchanges without LDS.  lane_x8: the value of lane l ^ 8 (DPP
// row_ror:8 within each 16-lane row).  swap16 / swap32 (gfx950
// v_permlane16_swap / v_permlane32_swap) pair lane l with lane l ^ 16 (l ^ 32)
// and return, on the lane of the pair whose bit is clear, {own x, partner's
// x}, and on the lane whose bit is set, {partner's y, own y}.  So .x + .y sums
// the pair's x on the lower lane and the pair's y on the upper lane (a
// reduce-scatter step), and with x = y both lanes get {own, partner}.
__device__ __forceinline__ float lane_x8(float x) { return dpp<0x128>(x); }
__device__ __forceinline__ float2 swap16(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap32(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_max3_f32 without the NaN-quieting canonicalisations fmaxf adds for values
// the compiler cannot prove canonical (MFMA results).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group,
// lane a + 4e (a, e in [0, 4)) supplies the address of four 16-bit values; lane
// 4a + c receives value c of the lanes a, a + 4, a + 8, a + 12, in that order.
// `base` points into LDS; `off` is a byte offset.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* base, uint32_t off) {
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const lds_char* b = (const lds_char*)(base);
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + off));
    return __builtin_bit_cast(uint2, r);
}

// s_waitcnt immediate (gfx9 encoding) waiting until at most N vector-memory
// operations are outstanding; expcnt and lgkmcnt are left at their maximum.
template <int N>
constexpr int waitcnt_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 0xF) | ((N >> 4) << 14) | 0x0F70;
}

// Zero in a VGPR the compiler cannot see through.  An atomic on an address
// offset by it is not turned into a wave-aggregated atomic (whose expansion
// waits for the result at once); the result's wait lands at its first use.
__device__ __forceinline__ int opaque_zero() {
    int v;
    asm volatile("v_mov_b32 %0, 0" : "=v"(v));
    return v;
}

// Lane index, read by an instruction the compiler neither hoists nor merges.
__device__ __forceinline__ int lane_id_volatile() {
    int v;
    asm volatile(
        "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
        "v_mbcnt_hi_u32_b32 %0, -1, %0"
        : "=v"(v));
    return v;
}

// Direct global -> LDS copy of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) (lds is wave-uniform, passed in M0).  Issued from
// inline assembly so that the compiler does not guard later LDS reads with waits
// on these loads: the pipeline orders them itself (s_waitcnt vmcnt + s_barrier).
// M0 is saved and restored around the copy.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(g)
        : "memory");
}

// Buffer resource (raw, 32-bit data format) over `bytes` bytes at `base`.
// All inputs must be wave-uniform: the result lives in SGPRs.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = uint64_t(uintptr_t(base));
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(uint32_t(a));
    r.y = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xFFFFu);   // base[47:32]; stride 0, no swizzle
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = uint32_t(kBufferWord3);
    return r;
}

// Agent-scope coherent (sc1) stores and loads of partial triples.  Partials
// are stored this way whenever the arrays fit 32-bit byte offsets (p.part_wt):
// the store writes through the writer's L2, so no dirty partial lines are left
// for the write-back at the end of the launch (measured: 1.7 us less per call
// on the Llama-3-8B-shaped layer, 0.4-0.6 % less on the larger batches), and
// plans that merge inside the forward launch need exactly this, since a
// partial written on one XCD is read by the task that completes its (query,
// KV head) on any other XCD.  The loads (that merge only) are not served
// stale from the reader's L2.  `rsrc` spans a whole partial array; `off` is a
// byte offset.  Cache policy 16 is sc1 on gfx950.
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, int(bytes), kBufferWord3);
}
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float a) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, off, 0, kCpolSc1);
}
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 a) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(a.x), __float_as_uint(a.y)}, r, off, 0, kCpolSc1);
}
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 a) {
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w)}, r, off, 0,
        kCpolSc1);
}
__device__ __forceinline__ float2 load_sc1_f2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolSc1);
    return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
__device__ __forceinline__ float4 load_sc1_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Buffer -> LDS copy of 16 bytes per lane: lane i reads bytes [voff, voff + 16)
// of the resource and writes LDS bytes [lds + 16 i, lds + 16 i + 16); dwords
// past the resource's size are written as zeros.  Inline assembly for the same
// reason as dma16; M0 is saved and restored around the copy.
__device__ __forceinline__ void dma16_buf(u32x4 rsrc, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc)
        : "memory");
}

// Schedule arrays are read-only for a whole launch: reading them through the
// constant address space lets uniform reads become scalar (SMEM) loads, which
// do not count against vmcnt and so never stall the in-flight KV loads.
#define KV_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const KV_CONST T* cptr(const T* x) {
    return (const KV_CONST T*)(x);
}

// A task as the kernels see it: header fields as wave-uniform values, entries
// and block ids left in the LDS copy of the task's descriptor.
struct TaskView {
    int kind, tile, head, n_tokens, n_q, n_rows, nblk, lim_all;
    const int32_t* ent;   // LDS: n_q entries of 4 words (query, dest, limit, 0)
    const int32_t* blk;   // LDS: nblk block ids
};

__device__ __forceinline__ TaskView view_of(const int32_t* d) {
    TaskView v;
    v.kind = __builtin_amdgcn_readfirstlane(d[kDescKind]);
    v.tile = __builtin_amdgcn_readfirstlane(d[kDescTile]);
    v.head = __builtin_amdgcn_readfirstlane(d[kDescHead]);
    v.n_tokens = __builtin_amdgcn_readfirstlane(d[kDescTokens]);
    v.n_q = __builtin_amdgcn_readfirstlane(d[kDescNq]);
    v.n_rows = __builtin_amdgcn_readfirstlane(d[kDescRows]);
    v.nblk = __builtin_amdgcn_readfirstlane(d[kDescBlocks]);
    v.lim_all = __builtin_amdgcn_readfirstlane(d[kDescLimAll]);
    v.ent = d + kDescHeader;
    v.blk = d + kDescHeader + 4 * v.n_q;
    return v;
}

__device__ __forceinline__ Entry entry_of(const TaskView& v, int i) {
    const int4 e4 = *reinterpret_cast<const int4*>(v.ent + 4 * i);
    Entry e;
    e.query = e4.x;
    e.dest = e4.y;
    e.limit = e4.z;
    e.pad = 0;
    return e;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// ============================================================================
// Online-softmax combination of a (query, q head) row's partial triples (PAT
// review, merge stage), for the four consecutive head-dim values at offset e0
// of the head: partial k sits in slot slot0 + k Hq.  Updates the running
// (M, L, A) in place, partials read BATCH at a time with every load in flight
// (the batch size groups the loads only; the arithmetic is the same):
//   M' = max(M, m_k);  A = A 2^(M - M') + 2^(m_k - M') acc_k;  L likewise with l_k.
// SC1 reads with agent-scope coherent loads (the forward's own merges).  Both
// the merge launch and the forward's merges use this one function, so a row
// comes out bit for bit the same either way.
// ============================================================================
template <int D, bool SC1, int BATCH>
__device__ __forceinline__ void merge_partials(const DevPlan& p, int Hq, size_t slot0, int n, int e0, float& M,
                                               float& L, float4& A) {
    const __amdgpu_buffer_rsrc_t rml = part_rsrc(p.part_ml, p.part_ml_bytes);
    const __amdgpu_buffer_rsrc_t racc = part_rsrc(p.part_acc, p.part_acc_bytes);
    for (int ib = 0; ib < n; ib += BATCH) {
        float2 ml[BATCH];
        float4 ac[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const size_t slot = slot0 + size_t(min(ib + j, n - 1)) * Hq;
            if constexpr (SC1) {
                ml[j] = load_sc1_f2(rml, uint32_t(slot * 8));
                ac[j] = load_sc1_f4(racc, uint32_t((slot * D + e0) * 4));
            } else {
                ml[j] = *reinterpret_cast<const float2*>(p.part_ml + slot * 2);
                ac[j] = *reinterpret_cast<const float4*>(p.part_acc + slot * D + e0);
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            // past the row's last partial: no change (weight 0, same max)
            const float mj = ib + j < n ? ml[j].x : -INFINITY;
            const float Mn = fmaxf(M, mj);
            const float so = fast_exp2(M - Mn);     // 0 while M is -inf
            const float sn = fast_exp2(mj - Mn);    // 0 past the last partial
            L = L * so + sn * ml[j].y;
            A.x = fmaf(sn, ac[j].x, A.x * so);
            A.y = fmaf(sn, ac[j].y, A.y * so);
            A.z = fmaf(sn, ac[j].z, A.z * so);
            A.w = fmaf(sn, ac[j].w, A.w * so);
            M = Mn;
        }
    }
}

// One wave merges the q heads of KV head g of merge record `rec` (wave-uniform)
// into out: that query's G rows, 256 floats per pass.
template <int D>
__device__ __forceinline__ void merge_unit(const DevPlan& p, const Dims& dm, int rec, int g, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int Hq = dm.num_q_heads;
    const KV_CONST MergeRec* r = cptr(p.merge_rec) + rec;
    const int b = r->query, n = r->count;
    const size_t first = size_t(r->first);
    const int cols = dm.group * D;
    for (int c0 = 0; c0 < cols; c0 += 256) {
        const int cc = c0 + 4 * lane;
        if (cc < cols) {
            const int col = g * cols + cc;
            const int h = col / D;
            float M = -INFINITY, L = 0.f;
            float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
            merge_partials<D, true, 16>(p, Hq, first + h, n, col - h * D, M, L, A);
            const float inv = 1.f / L;
            *reinterpret_cast<float4*>(out + size_t(b) * Hq * D + col) =
                make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
        }
    }
}

// Arrival of one task's partials of KV head g for the merge record `rec` (one
// lane): returns true for the task that completes the (record, head), which
// then merges it.  Its counter goes back to zero for the next launch.  The
// caller has waited for its own sc1 partial stores (s_waitcnt vmcnt(0)).
__device__ __forceinline__ bool arrive_last(const DevPlan& p, int Hkv, int rec, int g) {
    int* c = p.arrive + size_t(rec) * Hkv + g;
    const int n = p.merge_rec[rec].count;
    const int old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old != n - 1) return false;
    __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// ============================================================================
// VALU stream: a wave runs the VALU tasks of its workgroup's list for KV head
// (task head + wave) as one continuous stream of 16-token blocks.  Its
// kValuRing-deep register ring crosses task boundaries, so blocks of the next
// task are in flight while the current one finishes and nothing drains
// between tasks.  The list's descriptors sit in an LDS window; the q rows of a
// task are copied into one of four per-wave LDS slots by DMA right before the
// loads of its first block.
// Lane = 8 * t + c: token slots t and t + 8 of each 16-token block, and the
// head-dim chunk set of c (elements [8c, 8c+8) and, for D = 128, [64+8c, 64+8c+8)),
// so every load instruction reads whole 128-byte rows of a block.
// ============================================================================
//
// SPLIT (the VALU_SPLIT tile): the wave runs the list's VALU_SPLIT tasks
// instead, all four waves on the task's one KV head, wave w on blocks
// [w nb / 4, (w + 1) nb / 4) of it.  At the end of each task the waves put
// their (m, l, acc) rows into `cbuf` (LDS) and, between two workgroup
// barriers, combine them with the online-softmax rule and store.  Every wave
// has at least one block of every such task (the planner emits the tile for 4
// or more blocks; shorter ones are skipped here by every wave alike), so all
// waves reach the same barriers.
template <int D, int R, bool SPLIT>
__device__ __forceinline__ void valu_stream(const DevPlan& p, const Dims& dm, const int32_t* win, int n_words,
                                            uint16_t* qs, float* cbuf, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                            float* __restrict__ out) {
    constexpr int NPC = D / 64;      // 16-byte pieces per token per lane
    constexpr int NE = 8 * NPC;      // elements per token per lane
    constexpr int LPB = 2 * NPC * 2; // loads per block per lane (2 token slots, NPC pieces, K and V)
    constexpr int NR = kValuRing;    // load ring depth (blocks); also the q slots per wave
    static_assert(NR >= 2 && NR <= 4, "the LDS layout holds four q slots per wave");
    constexpr int QSLOT = R * D;     // bf16 elements of one q slot
    constexpr int QCH = QSLOT / 8;   // its 16-byte chunks
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int Hkv = dm.num_kv_heads;
    const int Hq = dm.num_q_heads;
    const int G = dm.group;
    const int t = lane >> 3, c = lane & 7;
    const size_t head_elems = size_t(16) * D;
    const size_t blk_elems = size_t(Hkv) * head_elems;
    const float sl2 = dm.scale_log2;
    const uint32_t qs_lds = uint32_t(uintptr_t(qs));

    auto hdr = [&](int off, int f) { return __builtin_amdgcn_readfirstlane(win[off + f]); };
    // this wave's KV head of the task at `off`, and its blocks [lo, hi) of the task's nb
    auto head_of = [&](int off) { return hdr(off, kDescHead) + (SPLIT ? 0 : wave); };
    auto range_lo = [&](int nb) { return SPLIT ? (wave * nb) / kWaves : 0; };
    auto range_hi = [&](int nb) { return SPLIT ? ((wave + 1) * nb) / kWaves : nb; };
    // first task at or after `off` that this wave runs: VALU_SPLIT tasks of 4 or
    // more blocks (SPLIT), else VALU tasks that have a KV head for this wave
    auto skip = [&](int off) {
        while (off < n_words) {
            const bool split = hdr(off, kDescKind) == KVATTN_VARIANT_VALU_SPLIT;
            if (SPLIT ? split && hdr(off, kDescBlocks) >= kWaves : !split && hdr(off, kDescHead) + wave < Hkv) break;
            off += hdr(off, kDescWords);
        }
        return off;
    };
    // copy the q rows of the task at `off` into slot `s` of this wave
    auto fetch_q = [&](int off, int s) {
        const int nrows = hdr(off, kDescRows);
        const int g = head_of(off);
        // The lane index is re-read here so that the per-lane terms below are
        // not hoisted out of the stream loop as live registers: spilled, their
        // reload would wait for every load in flight.
        const int ln = lane_id_volatile();
#pragma unroll
        for (int c0 = 0; c0 < QCH; c0 += 64) {
            const int ch = c0 + ln;
            const int r = ch / (D / 8), pc = ch % (D / 8);
            if (ch < QCH && r < nrows) {
                const int query = win[off + kDescHeader + 4 * (r / G)];
                const uint32_t e = uint32_t((query * Hq + g * G + r % G) * D + pc * 8);   // q holds < 2^31 elements
                dma16(q + e, qs_lds + uint32_t((s * QSLOT + c0 * 8) * 2));
            }
        }
    };

    // ---- load side
    int l_off = skip(0);
    int l_blk = 0, l_slot = 0;
    int l_lo = 0, l_hi = 0, l_ntok = 0, l_bids = 0, l_g = 0;
    auto l_enter = [&]() {
        if (l_off < n_words) {
            const int nb = hdr(l_off, kDescBlocks);
            l_lo = range_lo(nb);
            l_hi = range_hi(nb);
            l_blk = l_lo;
            l_ntok = hdr(l_off, kDescTokens);
            l_bids = l_off + kDescHeader + 4 * hdr(l_off, kDescNq);
            l_g = head_of(l_off);
        }
    };
    l_enter();

    // A block's K and V slices of KV head l_g are read through buffer resources
    // whose size covers the block's valid tokens only: the hardware returns
    // zeros for token slots past the range and for everything past the end of
    // the stream (size 0), so the ring below has no branches around its loads
    // (the compiler keeps them in flight) and needs no 64-bit per-lane addresses.
    int voff[2][NPC];   // byte offsets of this lane's pieces within a head slice
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int pc = 0; pc < NPC; ++pc) voff[tt][pc] = ((t + 8 * tt) * D + pc * 64 + 8 * c) * 2;
    auto load_block = [&](uint4 (&kb)[2][NPC], uint4 (&vb)[2][NPC]) {
        const bool live = l_off < n_words;
        // A task's q rows are copied right before its first block's loads: the
        // copy is then older than those loads, and at most NR - 1 tasks (the
        // blocks still in the ring) are pending, so NR slots never collide.
        if (live && l_blk == l_lo) fetch_q(l_off, l_slot);
        const int blk = live ? __builtin_amdgcn_readfirstlane(win[l_bids + l_blk]) : 0;
        const int valid = live ? min(16, l_ntok - l_blk * 16) : 0;
        const size_t o = size_t(blk) * blk_elems + size_t(l_g) * head_elems;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + o), 0, valid * D * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + o), 0, valid * D * 2, kBufferWord3);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rk, voff[tt][pc], 0, 0);
                const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[tt][pc], 0, 0);
                kb[tt][pc] = make_uint4(a.x, a.y, a.z, a.w);
                vb[tt][pc] = make_uint4(b.x, b.y, b.z, b.w);
            }
        }
        if (live && ++l_blk == l_hi) {
            l_off = skip(l_off + hdr(l_off, kDescWords));
            l_slot = (l_slot + 1) & 3;
            l_enter();
        }
    };

    // ---- process side: the stream ends when the last task's last block is
    // processed (p_off past the window); no load waits on a count of blocks
    int p_off = l_off;
    [[maybe_unused]] int n_done = 0;   // blocks processed (trace records only)
    int p_blk = -1, p_slot = 0, p_hi = 0;   // p_blk < 0: the next block starts a task
    int limit[R];
    float m[R], l[R], acc[R][NE];

    auto begin_task = [&]() {
        // the q copy of this task is older than its first block's loads, which
        // are complete once at most two blocks' loads remain outstanding
        __builtin_amdgcn_s_waitcnt(waitcnt_vm<(NR - 1) * LPB>());
        __builtin_amdgcn_sched_barrier(0);   // no LDS read of the slot moves above the wait
        const int nb = hdr(p_off, kDescBlocks);
        p_blk = range_lo(nb);
        p_hi = range_hi(nb);
        const int nrows = hdr(p_off, kDescRows);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // rows past the task's rows read stale q but are fully masked (limit 0)
            limit[r] = r < nrows ? win[p_off + kDescHeader + 4 * (r / G) + 2] : 0;
            m[r] = kNegSentinel;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[r][e] = 0.f;
        }
    };

    auto process = [&](int k, const uint4 (&kb)[2][NPC], const uint4 (&vb)[2][NPC]) {
        // q rows come from the task's LDS slot (every lane of a chunk set reads
        // the same 16 bytes), which keeps the register file for the load ring
        const uint16_t* qsl = qs + p_slot * QSLOT;
        float s[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const uint4 qq = *reinterpret_cast<const uint4*>(qsl + r * D + pc * 64 + 8 * c);
                a0 = dot2_bf16(qq.x, kb[0][pc].x, a0);
                a0 = dot2_bf16(qq.y, kb[0][pc].y, a0);
                a0 = dot2_bf16(qq.z, kb[0][pc].z, a0);
                a0 = dot2_bf16(qq.w, kb[0][pc].w, a0);
                a1 = dot2_bf16(qq.x, kb[1][pc].x, a1);
                a1 = dot2_bf16(qq.y, kb[1][pc].y, a1);
                a1 = dot2_bf16(qq.z, kb[1][pc].z, a1);
                a1 = dot2_bf16(qq.w, kb[1][pc].w, a1);
            }
            s[r][0] = octet_sum(a0);
            s[r][1] = octet_sum(a1);
        }
        bool need = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int tok = k * 16 + t + 8 * tt;
                s[r][tt] = tok < limit[r] ? s[r][tt] * sl2 : -INFINITY;
            }
            need |= fmaxf(s[r][0], s[r][1]) > m[r] + kRescaleLog2;
        }
        if (__any(need)) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float mn = fmaxf(m[r], fmaxf(s[r][0], s[r][1]));
                const float alpha = fast_exp2(m[r] - mn);
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[r][e] *= alpha;
                m[r] = mn;
            }
        }
        float pr[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            pr[r][0] = fast_exp2(s[r][0] - m[r]);
            pr[r][1] = fast_exp2(s[r][1] - m[r]);
            l[r] += pr[r][0] + pr[r][1];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const uint32_t w4[4] = {vb[tt][pc].x, vb[tt][pc].y, vb[tt][pc].z, vb[tt][pc].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float v0 = bf_lo(w4[w]), v1 = bf_hi(w4[w]);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        acc[r][pc * 8 + 2 * w] = fmaf(pr[r][tt], v0, acc[r][pc * 8 + 2 * w]);
                        acc[r][pc * 8 + 2 * w + 1] = fmaf(pr[r][tt], v1, acc[r][pc * 8 + 2 * w + 1]);
                    }
                }
            }
        }
    };

    // combine the 8 token lanes of each chunk set (lanes c, c+8, ..., c+56); the
    // results stay in acc[r][0 .. NE/8), ltot, mrow until store_task writes them
    float ltot[R], mrow[R];
    auto end_task = [&]() {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float M = m[r];
            M = fmaxf(M, lane_x8(M));
            float2 s = swap16(M, M);
            M = fmaxf(s.x, s.y);
            s = swap32(M, M);
            M = fmaxf(s.x, s.y);
            const float f = fast_exp2(m[r] - M);
            float lr = l[r] * f;
            lr += lane_x8(lr);
            s = swap16(lr, lr);
            lr = s.x + s.y;
            s = swap32(lr, lr);
            lr = s.x + s.y;
            ltot[r] = lr;
            mrow[r] = M;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[r][e] *= f;
        }
        // reduce-scatter over t: after three halving exchanges each lane owns NE/8
        // elements (lanes with bit 32 set keep the upper half of acc, and so on);
        // the first two exchanges are lane swaps, the last a DPP read
        const bool u8 = (lane & 8) != 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < NE / 2; ++i) {
                const float2 s = swap32(acc[r][i], acc[r][NE / 2 + i]);
                acc[r][i] = s.x + s.y;
            }
#pragma unroll
            for (int i = 0; i < NE / 4; ++i) {
                const float2 s = swap16(acc[r][i], acc[r][NE / 4 + i]);
                acc[r][i] = s.x + s.y;
            }
#pragma unroll
            for (int i = 0; i < NE / 8; ++i) {
                const float send = u8 ? acc[r][i] : acc[r][NE / 8 + i];
                const float keep = u8 ? acc[r][NE / 8 + i] : acc[r][i];
                acc[r][i] = keep + lane_x8(send);
            }
        }
    };
    // write the results of the task at `off` (output rows or partial triples)
    auto store_task = [&](int off) {
        const int nrows = hdr(off, kDescRows);
        const int g = head_of(off);
        const bool u32 = (lane & 32) != 0, u16 = (lane & 16) != 0, u8 = (lane & 8) != 0;
        const int ebase = (u32 ? NE / 2 : 0) + (u16 ? NE / 4 : 0) + (u8 ? NE / 8 : 0);
        // element e of chunk set c is head-dim index 8c + e (e < 8) or 64 + 8c + (e - 8)
        const int d0 = (ebase < 8) ? 8 * c + ebase : 64 + 8 * c + (ebase - 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nrows) continue;
            const int4 e = *reinterpret_cast<const int4*>(win + off + kDescHeader + 4 * (r / G));
            const int h = g * G + r % G;
            if (e.y < 0) {
                float* o = out + (size_t(e.x) * Hq + h) * D + d0;
                const float inv = 1.f / ltot[r];
                if constexpr (NE / 8 == 2) {
                    *reinterpret_cast<float2*>(o) = make_float2(acc[r][0] * inv, acc[r][1] * inv);
                } else {
                    o[0] = acc[r][0] * inv;
                }
            } else if (p.part_wt) {
                // partial triple, written through (read by the merge launch, or merged in
                // this launch possibly on another XCD)
                const size_t sl = size_t(e.y) + h;
                const __amdgpu_buffer_rsrc_t racc = part_rsrc(p.part_acc, p.part_acc_bytes);
                const uint32_t o = uint32_t((sl * D + d0) * 4);
                if constexpr (NE / 8 == 2) {
                    store_sc1(racc, o, make_float2(acc[r][0], acc[r][1]));
                } else {
                    store_sc1(racc, o, acc[r][0]);
                }
                if (lane == 0)
                    store_sc1(part_rsrc(p.part_ml, p.part_ml_bytes), uint32_t(sl * 8), make_float2(mrow[r], ltot[r]));
            } else {
                const size_t sl = size_t(e.y) + h;
                float* o = p.part_acc + sl * D + d0;
                if constexpr (NE / 8 == 2) {
                    *reinterpret_cast<float2*>(o) = make_float2(acc[r][0], acc[r][1]);
                } else {
                    o[0] = acc[r][0];
                }
                if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + sl * 2) = make_float2(mrow[r], ltot[r]);
            }
        }
    };

    // A finished task's stores are issued after the next block's loads: vmcnt
    // retires loads and stores in issue order, so a store issued before a load
    // would make the wait for that load also wait for the store's ack.  Issued
    // after it, the stores have NR block-times to complete before any wait
    // depends on them.
    int f_off = -1;   // task whose results await their stores
    // SPLIT: the four waves' rows of the task at `off` combined through LDS and stored
    auto split_combine = [&](int off) {
        const int nrows = hdr(off, kDescRows);
        const int g = hdr(off, kDescHead);
        constexpr int RS = D + 2;   // floats per row in cbuf: acc[D], m, l
        const bool u32 = (lane & 32) != 0, u16 = (lane & 16) != 0, u8 = (lane & 8) != 0;
        const int ebase = (u32 ? NE / 2 : 0) + (u16 ? NE / 4 : 0) + (u8 ? NE / 8 : 0);
        const int d0 = (ebase < 8) ? 8 * c + ebase : 64 + 8 * c + (ebase - 8);
        float* mine = cbuf + wave * R * RS;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nrows) continue;
#pragma unroll
            for (int i = 0; i < NE / 8; ++i) mine[r * RS + d0 + i] = acc[r][i];
            if (lane == 0) {
                mine[r * RS + D] = mrow[r];
                mine[r * RS + D + 1] = ltot[r];
            }
        }
        __syncthreads();
        for (int e = int(threadIdx.x); e < nrows * D; e += 64 * kWaves) {
            const int r = e / D, d = e - r * D;
            float M = cbuf[r * RS + D];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, cbuf[(w * R + r) * RS + D]);
            float L = 0.f, A = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float* x = cbuf + (w * R + r) * RS;
                const float f = fast_exp2(x[D] - M);
                L = fmaf(f, x[D + 1], L);
                A = fmaf(f, x[d], A);
            }
            const int query = win[off + kDescHeader + 4 * (r / G)];
            const int dest = win[off + kDescHeader + 4 * (r / G) + 1];
            const int h = g * G + r % G;
            if (dest < 0) {
                out[(size_t(query) * Hq + h) * D + d] = A / L;
            } else {
                const size_t sl = size_t(dest) + h;
                if (p.part_wt) {
                    store_sc1(part_rsrc(p.part_acc, p.part_acc_bytes), uint32_t((sl * D + d) * 4), A);
                    if (d == 0) store_sc1(part_rsrc(p.part_ml, p.part_ml_bytes), uint32_t(sl * 8), make_float2(M, L));
                } else {
                    p.part_acc[sl * D + d] = A;
                    if (d == 0) *reinterpret_cast<float2*>(p.part_ml + sl * 2) = make_float2(M, L);
                }
            }
        }
        __syncthreads();   // cbuf is free for the next task
    };
    auto proc_block = [&](const uint4 (&kb)[2][NPC], const uint4 (&vb)[2][NPC]) {
        if (p_blk < 0) begin_task();
        process(p_blk, kb, vb);
        if constexpr (KV_TRACE_ON) ++n_done;
        if (++p_blk == p_hi) {
            end_task();
            if constexpr (SPLIT) {
                split_combine(p_off);
            } else {
                f_off = p_off;
            }
            p_off = skip(p_off + hdr(p_off, kDescWords));
            p_blk = -1;
            p_slot = (p_slot + 1) & 3;
        }
    };
    auto flush = [&]() {
        if (f_off >= 0) {
            store_task(f_off);
            f_off = -1;
        }
    };

    // NR-deep register ring across the whole stream; scheduling barriers keep
    // each refill after the compute that frees its registers, so NR - 1 blocks
    // stay in flight and register pressure stays bounded
    uint4 kr[NR][2][NPC], vr[NR][2][NPC];
#pragma unroll
    for (int u = 0; u < NR; ++u) load_block(kr[u], vr[u]);
    while (p_off < n_words) {
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            if (p_off < n_words) proc_block(kr[u], vr[u]);
            __builtin_amdgcn_sched_barrier(0);
            load_block(kr[u], vr[u]);
            __builtin_amdgcn_sched_barrier(0);
            flush();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    flush();
    if constexpr (KV_TRACE_ON && !SPLIT) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
        if (lane == 0) KV_TRACE(blockIdx.x, 40 + wave, 4, uint32_t(n_done));
    }

    // Fused merge: the stream's partial stores are complete (sc1: performed at
    // agent scope) before its arrivals; the task completing a (query, KV head)
    // merges it.  Arrivals come at the end of the stream, where waiting for
    // every outstanding store costs nothing.
    if (!SPLIT && p.arrive) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // the stream's partial entries go to lanes in order, up to 64 arrivals
        // in flight at once; then the units this wave completed are merged
        int my_rec = -1, my_g = 0, na = 0;
        auto arrive_batch = [&]() {
            const bool last = my_rec >= 0 && arrive_last(p, Hkv, my_rec, my_g);
            uint64_t mask = __ballot(last);
            while (mask) {
                const int i = __builtin_ctzll(mask);
                mask &= mask - 1;
                merge_unit<D>(p, dm, __builtin_amdgcn_readlane(my_rec, i), __builtin_amdgcn_readlane(my_g, i), out);
            }
            my_rec = -1;
        };
        for (int off = skip(0); off < n_words; off = skip(off + hdr(off, kDescWords))) {
            const int nq = hdr(off, kDescNq);
            const int g = head_of(off);
            for (int e = 0; e < nq; ++e) {
                const int dest = hdr(off, kDescHeader + 4 * e + 1);
                if (dest < 0) continue;
                if (lane == (na & 63)) {
                    my_rec = win[off + kDescHeader + 4 * e + 3];
                    my_g = g;
                }
                if ((++na & 63) == 0) arrive_batch();
            }
        }
        if (na & 63) arrive_batch();
    }
}

// ============================================================================
// MFMA task: the workgroup's 4 waves share one KV head's tiles; wave w owns
// rows [16 t w, 16 t (w + 1)) as t = 1 or 2 sixteen-row tiles.  Per 32-token tile:
//   S^T[16 tok x 16 rows] = K[16 x 32 d] . Q^T[32 d x 16 rows]   (4 k-steps at D = 128)
//   O^T[16 d x 16 rows]  += V^T[16 d x 32 tok] . P^T[32 tok x 16 rows]
// Output tile j holds head dims [16j, 16j + 16).  Its A operand V^T (16 d x 32
// tokens) comes straight from the row-major V tile through two transposing LDS
// reads (tokens 4lg + e, then 16 + 4lg + e), the token order of the P^T operand.
// P is split into bf16 hi + lo parts (two MFMAs) so the weights keep ~16 bits.
// K and V tiles live in LDS in rows of D/8 16-byte chunks, permuted per token
// row so that both reads are bank-conflict free: K chunk c of token t sits at
// c ^ (t mod D/8) (16 row-strided 16-byte reads), V chunk c at c ^ vswz(t) (the
// transposing read takes 4 or 8 rows at one 32-byte column).
// ============================================================================
// V chunk permutation of token row t (t mod 16 suffices): XOR with an even
// value, so the two chunks of a 32-byte column stay together, and the rows
// t = 0..7 land that column on 8 distinct 32-byte bank groups (4 at D = 64).
template <int D>
__device__ __forceinline__ int vswz(int t) {
    if constexpr (D == 128)
        return ((t & 3) << 1) | (((t >> 2) & 1) << 3);
    else
        return ((t & 3) ^ ((t >> 2) & 1)) << 1;
}

template <int D, int TPW>
__device__ __forceinline__ void mfma_task(const DevPlan& p, const Dims& dm, const TaskView& it, int g,
                                          const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                          const uint16_t* __restrict__ vc, float* __restrict__ out,
                                          uint16_t* s_kv) {
    constexpr int NW = kWaves;
    constexpr int TT = kMfmaTileTokens;    // 32 tokens per stage
    constexpr int CPR = D / 8;             // 16-byte chunks per token row
    constexpr int TCH = TT * CPR;          // chunks per K (or V) tile
    constexpr int KS = D / 32;             // QK k-steps
    constexpr int NDT = D / 16;            // output tiles
    constexpr int NT = 64 * NW;            // threads
    constexpr int LPT = TCH >= NT ? TCH / NT : 1;   // DMA chunks per thread per tensor and tile
    constexpr int NS = kMfmaStages;        // LDS stages: NS - 1 tiles in flight
    constexpr int STAGE = 2 * TT * D;      // elements per stage (K tile then V tile)
    static_assert(TCH % NT == 0 || NT % TCH == 0, "tile chunks must split evenly over the workgroup");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int Hkv = dm.num_kv_heads;
    const int G = dm.group;
    const int n_tok = it.n_tokens;
    const int nblk = it.nblk;
    const int ntiles = (n_tok + TT - 1) / TT;
    const int row0 = wave * 16 * TPW;       // TPW sixteen-row tiles per wave
    const int32_t* s_blk = it.blk;          // block ids, in LDS

    // ---- Q operands (B of S^T = K Q^T): lane -> row lr of the tile, d = 32s + 8lg .. +7.
    // Rows past the item's rows get q = 0: they are computed but never stored.
    bf16x8 qop[TPW][KS];
    int lim[TPW];
    const bool active = row0 < it.n_rows;   // wave-uniform
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
        const int r = row0 + rt * 16 + lr;
        if (r < it.n_rows) {
            const Entry e = entry_of(it, r / G);
            const int h = g * G + r % G;
            const uint16_t* qrow = q + (size_t(e.query) * dm.num_q_heads + h) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) qop[rt][s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * lg);
            lim[rt] = e.limit;
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s) qop[rt][s] = bf16x8{};
            lim[rt] = 0;
        }
    }
    // tokens every row of the item attends to: tiles below this need no mask
    const int lim_all = it.lim_all;
    // Complete every setup load here: the tile loop below must see no older
    // vector-memory operation, or waits on it would also drain the tile DMA.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());

    // ---- loop-invariant DMA geometry
    const size_t head_elems = size_t(16) * D;
    const size_t blk_elems = size_t(Hkv) * head_elems;
    const uint16_t* kh = kc + size_t(g) * head_elems;
    const uint16_t* vh = vc + size_t(g) * head_elems;
    // chunk u of this thread is token tok0 + u * (NT / CPR): the same row offset in
    // every u, since NT / CPR is a multiple of 16 (or LPT is 1)
    static_assert(LPT == 1 || (NT / CPR) % 16 == 0, "DMA chunk stride");
    // Each copy instruction of a wave covers 64 consecutive chunks, i.e. whole
    // token rows of one block (16 rows at D = 128 per u, 8 rows at D = 64 per
    // wave), so the block and its buffer resource are wave-uniform.  A block's
    // resource spans its valid tokens: rows past the range land in LDS as zeros.
    const int tok0 = tid / CPR;
    const uint32_t voff_k = uint32_t((tok0 & 15) * D + ((tid % CPR) ^ (tok0 & (CPR - 1))) * 8) * 2;
    const uint32_t voff_v = uint32_t((tok0 & 15) * D + ((tid % CPR) ^ vswz<D>(tok0)) * 8) * 2;
    const uint32_t lds_base = uint32_t(uintptr_t(s_kv));
    auto issue_tile = [&](int i, int stage) {
        const uint32_t st = lds_base + uint32_t(stage * STAGE * 2);
        const int kb = 2 * i;
        const int blk0 = __builtin_amdgcn_readfirstlane(s_blk[kb]);
        const int blk1 = __builtin_amdgcn_readfirstlane(kb + 1 < nblk ? s_blk[kb + 1] : blk0);
        const int rem = n_tok - kb * kBlock;   // tokens from this tile's first block on (>= 1)
        const uint32_t bytes0 = uint32_t(min(rem, kBlock)) * D * 2;
        const uint32_t bytes1 = uint32_t(max(0, min(rem - kBlock, kBlock))) * D * 2;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            if (u * NT + wave * 64 >= TCH) continue;    // wave-uniform: waves past the tile issue nothing
            const bool second = (u * NT + wave * 64) / CPR >= kBlock;   // wave-uniform
            const size_t ob = size_t(second ? blk1 : blk0) * blk_elems;
            const uint32_t nb = second ? bytes1 : bytes0;
            const uint32_t dst = st + uint32_t((u * NT + wave * 64) * 16);
            dma16_buf(raw_rsrc(kh + ob, nb), voff_k, dst);
            dma16_buf(raw_rsrc(vh + ob, nb), voff_v, dst + TT * D * 2);
        }
    };

    float mref[TPW], lsum[TPW];
    f32x4 acc[TPW][NDT];
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
        mref[rt] = kNegSentinel;
        lsum[rt] = 0.f;
#pragma unroll
        for (int j = 0; j < NDT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = dm.scale_log2;

    // per-lane LDS offsets of the K operand (A of QK, elements) and of the
    // transposing V reads (bytes, output tile j) for token half 0; half 1 adds 16
    // rows (both permutations only see token mod 16, which the halves share).
    // Lane a + 4e of a 16-lane group addresses token 4lg + e, head dims
    // 16j + 4a .. 16j + 4a + 3.
    constexpr int HALF = 16 * CPR * 8;
    int koff[KS];
    uint32_t vtr[NDT];
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = (lr * CPR + ((4 * s + lg) ^ (lr & (CPR - 1)))) * 8;
    {
        const int t = 4 * lg + (lr >> 2);
        const int sw = vswz<D>(t);
        // vtr[j]: head dims 16j + 4 (lr mod 4) .. + 3 of token t, in V chunk 2j + (lr mod 4) / 2
#pragma unroll
        for (int j = 0; j < NDT; ++j)
            vtr[j] = uint32_t(2 * (TT * D + t * D) + ((2 * j + ((lr & 3) >> 1)) ^ sw) * 16 + (lr & 1) * 8);
    }

    auto compute = [&](int i, const uint16_t* sb) {
        if (!active) return;
        // ---- LDS reads of the whole tile: K operands, then the V^T operands (lane
        // (m, lg) of output tile j gets head dim 16j + m of tokens 4lg + e and
        // 16 + 4lg + e), whose latency the QK products and the softmax hide
        bf16x8 kop[2][KS];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int s = 0; s < KS; ++s) kop[half][s] = *reinterpret_cast<const bf16x8*>(sb + koff[s] + half * HALF);
        uint2 vr[NDT][2];
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            vr[j][0] = lds_read_tr16(sb, vtr[j]);
            vr[j][1] = lds_read_tr16(sb, vtr[j] + 2 * HALF);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- S^T tiles (unscaled q.k)
        f32x4 sc[TPW][2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[half][s], qop[rt][s], a, 0, 0, 0);
                sc[rt][half] = a;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- mask (tail tiles only): token 16 half + 4 lg + e beyond the row's limit
        if ((i + 1) * TT > lim_all) {
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (i * TT + 16 * half + 4 * lg + e >= lim[rt]) sc[rt][half][e] = -INFINITY;
        }
        // ---- lazy running max in log2 units
        bool need = false;
        float tmax[TPW];
#pragma unroll
        for (int rt = 0; rt < TPW; ++rt) {
            const float m3a = max3f(sc[rt][0][0], sc[rt][0][1], sc[rt][0][2]);
            const float m3b = max3f(sc[rt][0][3], sc[rt][1][0], sc[rt][1][1]);
            tmax[rt] = max3f(m3a, m3b, fmaxf(sc[rt][1][2], sc[rt][1][3])) * sl2;
            need |= tmax[rt] > mref[rt] + kRescaleLog2;
        }
        if (__any(need)) {
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                float rm = tmax[rt];
                float2 s = swap16(rm, rm);
                rm = fmaxf(s.x, s.y);
                s = swap32(rm, rm);
                rm = fmaxf(s.x, s.y);
                const float mn = fmaxf(mref[rt], rm);
                const float alpha = fast_exp2(mref[rt] - mn);
                lsum[rt] *= alpha;
#pragma unroll
                for (int j = 0; j < NDT; ++j) acc[rt][j] *= alpha;
                mref[rt] = mn;
            }
        }
        // ---- P^T operands (bf16 hi + lo): token tau(lg, u) = 4lg + u (u < 4) or 16 + 4lg + (u - 4)
        bf16x8 phi[TPW], plo[TPW];
#pragma unroll
        for (int rt = 0; rt < TPW; ++rt) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = fast_exp2(fmaf(sc[rt][0][e], sl2, -mref[rt]));
                pv[4 + e] = fast_exp2(fmaf(sc[rt][1][e], sl2, -mref[rt]));
            }
            lsum[rt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                hi[x] = pack_bf16(pv[2 * x], pv[2 * x + 1]);
                // low half moved up by v_perm_b32 (bytes 4, 5 are the first operand's low
                // half; selector 0x0c gives a zero byte), which the compiler does not
                // rewrite into a second conversion
                const float h0 = __uint_as_float(__builtin_amdgcn_perm(hi[x], 0u, 0x05040c0cu));
                lo[x] = pack_bf16(pv[2 * x] - h0, pv[2 * x + 1] - bf_hi(hi[x]));
            }
            phi[rt] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            plo[rt] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- O^T += V^T P^T
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            const bf16x8 vt = __builtin_bit_cast(bf16x8, make_uint4(vr[j][0].x, vr[j][0].y, vr[j][1].x, vr[j][1].y));
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, phi[rt], acc[rt][j], 0, 0, 0);
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, plo[rt], acc[rt][j], 0, 0, 0);
            }
        }
    };

    if constexpr (TPW == 1) {
        // ---- Register-staged pipeline (16 rows per wave): tile i + RT is loaded into
        // VGPRs while tile i is computed, and each tile is written to LDS by the
        // workgroup just before its barrier.  Measured streaming these 32-token
        // tiles alone (2 workgroups per CU, 8 GiB): three 16 KB tiles in registers
        // 6.30-6.40 TB/s, where buffer->LDS copies with three tiles in flight reach
        // 5.79-5.84 TB/s.  The tiles take 16 LPT VGPRs each, which fits next to one
        // sixteen-row tile per wave but not two.  The LDS layout is the DMA path's:
        // thread c of a copy holds chunk c of the stage, read from the permuted
        // global offset.
        constexpr int RT = 3;                   // tiles in flight (and LDS stages used)
        static_assert(RT <= NS, "register-staged tiles use the MFMA stage buffer");
        static_assert(TCH % NT == 0, "every thread holds LPT chunks of each tile");
        struct RegTile {
            u32x4 k[LPT], v[LPT];
        };
        // loads of tile i; past the task's last tile the resources are empty, so the
        // loads read nothing from memory and return zeros (the loop stays branch-free)
        auto load_tile = [&](int i, RegTile& t) {
            const bool live = i < ntiles;      // wave-uniform
            const int kb = live ? 2 * i : 0;
            const int blk0 = __builtin_amdgcn_readfirstlane(s_blk[kb]);
            const int blk1 = __builtin_amdgcn_readfirstlane(kb + 1 < nblk ? s_blk[kb + 1] : blk0);
            const int rem = live ? n_tok - kb * kBlock : 0;
            const uint32_t bytes0 = uint32_t(min(rem, kBlock)) * D * 2;
            const uint32_t bytes1 = uint32_t(max(0, min(rem - kBlock, kBlock))) * D * 2;
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const bool second = (u * NT + wave * 64) / CPR >= kBlock;   // wave-uniform
                const size_t ob = size_t(second ? blk1 : blk0) * blk_elems;
                const int nb = int(second ? bytes1 : bytes0);
                const __amdgpu_buffer_rsrc_t rk =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh + ob), 0, nb, kBufferWord3);
                const __amdgpu_buffer_rsrc_t rv =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vh + ob), 0, nb, kBufferWord3);
                t.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k, 0, 0);
                t.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, 0, 0);
            }
        };
        auto write_tile = [&](const RegTile& t, int stage) {
            uint16_t* sb = s_kv + stage * STAGE;
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                *reinterpret_cast<u32x4*>(sb + (u * NT + tid) * 8) = t.k[u];
                *reinterpret_cast<u32x4*>(sb + TT * D + (u * NT + tid) * 8) = t.v[u];
            }
        };
        // One step: tile i (held in t) is written to LDS stage st, and t takes the
        // loads of tile i + RT.  Stage st last held tile i - RT, which every wave
        // finished before it passed the previous step's barrier; after this step's
        // barrier every wave's part of tile i is in LDS.
        auto step = [&](RegTile& t, int i, int st) {
            write_tile(t, st);
            load_tile(i + RT, t);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (i < ntiles) compute(i, s_kv + st * STAGE);
            __builtin_amdgcn_sched_barrier(0);
        };
        RegTile t0, t1, t2;
        load_tile(0, t0);
        load_tile(1, t1);
        load_tile(2, t2);
        for (int i0 = 0; i0 < ntiles; i0 += RT) {
            step(t0, i0, 0);
            step(t1, i0 + 1, 1);
            step(t2, i0 + 2, 2);
        }
    } else {
        // ---- NS-stage pipeline: tiles i+1 .. i+NS-1 stream in while tile i is computed ----
    // Unrolled by NS so that every stage offset is a constant: LDS reads then
        // take it in their offset field instead of a vector add per address.
        static_assert(NS == 4, "the wait counts below assume at most two younger tiles");
    #pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (i < ntiles) issue_tile(i, i);
        for (int i0 = 0; i0 < ntiles; i0 += NS) {
    #pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int i = i0 + st;
                if (i < ntiles) {
                    // this thread's DMA for tile i is complete once at most the loads of the
                    // (up to NS - 2) younger tiles remain outstanding
                    const int younger = min(ntiles - 1 - i, NS - 2);
                    if (younger >= 2) {
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm<4 * LPT>());
                    } else if (younger == 1) {
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm<2 * LPT>());
                    } else {
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
                    }
                    __builtin_amdgcn_s_barrier();   // every wave's DMA for tile i landed; tile i-1 is consumed
                    if (i + NS - 1 < ntiles) issue_tile(i + NS - 1, (st + NS - 1) % NS);
                    compute(i, s_kv + st * STAGE);
                }
            }
        }
    }

    // ---- epilogue: lane holds row lr of each tile and, in output tile j, head dims 16j + 4lg + e
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
        if (!active) continue;
        float lt = lsum[rt];
        float2 s = swap16(lt, lt);
        lt = s.x + s.y;
        s = swap32(lt, lt);
        lt = s.x + s.y;
        const int r = row0 + rt * 16 + lr;
        if (r >= it.n_rows) continue;
        const Entry e = entry_of(it, r / G);
        const int h = g * G + r % G;
        if (e.dest >= 0 && p.part_wt) {
            // partial triple, written through (see store_sc1)
            const size_t slot = size_t(e.dest) + h;
            if (lg == 0)
                store_sc1(part_rsrc(p.part_ml, p.part_ml_bytes), uint32_t(slot * 8), make_float2(mref[rt], lt));
            const __amdgpu_buffer_rsrc_t racc = part_rsrc(p.part_acc, p.part_acc_bytes);
#pragma unroll
            for (int j = 0; j < NDT; ++j)
                store_sc1(racc, uint32_t((slot * D + 16 * j + 4 * lg) * 4),
                          make_float4(acc[rt][j][0], acc[rt][j][1], acc[rt][j][2], acc[rt][j][3]));
            continue;
        }
        float* dst;
        float scale;
        if (e.dest < 0) {
            dst = out + (size_t(e.query) * dm.num_q_heads + h) * D;
            scale = 1.f / lt;
        } else {
            const size_t slot = size_t(e.dest) + h;
            dst = p.part_acc + slot * D;
            scale = 1.f;
            if (lg == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(mref[rt], lt);
        }
#pragma unroll
        for (int j = 0; j < NDT; ++j)
            *reinterpret_cast<float4*>(dst + 16 * j + 4 * lg) =
                make_float4(acc[rt][j][0] * scale, acc[rt][j][1] * scale, acc[rt][j][2] * scale, acc[rt][j][3] * scale);
    }
}

// ============================================================================
// Persistent forward kernel: workgroup w runs static list w (and w + gridDim.x,
// ... when fewer workgroups are resident than lists): its MFMA tasks, then its
// VALU tasks as continuous per-wave streams.  VALU and MFMA tasks share one
// launch, so the MFMA work of packed groups runs side by side with the
// bandwidth-bound private tails (the goal of the PAT review's multi-stream
// forward: no execution bubbles), without cross-stream synchronisation.
// ============================================================================

// Copy `words` (a multiple of 4) int32 words of descriptors into LDS by direct
// global -> LDS DMA, 16 bytes per lane.  Completion is awaited by the caller
// (s_waitcnt vmcnt(0) and a barrier).
__device__ __forceinline__ void fetch_desc(const int32_t* src, int words, int32_t* dst) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = words >> 2;
    const uint32_t base = uint32_t(uintptr_t(dst));
    for (int r0 = 0; r0 < n16; r0 += 64 * kWaves) {
        const int c = r0 + tid;
        if (c < n16) dma16(src + 4 * c, base + uint32_t(16 * (r0 + 64 * wave)));
    }
}

__device__ __forceinline__ void wait_all_and_sync() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
    __syncthreads();
}

// Fused merge after an MFMA task (every wave's partial stores complete): one
// arrival per query entry on the task's KV head; the waves merge the
// (query, KV head) units this task completed.
template <int D>
__device__ __forceinline__ void mfma_arrivals(const DevPlan& p, const Dims& dm, const TaskView& it,
                                              float* __restrict__ out, int* s_last, int* s_nlast) {
    const int g = it.head;
    if (threadIdx.x == 0) *s_nlast = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < it.n_q; e += 64 * kWaves) {
        const int4 en = *reinterpret_cast<const int4*>(it.ent + 4 * e);
        if (en.y >= 0 && arrive_last(p, dm.num_kv_heads, en.w, g)) s_last[atomicAdd(s_nlast, 1)] = en.w;
    }
    __syncthreads();
    const int nl = __builtin_amdgcn_readfirstlane(*s_nlast);
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    for (int i = wave; i < nl; i += kWaves) merge_unit<D>(p, dm, __builtin_amdgcn_readfirstlane(s_last[i]), g, out);
    __syncthreads();   // s_last is free for the next task
}

template <int D, int R, int TPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_kernel(
    DevPlan p, Dims dm, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ out) {
    constexpr int TT = kMfmaTileTokens;
    constexpr int KV_ELEMS = kMfmaStages * 2 * TT * D;
    constexpr int WIN = valu_window_words(D, R);
    static_assert(KV_ELEMS * 2 == WIN * 4 + kWaves * 4 * R * D * 2, "VALU window layout");
    __shared__ __attribute__((aligned(16))) uint16_t s_kv[KV_ELEMS];
    __shared__ __attribute__((aligned(16))) int32_t s_desc[2][kDescMaxWords];
    __shared__ int s_last[kMaxItemQueries + 1];   // fused merge: units an MFMA task completed, and their count
    static_assert(kWaves * R * (D + 2) * 4 <= int(sizeof(s_desc)), "VALU_SPLIT combine rows fit the descriptor buffers");
    static_assert(D != 128 || KV_ELEMS * 2 + sizeof(s_desc) + sizeof(s_last) + 64 <= 80 * 1024,
                  "two workgroups per CU");
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    // All control flow below is wave-uniform: the loops hold barriers, so
    // lane-divergent branches must stay out of their exits and back edges.
    //
    // Lists [0, gridDim.x) run one per workgroup; the rest are claimed in order
    // from a counter in the workspace.  A workgroup asks for its next list when
    // it starts one (the atomic's latency hides behind the list's first loads)
    // and reads the answer when the list ends.  The claims of a launch draw
    // 0 .. n_lists - 1 once each (valid ones, plus one failing claim per
    // workgroup), so the workgroup that draws n_lists - 1 made the launch's
    // last claim and returns the counter to zero for the next launch.
    __shared__ int s_next[2];
    const bool claims = p.n_lists > int(gridDim.x);
    int w = blockIdx.x;
    [[maybe_unused]] int nev = 0;   // trace records of this workgroup slot
    if (threadIdx.x == 0) KV_TRACE(blockIdx.x, nev++, 0, uint32_t(w));
    for (int round = 0; w < p.n_lists; ++round) {
        int ticket = 0;
        if (claims && threadIdx.x == 0) ticket = atomicAdd(p.claim + opaque_zero(), 1);
        const KV_CONST int32_t* lp = cptr(p.list_ptr) + 3 * w;
        const int m0 = lp[0], v0 = lp[1], e0 = lp[2];
        // ---- MFMA tasks: the next descriptor lies right after the current one
        // and is copied into the other LDS buffer before the current task's
        // first KV load, so it has landed when the task ends.
        if (m0 < v0) {
            int off = m0, buf = 0;
            fetch_desc(p.desc + off, min(kDescMaxWords, v0 - off), s_desc[0]);
            wait_all_and_sync();
            while (true) {
                const int32_t* d = s_desc[buf];
                const int words = __builtin_amdgcn_readfirstlane(d[kDescWords]);
                const int next_words = __builtin_amdgcn_readfirstlane(d[kDescNextWords]);
                const int noff = off + words;
                if (noff < v0) fetch_desc(p.desc + noff, next_words, s_desc[buf ^ 1]);
                const TaskView it = view_of(d);
                if (threadIdx.x == 0) KV_TRACE(blockIdx.x, nev++, 1, uint32_t(it.n_tokens) | (uint32_t(it.n_rows) << 20));
                mfma_task<D, TPW>(p, dm, it, it.head, q, kc, vc, out, s_kv);
                wait_all_and_sync();   // the prefetched descriptor landed; this task's LDS is free
                if (threadIdx.x == 0) KV_TRACE(blockIdx.x, nev++, 2, 0u);
                if (p.arrive) mfma_arrivals<D>(p, dm, it, out, s_last, s_last + kMaxItemQueries);
                if (noff >= v0) break;
                off = noff;
                buf ^= 1;
            }
        }
        // ---- VALU tasks: the descriptors go into the LDS window in one piece,
        // then every wave streams its KV head of each task.
        if (v0 < e0) {
            int32_t* win = reinterpret_cast<int32_t*>(s_kv);
            fetch_desc(p.desc + v0, e0 - v0, win);
            wait_all_and_sync();
            if (threadIdx.x == 0) KV_TRACE(blockIdx.x, nev++, 3, uint32_t(e0 - v0));
            uint16_t* qs = s_kv + 2 * WIN + wave * 4 * R * D;
            float* cbuf = reinterpret_cast<float*>(&s_desc[0][0]);   // the descriptor buffers are idle here
            valu_stream<D, R, false>(p, dm, win, e0 - v0, qs, cbuf, q, kc, vc, out);
            wait_all_and_sync();   // the window is free for the next list ...
            if (p.has_split) {     // ... after the VALU_SPLIT tasks, if the plan has any
                valu_stream<D, R, true>(p, dm, win, e0 - v0, qs, cbuf, q, kc, vc, out);
                wait_all_and_sync();
            }
            if (threadIdx.x == 0) KV_TRACE(blockIdx.x, nev++, 5, 0u);
        }
        if (!claims) break;
        if (threadIdx.x == 0) {
            if (ticket == p.n_lists - 1) __hip_atomic_store(p.claim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_next[round & 1] = int(gridDim.x) + ticket;
        }
        __syncthreads();
        w = __builtin_amdgcn_readfirstlane(s_next[round & 1]);
    }
}

// ============================================================================
// Merge (one wave per workgroup): workgroup (query, y) combines, for the 256
// output floats [256 y, 256 y + 256) of the query's [Hq][D] block, all partial
// triples of the query in one pass with the online-softmax rule:
//   M' = max(M, m_i);  A = A 2^(M - M') + 2^(m_i - M') acc_i;  L likewise with l_i
// and writes A / L.  A query's partials are consecutive [Hq][D] blocks of
// slots (partial k of q head h in slot first + k Hq + h), located from one
// record.  Partials are read in batches of eight with every load in flight.
//
// With the fused KV append (NEW), the query's newest token, which the forward
// did not read, starts the combination as one more partial: m = q.k_new in log2
// units, l = 1, acc = v_new.  Its score is a dot product over the head's D/4
// lanes (one aligned lane group of the wave); the lanes of the first q head of
// each KV head also copy k_new / v_new into the token's paged slot.
// ============================================================================
template <int D, bool NEW>
__global__ __launch_bounds__(64) void merge_kernel(DevPlan p, Dims dm, NewTokens nt, float* __restrict__ out) {
    const int Hq = dm.num_q_heads;
    const int mq = blockIdx.x;
    const int col = int(blockIdx.y) * 256 + 4 * int(threadIdx.x);   // float index in [Hq][D]
    if (col >= Hq * D) return;     // whole heads: a head's lanes leave together
    const int h = col / D;
    // the query, its first partial slot and its partial count (one scalar load)
    const KV_CONST MergeRec* rec = cptr(p.merge_rec) + mq;
    const int b = rec->query, n = rec->count;
    const size_t slot0 = size_t(rec->first) + h;
    float M = -INFINITY, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (NEW) {
        const int hk = h / dm.group, e0 = col - h * D;
        const size_t kv = (size_t(b) * dm.num_kv_heads + hk) * D + e0;
        const uint2 qw = *reinterpret_cast<const uint2*>(nt.q + size_t(b) * Hq * D + col);
        const uint2 kw = *reinterpret_cast<const uint2*>(nt.k_new + kv);
        const uint2 vw = *reinterpret_cast<const uint2*>(nt.v_new + kv);
        float dot = dot2_bf16(qw.y, kw.y, dot2_bf16(qw.x, kw.x, 0.f));
#pragma unroll
        for (int o = D / 8; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
        M = dot * dm.scale_log2;
        L = 1.f;
        A = make_float4(bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y));
        if (h % dm.group == 0) {
            const int code = rec->new_slot;   // block * 16 + slot
            const size_t at = ((size_t(code >> 4) * dm.num_kv_heads + hk) * 16 + (code & 15)) * D + e0;
            *reinterpret_cast<uint2*>(nt.k_cache + at) = kw;
            *reinterpret_cast<uint2*>(nt.v_cache + at) = vw;
        }
    }
    merge_partials<D, false, 8>(p, Hq, slot0, n, col - h * D, M, L, A);
    const float inv = 1.f / L;
    *reinterpret_cast<float4*>(out + size_t(b) * Hq * D + col) = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
}

// Grid of a persistent launch: the workgroups the device holds at once
// (occupancy API x CUs), or fewer when there are fewer static lists.
template <typename K>
int persistent_grid(K kernel, int* cache, int n_lists) {
    if (*cache == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess) return -1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess) return -1;
        *cache = cus * (per_cu > 0 ? per_cu : 1);
    }
    return n_lists < *cache ? n_lists : *cache;
}

template <int D, int R, int TPW>
int launch_fwd_t(const DevPlan& p, const Dims& d, int n_tasks, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, float* out, hipStream_t s) {
    static int slots = 0;
    (void)n_tasks;
    // one workgroup per list when they all fit at once; otherwise the
    // workgroups claim the lists past the grid as they finish theirs
    const int grid = persistent_grid(fwd_kernel<D, R, TPW>, &slots, p.n_lists);
    if (grid < 0) return int(hipErrorInvalidDevice);
    hipLaunchKernelGGL((fwd_kernel<D, R, TPW>), dim3(grid), dim3(256), 0, s, p, d, q, k, v, out);
    return int(hipGetLastError());
}

// Measurement helper, not part of the attention path: a plain streaming read
// of two buffers (the K and V pools), split into one contiguous share per
// workgroup of NT threads, DEPTH 16-byte loads per lane in flight, XOR-folded
// into one word per thread so the loads are not removed.  It gives the
// bandwidth the memory system delivers for the pools' bytes at the same size.
template <int DEPTH, int NT>
__global__ __launch_bounds__(NT) void read_probe_kernel(const u32x4* __restrict__ a, size_t na,
                                                        const u32x4* __restrict__ b, size_t nb, uint32_t* sink) {
    const size_t n = na + nb;
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t s0 = per * blockIdx.x, s1 = min(n, s0 + per);
    uint32_t x = 0;
    for (size_t i = s0 + threadIdx.x; i < s1; i += size_t(NT) * DEPTH) {
        // addresses are selected, never the loads: all DEPTH loads stay in flight
        u32x4 v[DEPTH];
        bool ok[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const size_t j = i + size_t(d) * NT;
            ok[d] = j < s1;
            const size_t jj = ok[d] ? j : i;          // i < s1: a valid element
            const u32x4* src = jj < na ? a + jj : b + (jj - na);
            v[d] = *src;
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (ok[d]) x ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    sink[size_t(blockIdx.x) * NT + threadIdx.x] = x;
}

// Static device scratch of kvattn_decode_noalloc: the schedule blob and the
// partial triples of the plan being decoded, for callers that cannot allocate.
// Every device the library runs on holds its own copy until the process ends.
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

}  // namespace

int scratch_device_pointer(void** ptr) {
    // One address per device, looked up once with that device current.  In host
    // code `scratch` names a host-side stand-in, not device memory: only the
    // address returned by hipGetSymbolAddress may reach a kernel or a copy.
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return int(e);
    if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return int(e);
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return int(hipSuccess);
}

#ifdef KVATTN_TASK_TRACE
// Trace builds only: the device buffer that receives the records (NULL: off).
extern "C" int kvattn_trace_set(void* p) {
    return int(hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &p, sizeof(p)));
}
#endif

int launch_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, int grid,
                      int depth, int threads, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* pa = static_cast<const u32x4*>(a);
    const u32x4* pb = static_cast<const u32x4*>(b);
#define KV_PROBE(DD, TT)                                                                                           \
    if (depth == DD && threads == TT) {                                                                           \
        hipLaunchKernelGGL((read_probe_kernel<DD, TT>), dim3(grid), dim3(TT), 0, s, pa, a_bytes / 16, pb, b_bytes / 16, \
                           sink);                                                                                 \
        return int(hipGetLastError());                                                                            \
    }
    KV_PROBE(2, 256) KV_PROBE(4, 256) KV_PROBE(8, 256) KV_PROBE(2, 512) KV_PROBE(4, 512) KV_PROBE(8, 512)
    KV_PROBE(2, 1024) KV_PROBE(4, 1024) KV_PROBE(8, 1024)
#undef KV_PROBE
    return int(hipErrorInvalidValue);
}

int launch_forward(const DevPlan& p, const Dims& d, int valu_rows, int mfma_tiles, int n_tasks,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n_tasks <= 0) return 0;
#define KV_FWD(DD, RR, TP)                                           \
    if (d.head_dim == DD && valu_rows == RR && mfma_tiles == TP) \
        return launch_fwd_t<DD, RR, TP>(p, d, n_tasks, q, k, v, out, s);
    KV_FWD(128, 1, 1) KV_FWD(128, 2, 1) KV_FWD(128, 4, 1)
    KV_FWD(128, 1, 2) KV_FWD(128, 2, 2) KV_FWD(128, 4, 2)
    KV_FWD(64, 1, 1) KV_FWD(64, 2, 1) KV_FWD(64, 4, 1) KV_FWD(64, 8, 1)
    KV_FWD(64, 1, 2) KV_FWD(64, 2, 2) KV_FWD(64, 4, 2) KV_FWD(64, 8, 2)
#undef KV_FWD
    return int(hipErrorInvalidValue);
}

int launch_merge(const DevPlan& p, const Dims& d, int q_count, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (q_count <= 0) return 0;
    const unsigned ny = unsigned((d.num_q_heads * d.head_dim + 255) / 256);
    const NewTokens none{};
    if (d.head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<128, false>), dim3(q_count, ny), dim3(64), 0, s, p, d, none, out);
    else if (d.head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64, false>), dim3(q_count, ny), dim3(64), 0, s, p, d, none, out);
    else
        return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

int launch_merge_append(const DevPlan& p, const Dims& d, int q_count, const NewTokens& nt, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (q_count <= 0) return 0;
    const unsigned ny = unsigned((d.num_q_heads * d.head_dim + 255) / 256);
    if (d.head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<128, true>), dim3(q_count, ny), dim3(64), 0, s, p, d, nt, out);
    else if (d.head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64, true>), dim3(q_count, ny), dim3(64), 0, s, p, d, nt, out);
    else
        return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

}  // namespace kvattn
