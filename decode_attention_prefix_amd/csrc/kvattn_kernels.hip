// gfx950 (MI355X) kernels of the forward and merge stages.
//
// Forward (PAT review, forward stage: multi-tile kernels picked per work item,
// long KV split into chunks, several kernels kept busy at once to cut
// bubbles): one persistent launch whose workgroups pull tasks from per-XCD
// queues.  A task is one item (a run of paged KV blocks and the query rows
// attending to it) on one KV head (MFMA path) or four KV heads (VALU path); it
// yields either final output rows or partial triples (m, l, acc), m in log2
// units.
//   * VALU path -- at most 8 rows per KV head (a single query's GQA group, or a
//                  few queries of a small pack).  Bandwidth bound: q K^T with
//                  v_dot2_f32_bf16, p V with fp32 FMAs, 16-byte coalesced loads
//                  straight into registers, 8-lane DPP reductions.
//   * MFMA path -- packed groups (up to 128 rows per KV head): S^T = K Q^T and
//                  O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, K/V tiles staged
//                  in LDS by direct global->LDS DMA, three stages deep.
// Merge (PAT review, merge stage: online-softmax combination of the per-
// workgroup partial results of a query): one workgroup per query, all heads.
//
// Scores are kept in log2 units (q.k * scale * log2 e) so every exponential is
// a single v_exp_f32.  The running max is refreshed lazily: a row is rescaled
// only when a new score exceeds the reference by more than kRescaleLog2, so
// exponentials stay below 2^kRescaleLog2 and the result is unchanged.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvattn_internal.h"

namespace kvattn {
namespace {

constexpr float kRescaleLog2 = 8.0f;
constexpr float kNegSentinel = -1.0e30f;   // "no score yet"; finite so m - m stays 0

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate (gfx9 encoding) waiting until at most N vector-memory
// operations are outstanding; expcnt and lgkmcnt are left at their maximum.
template <int N>
constexpr int waitcnt_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 0xF) | ((N >> 4) << 14) | 0x0F70;
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
// VALU stream: a wave runs the VALU tasks of its workgroup's list for KV head
// (task head + wave) as one continuous stream of 16-token blocks.  Its
// three-deep register ring crosses task boundaries, so blocks of the next
// task are in flight while the current one finishes and nothing drains
// between tasks.  The list's descriptors sit in an LDS window; the q rows of a
// task are copied into one of four per-wave LDS slots by DMA when the load
// side enters the task, ahead of its first block.
// Lane = 8 * t + c: token slots t and t + 8 of each 16-token block, and the
// head-dim chunk set of c (elements [8c, 8c+8) and, for D = 128, [64+8c, 64+8c+8)),
// so every load instruction reads whole 128-byte rows of a block.
// ============================================================================
template <int D, int R>
__device__ __forceinline__ void valu_stream(const DevPlan& p, const Dims& dm, const int32_t* win, int n_words,
                                            uint16_t* qs, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                            float* __restrict__ out) {
    constexpr int NPC = D / 64;      // 16-byte pieces per token per lane
    constexpr int NE = 8 * NPC;      // elements per token per lane
    constexpr int NWD = NE / 2;      // bf16 pairs per token per lane
    constexpr int LPB = 2 * NPC * 2; // loads per block per lane (2 token slots, NPC pieces, K and V)
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
    // first task at or after `off` that has a KV head for this wave
    auto skip = [&](int off) {
        while (off < n_words && hdr(off, kDescHead) + wave >= Hkv) off += hdr(off, kDescWords);
        return off;
    };
    // copy the q rows of the task at `off` into slot `s` of this wave
    auto fetch_q = [&](int off, int s) {
        const int nrows = hdr(off, kDescRows);
        const int g = hdr(off, kDescHead) + wave;
#pragma unroll
        for (int c0 = 0; c0 < QCH; c0 += 64) {
            const int ch = c0 + lane;
            const int r = ch / (D / 8), pc = ch % (D / 8);
            if (ch < QCH && r < nrows) {
                const int query = win[off + kDescHeader + 4 * (r / G)];
                const uint16_t* src = q + (size_t(query) * Hq + g * G + r % G) * D + pc * 8;
                dma16(src, qs_lds + uint32_t((s * QSLOT + c0 * 8) * 2));
            }
        }
    };

    // ---- load side
    int l_off = skip(0);
    int l_blk = 0, l_slot = 0;
    int l_nblk = 0, l_ntok = 0, l_bids = 0, l_g = 0;
    auto l_enter = [&]() {
        if (l_off < n_words) {
            l_nblk = hdr(l_off, kDescBlocks);
            l_ntok = hdr(l_off, kDescTokens);
            l_bids = l_off + kDescHeader + 4 * hdr(l_off, kDescNq);
            l_g = hdr(l_off, kDescHead) + wave;
            fetch_q(l_off, l_slot);
        }
    };
    l_enter();
    int total = 0;   // blocks of this wave's stream
    for (int off = l_off; off < n_words; off = skip(off + hdr(off, kDescWords))) total += hdr(off, kDescBlocks);

    // Past the end of the stream the loads come from the zero page, so the ring
    // below needs no branches around its loads (the compiler keeps them in flight).
    auto load_block = [&](uint4 (&kb)[2][NPC], uint4 (&vb)[2][NPC]) {
        const bool live = l_off < n_words;
        const int blk = live ? __builtin_amdgcn_readfirstlane(win[l_bids + l_blk]) : 0;
        const uint16_t* kbase = kc + size_t(blk) * blk_elems + size_t(l_g) * head_elems;
        const uint16_t* vbase = vc + size_t(blk) * blk_elems + size_t(l_g) * head_elems;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int slot = t + 8 * tt;
            const bool ok = live && l_blk * 16 + slot < l_ntok;
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const int o = slot * D + pc * 64 + 8 * c;
                kb[tt][pc] = *reinterpret_cast<const uint4*>(ok ? kbase + o : p.zero);
                vb[tt][pc] = *reinterpret_cast<const uint4*>(ok ? vbase + o : p.zero);
            }
        }
        if (live && ++l_blk == l_nblk) {
            l_off = skip(l_off + hdr(l_off, kDescWords));
            l_blk = 0;
            l_slot = (l_slot + 1) & 3;
            l_enter();
        }
    };

    // ---- process side
    int p_off = skip(0);
    int p_blk = 0, p_slot = 0, p_nblk = 0;
    uint32_t qv[R][NWD];
    int limit[R];
    float m[R], l[R], acc[R][NE];

    auto begin_task = [&]() {
        // the q copy of this task is older than its first block's loads, which
        // are complete once at most two blocks' loads remain outstanding
        __builtin_amdgcn_s_waitcnt(waitcnt_vm<2 * LPB>());
        __builtin_amdgcn_sched_barrier(0);   // no LDS read of the slot moves above the wait
        p_nblk = hdr(p_off, kDescBlocks);
        const int nrows = hdr(p_off, kDescRows);
        const uint16_t* qsl = qs + p_slot * QSLOT;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nrows) {
#pragma unroll
                for (int pc = 0; pc < NPC; ++pc) {
                    const uint4 v = *reinterpret_cast<const uint4*>(qsl + r * D + pc * 64 + 8 * c);
                    qv[r][4 * pc + 0] = v.x;
                    qv[r][4 * pc + 1] = v.y;
                    qv[r][4 * pc + 2] = v.z;
                    qv[r][4 * pc + 3] = v.w;
                }
                limit[r] = win[p_off + kDescHeader + 4 * (r / G) + 2];
            } else {
#pragma unroll
                for (int w = 0; w < NWD; ++w) qv[r][w] = 0u;
                limit[r] = 0;
            }
            m[r] = kNegSentinel;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[r][e] = 0.f;
        }
    };

    auto process = [&](int k, const uint4 (&kb)[2][NPC], const uint4 (&vb)[2][NPC]) {
        float s[R][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float a = 0.f;
#pragma unroll
                for (int pc = 0; pc < NPC; ++pc) {
                    a = dot2_bf16(qv[r][4 * pc + 0], kb[tt][pc].x, a);
                    a = dot2_bf16(qv[r][4 * pc + 1], kb[tt][pc].y, a);
                    a = dot2_bf16(qv[r][4 * pc + 2], kb[tt][pc].z, a);
                    a = dot2_bf16(qv[r][4 * pc + 3], kb[tt][pc].w, a);
                }
                s[r][tt] = octet_sum(a);
            }
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

    // combine the 8 token lanes of each chunk set (lanes c, c+8, ..., c+56) and store
    auto end_task = [&]() {
        const int nrows = hdr(p_off, kDescRows);
        const int g = hdr(p_off, kDescHead) + wave;
        float ltot[R], mrow[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float M = m[r];
            M = fmaxf(M, __shfl_xor(M, 8));
            M = fmaxf(M, __shfl_xor(M, 16));
            M = fmaxf(M, __shfl_xor(M, 32));
            const float f = fast_exp2(m[r] - M);
            float lr = l[r] * f;
            lr += __shfl_xor(lr, 8);
            lr += __shfl_xor(lr, 16);
            lr += __shfl_xor(lr, 32);
            ltot[r] = lr;
            mrow[r] = M;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[r][e] *= f;
        }
        // reduce-scatter over t: after three halving exchanges each lane owns NE/8 elements
        const bool u32 = (lane & 32) != 0, u16 = (lane & 16) != 0, u8 = (lane & 8) != 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < NE / 2; ++i) {
                const float send = u32 ? acc[r][i] : acc[r][NE / 2 + i];
                const float keep = u32 ? acc[r][NE / 2 + i] : acc[r][i];
                acc[r][i] = keep + __shfl_xor(send, 32);
            }
#pragma unroll
            for (int i = 0; i < NE / 4; ++i) {
                const float send = u16 ? acc[r][i] : acc[r][NE / 4 + i];
                const float keep = u16 ? acc[r][NE / 4 + i] : acc[r][i];
                acc[r][i] = keep + __shfl_xor(send, 16);
            }
#pragma unroll
            for (int i = 0; i < NE / 8; ++i) {
                const float send = u8 ? acc[r][i] : acc[r][NE / 8 + i];
                const float keep = u8 ? acc[r][NE / 8 + i] : acc[r][i];
                acc[r][i] = keep + __shfl_xor(send, 8);
            }
        }
        const int ebase = (u32 ? NE / 2 : 0) + (u16 ? NE / 4 : 0) + (u8 ? NE / 8 : 0);
        // element e of chunk set c is head-dim index 8c + e (e < 8) or 64 + 8c + (e - 8)
        const int d0 = (ebase < 8) ? 8 * c + ebase : 64 + 8 * c + (ebase - 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nrows) continue;
            const int4 e = *reinterpret_cast<const int4*>(win + p_off + kDescHeader + 4 * (r / G));
            const int h = g * G + r % G;
            if (e.y < 0) {
                float* o = out + (size_t(e.x) * Hq + h) * D + d0;
                const float inv = 1.f / ltot[r];
                if constexpr (NE / 8 == 2) {
                    *reinterpret_cast<float2*>(o) = make_float2(acc[r][0] * inv, acc[r][1] * inv);
                } else {
                    o[0] = acc[r][0] * inv;
                }
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

    auto proc_block = [&](const uint4 (&kb)[2][NPC], const uint4 (&vb)[2][NPC]) {
        if (p_blk == 0) begin_task();
        process(p_blk, kb, vb);
        if (++p_blk == p_nblk) {
            end_task();
            p_off = skip(p_off + hdr(p_off, kDescWords));
            p_blk = 0;
            p_slot = (p_slot + 1) & 3;
        }
    };

    // three-deep register ring across the whole stream
    uint4 k0[2][NPC], v0[2][NPC], k1[2][NPC], v1[2][NPC], k2[2][NPC], v2[2][NPC];
    load_block(k0, v0);
    load_block(k1, v1);
    load_block(k2, v2);
    // scheduling barriers keep each refill after the compute that frees its registers,
    // so two blocks stay in flight and register pressure stays bounded
    for (int j = 0; j < total; j += 3) {
        proc_block(k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < total) proc_block(k1, v1);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k1, v1);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 2 < total) proc_block(k2, v2);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k2, v2);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ============================================================================
// MFMA task: the workgroup's 4 waves share one KV head's tiles; wave w owns
// rows [16 t w, 16 t (w + 1)) as t = 1 or 2 sixteen-row tiles.  Per 32-token tile:
//   S^T[16 tok x 16 rows] = K[16 x 32 d] . Q^T[32 d x 16 rows]   (4 k-steps at D = 128)
//   O^T[16 d x 16 rows]  += V^T[16 d x 32 tok] . P^T[32 tok x 16 rows]
// The head-dim index of O^T row m in output tile j is 8m + j (D = 128) or 4m + j
// (D = 64), so each lane reads 16 (8) contiguous bytes of a V row and an 8 x 8
// (8 x 4) register transpose yields the A operands of every output tile.
// P is split into bf16 hi + lo parts (two MFMAs) so the weights keep ~16 bits.
// K and V tiles live in LDS in rows of D/8 16-byte chunks, chunk index XOR
// (token mod D/8) to keep the 16 row-strided reads of an operand conflict free.
// ============================================================================
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

    // ---- loop-invariant DMA geometry: chunk u of this thread is token tok_u, row offset off_u
    const size_t head_elems = size_t(16) * D;
    const size_t blk_elems = size_t(Hkv) * head_elems;
    const uint16_t* kh = kc + size_t(g) * head_elems;
    const uint16_t* vh = vc + size_t(g) * head_elems;
    // chunk u of this thread is token tok0 + u * (NT / CPR): the same row offset in
    // every u, since NT / CPR is a multiple of 16 (or LPT is 1)
    static_assert(LPT == 1 || (NT / CPR) % 16 == 0, "DMA chunk stride");
    const int tok0 = tid / CPR;
    const int off0 = (tok0 & 15) * D + ((tid % CPR) ^ (tok0 & (CPR - 1))) * 8;
    const uint32_t lds_base = uint32_t(uintptr_t(s_kv));
    auto issue_tile = [&](int i) {
        const uint32_t st = lds_base + uint32_t((i % NS) * STAGE * 2);
        const int kb = 2 * i;
        const int blk0 = __builtin_amdgcn_readfirstlane(s_blk[kb]);
        const int blk1 = __builtin_amdgcn_readfirstlane(kb + 1 < nblk ? s_blk[kb + 1] : blk0);
        const size_t o0 = size_t(blk0) * blk_elems, o1 = size_t(blk1) * blk_elems;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            if (u * NT + wave * 64 >= TCH) continue;    // wave-uniform: waves past the tile issue nothing
            const int tok = tok0 + u * (NT / CPR);
            const bool ok = i * TT + tok < n_tok;
            const size_t o = (tok < 16 ? o0 : o1) + off0;
            const uint32_t dst = st + uint32_t((u * NT + wave * 64) * 16);
            dma16(ok ? static_cast<const void*>(kh + o) : static_cast<const void*>(p.zero), dst);
            dma16(ok ? static_cast<const void*>(vh + o) : static_cast<const void*>(p.zero), dst + TT * D * 2);
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

    // per-lane LDS element offsets of the K (A of QK) and V (to be transposed)
    // operands for token half 0; half 1 adds 16 rows (the XOR swizzle only sees
    // token mod 16, which both halves share)
    constexpr int HALF = 16 * CPR * 8;
    int koff[KS], voff[4];
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = (lr * CPR + ((4 * s + lg) ^ (lr & (CPR - 1)))) * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int tok = 4 * lg + u;
        if constexpr (D == 128)
            voff[u] = TT * D + (tok * CPR + (lr ^ (tok & (CPR - 1)))) * 8;
        else
            voff[u] = TT * D + (tok * CPR + ((lr >> 1) ^ (tok & (CPR - 1)))) * 8 + (lr & 1) * 4;
    }

    auto compute = [&](int i, const uint16_t* sb) {
        if (!active) return;
        // ---- S^T tiles (unscaled q.k)
        f32x4 sc[TPW][2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 kop[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) kop[s] = *reinterpret_cast<const bf16x8*>(sb + koff[s] + half * HALF);
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[s], qop[rt][s], a, 0, 0, 0);
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
            const float m4a = fmaxf(fmaxf(sc[rt][0][0], sc[rt][0][1]), fmaxf(sc[rt][0][2], sc[rt][0][3]));
            const float m4b = fmaxf(fmaxf(sc[rt][1][0], sc[rt][1][1]), fmaxf(sc[rt][1][2], sc[rt][1][3]));
            tmax[rt] = fmaxf(m4a, m4b) * sl2;
            need |= tmax[rt] > mref[rt] + kRescaleLog2;
        }
        if (__any(need)) {
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                float rm = tmax[rt];
                rm = fmaxf(rm, __shfl_xor(rm, 16));
                rm = fmaxf(rm, __shfl_xor(rm, 32));
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
                lo[x] = pack_bf16(pv[2 * x] - bf_lo(hi[x]), pv[2 * x + 1] - bf_hi(hi[x]));
            }
            phi[rt] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            plo[rt] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- V^T operands, built one output tile at a time from an 8 x 8 (8 x 4) register block
        constexpr int RAWW = D == 128 ? 4 : 2;   // dwords per lane per token
        uint32_t raw[8][RAWW];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint16_t* src = sb + voff[u & 3] + (u >> 2) * HALF;
            if constexpr (D == 128) {
                const uint4 r4 = *reinterpret_cast<const uint4*>(src);
                raw[u][0] = r4.x; raw[u][1] = r4.y; raw[u][2] = r4.z; raw[u][3] = r4.w;
            } else {
                const uint2 r2 = *reinterpret_cast<const uint2*>(src);
                raw[u][0] = r2.x; raw[u][1] = r2.y;
            }
        }
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                w[x] = __builtin_amdgcn_perm(raw[2 * x + 1][j >> 1], raw[2 * x][j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
            const bf16x8 vt = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
            for (int rt = 0; rt < TPW; ++rt) {
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, phi[rt], acc[rt][j], 0, 0, 0);
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, plo[rt], acc[rt][j], 0, 0, 0);
            }
        }
    };

    // ---- NS-stage pipeline: tiles i+1 .. i+NS-1 stream in while tile i is computed ----
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < ntiles) issue_tile(i);
    for (int i = 0; i < ntiles; ++i) {
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
        if (i + NS - 1 < ntiles) issue_tile(i + NS - 1);
        compute(i, s_kv + (i % NS) * STAGE);
    }

    // ---- epilogue: lane holds row lr of each tile, head dims of output tile j, row m = 4lg + e
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
        if (!active) continue;
        float lt = lsum[rt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int r = row0 + rt * 16 + lr;
        if (r >= it.n_rows) continue;
        const Entry e = entry_of(it, r / G);
        const int h = g * G + r % G;
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
        if constexpr (D == 128) {
            // d = 8 * (4lg + e) + j = 32lg + 8e + j
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                float4 a = make_float4(acc[rt][0][e4] * scale, acc[rt][1][e4] * scale, acc[rt][2][e4] * scale,
                                       acc[rt][3][e4] * scale);
                float4 b = make_float4(acc[rt][4][e4] * scale, acc[rt][5][e4] * scale, acc[rt][6][e4] * scale,
                                       acc[rt][7][e4] * scale);
                *reinterpret_cast<float4*>(dst + 32 * lg + 8 * e4) = a;
                *reinterpret_cast<float4*>(dst + 32 * lg + 8 * e4 + 4) = b;
            }
        } else {
            // d = 4 * (4lg + e) + j = 16lg + 4e + j
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                float4 a = make_float4(acc[rt][0][e4] * scale, acc[rt][1][e4] * scale, acc[rt][2][e4] * scale,
                                       acc[rt][3][e4] * scale);
                *reinterpret_cast<float4*>(dst + 16 * lg + 4 * e4) = a;
            }
        }
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
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    // All control flow below is wave-uniform: the loops hold barriers, so
    // lane-divergent branches must stay out of their exits and back edges.
    for (int w = blockIdx.x; w < p.n_lists; w += gridDim.x) {
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
                mfma_task<D, TPW>(p, dm, it, it.head, q, kc, vc, out, s_kv);
                wait_all_and_sync();   // the prefetched descriptor landed; this task's LDS is free
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
            uint16_t* qs = s_kv + 2 * WIN + wave * 4 * R * D;
            valu_stream<D, R>(p, dm, win, e0 - v0, qs, q, kc, vc, out);
            wait_all_and_sync();   // the window is free for the next list
        }
    }
}

// ============================================================================
// Merge: one workgroup per query with several partial triples, all q heads at
// once.  The slots of one item entry are consecutive (slot = dest + h), so each
// partial's accumulators for every head form one contiguous [Hq][D] block.
//   M_h = max_i m_ih, w_ih = 2^(m_ih - M_h) / sum_i 2^(m_ih - M_h) l_ih,
//   out[h] = sum_i w_ih acc_ih
// ============================================================================
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DevPlan p, Dims dm, float* __restrict__ out) {
    constexpr int COLS = 1024;              // floats of [Hq][D] per workgroup (blockIdx.y selects the block)
    constexpr int HB = COLS / D;            // heads per workgroup
    constexpr int MAXW = 4096;              // weights staged per batch of partials
    __shared__ float s_m[HB];
    __shared__ float s_inv[HB];
    __shared__ float s_w[MAXW];
    const int Hq = dm.num_q_heads;
    const int h_lo = int(blockIdx.y) * HB;
    const int nh = min(HB, Hq - h_lo);
    const int mq = blockIdx.x;
    const KV_CONST int32_t* mptr = cptr(p.merge_ptr);
    const KV_CONST int32_t* mdst = cptr(p.merge_dest);
    const int b = cptr(p.merge_query)[mq];
    const int i0 = mptr[mq], i1 = mptr[mq + 1];
    const int tid = threadIdx.x;
    // per head: M = max m_i, 1 / sum_i 2^(m_i - M) l_i  (one wave per head)
    for (int hh = tid >> 6; hh < nh; hh += 4) {
        const int h = h_lo + hh;
        float M = -INFINITY;
        for (int i = i0 + (tid & 63); i < i1; i += 64) M = fmaxf(M, p.part_ml[(size_t(mdst[i]) + h) * 2]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        float L = 0.f;
        for (int i = i0 + (tid & 63); i < i1; i += 64) {
            const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + (size_t(mdst[i]) + h) * 2);
            L += fast_exp2(ml.x - M) * ml.y;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
        if ((tid & 63) == 0) {
            s_m[hh] = M;
            s_inv[hh] = 1.f / L;
        }
    }
    const int n4 = nh * D / 4;              // float4 of this workgroup's block (<= 256)
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int per = MAXW / nh;
    const int hq = (4 * tid) / D;           // head of this thread's float4
    for (int ib = i0; ib < i1; ib += per) {
        const int nb = min(per, i1 - ib);
        __syncthreads();
        for (int x = tid; x < nb * nh; x += 256) {
            const int i = x / nh, hh = x % nh;
            const float m = p.part_ml[(size_t(mdst[ib + i]) + h_lo + hh) * 2];
            s_w[x] = fast_exp2(m - s_m[hh]) * s_inv[hh];
        }
        __syncthreads();
        if (tid < n4) {
            int i = 0;
            for (; i + 4 <= nb; i += 4) {
                float4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v[u] = reinterpret_cast<const float4*>(p.part_acc + (size_t(mdst[ib + i + u]) + h_lo) * D)[tid];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float w = s_w[(i + u) * nh + hq];
                    acc.x = fmaf(w, v[u].x, acc.x);
                    acc.y = fmaf(w, v[u].y, acc.y);
                    acc.z = fmaf(w, v[u].z, acc.z);
                    acc.w = fmaf(w, v[u].w, acc.w);
                }
            }
            for (; i < nb; ++i) {
                const float4 v = reinterpret_cast<const float4*>(p.part_acc + (size_t(mdst[ib + i]) + h_lo) * D)[tid];
                const float w = s_w[i * nh + hq];
                acc.x = fmaf(w, v.x, acc.x);
                acc.y = fmaf(w, v.y, acc.y);
                acc.z = fmaf(w, v.z, acc.z);
                acc.w = fmaf(w, v.w, acc.w);
            }
        }
    }
    if (tid < n4) reinterpret_cast<float4*>(out + (size_t(b) * Hq + h_lo) * D)[tid] = acc;
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
    // one workgroup per static list when they all fit at once; otherwise
    // workgroup w also runs lists w + grid, w + 2 grid, ...
    const int grid = persistent_grid(fwd_kernel<D, R, TPW>, &slots, p.n_lists);
    if (grid < 0) return int(hipErrorInvalidDevice);
    hipLaunchKernelGGL((fwd_kernel<D, R, TPW>), dim3(grid), dim3(256), 0, s, p, d, q, k, v, out);
    return int(hipGetLastError());
}

}  // namespace

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
    if (d.head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<128>), dim3(q_count, (d.num_q_heads + 7) / 8), dim3(256), 0, s, p, d, out);
    else if (d.head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64>), dim3(q_count, (d.num_q_heads + 15) / 16), dim3(256), 0, s, p, d, out);
    else
        return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

}  // namespace kvattn
