// gfx950 (MI355X) kernels of the forward and merge stages.
//
// Forward (PAT review, forward stage: multi-tile kernels picked per work item,
// long KV split into chunks): each work item reads one run of paged KV blocks
// for one KV head and attends the item's query rows over it, producing either
// the final output row or a partial triple (m, l, acc) with m in log2 units.
//   * fwd_valu  -- at most 8 rows per KV head (a single query's GQA group, or a
//                  few queries of a small pack).  Bandwidth bound: q K^T with
//                  v_dot2_f32_bf16, p V with fp32 FMAs, 16-byte coalesced loads
//                  straight into registers, 8-lane DPP reductions, online softmax.
//   * fwd_mfma  -- packed groups (up to 256 rows per KV head): S^T = K Q^T and
//                  O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, K/V tiles staged
//                  in LDS by direct global->LDS DMA, three stages deep.
// Merge (PAT review, merge stage: online-softmax combination of the per-
// workgroup partial results of a query): fwd rows with several partials.
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

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// ============================================================================
// VALU forward: one wave per (item, KV head); a workgroup holds 4 KV heads.
// Lane = 8 * t + c: token slots t and t + 8 of each 16-token block, and the
// head-dim chunk set of c (elements [8c, 8c+8) and, for D = 128, [64+8c, 64+8c+8)),
// so every load instruction reads whole 128-byte rows of a block.
// ============================================================================
template <int D, int R>
__global__ __launch_bounds__(256) void fwd_valu_kernel(DevPlan p, Dims dm, int item_begin,
                                                       const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kc,
                                                       const uint16_t* __restrict__ vc, float* __restrict__ out) {
    constexpr int NPC = D / 64;      // 16-byte pieces per token per lane
    constexpr int NE = 8 * NPC;      // elements per token per lane
    constexpr int NWD = NE / 2;      // bf16 pairs per token per lane
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Hkv = dm.num_kv_heads;
    const int n_hg = (Hkv + 3) >> 2;
    const int item_id = item_begin + int(blockIdx.x) / n_hg;
    const int g = (int(blockIdx.x) % n_hg) * 4 + wave;
    if (g >= Hkv) return;
    const Item it = p.items[item_id];
    const int G = dm.group;
    const int t = lane >> 3, c = lane & 7;

    uint32_t qv[R][NWD];
    int limit[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < it.n_rows) {
            const Entry e = p.entries[it.q_begin + r / G];
            const int h = g * G + r % G;
            const uint16_t* qrow = q + (size_t(e.query) * dm.num_q_heads + h) * D;
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const uint4 v = *reinterpret_cast<const uint4*>(qrow + pc * 64 + 8 * c);
                qv[r][4 * pc + 0] = v.x;
                qv[r][4 * pc + 1] = v.y;
                qv[r][4 * pc + 2] = v.z;
                qv[r][4 * pc + 3] = v.w;
            }
            limit[r] = e.limit;
        } else {
#pragma unroll
            for (int w = 0; w < NWD; ++w) qv[r][w] = 0u;
            limit[r] = 0;
        }
    }

    float m[R], l[R], acc[R][NE];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = kNegSentinel;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[r][e] = 0.f;
    }

    const int n_tok = it.n_tokens;
    const int nblk = (n_tok + 15) >> 4;
    const size_t head_elems = size_t(16) * D;
    const size_t blk_elems = size_t(Hkv) * head_elems;
    const int32_t* __restrict__ bids = p.block_ids + it.blk_begin;
    const float sl2 = dm.scale_log2;

    auto load_block = [&](int k, uint4 (&kb)[2][NPC], uint4 (&vb)[2][NPC]) {
        const int blk = bids[k];
        const uint16_t* kbase = kc + size_t(blk) * blk_elems + size_t(g) * head_elems;
        const uint16_t* vbase = vc + size_t(blk) * blk_elems + size_t(g) * head_elems;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int slot = t + 8 * tt;
            const bool ok = k * 16 + slot < n_tok;
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const int off = slot * D + pc * 64 + 8 * c;
                kb[tt][pc] = *reinterpret_cast<const uint4*>(ok ? kbase + off : p.zero);
                vb[tt][pc] = *reinterpret_cast<const uint4*>(ok ? vbase + off : p.zero);
            }
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

    // three-deep register ring: blocks k+1 and k+2 are in flight while k is processed
    uint4 k0[2][NPC], v0[2][NPC], k1[2][NPC], v1[2][NPC], k2[2][NPC], v2[2][NPC];
    load_block(0, k0, v0);
    if (nblk > 1) load_block(1, k1, v1);
    if (nblk > 2) load_block(2, k2, v2);
    for (int k = 0; k < nblk; k += 3) {
        process(k, k0, v0);
        if (k + 3 < nblk) load_block(k + 3, k0, v0);
        if (k + 1 < nblk) {
            process(k + 1, k1, v1);
            if (k + 4 < nblk) load_block(k + 4, k1, v1);
        }
        if (k + 2 < nblk) {
            process(k + 2, k2, v2);
            if (k + 5 < nblk) load_block(k + 5, k2, v2);
        }
    }

    // ---- combine the 8 token lanes of each chunk set (lanes c, c+8, ..., c+56) ----
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
        if (r >= it.n_rows) break;
        const Entry e = p.entries[it.q_begin + r / G];
        const int h = g * G + r % G;
        if (e.dest < 0) {
            float* o = out + (size_t(e.query) * dm.num_q_heads + h) * D + d0;
            const float inv = 1.f / ltot[r];
            if constexpr (NE / 8 == 2) {
                *reinterpret_cast<float2*>(o) = make_float2(acc[r][0] * inv, acc[r][1] * inv);
            } else {
                o[0] = acc[r][0] * inv;
            }
        } else {
            const size_t slot = size_t(e.dest) + h;
            float* o = p.part_acc + slot * D + d0;
            if constexpr (NE / 8 == 2) {
                *reinterpret_cast<float2*>(o) = make_float2(acc[r][0], acc[r][1]);
            } else {
                o[0] = acc[r][0];
            }
            if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(mrow[r], ltot[r]);
        }
    }
}

// ============================================================================
// MFMA forward: one workgroup of NW waves per (item, KV head); wave w owns rows
// [32w, 32w + 32) as two 16-row tiles.  Per 32-token tile:
//   S^T[16 tok x 16 rows] = K[16 x 32 d] . Q^T[32 d x 16 rows]   (4 k-steps at D = 128)
//   O^T[16 d x 16 rows]  += V^T[16 d x 32 tok] . P^T[32 tok x 16 rows]
// The head-dim index of O^T row m in output tile j is 8m + j (D = 128) or 4m + j
// (D = 64), so each lane reads 16 (8) contiguous bytes of a V row and an 8 x 8
// (8 x 4) register transpose yields the A operands of every output tile.
// P is split into bf16 hi + lo parts (two MFMAs) so the weights keep ~16 bits.
// K and V tiles live in LDS in rows of D/8 16-byte chunks, chunk index XOR
// (token mod D/8) to keep the 16 row-strided reads of an operand conflict free.
// ============================================================================
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_mfma_kernel(DevPlan p, Dims dm, int item_begin,
                                                           const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ kc,
                                                           const uint16_t* __restrict__ vc,
                                                           float* __restrict__ out) {
    constexpr int TT = kMfmaTileTokens;    // 32 tokens per stage
    constexpr int CPR = D / 8;             // 16-byte chunks per token row
    constexpr int TCH = TT * CPR;          // chunks per K (or V) tile
    constexpr int KS = D / 32;             // QK k-steps
    constexpr int NDT = D / 16;            // output tiles
    constexpr int NT = 64 * NW;            // threads
    constexpr int LPT = TCH >= NT ? TCH / NT : 1;   // DMA chunks per thread per tensor and tile
    constexpr int MAXBLK = kMaxItemBlocks;
    static_assert(TCH % NT == 0 || NT % TCH == 0, "tile chunks must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) uint16_t s_k0[TT * D], s_k1[TT * D], s_k2[TT * D];
    __shared__ __attribute__((aligned(16))) uint16_t s_v0[TT * D], s_v1[TT * D], s_v2[TT * D];
    __shared__ int32_t s_blk[MAXBLK];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int Hkv = dm.num_kv_heads;
    const int item_id = item_begin + int(blockIdx.x) / Hkv;
    const int g = int(blockIdx.x) % Hkv;
    const Item it = p.items[item_id];
    const int G = dm.group;
    const int n_tok = it.n_tokens;
    const int nblk = (n_tok + 15) >> 4;
    const int ntiles = (n_tok + TT - 1) / TT;

    for (int i = tid; i < nblk; i += NT) s_blk[i] = p.block_ids[it.blk_begin + i];

    // ---- Q operands (B of S^T = K Q^T): lane -> row lr of the tile, d = 32s + 8lg .. +7
    bf16x8 qop[2][KS];
    int lim[2];
    int nrt = 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = wave * 32 + rt * 16 + lr;
        if (r < it.n_rows) {
            const Entry e = p.entries[it.q_begin + r / G];
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
        if (wave * 32 + rt * 16 < it.n_rows) nrt = rt + 1;
    }
    __syncthreads();   // s_blk ready; all scalar and vector setup loads done

    const size_t head_elems = size_t(16) * D;
    const size_t blk_elems = size_t(Hkv) * head_elems;
    const size_t goff = size_t(g) * head_elems;

    auto issue_tile = [&](int i, uint16_t* sk, uint16_t* sv) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            if (u * NT + wave * 64 >= TCH) break;       // wave-uniform: waves past the tile issue nothing
            const int pos = u * NT + tid;               // physical chunk in the tile
            const int tok = pos / CPR, pc = pos % CPR;
            const int lc = pc ^ (tok & (CPR - 1));       // logical chunk held at pos
            const int gt = i * TT + tok;
            const uint16_t* ks = p.zero;
            const uint16_t* vs = p.zero;
            if (gt < n_tok) {
                const size_t off = size_t(s_blk[gt >> 4]) * blk_elems + goff + size_t(gt & 15) * D + lc * 8;
                ks = kc + off;
                vs = vc + off;
            }
            __builtin_amdgcn_global_load_lds(ks, (__attribute__((address_space(3))) void*)(sk + (u * NT + wave * 64) * 8),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vs, (__attribute__((address_space(3))) void*)(sv + (u * NT + wave * 64) * 8),
                                             16, 0, 0);
        }
    };

    float mref[2] = {kNegSentinel, kNegSentinel};
    float lsum[2] = {0.f, 0.f};
    f32x4 acc[2][NDT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < NDT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float sl2 = dm.scale_log2;

    auto compute = [&](int i, const uint16_t* sk, const uint16_t* sv) {
        if (nrt == 0) return;
        // K operands: token 16*half + lr, logical chunk 4s + lg
        bf16x8 kop[2][KS];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int tok = 16 * half + lr;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int pc = (4 * s + lg) ^ (tok & (CPR - 1));
                kop[half][s] = *reinterpret_cast<const bf16x8*>(sk + (tok * CPR + pc) * 8);
            }
        }
        f32x4 sc[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (rt >= nrt) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[half][s], qop[rt][s], a, 0, 0, 0);
                sc[rt][half] = a;
            }
        }
        // scale, mask, lazy max
        bool need = false;
        float tmax[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            tmax[rt] = -INFINITY;
            if (rt >= nrt) break;
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = i * TT + 16 * half + 4 * lg + e;
                    const float v = tok < lim[rt] ? sc[rt][half][e] * sl2 : -INFINITY;
                    sc[rt][half][e] = v;
                    tmax[rt] = fmaxf(tmax[rt], v);
                }
            need |= tmax[rt] > mref[rt] + kRescaleLog2;
        }
        if (__any(need)) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if (rt >= nrt) break;
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
        // V^T operands: tokens tau(lg, u) = 4lg + u (u < 4) or 16 + 4lg + (u - 4)
        bf16x8 vt[8];
        if constexpr (D == 128) {
            uint4 raw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int tok = (u < 4) ? 4 * lg + u : 16 + 4 * lg + (u - 4);
                const int pc = lr ^ (tok & (CPR - 1));
                raw[u] = *reinterpret_cast<const uint4*>(sv + (tok * CPR + pc) * 8);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t w[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t a = (&raw[2 * x].x)[j >> 1], b = (&raw[2 * x + 1].x)[j >> 1];
                    w[x] = __builtin_amdgcn_perm(b, a, (j & 1) ? 0x07060302u : 0x05040100u);
                }
                vt[j] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
        } else {
            uint2 raw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int tok = (u < 4) ? 4 * lg + u : 16 + 4 * lg + (u - 4);
                const int pc = (lr >> 1) ^ (tok & (CPR - 1));
                raw[u] = *reinterpret_cast<const uint2*>(sv + (tok * CPR + pc) * 8 + (lr & 1) * 4);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t w[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t a = (&raw[2 * x].x)[j >> 1], b = (&raw[2 * x + 1].x)[j >> 1];
                    w[x] = __builtin_amdgcn_perm(b, a, (j & 1) ? 0x07060302u : 0x05040100u);
                }
                vt[j] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (rt >= nrt) break;
            float pv[8];
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = fast_exp2(sc[rt][0][e] - mref[rt]);
                pv[4 + e] = fast_exp2(sc[rt][1][e] - mref[rt]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ps += pv[e];
            lsum[rt] += ps;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                hi[x] = pack_bf16(pv[2 * x], pv[2 * x + 1]);
                lo[x] = pack_bf16(pv[2 * x] - bf_lo(hi[x]), pv[2 * x + 1] - bf_hi(hi[x]));
            }
            const bf16x8 phi = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            const bf16x8 plo = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
            for (int j = 0; j < NDT; ++j) {
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[j], phi, acc[rt][j], 0, 0, 0);
                acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[j], plo, acc[rt][j], 0, 0, 0);
            }
        }
    };

    // ---- three-stage pipeline: tiles i+1 and i+2 stream in while i is computed ----
    issue_tile(0, s_k0, s_v0);
    if (ntiles > 1) issue_tile(1, s_k1, s_v1);
    for (int i = 0; i < ntiles; ++i) {
        // this thread's DMA for tile i is complete once at most the 2*LPT loads of
        // tile i+1 remain outstanding
        if (i + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm<2 * LPT>());
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
        }
        __builtin_amdgcn_s_barrier();   // every wave's DMA for tile i landed; tile i-1 is consumed
        const int st = i % 3;
        if (i + 2 < ntiles) {
            const int sn = (i + 2) % 3;
            issue_tile(i + 2, sn == 0 ? s_k0 : (sn == 1 ? s_k1 : s_k2), sn == 0 ? s_v0 : (sn == 1 ? s_v1 : s_v2));
        }
        compute(i, st == 0 ? s_k0 : (st == 1 ? s_k1 : s_k2), st == 0 ? s_v0 : (st == 1 ? s_v1 : s_v2));
    }

    // ---- epilogue: lane holds row lr of each tile, head dims of output tile j, row m = 4lg + e
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        if (rt >= nrt) break;
        float lt = lsum[rt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int r = wave * 32 + rt * 16 + lr;
        if (r >= it.n_rows) continue;
        const Entry e = p.entries[it.q_begin + r / G];
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
// Merge: one wave per (query, q head) with >= 2 partial triples.
//   M = max_i m_i, w_i = 2^(m_i - M), out = sum_i w_i acc_i / sum_i w_i l_i
// ============================================================================
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DevPlan p, Dims dm, int q_begin, int q_count,
                                                    float* __restrict__ out) {
    constexpr int PER = D / 64;
    const int Hq = dm.num_q_heads;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = int(blockIdx.x) * 4 + wave;
    if (row >= q_count * Hq) return;
    const int mq = q_begin + row / Hq;
    const int h = row % Hq;
    const int b = p.merge_query[mq];
    const int i0 = p.merge_ptr[mq], i1 = p.merge_ptr[mq + 1];
    float M = -INFINITY;
    for (int i = i0; i < i1; ++i) M = fmaxf(M, p.part_ml[(size_t(p.merge_dest[i]) + h) * 2]);
    float L = 0.f;
    float a[PER];
#pragma unroll
    for (int x = 0; x < PER; ++x) a[x] = 0.f;
    for (int i = i0; i < i1; ++i) {
        const size_t slot = size_t(p.merge_dest[i]) + h;
        const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + slot * 2);
        const float w = fast_exp2(ml.x - M);
        L += w * ml.y;
        const float* src = p.part_acc + slot * D + lane * PER;
        if constexpr (PER == 2) {
            const float2 v = *reinterpret_cast<const float2*>(src);
            a[0] = fmaf(w, v.x, a[0]);
            a[1] = fmaf(w, v.y, a[1]);
        } else {
            a[0] = fmaf(w, src[0], a[0]);
        }
    }
    const float inv = 1.f / L;
    float* o = out + (size_t(b) * Hq + h) * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<float2*>(o) = make_float2(a[0] * inv, a[1] * inv);
    } else {
        o[0] = a[0] * inv;
    }
}

template <int D, int R>
int launch_valu_t(const DevPlan& p, const Dims& d, int item_begin, int item_count, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, float* out, hipStream_t s) {
    const int n_hg = (d.num_kv_heads + 3) / 4;
    hipLaunchKernelGGL((fwd_valu_kernel<D, R>), dim3(item_count * n_hg), dim3(256), 0, s, p, d, item_begin, q, k, v,
                       out);
    return int(hipGetLastError());
}

template <int D, int NW>
int launch_mfma_t(const DevPlan& p, const Dims& d, int item_begin, int item_count, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, float* out, hipStream_t s) {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW>), dim3(item_count * d.num_kv_heads), dim3(64 * NW), 0, s, p, d,
                       item_begin, q, k, v, out);
    return int(hipGetLastError());
}

}  // namespace

int launch_forward_valu(const DevPlan& p, const Dims& d, int rows, int item_begin, int item_count,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (item_count <= 0) return 0;
#define KV_VALU(DD, RR) \
    if (d.head_dim == DD && rows == RR) return launch_valu_t<DD, RR>(p, d, item_begin, item_count, q, k, v, out, s);
    KV_VALU(128, 1) KV_VALU(128, 2) KV_VALU(128, 4) KV_VALU(128, 8)
    KV_VALU(64, 1) KV_VALU(64, 2) KV_VALU(64, 4) KV_VALU(64, 8)
#undef KV_VALU
    return int(hipErrorInvalidValue);
}

int launch_forward_mfma(const DevPlan& p, const Dims& d, int waves, int item_begin, int item_count,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (item_count <= 0) return 0;
#define KV_MFMA(DD, WW) \
    if (d.head_dim == DD && waves == WW) return launch_mfma_t<DD, WW>(p, d, item_begin, item_count, q, k, v, out, s);
    KV_MFMA(128, 1) KV_MFMA(128, 2) KV_MFMA(128, 4) KV_MFMA(128, 8)
    KV_MFMA(64, 1) KV_MFMA(64, 2) KV_MFMA(64, 4) KV_MFMA(64, 8)
#undef KV_MFMA
    return int(hipErrorInvalidValue);
}

int launch_merge(const DevPlan& p, const Dims& d, int q_begin, int q_count, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (q_count <= 0) return 0;
    const int rows = q_count * d.num_q_heads;
    const dim3 grid((rows + 3) / 4);
    if (d.head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(256), 0, s, p, d, q_begin, q_count, out);
    else if (d.head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(256), 0, s, p, d, q_begin, q_count, out);
    else
        return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

}  // namespace kvattn
