// Device pieces shared by the chain step kernels: the running-argmax words,
// the previous token, the top-k bound, the staging swizzle and the top-k
// insert of one scored tile.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

// Target id of chain column c: the column itself, or d2t[c] for a reduced
// draft vocabulary (llama.cpp PR #26275, rework commit message: d2t holds
// absolute target ids and the draft logits are scattered at run time).
__device__ __forceinline__ long column_token(const int64_t* d2t, int c) {
    return d2t ? (long)d2t[c] : (long)c;
}

// The running argmax words (kernels.hpp, kWinnerWays): the word workgroup g
// raises for block b of slot j, and the argmax key of that block and slot.
__device__ __forceinline__ u64* winner_word(u64* winners, int wstride, int j, int g, int b) {
    return winners + ((long)j * kWinnerWays + g % kWinnerWays) * wstride + b;
}
__device__ __forceinline__ u64 winner_key(const u64* winners, int wstride, int j, int b) {
    const u64* w = winners + (long)j * kWinnerWays * wstride + b;
    u64 k[kWinnerWays];
#pragma unroll
    for (int i = 0; i < kWinnerWays; ++i) k[i] = w[(long)i * wstride];   // loads issued together
    u64 m = k[0];
#pragma unroll
    for (int i = 1; i < kWinnerWays; ++i) m = k[i] > m ? k[i] : m;
    return m;
}

// The previous token of block b for slot j: the anchor, or the target id of
// the previous slot's argmax column. A value outside [0, vocab) is replaced
// by 0 and reported (when `report`) in the flags word.
__device__ __forceinline__ int prev_token(const ChainArgs& a, int j, int b, bool report) {
    long t;
    uint32_t bad;
    if (j == 0) {
        t = a.anchors[b];
        bad = kFlagBadAnchor;
    } else {
        const int c = key_id(winner_key(a.winners, a.wstride, j - 1, b));
        t = (c >= 0 && c < a.V) ? column_token(a.d2t, c) : -1;
        bad = kFlagBadD2t;
    }
    if (t >= 0 && t < a.vocab) return (int)t;
    if (report) atomicOr(a.flags, bad);
    return 0;
}

// The previous tokens of a group of 32 blocks through LDS. A step kernel
// copies the words they come from (slot j > 0: the previous slot's
// kWinnerWays running-argmax words of blocks gbase .. gbase + 31, 2 KB;
// slot 0: the anchors) direct to LDS ahead of the tile copies, which do not
// depend on them; waits for them with an explicit count (loads complete in
// issue order, so the tiles stay in flight); and reads them back. A register
// load among the copies would instead be waited for with every copy in
// flight. kPrevChunks 16-byte chunks hold one group's copy. The caller
// copies only for a group that holds a block (gbase < B): its 32 words of a
// way then lie inside the way's row (winners_stride rounds B up to 32).
constexpr int kPrevChunks = 128;

__device__ __forceinline__ void copy_prev(const ChainArgs& a, int j, int gbase, lds_char* dst) {
    const int lane = threadIdx.x & 63;
    if (j == 0) {
        // lane l's anchor to byte 4 l: lanes 0-31 hold blocks gbase + l
        const int b = min(gbase + (lane & 31), a.B - 1);
        __builtin_amdgcn_global_load_lds((const void*)(a.anchors + b), (lds_ptr)dst, 4, 0, 0);
    } else {
        // chunk 64 i + l: way 4 i + l / 16, blocks gbase + 2 (l % 16) and the next
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int way = 4 * i + (lane >> 4);
            const unsigned long long* w =
                a.winners + ((long)(j - 1) * kWinnerWays + way) * a.wstride + gbase + 2 * (lane & 15);
            __builtin_amdgcn_global_load_lds((const void*)w, (lds_ptr)(dst + i * 64 * 16), 16, 0, 0);
        }
    }
}

// The previous token of block gbase + k from copy_prev's copy at src (after
// the wait for it), as prev_token gives it.
__device__ __forceinline__ int prev_from_copy(const ChainArgs& a, int j, const void* src, int k, bool report) {
    typedef const __attribute__((address_space(3))) int32_t lds_i32;
    typedef const __attribute__((address_space(3))) unsigned long long lds_u64;
    long t;
    uint32_t bad;
    if (j == 0) {
        t = ((lds_i32*)src)[k];
        bad = kFlagBadAnchor;
    } else {
        lds_u64* w = (lds_u64*)src;
        unsigned long long m = w[k];
#pragma unroll
        for (int i = 1; i < kWinnerWays; ++i) {
            const unsigned long long x = w[i * 32 + k];
            m = x > m ? x : m;
        }
        const int c = key_id(m);
        if (c < 0 || c >= a.V) {
            t = -1;
        } else if (a.d2t == nullptr) {
            t = c;
        } else {
            // A register load among the copies: this path waits for every
            // load in flight here, so that the paths without one do not
            // inherit the wait where they join.
            t = a.d2t[c];
            wait_vmcnt<0>();
        }
        bad = kFlagBadD2t;
    }
    if (t >= 0 && t < a.vocab) return (int)t;
    if (report) atomicOr(a.flags, bad);
    return 0;
}

// Adaptive gate: block b was cut before slot j (its confidence fell below its
// threshold at a slot < j + 1), so slot j is not drafted for it. The chain
// then streams no logits row for it, inserts and publishes nothing for it,
// and reads no previous token for it (it published none).
__device__ __forceinline__ bool block_cut(const ChainArgs& a, int b, int j) {
    return a.stop != nullptr && a.lengths[b] <= j;
}

// Lower bound on the KL-th best biased score of one slot of one block, from
// which its top-k filter starts. The row's KL largest slab maxima are the
// projections of KL distinct columns (the slabs are disjoint), and the
// Markov term of any column is at most |markov_w2[v]| |u| in magnitude
// (Cauchy-Schwarz, u = markov_w1[prev]), so those KL columns score at least
// kth - |w2|max |u|. The scores are fp32 sums of r + 1 terms, within
// (r + 1) 2^-24 (|z| + |bias|) of exact (r <= 256: below 2e-5 relative), and
// the norms carry a few ulps: the margins below cover both. -inf without a
// k-th slab.
__device__ __forceinline__ float chain_bound(float kth, float w2n2, float un2) {
    const float mk = sqrtf(w2n2) * sqrtf(un2);
    return kth - mk * 1.001f - 1e-4f * (1.0f + fabsf(kth));
}

// Squared norm of this lane's block's markov_w1 row from its MFMA B-operand
// share (rank chunks 16 s + 8 (lane / 32) .. + 8) and its partner lane's.
template <int RS>
__device__ __forceinline__ float w1_norm2(const u32x4 (&u)[RS > 0 ? RS : 1]) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < RS; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = bf16_lo(u[i][q]), hi = bf16_hi(u[i][q]);
            s += lo * lo;
            s += hi * hi;
        }
    return s + __shfl_xor(s, 32, kWave);
}

// Swizzle of a staged row of R 16-byte chunks: chunk c of row `row` is stored
// at c ^ swz_rows<R>(row). MFMA operand reads take one chunk of 32
// consecutive rows; the permutation spreads any 8 (32-bank view) or 16
// (64-bank view) consecutive rows over distinct banks.
template <int R>
__device__ __forceinline__ int swz_rows(int row) {
    if constexpr (R >= 16) return row & 15;
    else if constexpr (R == 8) return (row ^ (row >> 3)) & 7;
    else if constexpr (R == 4) return (((row >> 1) ^ (row >> 3)) & 1) | (((row >> 2) & 1) << 1);
    else if constexpr (R == 2) return ((row >> 2) ^ (row >> 3)) & 1;
    else return 0;
}

typedef const volatile __attribute__((address_space(3))) float lds_vfloat;
typedef __attribute__((address_space(3))) float lds_float;

// Inserts a lane's 16 biased scores of one 32-column tile into its running
// top-KL list. acc[4q + e] is the score of column vt + 8q + 4 (lane / 32) + e
// of the lane's block (the 32x32 accumulator layout): the column rises with
// the index. `plain` inserts every column inside V (the ragged last tile; the
// first tile of a top-k list with no bound known). Otherwise, for KL > 1, a
// filter keeps the scores that can still enter the list. VW waves score the
// same blocks over other columns and share their bounds through LDS: this
// wave (index vb among them) publishes its bound for the lane's block at
// thr_mine and reads the others' at thr_grp[w * 32 + lane % 32].
template <int KL, int VW>
__device__ __forceinline__ void insert_scores(u64 (&list)[KL], const f32x16& acc, int vt, int V, bool active,
                                              bool plain, float tau, lds_float* thr_mine, lds_vfloat* thr_grp,
                                              int vb) {
    const int lane = threadIdx.x & 63;
    const int lrow = lane & 31, lhalf = lane >> 5;
    float z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = acc[e];
    const int vlane = vt + 4 * lhalf;
    if (plain) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int v = vlane + 8 * (e >> 2) + (e & 3);
            topk_insert<KL>(list, (active && v < V) ? make_key(z[e], v) : 0ull);
        }
    } else if constexpr (KL == 1) {
        // Argmax of the lane's 16 columns: a strictly greater score moves
        // the pick, so equal scores keep the lower column.
        float best = z[0];
        int be = 0;
#pragma unroll
        for (int e = 1; e < 16; ++e) {
            const bool gt = z[e] > best;
            best = gt ? z[e] : best;
            be = gt ? e : be;
        }
        const u64 key = make_key(best, vlane + 8 * (be >> 2) + (be & 3));
        if (active && key > list[0]) list[0] = key;
    } else {
        // Filtered inserts. A score below a bound that KL distinct columns
        // of the block reach cannot be among its best KL. Bounds: the KL-th
        // best of the union of this lane's list and the partner lane's (both
        // decreasing: the largest over the splits of KL between them of the
        // smaller of the two closing entries), tau, and the bounds the other
        // waves of the block last published. A score equal to the bound
        // passes, so the full key comparison settles ties by column. Hits are
        // inserted in rounds, one per lane per round.
        float sa[KL], sb[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            sa[i] = list[i] != 0ull ? key_score(list[i]) : -INFINITY;
            sb[i] = __shfl_xor(sa[i], 32, kWave);
        }
        float thr = fmaxf(sa[KL - 1], sb[KL - 1]);
#pragma unroll
        for (int i = 1; i < KL; ++i) thr = fmaxf(thr, fminf(sa[i - 1], sb[KL - 1 - i]));
        thr = fmaxf(thr, tau);
        if (lhalf == 0 && active) *thr_mine = thr;
#pragma unroll
        for (int w = 0; w < VW; ++w)
            if (w != vb) thr = fmaxf(thr, thr_grp[w * 32 + lrow]);
        float zmax = z[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) zmax = fmaxf(zmax, z[e]);
        if (__any(active && zmax >= thr)) {
            unsigned hits = 0u;
#pragma unroll
            for (int e = 0; e < 16; ++e) hits |= (z[e] >= thr ? 1u : 0u) << e;
            if (!active) hits = 0u;
            // Every lane runs every round (no branch): a lane whose hits are
            // done inserts the empty key 0, which changes nothing.
            while (__any(hits != 0u)) {
                const bool has = hits != 0u;
                const int e = __builtin_ctz(hits | 0x10000u);
                hits &= hits - 1u;
                // z[e] by a select tree on the bits of e
                const u64 m0 = __builtin_amdgcn_ballot_w64((e & 1) != 0);
                const u64 m1 = __builtin_amdgcn_ballot_w64((e & 2) != 0);
                const u64 m2 = __builtin_amdgcn_ballot_w64((e & 4) != 0);
                const u64 m3 = __builtin_amdgcn_ballot_w64((e & 8) != 0);
                float s8[8], s4[4], s2[2];
#pragma unroll
                for (int i = 0; i < 8; ++i) s8[i] = lane_select(z[2 * i + 1], z[2 * i], m0);
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[i] = lane_select(s8[2 * i + 1], s8[2 * i], m1);
#pragma unroll
                for (int i = 0; i < 2; ++i) s2[i] = lane_select(s4[2 * i + 1], s4[2 * i], m2);
                const float ze = lane_select(s2[1], s2[0], m3);
                topk_insert<KL>(list, has ? make_key(ze, vlane + 8 * (e >> 2) + (e & 3)) : 0ull);
            }
        }
    }
}

}  // namespace

}  // namespace dspark
