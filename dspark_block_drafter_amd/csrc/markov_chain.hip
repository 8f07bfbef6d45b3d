// Markov chain, candidates and confidence truncation.
//
// Chain (llama.cpp commit 6fed9f6 "spec: add DSpark speculative decoding",
// the chained-bias formula): for prediction slot j of block b,
//   z'[v] = logits[b * n_pred + j][v] + sum_k markov_w2[v][k] * markov_w1[prev][k]
// with prev = anchor[b] for j = 0 and prev = argmax z' of slot j - 1 after
// that; every block advances in the same launch (the chain is vectorised
// across blocks). The same biased scores feed the top-k candidate lattice
// (lucebox PR #626 "feat(qwen38): add adaptive concurrent DSpark
// speculation", description).
//
// One launch per slot j. A workgroup owns a contiguous range of vocabulary
// columns for up to 64 blocks. It stages, with coalesced direct-to-LDS loads,
// the markov_w2 rows of its columns and the slot-j logits of its blocks,
// through a ring shared by its four waves (chain_step_pipe) or one private
// ring per wave (chain_step_wave); the rank-r rows markov_w1[prev_b] become
// the MFMA B operand. The [v x b] bias tile is one bf16 MFMA product per 32
// columns with the logits as accumulator input, and every lane keeps a
// running top-k for its block. The 32x32 accumulator layout gives every lane
// a single block b and 16 vocabulary ids, so the per-lane lists see their ids
// in increasing order. Lists are merged across the two lanes that share b,
// then across the waves through LDS; the workgroup's best key goes to a
// 64-bit atomicMax on one of the slot's running-argmax words for b (keys
// order by score, then lower id), and its list to the partials used to
// assemble the candidates after the last slot. chain_step_direct reads its
// operands straight from global memory for any V.
#include "common.hpp"
#include "kernels.hpp"
#include "chain_parts.hpp"

namespace dspark {

namespace {

constexpr int kWaves = 4;
// finalize runs two waves per (block, slot) from this many pairs on, one
// workgroup per pair below it.
constexpr long kFinalWavePairs = 512;
static_assert(kChainTileV == kWaves * 32, "one 32-column block per wave");

__global__ __launch_bounds__(256) void chain_init(u64* winners, int n, uint32_t* flags,
                                                  int32_t* lengths, int B, int n_pred,
                                                  uint32_t* w2n2, uint32_t* w1n2) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) winners[i] = 0ull;
    if (i < B) lengths[i] = n_pred;
    if (i == 0) {
        *flags = 0u;
        if (w2n2) *w2n2 = 0u;
        if (w1n2) *w1n2 = 0u;
    }
}

// ---- pieces shared by the two step kernels ----------------------------------

// prev_b for slot j (anchor, or the previous slot's argmax) and the lane's
// share of markov_w1[prev_b] as MFMA B operand: u[nb][s] holds
// W1[prev][16 s + 8 (lane / 32) .. + 8] for block bbase + 32 nb + lane % 32.
template <int NB, int RS>
__device__ __forceinline__ void gather_w1(const ChainArgs& a, int j, int bbase, int lrow, int lhalf,
                                          u32x4 (&u)[NB][RS], int (&bl)[NB]) {
    const int B = a.B, r = a.r;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int b = bbase + nb * 32 + lrow;
        bl[nb] = b;
        const int prev = b < B ? prev_token(a, j, b, true) : 0;
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int k0 = s * 16 + lhalf * 8;
            u[nb][s] = (b < B && k0 < r)
                           ? *reinterpret_cast<const u32x4*>(a.w1 + (long)prev * r + k0)
                           : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Merge the per-lane lists of a workgroup into one list per block and publish
// it: partial list (top_k > 1) and atomicMax on the slot's argmax word.
template <int NB, int KL>
__device__ __forceinline__ void publish(const ChainArgs& a, int j, int bbase, u64 (&list)[NB][KL],
                                        u64 (*s_list)[NB * 32][KL]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    // the two lanes that hold the same block (lane, lane ^ 32)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[nb][i], 32);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list[nb], other[i]);
    }
    if (lhalf == 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < KL; ++i) s_list[wave][nb * 32 + lrow][i] = list[nb][i];
    }
    __syncthreads();
    const int t = threadIdx.x;
    const int B = a.B;
    if (t < NB * 32) {
        const int b = bbase + t;
        if (b < B) {
            u64 m[KL];
#pragma unroll
            for (int i = 0; i < KL; ++i) m[i] = s_list[0][t][i];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
#pragma unroll
                for (int i = 0; i < KL; ++i) topk_insert<KL>(m, s_list[w][t][i]);
            if (a.top_k > 1) {
                u64* p = a.partials + (((long)j * B + b) * a.nwg + blockIdx.x) * a.top_k;
#pragma unroll
                for (int i = 0; i < KL; ++i)
                    if (i < a.top_k) p[i] = m[i];
            }
            if (m[0] != 0ull) atomicMax(winner_word(a.winners, a.wstride, j, blockIdx.x, b), m[0]);
        }
    }
}

// ---- top-k bound from the projection's row-maximum bins ----------------------

// Insert x into the decreasing list top[0..KL).
template <int KL>
__device__ __forceinline__ void top_insert_f32(float (&top)[KL], float x) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
        const float hi = fmaxf(x, top[i]);
        x = fminf(x, top[i]);
        top[i] = hi;
    }
}

// The k-th largest slab maximum of every row: one workgroup per row; each
// thread keeps the KL largest of its share of the slabs (up to 16 loads in
// flight), then the lists are merged across the wave and the four waves.
// -inf when the row has fewer than KL slabs.
template <int KL>
__global__ __launch_bounds__(256) void row_kth(const float* smax, int nslab, float* kth) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = smax + (long)blockIdx.x * nslab;
    float top[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) top[i] = -INFINITY;
    for (int s0 = 0; s0 < nslab; s0 += 256 * 16) {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int s = s0 + u * 256 + tid;
            x[u] = s < nslab ? row[s] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) top_insert_f32<KL>(top, x[u]);
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) {
        float other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = __shfl_xor(top[i], mask, kWave);
#pragma unroll
        for (int i = 0; i < KL; ++i) top_insert_f32<KL>(top, other[i]);
    }
    __shared__ float s_top[kWaves][KL];
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < KL; ++i) s_top[wave][i] = top[i];
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
#pragma unroll
            for (int i = 0; i < KL; ++i) top_insert_f32<KL>(top, s_top[w][i]);
        kth[blockIdx.x] = top[KL - 1];
    }
}

// Direct-to-LDS copy, by wave 0, of the k-th slab maxima of slot j of blocks
// bbase + lane into s_kth[64] (blocks past B repeat block B - 1), and, by the
// last wave, of the markov_w2 (and, with s_w1n2, markov_w1) norm word into
// all 64 words of s_w2n2 (s_w1n2).
// The destinations are addressed through bases the compiler cannot trace to
// the arrays (the readers wait explicitly): a copy it can attribute to an
// array makes it wait for every copy in flight before any later LDS read it
// cannot tell apart from that array.
__device__ __forceinline__ void load_bound(const ChainArgs& a, int j, int bbase, float* s_kth,
                                           uint32_t* s_w2n2, int wave, int lane, uint32_t* s_w1n2 = nullptr) {
    if (wave == 0) {
        const int b = min(bbase + lane, a.B - 1);
        lds_char* d = (lds_char*)(lds_ptr)s_kth;
        asm volatile("" : "+s"(d));
        __builtin_amdgcn_global_load_lds((const void*)(a.kth + (long)b * a.n_pred + j), (lds_ptr)d, 4, 0, 0);
    }
    if (wave == kWaves - 1) {
        lds_char* d = (lds_char*)(lds_ptr)s_w2n2;
        asm volatile("" : "+s"(d));
        __builtin_amdgcn_global_load_lds((const void*)a.w2n2, (lds_ptr)d, 4, 0, 0);
        if (s_w1n2 && a.w1n2) {
            lds_char* d1 = (lds_char*)(lds_ptr)s_w1n2;
            asm volatile("" : "+s"(d1));
            __builtin_amdgcn_global_load_lds((const void*)a.w1n2, (lds_ptr)d1, 4, 0, 0);
        }
    }
}

// ---- step kernel for V % 4 == 0: operands staged through LDS -----------------

// Workgroup g streams the vocabulary range of tiles [t0, t1) (TS = 32 VW
// columns each) for up to 64 blocks. Every tile's markov_w2 rows and slot-j
// logits go through an NS-deep ring of LDS stages filled by direct-to-LDS
// loads, so NS - 1 tiles are in flight while one is scored. Wave w scores the
// 32-column block w % VW of the tile for block group w / VW (VW = 4 when one
// group of 32 blocks suffices, else 2). The workgroup publishes once per
// slot, after its whole range.
template <int NB, int KL, int RS, int NS, int VW>
__global__ __launch_bounds__(256) void chain_step_pipe(ChainArgs a, int j) {
    constexpr int TS = 32 * VW;             // columns per tile
    static_assert(VW * NB <= kWaves && (VW == 2 || VW == 4), "wave split");
    constexpr int WR = 2 * RS;              // 16-byte chunks per staged markov_w2 row
    constexpr int WRd = WR > 0 ? WR : 1;    // (divisor; only used when RS > 0)
    constexpr int LR = TS / 4;              // 16-byte chunks per staged logits row
    constexpr int W_SLOTS = RS > 0 ? TS * WR : 0;
    constexpr int L_SLOTS = NB * 32 * LR;
    constexpr int STAGE = W_SLOTS + L_SLOTS;
    constexpr int W_INST = W_SLOTS / 64, L_INST = L_SLOTS / 64;
    constexpr int LW = (W_INST + L_INST) / kWaves;  // loads per wave per tile
    static_assert((W_INST + L_INST) % kWaves == 0, "tile loads must split over waves");
    static_assert(NS >= 2 && (NS - 1) * LW < 64, "pipeline depth");
    static_assert(kWaves * KL * NB * 32 * 8 <= NS * STAGE * 16, "list merge reuses the ring");
    __shared__ u32x4 ring[NS][STAGE];
    // Last-entry score of each wave's lists, per block: a lower bound of the
    // block's KL-th best score in this workgroup, shared with the waves that
    // score the other columns of the same blocks.
    __shared__ float s_thr[kWaves][32];
    // The slot's k-th slab maxima of its blocks and the markov_w2 norm word
    // (the top-k bound), copied in by the prologue.
    __shared__ float s_kth[64];
    __shared__ uint32_t s_w2n2[64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int vb = wave % VW, nbw = wave / VW;       // this wave's 32-column block / block group
    // adaptive gate: every block was cut before this slot
    if (a.stop && j >= *a.stop) return;
    const int bbase = blockIdx.y * NB * 32;
    // the bound's copies go first: the prologue's waits cover them
    const bool bounded = KL > 1 && a.kth != nullptr;
    if constexpr (KL > 1)
        if (bounded) load_bound(a, j, bbase, s_kth, s_w2n2, wave, lane);
    const int B = a.B, V = a.V, r = a.r;
    const int nT = (V + TS - 1) / TS, G = gridDim.x, g = blockIdx.x;
    const int t0 = (int)((long)nT * g / G), t1 = (int)((long)nT * (g + 1) / G);
    const int n = t1 - t0;

    // This lane's fixed part of each of its LW loads per tile.
    const char* src[LW];
    int dst[LW];
    long step[LW];   // bytes to advance per tile
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int inst = wave + i * kWaves;
        if (inst < W_INST) {
            const int slot = inst * 64 + lane, row = slot / WRd;
            const int c = (slot % WRd) ^ swz_rows<WR>(row);
            const int k = c * 8 < r ? c * 8 : 0;   // rank padding: any valid chunk
            src[i] = reinterpret_cast<const char*>(a.w2 + (long)row * r + k);
            step[i] = (long)TS * r * 2;
            dst[i] = inst * 64;
        } else {
            const int slot = (inst - W_INST) * 64 + lane, row = slot / LR;
            const int c = (slot % LR) ^ swz_rows<LR>(row);
            int b = min(bbase + row, B - 1);
            if (block_cut(a, b, j)) b = bbase;   // one shared row for every cut block
            src[i] = reinterpret_cast<const char*>(a.logits + ((long)b * a.n_pred + j) * V + 4 * c);
            step[i] = (long)TS * 4;
            dst[i] = W_SLOTS + (inst - W_INST) * 64;
        }
    }
    // The copies into the ring address it through a base the compiler cannot
    // trace to the array: a copy it can attribute to the ring would make the
    // next LDS read of the ring wait for every load in flight (vmcnt(0)),
    // which drains the ring. The explicit waits below order the reads. (The
    // address arithmetic stays inline: moved into a helper called from the
    // lambdas, the host pass stops emitting this kernel's launch stub.)
    lds_char* ring_dma = (lds_char*)(lds_ptr)&ring[0][0];
    asm volatile("" : "+s"(ring_dma));
    // Load i of a wave is a markov_w2 load for i < W_INST / kWaves, a logits
    // load after. The logits are read once: those loads are non-temporal, so
    // they do not push markov_w2 (read again by every slot) out of the caches.
    static_assert(W_INST % kWaves == 0, "the first loads of every wave are the markov_w2 ones");
    auto copy = [&](int i, const void* p, int st) __attribute__((always_inline)) {
        lds_ptr d = (lds_ptr)(ring_dma + (st * STAGE + dst[i]) * 16);
        if (i < W_INST / kWaves) __builtin_amdgcn_global_load_lds(p, d, 16, 0, 0);
        else __builtin_amdgcn_global_load_lds(p, d, 16, 0, kLoadNT);
    };
    // Columns past V: markov_w2 rows are clamped to row V-1, logits to the
    // last 16-byte chunk of the row; such columns are never scored.
    auto issue = [&](int st, int t) __attribute__((always_inline)) {
        const int v0 = t * TS;
        if (v0 + TS <= V) {   // whole tile inside the vocabulary: no clamping
#pragma unroll
            for (int i = 0; i < LW; ++i) copy(i, src[i] + (long)t * step[i], st);
            return;
        }
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            const char* p = src[i] + (long)t * step[i];
            if (i * kWaves + wave < W_INST) {
                const int row = ((i * kWaves + wave) * 64 + lane) / WRd;
                if (v0 + row >= V) p -= (long)(v0 + row - (V - 1)) * r * 2;
            } else {
                const int slot = ((i * kWaves + wave) - W_INST) * 64 + lane;
                const int c = (slot % LR) ^ swz_rows<LR>(slot / LR);
                if (v0 + 4 * c > V - 4) p -= (long)(v0 + 4 * c - (V - 4)) * 4;
            }
            copy(i, p, st);
        }
    };

    // Previous token of this lane's block (anchor, or the last slot's argmax).
    const int bme = bbase + nbw * 32 + lrow;
    const bool live = bme < B && !block_cut(a, bme, j);
    // The copy of the previous tokens' words (each wave its own, after the
    // W1 rows in stage NS-1), tiles 0 .. NS-2, then the tokens and the
    // markov_w1 rows of prev (MFMA B operand; their address needs prev). The
    // words land first, so the tiles stream during the tokens' two round
    // trips. The loop starts once all of these have landed. The W1 rows
    // travel direct to LDS like the tiles (a register load would need a wait
    // for every older load, the whole ring), into stage NS-1, which the first
    // step refills only after the barrier that follows their reads: one copy
    // per block group, loaded by its first wave. A workgroup owns n >= 1
    // tiles (there are at most as many workgroups as tiles), and a stage past
    // n - 1 gets a second copy of the last tile, which no iteration reads, so
    // the number of loads in flight is fixed. Lanes of blocks past B read row
    // 0 (their scores are never inserted); chunks past the rank are zeroed
    // when read. (Without markov_w1 rows, r = 0, the token is read directly.)
    static_assert(NS >= 2, "a stage in use and one in flight at least");
    static_assert(NB * RS * 64 <= STAGE, "W1 rows fit stage NS - 1");
    constexpr int PREV_OFF = NB * RS * 64;   // the waves' copies of the previous tokens' words
    static_assert(RS == 0 || PREV_OFF + kWaves * kPrevChunks <= STAGE, "previous tokens fit stage NS - 1");
    int prev = 0;
    if constexpr (RS > 0) {
        if (nbw < NB && bbase + nbw * 32 < B)
            copy_prev(a, j, bbase + nbw * 32, ring_dma + ((NS - 1) * STAGE + PREV_OFF + wave * kPrevChunks) * 16);
    } else {
        prev = (live && nbw < NB) ? prev_token(a, j, bme, vb == 0) : 0;
    }
    issue(0, t0);
#pragma unroll
    for (int t = 1; t < NS - 1; ++t) issue(t, t0 + min(t, n - 1));
    if constexpr (RS > 0) {
        wait_vmcnt<(NS - 1) * LW>();   // the words: older than every tile copy
        asm volatile("" ::: "memory");
        // (read through the copies' base: an address the compiler can trace
        // to the ring would make it wait for every copy in flight first)
        if (live && nbw < NB)
            prev = prev_from_copy(a, j, (const void*)(ring_dma + ((NS - 1) * STAGE + PREV_OFF + wave * kPrevChunks) * 16),
                                  lrow, vb == 0);
        if (vb == 0 && nbw < NB) {
#pragma unroll
            for (int s = 0; s < RS; ++s) {
                const int k0 = s * 16 + lhalf * 8;
                __builtin_amdgcn_global_load_lds((const void*)(a.w1 + (long)prev * r + (k0 < r ? k0 : 0)),
                                                 (lds_ptr)(ring_dma + ((NS - 1) * STAGE + (nbw * RS + s) * 64) * 16), 16, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();
    u32x4 u[RS > 0 ? RS : 1];   // W1 rows (MFMA B operand), read after the barrier

    // MFMA runs on whole waves: only the wave-uniform part of the condition may
    // guard it; blocks past B are masked at the inserts.
    const bool wave_on = nbw < NB;
    const bool active = wave_on && live;

    u64 list[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) list[i] = 0ull;
    if (lhalf == 0) s_thr[wave][lrow] = -INFINITY;
    float tau = -INFINITY;   // the block's top-k bound (set once u is read)

    // Software pipeline over tiles: the bias product of tile it + 1 (LDS
    // reads + MFMA) is issued before the top-k work of tile it, so the matrix
    // pipe runs while the wave inserts. Tile it + NS - 1 is loaded into the
    // stage of tile it - 1, which every wave finished reading (score of tile
    // it - 1, one iteration earlier) before it passed the previous barrier.
    // The slot-j logits of a tile enter the MFMA as its accumulator input, so
    // the accumulator ends as the biased score z = logits + W2 . W1[prev].
    struct Scores { f32x16 acc; };
    auto score = [&](int st_, Scores& sc) __attribute__((always_inline)) {
        const u32x4* stg = ring[st_];
        const int vrow = vb * 32 + lrow;
        const int row = nbw * 32 + lrow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = vb * 8 + 2 * q + lhalf;
            const f32x4 x = __builtin_bit_cast(f32x4, stg[W_SLOTS + row * LR + (c ^ swz_rows<LR>(row))]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc.acc[4 * q + e] = x[e];
        }
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const u32x4 w = stg[vrow * WR + ((2 * s + lhalf) ^ swz_rows<WR>(vrow))];
            sc.acc = mfma32x32x16(w, u[s], sc.acc);
        }
    };
    auto consume = [&](int it, const Scores& sc) __attribute__((always_inline)) {
        const int vt = (t0 + it) * TS + vb * 32;
        // z[4q + e] is the biased score of column vt + 8q + 4(lane/32) + e;
        // the column rises with the index.
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = sc.acc[e];
        const int vlane = vt + 4 * lhalf;
        const bool full = vt + 32 <= V;
        if (!full || (KL > 1 && it == 0 && !bounded)) {
            // plain inserts (the ragged last tile; the first tile of top-k
            // lists when no bound is known)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int v = vlane + 8 * (e >> 2) + (e & 3);
                topk_insert<KL>(list, (active && v < V) ? make_key(z[e], v) : 0ull);
            }
        } else if constexpr (KL == 1) {
            // Argmax of the lane's 16 columns: a strictly greater score moves
            // the pick, so equal scores keep the lower column, as the key
            // order does.
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
            // Filtered inserts: a score cannot be among the block's best KL
            // if KL other columns of the block score above it. The bound is
            // the KL-th best of the union of this lane's list and the partner
            // lane's (both decreasing: the largest over the splits of KL
            // between them of the smaller of the two entries that close the
            // split), published for the other waves of the block group, and
            // raised to their last published bounds. A score equal to the
            // bound passes, so the full key comparison settles ties by
            // column. Hits are inserted in rounds, one per lane per round.
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
            if (lhalf == 0) s_thr[wave][lrow] = thr;
#pragma unroll
            for (int w = 0; w < VW; ++w) thr = fmaxf(thr, s_thr[nbw * VW + w][lrow]);
            float zmax = z[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) zmax = fmaxf(zmax, z[e]);
            if (__any(active && zmax >= thr)) {
                unsigned hits = 0u;
#pragma unroll
                for (int e = 0; e < 16; ++e) hits |= (z[e] >= thr ? 1u : 0u) << e;
                if (!active) hits = 0u;
                // Every lane runs every round (no branch): a lane whose hits
                // are done inserts the empty key 0, which changes nothing.
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
    };
    // one iteration: bring tile it + 1 in and score it, then consume tile it.
    // The first one refills stage NS - 1 after its barrier, once every wave
    // holds its W1 rows from there; tiles 1 .. NS - 2 came from the prologue.
    auto step_tile = [&](int it, int& st, const Scores& cur, Scores& nxt, bool first)
                         __attribute__((always_inline)) {
        const int nst = st + 1 == NS ? 0 : st + 1;
        if (it + 1 < n) {
            if (first) {
                wait_vmcnt<(NS >= 3 ? (NS - 3) * LW : 0)>();
            } else {
                if (it + NS - 1 < n) issue((st + NS - 1) % NS, t0 + it + NS - 1);
                wait_stages<LW, NS - 2>(min(NS - 2, n - 2 - it));
            }
            // The logits of tile it were read into registers before this
            // barrier; their reads must have landed before any wave refills
            // that stage after it.
            wait_lds_reads();
            block_barrier();
            if (first && NS - 1 < n) issue(NS - 1, t0 + NS - 1);
            if (wave_on) score(nst, nxt);
        }
        if (wave_on) consume(it, cur);
        st = nst;
    };

    // Tile 0 and the W1 rows have landed for every wave after this barrier
    // (tiles 1 .. NS - 2 may still fly: the loop waits for each before
    // reading it); stage NS - 1 is refilled by the first step.
    int st = 0;
    Scores S0, S1;
    block_barrier();
    if (wave_on) {
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            u[s] = ring[NS - 1][(nbw * RS + s) * 64 + lane];
            if (s * 16 + lhalf * 8 >= r) u[s] = u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (KL > 1) {
            if (bounded) {
                const float un2 = w1_norm2<RS>(u);
                tau = chain_bound(s_kth[nbw * 32 + lrow], __uint_as_float(s_w2n2[0]), un2);
            }
        }
        score(0, S0);
    }
    if constexpr (NS >= 3) {
        step_tile(0, st, S0, S1, true);
        for (int it = 1; it < n; it += 2) {
            step_tile(it, st, S1, S0, false);
            if (it + 1 < n) step_tile(it + 1, st, S0, S1, false);
        }
    } else {
        // Two stages (two workgroups per CU): tile t sits in stage t & 1.
        // Tile it + 1 is loaded while the wave inserts tile it; it goes to
        // the stage of tile it - 1, which every wave finished reading before
        // the previous barrier. Stage 1 first held the W1 rows: every wave
        // has read them before this barrier.
        wait_lds_reads();
        block_barrier();
        auto step2 = [&](int it, const Scores& cur, Scores& nxt) __attribute__((always_inline)) {
            if (it + 1 < n) issue((it + 1) & 1, t0 + it + 1);
            if (wave_on) consume(it, cur);
            if (it + 1 < n) {
                wait_vmcnt<0>();
                wait_lds_reads();
                block_barrier();
                if (wave_on) score((it + 1) & 1, nxt);
            }
        };
        for (int it = 0; it < n; it += 2) {
            step2(it, S0, S1);
            if (it + 1 < n) step2(it + 1, S1, S0);
        }
    }

    // Merge: the lane pair that holds the same block, then the VW waves of
    // the block group (their lists go through the ring, free by now).
    {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[i], 32);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list, other[i]);
    }
    u64* s_list = reinterpret_cast<u64*>(&ring[0][0]);  // [wave][32][KL]
    wait_vmcnt<0>();   // with n == 1 the extra copies of the prologue may still fly
    __syncthreads();
    if (lhalf == 0) {
#pragma unroll
        for (int i = 0; i < KL; ++i) s_list[(wave * 32 + lrow) * KL + i] = list[i];
    }
    __syncthreads();
    if (vb == 0 && lhalf == 0 && active) {
#pragma unroll
        for (int w = 1; w < VW; ++w)
#pragma unroll
            for (int i = 0; i < KL; ++i) topk_insert<KL>(list, s_list[((wave + w) * 32 + lrow) * KL + i]);
        const int b = bme;
        if (a.top_k > 1) {
            u64* p = a.partials + (((long)j * B + b) * a.nwg + g) * a.top_k;
#pragma unroll
            for (int i = 0; i < KL; ++i)
                if (i < a.top_k) p[i] = list[i];
        }
        if (list[0] != 0ull) atomicMax(winner_word(a.winners, a.wstride, j, g, b), list[0]);
    }
}

// ---- step kernel for V % 4 == 0: a private ring per wave ----------------------

// The workgroup's range of tiles [t0, t1) (TS = 32 VW columns per tile) is
// cut into VW contiguous runs of 32-column steps; wave w scores run w % VW
// for the block group w / VW (VW = 2 for two groups of 32 blocks, 4 for one
// group). Each wave streams its own markov_w2 rows and slot-j logits rows
// (LROWS of them: only the group's blocks that exist) through its own
// NS-stage LDS ring of direct-to-LDS copies, so its loop needs no workgroup
// barrier: a slow insert round holds up only that wave, and all NS stages are
// in flight while it inserts (a stage is refilled as soon as its step has
// been read into the accumulators). With two block groups the two waves of a
// run both copy its markov_w2 rows (the second copy is an L2 hit). The waves
// that score the same blocks share their top-k bounds through LDS without
// synchronisation: every published value is a valid bound whenever it is
// read. The workgroup merges and publishes once per slot.
template <int NB, int KL, int RS, int NS, int LROWS>
__global__ __launch_bounds__(256) void chain_step_wave(ChainArgs a, int j) {
    constexpr int VW = kWaves / NB;         // 32-column blocks per tile
    constexpr int TS = 32 * VW;             // columns per tile
    constexpr int WR = 2 * RS;              // 16-byte chunks per staged markov_w2 row
    constexpr int WRd = WR > 0 ? WR : 1;
    constexpr int LR = 8;                   // 16-byte chunks per staged logits row (32 columns)
    constexpr int W_SLOTS = 32 * WR;
    constexpr int L_SLOTS = LROWS * LR;     // the logits rows of the group's blocks that exist
    constexpr int STAGE = W_SLOTS + L_SLOTS;
    constexpr int W_INST = W_SLOTS / 64, L_INST = L_SLOTS / 64;
    constexpr int LW = W_INST + L_INST;     // copies per tile per wave
    static_assert(NB == 1 || NB == 2, "one or two block groups");
    static_assert(NS >= 2 && NS * LW + RS < 64, "vmcnt range");
    static_assert(LROWS == 8 || LROWS == 16 || LROWS == 32, "staged logits rows");
    static_assert(RS * 64 <= STAGE, "W1 rows fit one stage");
    static_assert(KL * 32 * 8 <= NS * STAGE * 16, "list merge reuses a wave's ring");
    __shared__ u32x4 ring[kWaves][NS][STAGE];
    // Top-k bound of each wave's lane pairs, per block (see consume below).
    __shared__ float s_thr[kWaves][32];
    // The slot's k-th slab maxima of its blocks and the markov_w2 norm word
    // (the top-k bound).
    __shared__ float s_kth[64];
    __shared__ uint32_t s_w2n2[64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int vb = wave % VW, nbw = wave / VW;
    if (a.stop && j >= *a.stop) return;   // adaptive gate: every block was cut
    const int bbase = blockIdx.y * NB * 32;
    const bool bounded = KL > 1 && a.kth != nullptr;
    if constexpr (KL > 1)
        if (bounded) load_bound(a, j, bbase, s_kth, s_w2n2, wave, lane);
    const int B = a.B, V = a.V, r = a.r;
    const int nT = (V + TS - 1) / TS, G = gridDim.x, g = blockIdx.x;
    const int t0 = (int)((long)nT * g / G), t1 = (int)((long)nT * (g + 1) / G);
    const int n = t1 - t0;                  // >= 1: there are at most as many workgroups as tiles

    // The workgroup's columns [t0 TS, t1 TS) are cut into VW contiguous runs
    // of n 32-column steps, one per column block: wave vb streams columns
    // cbase + 32 it, it = 0 .. n-1, so each wave reads its markov_w2 and
    // logits rows front to back.
    const int cbase = (t0 * VW + vb * n) * 32;
    // This lane's fixed part of each of its LW copies per step (step 0).
    const char* src[LW];
    int dst[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        if (i < W_INST) {
            const int slot = i * 64 + lane, row = slot / WRd;
            const int c = (slot % WRd) ^ swz_rows<WR>(row);
            const int k = c * 8 < r ? c * 8 : 0;   // rank padding: any valid chunk
            src[i] = reinterpret_cast<const char*>(a.w2 + (long)(cbase + row) * r + k);
        } else {
            const int slot = (i - W_INST) * 64 + lane, row = slot / LR;
            const int c = (slot % LR) ^ swz_rows<LR>(row);
            int b = min(bbase + nbw * 32 + row, B - 1);
            if (block_cut(a, b, j)) b = bbase + nbw * 32;   // one shared row for every cut block
            src[i] = reinterpret_cast<const char*>(a.logits + ((long)b * a.n_pred + j) * V + cbase + 4 * c);
        }
        dst[i] = i * 64;
    }
    // Copies address the ring through a base the compiler cannot trace to the
    // array (as in chain_step_pipe): the explicit waits order the reads.
    lds_char* ring_dma = (lds_char*)(lds_ptr)&ring[wave][0][0];
    asm volatile("" : "+s"(ring_dma));
    auto copy = [&](int i, const void* p, int st) __attribute__((always_inline)) {
        lds_ptr d = (lds_ptr)(ring_dma + (st * STAGE + dst[i]) * 16);
        if (i < W_INST) __builtin_amdgcn_global_load_lds(p, d, 16, 0, 0);
        else __builtin_amdgcn_global_load_lds(p, d, 16, 0, kLoadNT);
    };
    // Columns past V: markov_w2 rows are clamped to row V-1, logits to the
    // last 16-byte chunk of the row; such columns are never scored.
    auto issue = [&](int st, int t) __attribute__((always_inline)) {
        const int v0 = cbase + t * 32;
        if (v0 + 32 <= V) {
#pragma unroll
            for (int i = 0; i < LW; ++i) copy(i, src[i] + (long)t * (i < W_INST ? 64 * r : 128), st);
            return;
        }
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            const char* p = src[i] + (long)t * (i < W_INST ? 64 * r : 128);
            if (i < W_INST) {
                const int row = (i * 64 + lane) / WRd;
                if (v0 + row >= V) p -= (long)(v0 + row - (V - 1)) * r * 2;
            } else {
                const int slot = (i - W_INST) * 64 + lane;
                const int c = (slot % LR) ^ swz_rows<LR>(slot / LR);
                if (v0 + 4 * c > V - 4) p -= (long)(v0 + 4 * c - (V - 4)) * 4;
            }
            copy(i, p, st);
        }
    };

    const int bme = bbase + nbw * 32 + lrow;
    const bool active = bme < B && !block_cut(a, bme, j);
    // The copy of the previous tokens' words into stage NS-1, tiles 0 .. NS-2,
    // then the tokens and the markov_w1 rows of prev (the MFMA B operand)
    // into stage NS-1 over the read copy. The words land first, so the tiles
    // stream during the tokens' two round trips. Once all of these (and the
    // bound's copies) have landed and every wave has set its bounds, the rows
    // go to registers and tile NS-1 into stage NS-1. A stage past the last
    // tile gets a second copy of it (no iteration reads it), so the number of
    // copies in flight is fixed. Chunks past the rank are zeroed when read.
    // (Without markov_w1 rows, r = 0, the token is read directly.)
    static_assert(RS == 0 || kPrevChunks <= STAGE, "previous tokens fit a stage");
    int prev = 0;
    if constexpr (RS > 0) {
        if (bbase + nbw * 32 < B) copy_prev(a, j, bbase + nbw * 32, ring_dma + (NS - 1) * STAGE * 16);
    } else {
        prev = active ? prev_token(a, j, bme, vb == 0) : 0;
    }
    issue(0, 0);
#pragma unroll
    for (int t = 1; t < NS - 1; ++t) issue(t, min(t, n - 1));
    if constexpr (RS > 0) {
        wait_vmcnt<(NS - 1) * LW>();   // the words: older than every tile copy
        asm volatile("" ::: "memory");
        if (active) prev = prev_from_copy(a, j, (const void*)(ring_dma + (NS - 1) * STAGE * 16), lrow, vb == 0);
        wait_lds_reads();   // the copy is read before the W1 rows replace it
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int k0 = s * 16 + lhalf * 8;
            __builtin_amdgcn_global_load_lds((const void*)(a.w1 + (long)prev * r + (k0 < r ? k0 : 0)),
                                             (lds_ptr)(ring_dma + ((NS - 1) * STAGE + s * 64) * 16), 16, 0, 0);
        }
    }
    if (lhalf == 0) s_thr[wave][lrow] = -INFINITY;
    wait_lds_reads();
    wait_vmcnt<0>();   // tiles 0 .. NS-2, the W1 rows, the bound's copies
    block_barrier();   // every bound is set before any wave reads it
    asm volatile("" ::: "memory");
    u32x4 u[RS > 0 ? RS : 1];
#pragma unroll
    for (int s = 0; s < RS; ++s) {
        u[s] = ring[wave][NS - 1][s * 64 + lane];
        if (s * 16 + lhalf * 8 >= r) u[s] = u32x4{0u, 0u, 0u, 0u};
    }
    float tau = -INFINITY;   // the block's top-k bound
    if constexpr (KL > 1) {
        if (bounded) {
            const float un2 = w1_norm2<RS>(u);
            tau = chain_bound(s_kth[nbw * 32 + lrow], __uint_as_float(s_w2n2[0]), un2);
        }
    }
    asm volatile("" ::: "memory");
    wait_lds_reads();
    asm volatile("" ::: "memory");
    issue(NS - 1, min(NS - 1, n - 1));

    u64 list[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) list[i] = 0ull;
    // (an LDS-qualified pointer: a generic one would become a flat load,
    // which waits for every copy in flight)
    lds_vfloat* thr_v = (lds_vfloat*)&s_thr[0][0];

    // The slot-j logits of a tile enter the MFMA as its accumulator input,
    // so the accumulator ends as the biased score z = logits + W2 . W1[prev].
    auto score = [&](int st_, f32x16& acc) __attribute__((always_inline)) {
        const u32x4* stg = ring[wave][st_];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 2 * q + lhalf;
            // rows past LROWS hold no block: their lanes score zeros
            const int lr = lrow < LROWS ? lrow : 0;
            f32x4 x = __builtin_bit_cast(f32x4, stg[W_SLOTS + lr * LR + (c ^ swz_rows<LR>(lr))]);
            if (LROWS < 32 && lrow >= LROWS) x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] = x[e];
        }
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const u32x4 w = stg[lrow * WR + ((2 * s + lhalf) ^ swz_rows<WR>(lrow))];
            acc = mfma32x32x16(w, u[s], acc);
        }
    };
    auto consume = [&](int it, const f32x16& acc) __attribute__((always_inline)) {
        const int vt = cbase + it * 32;
        const bool plain = vt + 32 > V || (KL > 1 && it == 0 && !bounded);
        insert_scores<KL, VW>(list, acc, vt, V, active, plain, tau, (lds_float*)&s_thr[wave][lrow],
                              thr_v + nbw * VW * 32, vb);
    };
    // One iteration: the stage of tile it (already read into `cur`) is
    // refilled with tile it + NS, tile it + 1 is waited for and scored, then
    // tile it is consumed, so the matrix pipe and every stage's copy run while
    // the wave inserts.
    auto step_tile = [&](int it, int& st, const f32x16& cur, f32x16& nxt) __attribute__((always_inline)) {
        if (it + NS < n) {
            wait_lds_reads();
            asm volatile("" ::: "memory");
            issue(st, it + NS);
        }
        const int nst = st + 1 == NS ? 0 : st + 1;
        if (it + 1 < n) {
            // copies issued after tile it + 1: the prologue's NS tiles (with
            // copies of the last tile when n < NS), then one per iteration
            const int newer = n >= NS ? min(NS - 1, n - 2 - it) : NS - 2 - it;
            wait_stages<LW, NS - 1>(newer);
            asm volatile("" ::: "memory");
            score(nst, nxt);
        }
        consume(it, cur);
        st = nst;
    };
    int st = 0;
    f32x16 S0, S1;
    score(0, S0);
    for (int it = 0; it < n; it += 2) {
        step_tile(it, st, S0, S1);
        if (it + 1 < n) step_tile(it + 1, st, S1, S0);
    }

    // Merge: the lane pair that holds the same block, then the VW waves of
    // the block group through LDS (each wave's list in its own ring, whose
    // copies have all landed).
    {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[i], 32);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list, other[i]);
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    if (lhalf == 0) {
        u64* s_list = reinterpret_cast<u64*>(&ring[wave][0][0]);
#pragma unroll
        for (int i = 0; i < KL; ++i) s_list[lrow * KL + i] = list[i];
    }
    __syncthreads();
    if (vb == 0 && lhalf == 0 && active) {
#pragma unroll
        for (int w = 1; w < VW; ++w) {
            const u64* o = reinterpret_cast<const u64*>(&ring[wave + w][0][0]);
#pragma unroll
            for (int i = 0; i < KL; ++i) topk_insert<KL>(list, o[lrow * KL + i]);
        }
        if (a.top_k > 1) {
            u64* p = a.partials + (((long)j * B + bme) * a.nwg + g) * a.top_k;
#pragma unroll
            for (int i = 0; i < KL; ++i)
                if (i < a.top_k) p[i] = list[i];
        }
        if (list[0] != 0ull) atomicMax(winner_word(a.winners, a.wstride, j, g, bme), list[0]);
    }
}

// ---- pruned step kernel (after a projection that left slab maxima) ---------

// The step of a proposal whose projection left the slab maxima and the bins
// (kernels.hpp): per-wave rings as in chain_step_wave, but a wave streams only
// the kSlabCols-column slabs in which some block of its group can still reach
// its top k, and of those only the logits rows of such blocks.
//
// Skip rule. Let Bg = max_v |markov_w2[v]| max_p |markov_w1[p]| bound the
// Markov term of any column under any previous token (Cauchy-Schwarz). The
// KL columns behind the block's KL largest bins score at least kth - Bg, so
// its KL-th best score is at least that; a column c of slab s scores at most
// smax[s] + Bg. Slab s can therefore hold none of the block's top KL when
// smax[s] < kth - 2 Bg (less margins for the fp32 rounding of the scores and
// of the norms). Neither side depends on the previous token, so the skip
// masks are known before the Markov row is gathered. Inside a streamed slab
// the per-block filter of chain_step_wave applies, from the tighter bound
// with the block's own |markov_w1[prev]|.
//
// Work split: wave w of the G * VW waves of a block group owns a contiguous
// run of slabs; it examines them in passes of up to 64 (one per lane), and a
// pass streams the compacted list of the slabs some block needs, two 32-column
// steps each. A skipped block's logits rows are not read: its copies read one
// fixed 16-byte chunk instead (the slab maxima's first, hot in the caches),
// and its scores in that slab are ignored. No workgroup barrier inside the
// loop; the workgroup merges and publishes once per slot as chain_step_wave.
template <int NB, int KL, int RS, int NS, int LROWS>
__global__ __launch_bounds__(256) void chain_step_sparse(ChainArgs a, int j) {
    constexpr int VW = kWaves / NB;         // waves per block group
    constexpr int WR = 2 * RS;              // 16-byte chunks per staged markov_w2 row
    constexpr int WRd = WR > 0 ? WR : 1;
    constexpr int LR = 8;                   // 16-byte chunks per staged logits row (32 columns)
    constexpr int W_SLOTS = 32 * WR;
    constexpr int L_SLOTS = LROWS * LR;
    constexpr int STAGE = W_SLOTS + L_SLOTS;
    constexpr int W_INST = W_SLOTS / 64, L_INST = L_SLOTS / 64;
    constexpr int LW = W_INST + L_INST;     // copies per step per wave
    static_assert(NB == 1 || NB == 2, "one or two block groups");
    static_assert(NS >= 2 && NS * LW + RS < 64, "vmcnt range");
    static_assert(LROWS == 8 || LROWS == 16 || LROWS == 32, "staged logits rows");
    static_assert(RS * 64 <= STAGE, "W1 rows fit one stage");
    static_assert(KL * 32 * 8 <= NS * STAGE * 16, "list merge reuses a wave's ring");
    static_assert(kSlabCols == 64, "two 32-column steps per slab");
    __shared__ u32x4 ring[kWaves][NS][STAGE];
    __shared__ float s_thr[kWaves][32];            // top-k bounds shared by the waves of a group
    __shared__ float s_kth[64];                    // the blocks' k-th slab maxima
    __shared__ uint32_t s_w2n2[64], s_w1n2[64];    // the norm words (every word the same)
    __shared__ float s_skip[kWaves][32];           // per wave: skip threshold of each block
    __shared__ int s_slab[kWaves][64];             // per wave: the pass's needed slabs
    __shared__ uint32_t s_need[kWaves][64];        // and their block masks

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int vb = wave % VW, nbw = wave / VW;
    if (a.stop && j >= *a.stop) return;   // adaptive gate: every block was cut
    const int bbase = blockIdx.y * NB * 32;
    load_bound(a, j, bbase, s_kth, s_w2n2, wave, lane, s_w1n2);
    const int B = a.B, V = a.V, r = a.r;
    const int nS = (V + kSlabCols - 1) / kSlabCols;
    const long GW = (long)gridDim.x * VW, wg = (long)blockIdx.x * VW + vb;
    const int gbase = bbase + nbw * 32;      // first block of this wave's group
    // the wave's slabs (none for a group past the last block)
    const int sb0 = (int)(nS * wg / GW), sb1 = gbase < B ? (int)(nS * (wg + 1) / GW) : sb0;
    const int bme = gbase + lrow;
    const bool active = bme < B && !block_cut(a, bme, j);
    // blocks of the group that exist and are not cut, as a mask over the
    // group's 32 blocks (lanes 0-31 hold them)
    const uint32_t exist = (uint32_t)(__ballot(active) & 0xFFFFFFFFull);
    // slab maxima of the first pass (register loads issued before the wait
    // below, so they travel with the previous tokens): lane k reads slab
    // pb + k of each of the group's blocks that can exist (rows b * n_pred +
    // j; LROWS bounds them: B <= LROWS for one group)
    float sm[LROWS];
    auto load_smax = [&](int pb) __attribute__((always_inline)) {
        const int sl = min(pb + lane, sb1 - 1);   // (sb1 > pb whenever it is called)
        const float* col = a.smax + ((long)gbase * a.n_pred + j) * nS + sl;
#pragma unroll
        for (int k = 0; k < LROWS; ++k)
            // rows of blocks past B are not read (their row is clamped; the
            // need mask drops blocks outside `exist`). Nothing here uses the
            // values, so every load is issued before the first wait.
            sm[k] = col[(long)min(k, B - 1 - gbase) * a.n_pred * nS];
    };
    if (sb0 < sb1) load_smax(sb0);
    // (a compiler barrier: without it the first pass's loads are merged with
    // the loop's and issued after the wait below, one more round trip)
    asm volatile("" ::: "memory");
    const int prev = active ? prev_token(a, j, bme, vb == 0) : 0;
    if (lhalf == 0) s_thr[wave][lrow] = -INFINITY;
    wait_lds_reads();
    wait_vmcnt<0>();   // the bound's copies, the slab maxima and the previous tokens
    block_barrier();

    // Skip threshold of this lane's block (lanes 0-31), from the KL-th largest
    // bin and the global bound Bg of the Markov term.
    {
        const float kth = s_kth[nbw * 32 + lrow];
        const float bg = sqrtf(__uint_as_float(s_w2n2[0])) * sqrtf(__uint_as_float(s_w1n2[0]));
        const float skip = kth - 2.0f * bg * 1.001f - 2e-4f * (1.0f + fabsf(kth));
        if (lhalf == 0) s_skip[wave][lrow] = skip;
    }

    // Per-lane fixed part of the copies of a step: markov_w2 chunk (row offset
    // within the step, rank chunk) and logits chunk (block row, column).
    int w_row[W_INST > 0 ? W_INST : 1], w_k[W_INST > 0 ? W_INST : 1], l_row[L_INST], l_col[L_INST];
#pragma unroll
    for (int i = 0; i < W_INST; ++i) {
        const int slot = i * 64 + lane, row = slot / WRd;
        const int c = (slot % WRd) ^ swz_rows<WR>(row);
        w_row[i] = row;
        w_k[i] = c * 8 < r ? c * 8 : 0;   // rank padding: any valid chunk
    }
#pragma unroll
    for (int i = 0; i < L_INST; ++i) {
        const int slot = i * 64 + lane, row = slot / LR;
        l_row[i] = row;
        l_col[i] = 4 * ((slot % LR) ^ swz_rows<LR>(row));
    }
    lds_char* ring_dma = (lds_char*)(lds_ptr)&ring[wave][0][0];
    asm volatile("" : "+s"(ring_dma));
    lds_vfloat* thr_v = (lds_vfloat*)&s_thr[0][0];

    int my_slab = 0;          // lane k: slab of entry k of the pass's list
    uint32_t my_need = 0u;    // and its block mask
    // Step t of the pass: slab entry t / 2, columns v0 .. v0 + 31.
    auto step_slab = [&](int t) __attribute__((always_inline)) {
        return __builtin_amdgcn_readlane(my_slab, t >> 1);
    };
    auto step_need = [&](int t) __attribute__((always_inline)) {
        return (uint32_t)__builtin_amdgcn_readlane((int)my_need, t >> 1);
    };
    auto copy = [&](bool w, const void* p, int st, int slot0) __attribute__((always_inline)) {
        lds_ptr d = (lds_ptr)(ring_dma + (st * STAGE + slot0) * 16);
        if (w) __builtin_amdgcn_global_load_lds(p, d, 16, 0, 0);
        else __builtin_amdgcn_global_load_lds(p, d, 16, 0, kLoadNT);
    };
    const void* dummy = a.smax;
    auto issue = [&](int st, int t) __attribute__((always_inline)) {
        const int v0 = step_slab(t) * kSlabCols + (t & 1) * 32;
        const uint32_t need = step_need(t);
#pragma unroll
        for (int i = 0; i < W_INST; ++i) {
            const int row = min(v0 + w_row[i], V - 1);   // columns past V: row V - 1, never scored
            copy(true, a.w2 + (long)row * r + w_k[i], st, i * 64);
        }
#pragma unroll
        for (int i = 0; i < L_INST; ++i) {
            const int b = gbase + l_row[i];
            const int col = min(v0 + l_col[i], V - 4);
            const void* p = ((need >> l_row[i]) & 1u)
                                ? (const void*)(a.logits + ((long)b * a.n_pred + j) * V + col)
                                : dummy;
            copy(false, p, st, W_SLOTS + i * 64);
        }
    };

    u32x4 u[RS > 0 ? RS : 1];
    bool have_u = false;
    float tau = -INFINITY;   // the block's top-k bound (with its own markov_w1 row)
    u64 list[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) list[i] = 0ull;

    auto score = [&](int st_, f32x16& acc) __attribute__((always_inline)) {
        const u32x4* stg = ring[wave][st_];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 2 * q + lhalf;
            const int lr = lrow < LROWS ? lrow : 0;
            f32x4 x = __builtin_bit_cast(f32x4, stg[W_SLOTS + lr * LR + (c ^ swz_rows<LR>(lr))]);
            if (LROWS < 32 && lrow >= LROWS) x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] = x[e];
        }
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const u32x4 w = stg[lrow * WR + ((2 * s + lhalf) ^ swz_rows<WR>(lrow))];
            acc = mfma32x32x16(w, u[s], acc);
        }
    };
    auto consume = [&](int t, const f32x16& acc) __attribute__((always_inline)) {
        const int vt = step_slab(t) * kSlabCols + (t & 1) * 32;
        // this lane's block is streamed in this slab
        const bool on = active && ((step_need(t) >> lrow) & 1u);
        insert_scores<KL, VW>(list, acc, vt, V, on, vt + 32 > V, tau, (lds_float*)&s_thr[wave][lrow],
                              thr_v + nbw * VW * 32, vb);
    };

    for (int pb = sb0; pb < sb1; pb += 64) {
        if (pb != sb0) load_smax(pb);
        // the need masks of the pass's slabs (lane k: slab pb + k)
        uint32_t need = 0u;
        if (pb + lane < sb1) {
#pragma unroll
            for (int k = 0; k < LROWS; ++k) need |= (sm[k] >= s_skip[wave][k] ? 1u : 0u) << k;
            need &= exist;
        }
        // compact the slabs some block needs into entries 0 .. cnt - 1
        const u64 bal = __builtin_amdgcn_ballot_w64(need != 0u);
        const int cnt = __builtin_popcountll(bal);
        if (need != 0u) {
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            s_slab[wave][pos] = pb + lane;
            s_need[wave][pos] = need;
        }
        wait_lds_reads();
        my_slab = lane < cnt ? s_slab[wave][lane] : 0;
        my_need = lane < cnt ? s_need[wave][lane] : 0u;
        const int n = 2 * cnt;   // 32-column steps of the pass
        if (n == 0) continue;

        // Prologue: step 0, the markov_w1 rows of prev into stage NS - 1 (the
        // first pass with work only), steps 1 .. NS - 2; then step NS - 1 into
        // stage NS - 1 once the rows are in registers. A stage past the last
        // step gets a second copy of it (no iteration reads it), so the number
        // of copies in flight is fixed.
        issue(0, 0);
        const bool first = !have_u;
        if (first) {
#pragma unroll
            for (int s = 0; s < RS; ++s) {
                const int k0 = s * 16 + lhalf * 8;
                __builtin_amdgcn_global_load_lds((const void*)(a.w1 + (long)prev * r + (k0 < r ? k0 : 0)),
                                                 (lds_ptr)(ring_dma + ((NS - 1) * STAGE + s * 64) * 16), 16, 0, 0);
            }
        }
#pragma unroll
        for (int t = 1; t < NS - 1; ++t) issue(t, min(t, n - 1));
        wait_vmcnt<(NS - 2) * LW>();
        asm volatile("" ::: "memory");
        if (first) {
#pragma unroll
            for (int s = 0; s < RS; ++s) {
                u[s] = ring[wave][NS - 1][s * 64 + lane];
                if (s * 16 + lhalf * 8 >= r) u[s] = u32x4{0u, 0u, 0u, 0u};
            }
            have_u = true;
            if constexpr (KL > 1) {
                const float un2 = w1_norm2<RS>(u);
                tau = chain_bound(s_kth[nbw * 32 + lrow], __uint_as_float(s_w2n2[0]), un2);
            }
        }
        asm volatile("" ::: "memory");
        wait_lds_reads();
        asm volatile("" ::: "memory");
        issue(NS - 1, min(NS - 1, n - 1));

        auto step_tile = [&](int it, int& st, const f32x16& cur, f32x16& nxt) __attribute__((always_inline)) {
            if (it + NS < n) {
                wait_lds_reads();
                asm volatile("" ::: "memory");
                issue(st, it + NS);
            }
            const int nst = st + 1 == NS ? 0 : st + 1;
            if (it + 1 < n) {
                const int newer = n >= NS ? min(NS - 1, n - 2 - it) : NS - 2 - it;
                wait_stages<LW, NS - 1>(newer);
                asm volatile("" ::: "memory");
                score(nst, nxt);
            }
            consume(it, cur);
            st = nst;
        };
        int st = 0;
        f32x16 S0, S1;
        score(0, S0);
        for (int it = 0; it < n; it += 2) {
            step_tile(it, st, S0, S1);
            if (it + 1 < n) step_tile(it + 1, st, S1, S0);
        }
        // every copy of the pass (extra ones included) has landed and been
        // read before the next pass refills the ring
        wait_vmcnt<0>();
        wait_lds_reads();
        asm volatile("" ::: "memory");
    }

    // Merge: the lane pair that holds the same block, then the VW waves of
    // the block group through LDS (each wave's list in its own ring).
    {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[i], 32);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list, other[i]);
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    if (lhalf == 0) {
        u64* s_list = reinterpret_cast<u64*>(&ring[wave][0][0]);
#pragma unroll
        for (int i = 0; i < KL; ++i) s_list[lrow * KL + i] = list[i];
    }
    __syncthreads();
    if (vb == 0 && lhalf == 0 && active) {
#pragma unroll
        for (int w = 1; w < VW; ++w) {
            const u64* o = reinterpret_cast<const u64*>(&ring[wave + w][0][0]);
#pragma unroll
            for (int i = 0; i < KL; ++i) topk_insert<KL>(list, o[lrow * KL + i]);
        }
        const int g = blockIdx.x;
        if (a.top_k > 1) {
            u64* p = a.partials + (((long)j * B + bme) * a.nwg + g) * a.top_k;
#pragma unroll
            for (int i = 0; i < KL; ++i)
                if (i < a.top_k) p[i] = list[i];
        }
        if (list[0] != 0ull) atomicMax(winner_word(a.winners, a.wstride, j, g, bme), list[0]);
    }
}

// ---- step kernel for any V: operands read straight from global memory --------

template <int NB, int KL, int RS>
__global__ __launch_bounds__(256) void chain_step_direct(ChainArgs a, int j) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    if (a.stop && j >= *a.stop) return;   // adaptive gate: every block was cut
    const int bbase = blockIdx.y * NB * 32;
    const int B = a.B, V = a.V, r = a.r;
    __shared__ u64 s_list[kWaves][NB * 32][KL];

    u32x4 u[NB][RS];
    int bl[NB];
    gather_w1<NB, RS>(a, j, bbase, lrow, lhalf, u, bl);

    u64 list[NB][KL];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < KL; ++i) list[nb][i] = 0ull;

    const int v0 = blockIdx.x * kChainTileV + wave * 32;
    if (v0 < V) {
        const int vrow = v0 + lrow;
        u32x4 w[RS];
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int k0 = s * 16 + lhalf * 8;
            w[s] = (vrow < V && k0 < r) ? *reinterpret_cast<const u32x4*>(a.w2 + (long)vrow * r + k0)
                                        : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            // The logits enter the MFMA as accumulator input, as in the
            // pipelined kernel, so both kernels round the same sums.
            const int b = bl[nb];
            const float* row = a.logits + ((long)min(b, B - 1) * a.n_pred + j) * V;
            f32x16 acc;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int vq = v0 + 8 * q + 4 * lhalf;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * q + e] = (vq + e < V) ? row[vq + e] : 0.0f;
            }
            if (r > 0) {
#pragma unroll
                for (int s = 0; s < RS; ++s) acc = mfma32x32x16(w[s], u[nb][s], acc);
            }
            if (b >= B) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int vq = v0 + 8 * q + 4 * lhalf;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = vq + e;
                    topk_insert<KL>(list[nb], v < V ? make_key(acc[4 * q + e], v) : 0ull);
                }
            }
        }
    }
    publish<NB, KL>(a, j, bbase, list, s_list);
}

// ---- final assembly: one workgroup per (slot, block) --------------------------

// Confidence of one slot on one wave: float(sigmoid(hidden_row . conf_w)),
// fp32 hidden rounded to bf16 first.
template <bool F32>
__device__ __forceinline__ float slot_conf_dot(const void* hidden, const uint16_t* conf_w, long row, int H,
                                               int lane) {
    // Lane l sums h = 8l + 512i .. + 8 for i = 0, 1, ... in that order. The
    // loads of sixteen such chunks (H up to 8192 in one round) go out
    // together, raw, and are converted after (a chunk past H reads the lane's
    // first chunk again and adds nothing). The hidden dtype is a template
    // parameter: a branch on it among the loads would have them waited for
    // one chunk at a time.
    constexpr int U = 16;
    float s = 0.0f;
    for (int h0 = lane * 8; h0 < H; h0 += 64 * 8 * U) {
        u32x4 cw[U], hv[U];
        f32x4 hf[F32 ? U : 1][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int h = h0 + u * 64 * 8 < H ? h0 + u * 64 * 8 : lane * 8;
            cw[u] = *reinterpret_cast<const u32x4*>(conf_w + h);
            if constexpr (F32) {
                const f32x4* hp = reinterpret_cast<const f32x4*>(static_cast<const float*>(hidden) + row * H + h);
                hf[u][0] = hp[0];
                hf[u][1] = hp[1];
            } else {
                hv[u] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(hidden) + row * H + h);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (h0 + u * 64 * 8 >= H) break;
            if constexpr (F32) {
                // fp32 hidden values rounded to bf16 (RNE), as the projection reads them
                hv[u][0] = pack_bf16x2(hf[u][0][0], hf[u][0][1]);
                hv[u][1] = pack_bf16x2(hf[u][0][2], hf[u][0][3]);
                hv[u][2] = pack_bf16x2(hf[u][1][0], hf[u][1][1]);
                hv[u][3] = pack_bf16x2(hf[u][1][2], hf[u][1][3]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s += bf16_lo(hv[u][q]) * bf16_lo(cw[u][q]);
                s += bf16_hi(hv[u][q]) * bf16_hi(cw[u][q]);
            }
        }
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, 64);
    return s;
}
__device__ __forceinline__ float slot_conf(const void* hidden, int hidden_f32, const uint16_t* conf_w,
                                           long row, int H, int lane) {
    const float s = hidden_f32 ? slot_conf_dot<true>(hidden, conf_w, row, H, lane)
                               : slot_conf_dot<false>(hidden, conf_w, row, H, lane);
    return 1.0f / (1.0f + expf(-s));
}

// Output id of a key: the target id of its column (the column without d2t).
__device__ __forceinline__ int final_token(const FinalArgs& a, u64 key) {
    const int c = key_id(key);
    return (c >= 0 && c < a.V) ? (int)column_token(a.d2t, c) : c;
}

// Final step of a proposal, for every block b and slot j: the slot's
// confidence, with lengths[b] (preset to n_pred) lowered to j when conf <
// p_min so that it ends at the first such slot (llama.cpp commit 6fed9f6,
// "spec: add confidence-based draft pruning for DSpark" and "dspark: fold
// conf_min into p_min"); the token from the running argmax; and the
// candidates, merged from the per-workgroup partial lists. Two shapes, the
// same results:
//  * finalize_group: one workgroup per (slot, block), eight keys per thread
//    in flight, then a wave merge and an LDS merge;
//  * finalize_wave: two waves per (block, slot), two pairs per workgroup:
//    the candidates (16 keys per lane in flight, then a wave merge) on one,
//    the confidence on the other. With many pairs a workgroup per pair costs
//    more in launch and dispatch than in merging (at B = 64, 1024 pairs: 31
//    us, against 22 with one wave per pair and 14 with two); with few (B = 8:
//    128 pairs) it spreads the merge over more CUs (12 against 14.5 us).

template <int KL>
__global__ __launch_bounds__(256) void finalize_group(FinalArgs a) {
    const int j = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int B = a.B, n = a.n_pred, k = a.top_k;
    const long o = (long)b * n + j;
    const u64 win = winner_key(a.winners, a.wstride, j, b);
    __shared__ u64 s_list[kWaves][KL];

    // Adaptive gate: a slot past its block's cut was not drafted, and a block
    // keeps only its own number of candidates.
    const int kb = a.top_k_b ? min(max(a.top_k_b[b], 1), k) : k;
    if (a.gated && j >= a.lengths[b]) {
        for (int i = threadIdx.x; i < k; i += 256) {
            a.candidates[o * k + i] = -1;
            if (a.cand_logits) a.cand_logits[o * k + i] = -INFINITY;
        }
        if (threadIdx.x == 0) a.tokens[o] = -1;
        return;
    }

    if (k == 1) {
        if (threadIdx.x == 0) {
            const int t = final_token(a, win);
            a.tokens[o] = t;
            a.candidates[o] = t;
            if (a.cand_logits) a.cand_logits[o] = key_score(win);
        }
    } else {
        u64 list[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) list[i] = 0ull;
        const u64* p = a.partials + ((long)j * B + b) * a.nwg * k;
        const int cnt = a.nwg * k;
        // eight independent loads at a time, then their inserts
        for (int e0 = threadIdx.x; e0 < cnt; e0 += 256 * 8) {
            u64 kk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kk[u] = e0 + u * 256 < cnt ? p[e0 + u * 256] : 0ull;
#pragma unroll
            for (int u = 0; u < 8; ++u) topk_insert<KL>(list, kk[u]);
        }
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) {
            u64 other[KL];
#pragma unroll
            for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[i], mask);
#pragma unroll
            for (int i = 0; i < KL; ++i) topk_insert<KL>(list, other[i]);
        }
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < KL; ++i) s_list[wave][i] = list[i];
        }
        __syncthreads();
        if (threadIdx.x == 0) {
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
#pragma unroll
                for (int i = 0; i < KL; ++i) topk_insert<KL>(list, s_list[w][i]);
            a.tokens[o] = final_token(a, win);
            if (list[0] != win) atomicOr(a.flags, kFlagInternal);  // internal consistency check
#pragma unroll
            for (int i = 0; i < KL; ++i) {
                if (i < k) {
                    a.candidates[o * k + i] = i < kb ? final_token(a, list[i]) : -1;
                    if (a.cand_logits) a.cand_logits[o * k + i] = i < kb ? key_score(list[i]) : -INFINITY;
                }
            }
        }
    }

    // Confidence head on wave 1 (wave 0 may still be writing candidates);
    // with the adaptive gate it was computed before the chain.
    if (!a.gated && wave == 1 % kWaves) {
        float c = 1.0f;
        if (a.conf_w) {
            c = slot_conf(a.hidden, a.hidden_f32, a.conf_w, (long)b * a.L + a.i_first + j, a.H, lane);
            if (lane == 0 && c < a.p_min) atomicMin(a.lengths + b, j);
        }
        if (lane == 0 && a.conf) a.conf[o] = c;
    }
}

template <int KL>
__global__ __launch_bounds__(256) void finalize_wave(FinalArgs a) {
    // two waves per (block, slot), pair = b * n_pred + j the output row: the
    // candidates on the even wave and the confidence on the odd one, side by
    // side (in one wave the two ran one after the other: 6.7 + 10.6 us)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int B = a.B, n = a.n_pred, k = a.top_k;
    const long o = (long)blockIdx.x * (kWaves / 2) + (wave >> 1);
    if (o >= (long)B * n) return;
    const int b = (int)(o / n), j = (int)(o - (long)b * n);
    if (wave & 1) {
        // Confidence head (with the adaptive gate it was computed before the chain).
        if (!a.gated) {
            float c = 1.0f;
            if (a.conf_w) {
                c = slot_conf(a.hidden, a.hidden_f32, a.conf_w, (long)b * a.L + a.i_first + j, a.H, lane);
                if (lane == 0 && c < a.p_min) atomicMin(a.lengths + b, j);
            }
            if (lane == 0 && a.conf) a.conf[o] = c;
        }
        return;
    }

    // Adaptive gate: a slot past its block's cut was not drafted, and a block
    // keeps only its own number of candidates.
    const int kb = a.top_k_b ? min(max(a.top_k_b[b], 1), k) : k;
    if (a.gated && j >= a.lengths[b]) {
        for (int i = lane; i < k; i += kWave) {
            a.candidates[o * k + i] = -1;
            if (a.cand_logits) a.cand_logits[o * k + i] = -INFINITY;
        }
        if (lane == 0) a.tokens[o] = -1;
        return;
    }
    const u64 win = winner_key(a.winners, a.wstride, j, b);

    // the first keys of the partial lists, 16 per lane in flight
    constexpr int U = 16;
    const u64* p = a.partials + ((long)j * B + b) * a.nwg * k;
    const int cnt = k > 1 ? a.nwg * k : 0;
    u64 kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kk[u] = lane + u * kWave < cnt ? p[lane + u * kWave] : 0ull;

    if (k == 1) {
        if (lane == 0) {
            const int t = final_token(a, win);
            a.tokens[o] = t;
            a.candidates[o] = t;
            if (a.cand_logits) a.cand_logits[o] = key_score(win);
        }
        return;
    }
    u64 list[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) list[i] = 0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) topk_insert<KL>(list, kk[u]);
    for (int e0 = lane + U * kWave; e0 < cnt; e0 += U * kWave) {
#pragma unroll
        for (int u = 0; u < U; ++u) kk[u] = e0 + u * kWave < cnt ? p[e0 + u * kWave] : 0ull;
#pragma unroll
        for (int u = 0; u < U; ++u) topk_insert<KL>(list, kk[u]);
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[i], mask);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list, other[i]);
    }
    if (lane == 0) {
        a.tokens[o] = final_token(a, win);
        if (list[0] != win) atomicOr(a.flags, kFlagInternal);  // internal consistency check
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            if (i < k) {
                a.candidates[o * k + i] = i < kb ? final_token(a, list[i]) : -1;
                if (a.cand_logits) a.cand_logits[o * k + i] = i < kb ? key_score(list[i]) : -INFINITY;
            }
        }
    }
}

// ---- adaptive gate: confidences before the chain ------------------------------

// Slot j of block b on one wave: conf, and lengths[b] lowered to j when
// conf < p_min[b] (per-block thresholds).
__global__ __launch_bounds__(64) void conf_gate(GateArgs g) {
    const int j = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const float c = slot_conf(g.hidden, g.hidden_f32, g.conf_w, (long)b * g.L + g.i_first + j, g.H, lane);
    if (lane == 0) {
        if (g.conf) g.conf[(long)b * g.n_pred + j] = c;
        if (c < g.p_min[b]) atomicMin(g.lengths + b, j);
    }
}

// The number of slots the chain has to run: the longest surviving block.
__global__ __launch_bounds__(256) void gate_stop(const int32_t* lengths, int B, int32_t* stop) {
    __shared__ int s_max[kWaves];
    int m = 0;
    for (int b = threadIdx.x; b < B; b += 256) m = max(m, lengths[b]);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) m = max(m, __shfl_xor(m, mask, kWave));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = s_max[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t = max(t, s_max[w]);
        *stop = t;
    }
}

// Dispatch check: while set (on the calling host thread) launch_chain_step
// selects its kernel exactly as for a launch and then launches nothing.
thread_local bool g_dry_dispatch = false;

// The status of a launch that the selection reached.
inline hipError_t launched() { return g_dry_dispatch ? hipSuccess : hipGetLastError(); }

template <int NB, int KL>
hipError_t step_direct(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    const int rs = (a.r + 15) / 16;
#define DSPARK_STEP(RSV) \
    if (!g_dry_dispatch) hipLaunchKernelGGL((chain_step_direct<NB, KL, RSV>), grid, dim3(256), 0, s, a, j);
    if (rs <= 1) { DSPARK_STEP(1) }
    else if (rs <= 2) { DSPARK_STEP(2) }
    else if (rs <= 4) { DSPARK_STEP(4) }
    else if (rs <= 8) { DSPARK_STEP(8) }
    else { DSPARK_STEP(16) }
#undef DSPARK_STEP
    return launched();
}

template <int NB, int KL>
hipError_t step_pipe(const ChainArgs& a, int j, dim3 grid, bool two, hipStream_t s) {
    const int rs = (a.r + 15) / 16;
#define DSPARK_STEP(RSV, NSV, VWV) \
    if (!g_dry_dispatch) hipLaunchKernelGGL((chain_step_pipe<NB, KL, RSV, NSV, VWV>), grid, dim3(256), 0, s, a, j);
    // Two stages and two workgroups per CU (kChainPipeTwo: top-k lists over
    // two block groups, rank up to 128); three stages, one workgroup per CU,
    // for the widest rank (kChainPipeDeep).
    if (two) {
        if constexpr (NB == 2) {
            if (rs == 0) { DSPARK_STEP(0, 2, 2) }
            else if (rs <= 2) { DSPARK_STEP(2, 2, 2) }
            else if (rs <= 4) { DSPARK_STEP(4, 2, 2) }
            else if (rs <= 8) { DSPARK_STEP(8, 2, 2) }
            else return hipErrorInvalidValue;   // chain_form never picks this form for it
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        if (rs > 8) { DSPARK_STEP(16, 3, 2) }
        else return hipErrorInvalidValue;   // narrower ranks take the other forms
    }
#undef DSPARK_STEP
    return launched();
}

// Per-wave rings: as many stages as fit the workgroup's share of the CU's
// LDS (chain_wave_per_cu), at most 8.
template <int RS, int LROWS, int WPC>
constexpr int chain_wave_stages() {
    const int n = (WPC == 2 ? kChainWaveBudget2 : kChainWaveBudget1) / (4 * chain_wave_stage_bytes(RS, LROWS));
    return n > 8 ? 8 : n;
}

template <int NB, int KL, int LROWS>
hipError_t step_wave_rows(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    const int rs = chain_wave_rank(a.r);
    const bool two = chain_wave_per_cu(a.B, a.r, a.top_k) == 2;
#define DSPARK_STEP(RSV, WPCV)                                                                 \
    if (!g_dry_dispatch)                                                                       \
        hipLaunchKernelGGL((chain_step_wave<NB, KL, RSV, chain_wave_stages<RSV, LROWS, WPCV>(), LROWS>), \
                           grid, dim3(256), 0, s, a, j);
#define DSPARK_RANK(RSV)                                                                     \
    if constexpr (LROWS < 32 && chain_wave_stages<RSV, LROWS, 2>() >= 2) {                   \
        if (two) { DSPARK_STEP(RSV, 2) }                                                     \
        else { DSPARK_STEP(RSV, 1) }                                                         \
    } else {                                                                                 \
        DSPARK_STEP(RSV, 1)                                                                  \
    }
    if (rs == 0) { DSPARK_RANK(0) }
    else if (rs == 2) { DSPARK_RANK(2) }
    else if (rs == 4) { DSPARK_RANK(4) }
    else if (rs == 8) { DSPARK_RANK(8) }
    else return hipErrorInvalidValue;   // chain_form never picks this form for a wider rank
#undef DSPARK_RANK
#undef DSPARK_STEP
    return launched();
}

// Pruned form: as many stages as fit its budgets (chain_sparse_per_cu), at most 8.
template <int RS, int LROWS, int WPC>
constexpr int chain_sparse_stages() {
    const int n = (WPC == 2 ? kChainSparseBudget2 : kChainSparseBudget1) / (4 * chain_wave_stage_bytes(RS, LROWS));
    return n > 8 ? 8 : n;
}

template <int NB, int KL, int LROWS>
hipError_t step_sparse_rows(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    const int rs = chain_wave_rank(a.r);
    const bool two = chain_sparse_per_cu(a.B, a.r, a.top_k) == 2;
#define DSPARK_STEP(RSV, WPCV)                                                                     \
    if (!g_dry_dispatch)                                                                           \
        hipLaunchKernelGGL((chain_step_sparse<NB, KL, RSV, chain_sparse_stages<RSV, LROWS, WPCV>(), LROWS>), \
                           grid, dim3(256), 0, s, a, j);
#define DSPARK_RANK(RSV)                                                                         \
    if constexpr (LROWS < 32 && chain_sparse_stages<RSV, LROWS, 2>() >= 2) {                     \
        if (two) { DSPARK_STEP(RSV, 2) }                                                         \
        else { DSPARK_STEP(RSV, 1) }                                                             \
    } else {                                                                                     \
        DSPARK_STEP(RSV, 1)                                                                      \
    }
    if (rs == 0) { DSPARK_RANK(0) }
    else if (rs == 2) { DSPARK_RANK(2) }
    else if (rs == 4) { DSPARK_RANK(4) }
    else if (rs == 8) { DSPARK_RANK(8) }
    else return hipErrorInvalidValue;   // chain_sparse excludes wider ranks
#undef DSPARK_RANK
#undef DSPARK_STEP
    return launched();
}

template <int NB, int KL>
hipError_t step_sparse(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    if constexpr (NB == 1 && KL <= 4) {
        const int lr = chain_wave_rows(a.B, a.top_k);
        if (lr == 8) return step_sparse_rows<NB, KL, 8>(a, j, grid, s);
        if (lr == 16) return step_sparse_rows<NB, KL, 16>(a, j, grid, s);
    }
    return step_sparse_rows<NB, KL, 32>(a, j, grid, s);
}

template <int NB, int KL>
hipError_t step_wave(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    if constexpr (NB == 1 && KL <= 4) {
        const int lr = chain_wave_rows(a.B, a.top_k);
        if (lr == 8) return step_wave_rows<NB, KL, 8>(a, j, grid, s);
        if (lr == 16) return step_wave_rows<NB, KL, 16>(a, j, grid, s);
    }
    return step_wave_rows<NB, KL, 32>(a, j, grid, s);
}

template <int NB, int KL>
hipError_t step_form(const ChainArgs& a, int j, dim3 grid, ChainForm f, hipStream_t s) {
    switch (f) {
        case kChainWave:
            // (top-k lists over two block groups take the two-stage ring)
            if constexpr (NB == 2 && KL > 1) return hipErrorInvalidValue;
            else return step_wave<NB, KL>(a, j, grid, s);
        case kChainPipeTwo: return step_pipe<NB, KL>(a, j, grid, true, s);
        case kChainPipeDeep: return step_pipe<NB, KL>(a, j, grid, false, s);
        default: return step_direct<NB, KL>(a, j, grid, s);
    }
}

template <int NB>
hipError_t step_kl(const ChainArgs& a, int j, dim3 grid, ChainForm f, hipStream_t s) {
    if (a.sparse) {
        if (a.top_k == 1) return step_sparse<NB, 1>(a, j, grid, s);
        if (a.top_k <= 4) return step_sparse<NB, 4>(a, j, grid, s);
        if (a.top_k <= 8) return step_sparse<NB, 8>(a, j, grid, s);
        return step_sparse<NB, 16>(a, j, grid, s);
    }
    if (a.top_k == 1) return step_form<NB, 1>(a, j, grid, f, s);
    if (a.top_k <= 4) return step_form<NB, 4>(a, j, grid, f, s);
    if (a.top_k <= 8) return step_form<NB, 8>(a, j, grid, f, s);
    return step_form<NB, 16>(a, j, grid, f, s);
}

}  // namespace

hipError_t launch_chain_init(const ChainArgs& a, hipStream_t stream) {
    const int nw = a.n_pred * kWinnerWays * a.wstride;   // < 2^31 (checked on the host)
    const int n = nw > a.B ? nw : a.B;
    hipLaunchKernelGGL(chain_init, dim3((n + 255) / 256), dim3(256), 0, stream, a.winners, nw,
                       a.flags, a.lengths, a.B, a.n_pred, a.w2n2, a.w1n2);
    return hipGetLastError();
}

hipError_t launch_row_kth(const ChainArgs& a, hipStream_t stream) {
    const int M = a.B * a.n_pred, nslab = (a.V + a.slab_cols - 1) / a.slab_cols;
    const dim3 grid(M), block(256);
    if (a.top_k == 1) hipLaunchKernelGGL(row_kth<1>, grid, block, 0, stream, a.smax, nslab, a.kth);
    else if (a.top_k <= 4) hipLaunchKernelGGL(row_kth<4>, grid, block, 0, stream, a.smax, nslab, a.kth);
    else if (a.top_k <= 8) hipLaunchKernelGGL(row_kth<8>, grid, block, 0, stream, a.smax, nslab, a.kth);
    else hipLaunchKernelGGL(row_kth<16>, grid, block, 0, stream, a.smax, nslab, a.kth);
    return hipGetLastError();
}

void set_chain_dry_dispatch(bool on) { g_dry_dispatch = on; }

hipError_t launch_chain_step(const ChainArgs& a, int j, hipStream_t stream) {
    // Blocks are taken 64 at a time (two 32-wide MFMA column groups) so that a
    // markov_w2 tile is read once per step for all of them.
    const int nb = a.B > 32 ? 2 : 1;
    dim3 grid(a.nwg, (a.B + 32 * nb - 1) / (32 * nb));
    const ChainForm f = chain_form(a.B, a.V, a.r, a.top_k);
    return nb == 2 ? step_kl<2>(a, j, grid, f, stream) : step_kl<1>(a, j, grid, f, stream);
}

hipError_t launch_gate(const GateArgs& g, hipStream_t stream) {
    hipLaunchKernelGGL(conf_gate, dim3(g.n_pred, g.B), dim3(64), 0, stream, g);
    hipLaunchKernelGGL(gate_stop, dim3(1), dim3(256), 0, stream, g.lengths, g.B, g.stop);
    return hipGetLastError();
}

hipError_t launch_finalize(const FinalArgs& a, hipStream_t stream) {
    const long pairs = (long)a.B * a.n_pred;
    const dim3 block(256);
#define DSPARK_FINAL(KERNEL, GRID)                                                           \
    if (a.top_k <= 1) hipLaunchKernelGGL(KERNEL<1>, GRID, block, 0, stream, a);              \
    else if (a.top_k <= 4) hipLaunchKernelGGL(KERNEL<4>, GRID, block, 0, stream, a);         \
    else if (a.top_k <= 8) hipLaunchKernelGGL(KERNEL<8>, GRID, block, 0, stream, a);         \
    else hipLaunchKernelGGL(KERNEL<16>, GRID, block, 0, stream, a);
    if (pairs >= kFinalWavePairs) {
        DSPARK_FINAL(finalize_wave, dim3((unsigned)((pairs + kWaves / 2 - 1) / (kWaves / 2))))
    } else {
        DSPARK_FINAL(finalize_group, dim3(a.n_pred, a.B))
    }
#undef DSPARK_FINAL
    return hipGetLastError();
}

}  // namespace dspark
