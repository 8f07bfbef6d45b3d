// Host-side launchers of the gfx950 kernels (internal to libdspark).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// ---- lm_head projection ---------------------------------------------------
// Slab maxima: with them, the projection's epilogue also writes, for every
// row m and every slab of slab_cols columns, the largest projection of the
// row over the slab: smax[m][s], layout [M][ceil(N / slab_cols)]. A pass
// after the projection takes each row's k-th largest slab maximum (a lower
// bound on the row's k-th largest projection: the slabs are disjoint), and
// the chain bounds its top-k scores with it; the pruned chain form also
// skips slabs of kSlabCols columns in which no column can reach a block's
// top k. The four-wave projection kernel takes slabs of kSlabColsWide (one
// wave's columns) when the pruned form does not run: half the epilogue work.
constexpr int kSlabCols = 64;
constexpr int kSlabColsWide = 128;
// Whether launch_lmhead_gemm runs the four-wave kernel for these sizes
// (bf16 hidden, K % 64 == 0, M > 128, 32-bit buffer offsets).
inline bool gemm_four_wave(int M, int K, int L, int n_pred, bool hidden_f32) {
    const long hid_bytes = (long)((M + n_pred - 1) / n_pred) * L * K * 2;
    return !hidden_f32 && K % 64 == 0 && M > 128 && hid_bytes < 0xFFFFFFFFL && 256L * K * 2 < 0x7FFFFFFFL;
}

struct GemmArgs {
    const void* hidden;      // [B, L, H] bf16 bits or fp32
    const uint16_t* lm_head; // [V, H] bf16 bits
    const float* bias;       // [V] or nullptr
    float* out;              // [M, V], M = B * n_pred
    int M, N, K;             // M rows, N = V, K = H
    int L, n_pred, i_first;  // row m reads hidden row (m / n_pred) * L + i_first + m % n_pred
    float* smax;             // slab maxima [M][ceil(N / slab_cols)], or nullptr
    int slab_cols;           // kSlabCols, or kSlabColsWide for the four-wave kernel
    // With w2n2: the largest squared row norms of markov_w2 [w2_rows, w2_rank]
    // and markov_w1 [w1_rows, w2_rank] are raised into *w2n2 and *w1n2 (fp32
    // bits, zeroed before) by w2_groups extra workgroups after the tiles of
    // the launch (they run in its last, partly filled round).
    const uint16_t* w2;
    const uint16_t* w1;
    int w2_rows, w1_rows, w2_rank, w2_groups;
    uint32_t* w2n2;
    uint32_t* w1n2;
};
hipError_t launch_lmhead_gemm(const GemmArgs& a, bool hidden_f32, hipStream_t stream);

// ---- 4-bit lm_head ------------------------------------------------------------
// GGUF plain 4-bit blocks (kQ4Block weights: binary16 scale + 16 code bytes)
// and their packed form: V in tiles of 16 rows, H in quads of 4 blocks, a
// kQ4CodeRec-byte code record and a kQ4ScaleRec-byte scale record per (tile,
// quad); all code records first, then all scale records.
constexpr int kQ4Block = 32, kQ4BlockBytes = 18, kQ4CodeRec = 1024, kQ4ScaleRec = 128;
inline int q4_tiles(int V) { return (V + 15) / 16; }
inline int q4_quads(int H) { return (H / kQ4Block + 3) / 4; }
inline size_t q4_packed_bytes(int V, int H) {
    return (size_t)q4_tiles(V) * q4_quads(H) * (kQ4CodeRec + kQ4ScaleRec);
}

struct Q4PackArgs {
    const uint8_t* blocks;   // [V, G * kQ4BlockBytes]
    uint8_t* packed;         // q4_packed_bytes(V, H)
    int V, G, GQ, T16;       // G = H / 32 blocks per row, GQ = q4_quads(H), T16 = q4_tiles(V)
};
hipError_t launch_q4_pack(const Q4PackArgs& a, hipStream_t stream);

struct Q4Args {
    const void* hidden;      // [B, L, H] bf16 bits or fp32
    int hidden_f32;
    uint16_t* xp;            // [M, 128 * GQ] bf16 bits: hidden rows, each block in the MFMA's k order
    const uint8_t* packed;   // the packed head
    const float* bias;       // [V] or nullptr
    float* out;              // [M, V]
    float* smax;             // slab maxima [M][ceil(V / kSlabCols)] (the top-k bound), or nullptr
    // With w2n2: norm_groups extra workgroups after the projection's raise the
    // largest squared row norms of markov_w2 [w_rows, w_rank] (and, with w1n2,
    // of markov_w1) into the two words, zeroed before (as GemmArgs).
    const uint16_t* w2;
    const uint16_t* w1;
    int w_rows, w_rank, norm_groups;
    uint32_t* w2n2;
    uint32_t* w1n2;
    int M, V, H, G, GQ, T16;
    int L, n_pred, i_first;  // row m reads hidden row (m / n_pred) * L + i_first + m % n_pred
};
// The preparation of xp, then the projection.
hipError_t launch_lmhead_q4(const Q4Args& a, hipStream_t stream);

// ---- Markov chain -----------------------------------------------------------
// Chain step geometry. With V % 4 == 0 a workgroup streams a contiguous range
// of tiles of chain_tile(B, r) columns in one of three forms:
//  * kChainWave: every wave streams its own run of 32-column steps for its
//    own 32 blocks through a private LDS ring, with no workgroup barrier
//    inside the loop; one workgroup per CU (kChainCUs). Rank up to 128.
//  * kChainPipeTwo: one shared two-stage ring per workgroup, two workgroups
//    per CU (kChainMaxWGs).
//  * kChainPipeDeep: one shared three- or four-stage ring, one workgroup per CU.
// Otherwise (V % 4 != 0) the direct kernel runs one workgroup per kChainTileV
// columns. The per-wave form is the faster one for top-1 steps and for one
// block group (8-12% at the Gemma-4 and Qwen3-8B shapes, 3% on the B = 8 top-4
// tree). Top-k lists over two block groups stay on the two-per-CU ring: there
// a wave's inserts are the larger part of a step, and the second workgroup
// on the CU hides them (493 against 533 us per call at B = 64).
constexpr int kChainCUs = 256;
constexpr int kChainMaxWGs = 2 * kChainCUs;
constexpr int kChainTileV = 128;
enum ChainForm { kChainDirect, kChainWave, kChainPipeTwo, kChainPipeDeep };
inline bool chain_pipelined(int V) { return (V & 3) == 0; }
inline int chain_tile(int B, int r) { return (B <= 32 && r <= 128) ? 128 : 64; }
inline ChainForm chain_form(int B, int V, int r, int top_k) {
    if (!chain_pipelined(V)) return kChainDirect;
    if ((r + 15) / 16 > 8) return kChainPipeDeep;
    return (B > 32 && top_k > 1) ? kChainPipeTwo : kChainWave;
}
// Per-wave form: the logits rows a wave stages per step (only the blocks of
// its group that exist: 8, 16 or 32; top-k lists longer than 4 always take
// 32), and whether it runs two workgroups per CU: with 8 or 16 rows, when two
// workgroups of four waves with at least two stages each fit the CU's 160 KB
// (a stage is 32 markov_w2 rows of the rank, rounded up to 32, 64 or 128,
// plus the logits rows of 128 bytes). A second workgroup hides one's inserts
// and waits behind the other's: chain + finalize 330 -> 315 us on the B = 8
// top-4 tree, 57 -> 54 us at the Gemma shape, Qwen3-8B unchanged; staging
// fewer rows with one workgroup per CU and a deeper ring alone was slower
// (353 / 66 / 122 us).
inline int chain_wave_rows(int B, int top_k) {
    if (top_k > 4 || B > 16) return 32;
    return B <= 8 ? 8 : 16;
}
inline int chain_wave_rank(int r) {
    const int rs = (r + 15) / 16;
    return rs == 0 ? 0 : rs <= 2 ? 2 : rs <= 4 ? 4 : 8;
}
constexpr int chain_wave_stage_bytes(int RS, int LROWS) { return (64 * RS + 8 * LROWS) * 16; }
constexpr int kChainWaveBudget2 = 79 * 1024;    // per workgroup, two per CU
constexpr int kChainWaveBudget1 = 158 * 1024;   // one per CU
inline int chain_wave_per_cu(int B, int r, int top_k) {
    const int rows = chain_wave_rows(B, top_k);
    return rows < 32 && 4 * 2 * chain_wave_stage_bytes(chain_wave_rank(r), rows) <= kChainWaveBudget2 ? 2 : 1;
}
inline int chain_workgroups(int B, int V, int r, int top_k) {
    const ChainForm f = chain_form(B, V, r, top_k);
    if (f == kChainDirect) return (V + kChainTileV - 1) / kChainTileV;
    const int ts = chain_tile(B, r);
    const int nt = (V + ts - 1) / ts;
    const int cap = f == kChainPipeTwo ? kChainMaxWGs
                    : f == kChainWave ? kChainCUs * chain_wave_per_cu(B, r, top_k) : kChainCUs;
    return nt < cap ? nt : cap;
}
// Pruned form (chain_step_sparse: a propose call whose projection left the
// slab maxima; V % 4 == 0, rank up to 128): per-wave rings like kChainWave,
// with LDS budgets that leave room for the skip lists; at least one slab per
// wave where the vocabulary allows.
constexpr int kChainSparseBudget2 = 72 * 1024;   // per workgroup, two per CU
constexpr int kChainSparseBudget1 = 150 * 1024;  // one per CU
inline bool chain_sparse(int V, int r) { return chain_pipelined(V) && (r + 15) / 16 <= 8; }
inline int chain_sparse_per_cu(int B, int r, int top_k) {
    const int rows = chain_wave_rows(B, top_k);
    return rows < 32 && 4 * 2 * chain_wave_stage_bytes(chain_wave_rank(r), rows) <= kChainSparseBudget2 ? 2 : 1;
}
inline int chain_sparse_workgroups(int B, int V, int r, int top_k) {
    const int vw = B > 32 ? 2 : 4;   // waves per block group
    const int slabs = (V + kSlabCols - 1) / kSlabCols;
    const int want = (slabs + vw - 1) / vw;
    const int cap = kChainCUs * chain_sparse_per_cu(B, r, top_k);
    return want < cap ? want : cap;
}
// Upper bound of chain_workgroups over every rank (workspace sizing does not
// know r): the narrowest tile gives the most workgroups.
inline int chain_workgroups_max(int V) {
    if (chain_pipelined(V)) {
        const int nt = (V + 63) / 64;
        return nt < kChainMaxWGs ? nt : kChainMaxWGs;
    }
    return (V + kChainTileV - 1) / kChainTileV;
}
// The running argmax of a (slot, block) is spread over kWinnerWays 64-bit
// words, which workgroup g raises with atomicMax on word g % kWinnerWays;
// the argmax is the largest of them. Atomics on one address are serialised
// (256-512 per slot on one word cost 2-5 us per slot); spread, each word
// takes an eighth of them, and a reader loads eight words. (4 and 8 ways
// time the same; 16 and 32 lose more on the reads than they gain.) Word
// (j, k, b) sits at (j * kWinnerWays + k) * winners_stride(B) + b, so the
// words of one block are at least 256 bytes apart.
constexpr int kWinnerWays = 8;
inline int winners_stride(int B) { return (B + 31) / 32 * 32; }
// Flags word bits (the public values of DSPARK_FLAG_*).
constexpr uint32_t kFlagBadAnchor = 1u, kFlagInternal = 2u, kFlagBadD2t = 4u;

// The chain runs over V columns. Without a d2t table a column is a
// vocabulary id; with one (a reduced draft vocabulary), column c is draft id c
// and stands for target id d2t[c], and previous tokens (anchors included) are
// target ids in [0, vocab) that index markov_w1.
struct ChainArgs {
    const float* logits;       // [B * n_pred, V]
    const uint16_t* w1;        // [vocab, r] bf16 bits (nullptr iff r == 0)
    const uint16_t* w2;        // [V, r] bf16 bits
    const int64_t* d2t;        // [V] target id of each column, or nullptr (identity)
    const int32_t* anchors;    // [B]
    unsigned long long* winners;   // [n_pred, kWinnerWays, wstride] running argmax keys
    unsigned long long* partials;  // [n_pred, B, nwg, top_k] per-workgroup top-k keys (top_k > 1)
    uint32_t* flags;
    int32_t* lengths;          // [B], set to n_pred here, cut by the confidence head later
    int B, V, r, n_pred, top_k, nwg;
    int wstride;               // winners_stride(B)
    int vocab;                 // target vocabulary size (== V without d2t)
    const int32_t* stop;       // adaptive gate: slots from *stop on are skipped (nullptr: none)
    // Bound (after a projection of the same call), or nullptr: slab maxima
    // [B * n_pred][ceil(V / slab_cols)] (GemmArgs), the k-th largest slab
    // maximum of every row [B * n_pred] (row_kth, k = the list length), and
    // the largest squared row norms of markov_w2 and markov_w1 (fp32 bits;
    // markov_w1 only for the pruned form).
    const float* smax;
    float* kth;
    uint32_t* w2n2;
    uint32_t* w1n2;
    int slab_cols;
    // The pruned form runs the steps (chain_step_sparse): set only with smax,
    // kth, w2n2 and w1n2 all present (and chain_sparse(V, r)).
    int sparse;
};
// The k-th largest slab maximum of every row (after the projection).
hipError_t launch_row_kth(const ChainArgs& a, hipStream_t stream);
// Zeroes the running-argmax words, the flags and the norm words (when
// present) and presets lengths to n_pred; enqueued before the projection.
hipError_t launch_chain_init(const ChainArgs& a, hipStream_t stream);
hipError_t launch_chain_step(const ChainArgs& a, int j, hipStream_t stream);
// While on (on the calling host thread), launch_chain_step selects its kernel
// as for a launch, launches nothing and returns hipSuccess; a size for which
// no compiled kernel exists still returns hipErrorInvalidValue.
void set_chain_dry_dispatch(bool on);

struct FinalArgs {
    const unsigned long long* winners;   // as in ChainArgs
    const unsigned long long* partials;
    const void* hidden;        // [B, L, H] (confidence head only)
    const uint16_t* conf_w;    // [H] or nullptr
    const int64_t* d2t;        // as in ChainArgs: tokens and candidates are mapped through it
    int32_t* tokens;           // [B, n_pred]
    int32_t* candidates;       // [B, n_pred, top_k]
    float* cand_logits;        // [B, n_pred, top_k] or nullptr
    float* conf;               // [B, n_pred] or nullptr
    int32_t* lengths;          // [B]
    uint32_t* flags;
    int B, L, H, n_pred, i_first, top_k, nwg;
    int wstride;               // winners_stride(B)
    int V;                     // chain columns (keys outside [0, V) are never mapped)
    int hidden_f32;
    float p_min;
    int gated;                 // conf and lengths came from the adaptive gate; mask cut slots
    const int32_t* top_k_b;    // [B] candidates kept per block, or nullptr (all top_k)
};
hipError_t launch_finalize(const FinalArgs& a, hipStream_t stream);

// ---- adaptive gate -------------------------------------------------------------
struct GateArgs {
    const void* hidden;
    const uint16_t* conf_w;    // [H]
    const float* p_min;        // [B] per-block thresholds
    float* conf;               // [B, n_pred] or nullptr
    int32_t* lengths;          // [B], preset to n_pred
    int32_t* stop;             // one word: max over blocks of lengths
    int B, L, H, n_pred, i_first, hidden_f32;
};
hipError_t launch_gate(const GateArgs& g, hipStream_t stream);

// ---- greedy verification ---------------------------------------------------------
struct VerifyArgs {
    const int32_t* candidates; // [B, n_pred, top_k]
    const int32_t* lengths;    // [B], clamped to [0, n_pred]
    const int32_t* target;     // [B, n_pred]: the target's greedy token per slot
    int32_t* accepted;         // [B]
    int32_t* totals;           // [2]: sum of accepted, sum of the clamped lengths
    int B, n_pred, top_k;
    int width;                 // candidates checked per slot: 1 (the chain) or top_k (lattice)
};
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

}  // namespace dspark
