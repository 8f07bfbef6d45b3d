// lm_head projection: logits[m][n] = sum_k A[m][k] * lm_head[n][k] (+ bias[n]).
//
// A row m is the hidden state of prediction slot (m / n_pred, m % n_pred);
// both operands are K-contiguous (an "NT" product), which is exactly the
// operand layout the bf16 MFMA wants: every lane feeds 8 consecutive k of one
// row. The drafter shares the target's vocabulary head (onnxruntime-genai PR
// #2490 "Export DSpark block drafters for Qwen 3.5 and 3.8", DSpark commit
// message); the optional bias carries the -1e9 rows of an expanded reduced
// vocabulary (llama.cpp PR #26275 "dspark: support speculators-format
// checkpoints", first commit message).
//
// Design (gfx950): a BM x BN output tile per workgroup, K stepped by 64
// through double-buffered LDS (each row of a K step is 128 B = 8 chunks of
// 16 B, XOR-swizzled by the row's low three bits so that the 32 rows an MFMA
// operand read touches spread over the banks), 32x32x16 bf16 MFMA with fp32
// accumulators, and the next K step's global loads in flight while the
// current one is multiplied. Tiles are numbered so that the M tiles sharing
// one lm_head slab are dispatched together on one XCD (one L2).
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int BK = 64;

// Epilogue shared by the GEMM variants: + bias, fp32 store of the wave's
// FM x FN accumulator blocks. Per register, lanes 0-31 and 32-63 write 32
// consecutive columns of two rows (two whole 128-byte lines). Stores are
// non-temporal: the logits are streamed out once and should not evict the
// lm_head / hidden tiles from L2. The bias is read once per column before any
// store, and tiles that lie wholly inside the matrix store without predicates.
// An extra workgroup g (of a.w2_groups, numbered after the tiles) of a
// projection launch: its share of the markov_w2 and (when wanted) markov_w1
// row norms.
__device__ __forceinline__ void w2_norm_part(const GemmArgs& a, int g) {
    row_norm_part(a.w2, a.w2_rows, a.w2_rank, g, a.w2_groups, a.w2n2);
    if (a.w1n2 != nullptr) row_norm_part(a.w1, a.w1_rows, a.w2_rank, g, a.w2_groups, a.w1n2);
}

// Slab maxima (kernels.hpp) of SC columns of a wave's FM x FN block in the
// plain accumulator layout: the lane holds column nb + 32 j + lane % 32 and,
// in register g, row mb + 32 i + acc_row(g, lane). Per row and slab: the
// largest projection over the lane's columns of the slab, then over the 32
// lanes of the half wave (block_row_max), stored by the even lanes. A wave of
// 32 columns (FN == 1) holds half a 64-column slab: waves 2t and 2t + 1 (the
// same rows, neighbouring columns) combine their halves through LDS.
template <int FM, int FN, int NW, int SC>
__device__ __forceinline__ void slab_maxima(const GemmArgs& a, const f32x16 (&acc)[FM][FN],
                                            const float (&bn)[FN], int mb, int nb, int wave, int lane) {
    static_assert((FN == 1 && SC == 64) || FN % (SC / 32) == 0, "a wave holds half a slab or whole slabs");
    constexpr int JS = FN == 1 ? 1 : SC / 32;  // 32-column blocks per slab in the wave
    constexpr int SW = FN / JS;                // slabs (or half slabs) per wave
    const int lrow = lane & 31, N = a.N;
    const int nslab = (N + SC - 1) / SC;
    const int row = acc_row((lane >> 1) & 15, lane);   // the row this lane ends with
    float pick[FM][SW];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < SW; ++q) {
            float v[16];
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                v[g] = -INFINITY;
#pragma unroll
                for (int jj = 0; jj < JS; ++jj) {
                    const int j = q * JS + jj;
                    if (nb + j * 32 + lrow < N) v[g] = fmaxf(v[g], acc[i][j][g] + bn[j]);
                }
            }
            pick[i][q] = block_row_max(v, lane);
        }
    if constexpr (FN == 1) {
        static_assert(NW % 2 == 0, "waves pair up");
        __shared__ float s_half[NW][FM * 32];
        if ((lane & 1) == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) s_half[wave][i * 32 + row] = pick[i][0];
        }
        __syncthreads();
        if ((lane & 1) == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) pick[i][0] = fmaxf(pick[i][0], s_half[wave ^ 1][i * 32 + row]);
        }
        if (wave & 1) return;   // the even wave of the pair writes the slab
    }
    if (lane & 1) return;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = mb + i * 32 + row;
        if (m >= a.M) continue;
#pragma unroll
        for (int q = 0; q < SW; ++q) {
            const int n = nb + q * SC;
            if (n < N) a.smax[(long)m * nslab + n / SC] = pick[i][q];
        }
    }
}

template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                           int m0, int n0, int wm, int wn, int lane) {
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    const int M = a.M, N = a.N;
    const int lrow = lane & 31;
    float bn[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * TN + j * 32 + lrow;
        bn[j] = (a.bias != nullptr && n < N) ? a.bias[n] : 0.0f;
    }
    // The bias loads must be complete before the first store: otherwise the
    // wait inserted for them also waits for every store issued so far.
    __builtin_amdgcn_s_waitcnt(0);
    // (the layout puts waves wm * WN + wn and its neighbour wn ^ 1 on the same rows)
    if (a.smax != nullptr) {
        if constexpr (FN % (kSlabColsWide / 32) == 0) {
            if (a.slab_cols == kSlabColsWide) {
                slab_maxima<FM, FN, WM * WN, kSlabColsWide>(a, acc, bn, m0 + wm * TM, n0 + wn * TN,
                                                             wm * WN + wn, lane);
            } else {
                slab_maxima<FM, FN, WM * WN, kSlabCols>(a, acc, bn, m0 + wm * TM, n0 + wn * TN,
                                                        wm * WN + wn, lane);
            }
        } else {
            slab_maxima<FM, FN, WM * WN, kSlabCols>(a, acc, bn, m0 + wm * TM, n0 + wn * TN,
                                                    wm * WN + wn, lane);
        }
    }
    if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int mb = m0 + wm * TM + i * 32;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float* col = a.out + (n0 + wn * TN + j * 32 + lrow);
#pragma unroll
                for (int g = 0; g < 16; ++g)
                    __builtin_nontemporal_store(acc[i][j][g] + bn[j], col + (long)(mb + acc_row(g, lane)) * N);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int mb = m0 + wm * TM + i * 32;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 32 + lrow;
            float* col = a.out + n;
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int m = mb + acc_row(g, lane);
                if (m < M && n < N)
                    __builtin_nontemporal_store(acc[i][j][g] + bn[j], col + (long)m * N);
            }
        }
    }
}

template <bool F32A>
__device__ __forceinline__ u32x4 load_a_chunk(const void* base, long elem, bool valid) {
    if (!valid) return u32x4{0u, 0u, 0u, 0u};
    if constexpr (F32A) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
        f32x4 x0 = p[0], x1 = p[1];
        return u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                     pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
    } else {
        return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
    }
}

template <int BM, int BN, int WM, int WN, bool F32A, bool KFULL>
__global__ __launch_bounds__(64 * WM * WN) void lmhead_gemm(GemmArgs a) {
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA blocks per wave
    constexpr int AC = BM * 8 / NT, BC = BN * 8 / NT;  // 16-byte chunks per thread per K step
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile / thread mismatch");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");

    __shared__ u32x4 sA[2][BM * 8];
    __shared__ u32x4 sB[2][BN * 8];

    const int M = a.M, N = a.N, K = a.K;
    const int nMT = (M + BM - 1) / BM, nNT = (N + BN - 1) / BN, T = nMT * nNT;
    const int bid = blockIdx.x;
    if (bid >= T) {
        w2_norm_part(a, bid - T);
        return;
    }
    // XCD-aware order: dispatch sends block i to XCD i % 8; give each XCD a
    // contiguous run of tiles, M fastest, so the M tiles of an N slab share an L2.
    const int sid = xcd_unit(bid, T);
    const int m0 = (sid % nMT) * BM, n0 = (sid / nMT) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // Global-load descriptors, fixed for the whole K loop. Rows past M / N are
    // clamped onto the last valid row: they load real data whose products
    // land only in output rows / columns that are never stored.
    long a_off[AC], b_off[BC];
    int a_ch[AC], b_ch[BC], a_slot[AC], b_slot[BC];
#pragma unroll
    for (int c = 0; c < AC; ++c) {
        const int id = tid + c * NT, row = id >> 3, ch = id & 7;
        const int m = min(m0 + row, M - 1);
        const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
        a_off[c] = hrow * K + ch * 8;
        a_ch[c] = ch;
        a_slot[c] = row * 8 + (ch ^ (row & 7));
    }
#pragma unroll
    for (int c = 0; c < BC; ++c) {
        const int id = tid + c * NT, row = id >> 3, ch = id & 7;
        b_off[c] = (long)min(n0 + row, N - 1) * K + ch * 8;
        b_ch[c] = ch;
        b_slot[c] = row * 8 + (ch ^ (row & 7));
    }

    // Two register stages: tile t is staged in set t % 2 and LDS buffer t % 2,
    // so the loads of tile t + 2 are in flight while tile t is multiplied.
    u32x4 ra[2][AC], rb[2][BC];
    auto gload = [&](int set, int k0) {
#pragma unroll
        for (int c = 0; c < AC; ++c)
            ra[set][c] = load_a_chunk<F32A>(a.hidden, a_off[c] + k0, KFULL || k0 + a_ch[c] * 8 < K);
#pragma unroll
        for (int c = 0; c < BC; ++c) {
            const bool ok = KFULL || k0 + b_ch[c] * 8 < K;
            rb[set][c] = ok ? *reinterpret_cast<const u32x4*>(a.lm_head + b_off[c] + k0)
                            : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto lstore = [&](int set, int buf) {
#pragma unroll
        for (int c = 0; c < AC; ++c) sA[buf][a_slot[c]] = ra[set][c];
#pragma unroll
        for (int c = 0; c < BC; ++c) sB[buf][b_slot[c]] = rb[set][c];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int lrow = lane & 31, lhalf = lane >> 5;
    auto mma = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + lhalf;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + lrow;
                fa[i] = sA[buf][row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + lrow;
                fb[j] = sB[buf][row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        }
    };

    const int nK = (K + BK - 1) / BK;
    gload(0, 0);
    lstore(0, 0);
    if (nK > 1) gload(1, BK);
    __syncthreads();

    // Iteration kt: multiply tile kt (LDS buffer kt % 2); load tile kt + 2
    // into register set kt % 2; stage tile kt + 1 (set (kt+1) % 2) into the
    // other LDS buffer. Unrolled by two so that the register sets are static.
    for (int kt = 0; kt < nK; kt += 2) {
        if (kt + 2 < nK) gload(0, (kt + 2) * BK);
        mma(0);
        if (kt + 1 < nK) lstore(1, 1);
        __syncthreads();
        if (kt + 1 >= nK) break;
        if (kt + 3 < nK) gload(1, (kt + 3) * BK);
        mma(1);
        if (kt + 2 < nK) lstore(0, 0);
        __syncthreads();
    }

    store_tile<BM, BN, WM, WN>(a, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS pipeline (bf16 hidden, K % 32 == 0).
//
// K advances BKS (32 or 64) at a time through an NS-deep ring of LDS stages
// filled by global_load_lds_dwordx4 (each lane's 16 bytes land at LDS slot
// base + lane, no register staging), so NS - 1 stages of loads stay in flight
// while one is multiplied. A stage holds rows of BKS / 8 chunks of 16 B (64
// or 128 bytes: with 64 K values a row is one whole 128-byte line, fetched by
// one copy instead of two). With 4 chunks, chunk c of row r sits in physical
// slot c ^ h(r), h(r) = ((r>>1 ^ r>>3) & 1) | ((r>>2 & 1) << 1); with 8, in
// c ^ ((r ^ r>>3) & 7). Either spreads the same chunk of consecutive rows
// over distinct banks. The permutation is applied on the global side: the
// lane that owns slot p fetches the chunk that belongs there.
// Barriers are raw s_barrier with explicit vmcnt waits: a workgroup fence
// would drain every load in flight.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int swz(int row) {
    return (((row >> 1) ^ (row >> 3)) & 1) | (((row >> 2) & 1) << 1);
}


// Chunk swizzle for stage rows of CH 16-byte chunks (4: 32 K values per
// step, 8: 64, one 128-byte line).
template <int CH>
__device__ __forceinline__ int swz_ch(int row) {
    if constexpr (CH == 8) return (row ^ (row >> 3)) & 7;
    else return swz(row);
}

template <int BM, int BN, int WM, int WN, int NS, int BKS = 32>
__global__ __launch_bounds__(64 * WM * WN) void lmhead_gemm_dma(GemmArgs a) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CH = BKS / 8;                   // 16-byte chunks per stage row
    constexpr int IA = BM * CH / 64, IB = BN * CH / 64;   // 1 KB wave-loads per stage
    constexpr int LW = (IA + IB) / NW;            // loads per wave per stage
    static_assert(BKS == 32 || BKS == 64, "K step");
    static_assert((IA + IB) % NW == 0, "stage loads must split evenly over waves");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(NS >= 2 && (NS - 2) * LW < 64, "pipeline depth");

    // One ring for both operands: stage s holds A rows at slots [0, CH*BM) and
    // lm_head rows at [CH*BM, CH*(BM+BN)).
    __shared__ u32x4 smem[NS][(BM + BN) * CH];

    const int M = a.M, N = a.N, K = a.K;
    const int nMT = (M + BM - 1) / BM, nNT = (N + BN - 1) / BN, T = nMT * nNT;
    const int bid = blockIdx.x;
    if (bid >= T) {
        w2_norm_part(a, bid - T);
        return;
    }
    const int sid = xcd_unit(bid, T);
    const int m0 = (sid % nMT) * BM, n0 = (sid / nMT) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // This lane's source of each of its LW loads per stage (k offset 0).
    const uint16_t* src[LW];
    int dst[LW];        // first slot of the wave's 64-slot destination in a stage
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int inst = wave + i * NW;
        const int slot = (inst < IA ? inst : inst - IA) * 64 + lane;
        const int row = slot / CH, c = (slot % CH) ^ swz_ch<CH>(row);
        if (inst < IA) {
            const int m = min(m0 + row, M - 1);
            const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
            src[i] = static_cast<const uint16_t*>(a.hidden) + hrow * K + c * 8;
            dst[i] = (inst * 64);
        } else {
            src[i] = a.lm_head + (long)min(n0 + row, N - 1) * K + c * 8;
            dst[i] = BM * CH + (inst - IA) * 64;
        }
    }
    auto issue = [&](int stage, int k0) {
#pragma unroll
        for (int i = 0; i < LW; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(src[i] + k0), (lds_ptr)&smem[stage][dst[i]],
                                             16, 0, 0);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int lrow = lane & 31, lhalf = lane >> 5;
    auto mma = [&](int stage) {
#pragma unroll
        for (int ks = 0; ks < BKS / 16; ++ks) {
            const int ch = ks * 2 + lhalf;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + lrow;
                fa[i] = smem[stage][row * CH + (ch ^ swz_ch<CH>(row))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + lrow;
                fb[j] = smem[stage][(BM + row) * CH + (ch ^ swz_ch<CH>(row))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        }
    };

    const int nK = K / BKS;
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < nK) issue(t, t * BKS);

    int stage = 0;
    for (int kt = 0; kt < nK; ++kt) {
        // Tile kt must have landed: at most min(NS-2, nK-1-kt) newer tiles may still fly.
        wait_stages<LW, NS - 2>(min(NS - 2, nK - 1 - kt));
        // this wave's reads of stage kt-1 (previous iteration) have returned
        // before the barrier lets any wave refill that stage
        wait_lds_reads();
        block_barrier();  // every wave's part of tile kt is in LDS; stage kt-1 is free
        const int kn = kt + NS - 1;
        if (kn < nK) issue(kn % NS, kn * BKS);
        mma(stage);
        stage = stage + 1 == NS ? 0 : stage + 1;
    }

    store_tile<BM, BN, WM, WN>(a, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Four-wave pipeline for large M (bf16 hidden, K % 64 == 0).
//
// A 256 x 256 tile per workgroup of four waves; each wave owns a 128 x 128
// quarter (4 x 4 MFMA blocks, all 256 accumulator registers), which needs
// 8 operand reads from LDS per 16 MFMAs. K advances 64 at a time (a stage row
// is one 128-byte line, chunks swizzled as above). The hidden rows (A) are
// re-read by every lm_head slab and stay in L2, so their ring has two stages;
// the lm_head rows (B) come from HBM once and get three. Loads go straight
// into LDS through buffer loads (the per-lane state is a 32-bit offset; the
// lm_head descriptor covers exactly this tile's rows, so rows past N read as
// zero). One barrier per K step, at its start. The step is cut into four
// regions of 16 products; every region carries the LDS reads of the next
// k-substep and four of the global->LDS loads of later stages (A in the
// first two regions, B in the last two, all A before all B so one count
// waits for both), each after every other of the region's last eight
// products (sched_group_barrier). Four loads per region keep the four waves'
// requests at the texture unit's rate (eight A loads in one region were
// twice that and stalled the issuing waves: 2153 -> 2129 us). Past the last
// K step the loads repeat the last step into stages that are not read again,
// which keeps the step free of branches.
// ---------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, unsigned bytes) {
    // raw buffer (stride 0): accesses at or past `bytes` read as zero
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(256) void lmhead_gemm_w4(GemmArgs a) {
    constexpr int BM = 256, BN = 256, BKS = 64, CH = 8, FM = 4, FN = 4, NSA = 2, NSB = 3;
    constexpr int ASTG = BM * CH * 16, BSTG = BN * CH * 16;   // bytes per stage
    constexpr int LA = 8, LB = 8;                              // 1 KB loads per wave per stage
    __shared__ __attribute__((aligned(1024))) char smem[NSA * ASTG + NSB * BSTG];

    const int M = a.M, N = a.N, K = a.K;
    const int nMT = (M + BM - 1) / BM, nNT = (N + BN - 1) / BN, T = nMT * nNT;
    const int bid = blockIdx.x;
    if (bid >= T) {
        w2_norm_part(a, bid - T);
        return;
    }
    const int sid = xcd_unit(bid, T);
    const int m0 = (sid % nMT) * BM, n0 = (sid / nMT) * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Load i of this wave fills LDS slots (wave + 4 i) * 64 + lane of a stage:
    // row 32 i + 8 wave + lane / 8, position lane % 8, which holds the chunk
    // the swizzle puts there.
    const rsrc_t ra = make_rsrc(a.hidden, 0xFFFFFFFFu);
    const rsrc_t rb = make_rsrc(a.lm_head + (long)n0 * K, (unsigned)min(BN, N - n0) * K * 2);
    const int p = lane & 7, r8 = lane >> 3;
    unsigned aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int row = 32 * i + 8 * wave + r8;
        const int m = min(m0 + row, M - 1);
        const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
        aoff[i] = (unsigned)(hrow * K * 2 + (p ^ swz_ch<CH>(row)) * 16);
    }
    // lm_head rows are linear in i; the swizzle depends on i only by parity
    unsigned boff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = 32 * q + 8 * wave + r8;
        boff[q] = (unsigned)((8 * wave + r8) * K * 2 + (p ^ swz_ch<CH>(row)) * 16);
    }
    auto loadA = [&](int st, int kb, int i) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(smem + st * ASTG + (wave + 4 * i) * 1024), 16,
                                                 aoff[i], kb, 0, 0);
    };
    auto loadB = [&](int st, int kb, int i) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(smem + NSA * ASTG + st * BSTG + (wave + 4 * i) * 1024),
                                                 16, boff[i & 1], i * 32 * K * 2 + kb, 0, 0);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
    // Fragment i of A: rows wm*128 + 32 i + lrow (B likewise with wn); the
    // swizzle depends on i only by parity.
    const int lrow = lane & 31, lhalf = lane >> 5;
    int fa_base[2], fb_base[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        fa_base[q] = (wm * 128 + lrow) * 128 + (swz_ch<CH>(wm * 128 + 32 * q + lrow) << 4);
        fb_base[q] = (wn * 128 + lrow) * 128 + (swz_ch<CH>(wn * 128 + 32 * q + lrow) << 4);
    }
    auto rdA = [&](int sa, int ks, int i) __attribute__((always_inline)) {
        const int cx = (2 * ks + lhalf) << 4;
        return *reinterpret_cast<const u32x4*>(smem + sa * ASTG + i * 4096 + (fa_base[i & 1] ^ cx));
    };
    auto rdB = [&](int sb, int ks, int j) __attribute__((always_inline)) {
        const int cx = (2 * ks + lhalf) << 4;
        return *reinterpret_cast<const u32x4*>(smem + NSA * ASTG + sb * BSTG + j * 4096 + (fb_base[j & 1] ^ cx));
    };
    auto products = [&](const u32x4 (&fa)[FM], const u32x4 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
    };
    // Fragment reads of k-substep ks, in the order the products use them.
    auto reads = [&](u32x4 (&nfa)[FM], u32x4 (&nfb)[FN], int sa, int sb, int ks) __attribute__((always_inline)) {
        nfa[0] = rdA(sa, ks, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) nfb[j] = rdB(sb, ks, j);
#pragma unroll
        for (int i = 1; i < FM; ++i) nfa[i] = rdA(sa, ks, i);
    };
    // Issue order of a region: one LDS read after each of the first 8
    // products, then nv (0, 4 or 8) loads spread over the last 8. The loads
    // write LDS, so the compiler keeps them after the region's reads.
    auto pattern = [&](int nv) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
            if (q < 8)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
            else if (nv == 8 || (nv == 4 && q % 2 == 0))
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);    // one load
        }
    };

    const int nK = K / BKS;
    // Prologue: A(0), B(0), B(1). During step t, A(t+1) and then B(t+2) are
    // issued, so at the start of step t + 1 only B(t+2) may still fly.
#pragma unroll
    for (int i = 0; i < LA; ++i) loadA(0, 0, i);
#pragma unroll
    for (int i = 0; i < LB; ++i) loadB(0, 0, i);
#pragma unroll
    for (int i = 0; i < LB; ++i) loadB(1, min(1, nK - 1) * BKS * 2, i);

    u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa1[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < FN; ++j) fb1[j] = u32x4{0u, 0u, 0u, 0u};
    int sa = 0, sb = 0;
    for (int t = 0; t < nK; ++t) {
        // stage t has landed; every wave has finished reading stage t - 1
        wait_vmcnt<LB>();
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // A(t+1) and B(t+2) go to the stages of t - 1
        const int pa = sa ^ 1, pb = sb == 0 ? NSB - 1 : sb - 1;
        const int kA = min(t + 1, nK - 1) * BKS * 2, kB = min(t + 2, nK - 1) * BKS * 2;
        // region 1: k-substep 3 of step t - 1 (zero fragments at t = 0),
        // reads of (t, 0), first half of A(t+1)
        reads(fa0, fb0, sa, sb, 0);
#pragma unroll
        for (int i = 0; i < LA / 2; ++i) loadA(pa, kA, i);
        products(fa1, fb1);
        pattern(4);
        __builtin_amdgcn_sched_barrier(0);
        // region 2: (t, 0) products, reads of (t, 1), second half of A(t+1)
        reads(fa1, fb1, sa, sb, 1);
#pragma unroll
        for (int i = LA / 2; i < LA; ++i) loadA(pa, kA, i);
        products(fa0, fb0);
        pattern(4);
        __builtin_amdgcn_sched_barrier(0);
        // region 3: (t, 1) products, reads of (t, 2), first half of B(t+2)
        reads(fa0, fb0, sa, sb, 2);
#pragma unroll
        for (int i = 0; i < LB / 2; ++i) loadB(pb, kB, i);
        products(fa1, fb1);
        pattern(4);
        __builtin_amdgcn_sched_barrier(0);
        // region 4: (t, 2) products, reads of (t, 3), second half of B(t+2)
        reads(fa1, fb1, sa, sb, 3);
#pragma unroll
        for (int i = LB / 2; i < LB; ++i) loadB(pb, kB, i);
        products(fa0, fb0);
        pattern(4);
        __builtin_amdgcn_sched_barrier(0);
        // the reads of stage t have returned before the next barrier lets
        // other waves refill it
        wait_lds_reads();
        sa ^= 1;
        sb = sb + 1 == NSB ? 0 : sb + 1;
    }
    products(fa1, fb1);   // k-substep 3 of the last step
    store_tile<BM, BN, 2, 2>(a, acc, m0, n0, wm, wn, lane);
}

// Workgroups of a launch: the tiles, then the markov_w2 norm groups.
long launch_groups(const GemmArgs& a, int BM, int BN) {
    return (long)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) + (a.w2n2 != nullptr ? a.w2_groups : 0);
}

template <int BM, int BN, int WM, int WN, int NS, int BKS = 32>
hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
    const long tiles = launch_groups(a, BM, BN);
    if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((lmhead_gemm_dma<BM, BN, WM, WN, NS, BKS>), dim3((unsigned)tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, bool f32, hipStream_t s) {
    const long tiles = launch_groups(a, BM, BN);
    if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles), block(64 * WM * WN);
    const bool kfull = a.K % BK == 0;
    if (f32 && kfull)
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, true, true>), grid, block, 0, s, a);
    else if (f32)
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, true, false>), grid, block, 0, s, a);
    else if (kfull)
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_gemm(const GemmArgs& a, bool hidden_f32, hipStream_t stream) {
    if (!hidden_f32 && a.K % 32 == 0) {
        // buffer offsets are 32-bit: the hidden rows and one lm_head tile
        // must each span less than 4 GiB
        if (gemm_four_wave(a.M, a.K, a.L, a.n_pred, false)) {
            const long tiles = launch_groups(a, 256, 256);
            if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
            hipLaunchKernelGGL(lmhead_gemm_w4, dim3((unsigned)tiles), dim3(256), 0, stream, a);
            return hipGetLastError();
        }
        if (a.M > 128) return launch_dma<256, 256, 2, 4, 4>(a, stream);
        // Stage rows of 64 K values (one 128-byte line each) where K allows:
        // 6-15% faster than 32-value rows at M = 16, 24 and 128 (same sums).
        if (a.K % 64 == 0) {
            // 32 < M <= 128: 256 lm_head rows per tile (the hidden rows, read
            // again by every tile from L2, are a third of a step's copies
            // instead of half), eight waves; 10% faster than 128 rows at
            // M = 128. A vocabulary too small to give every CU a tile that
            // way keeps 128 rows.
            if (a.M > 32) {
                if ((a.N + 255) / 256 >= 256) return launch_dma<128, 256, 2, 4, 3, 64>(a, stream);
                return launch_dma<128, 128, 2, 2, 4, 64>(a, stream);
            }
            // M <= 32: 128 lm_head rows per tile and two workgroups per CU,
            // unless the last round of 2 x 256 workgroups would run less than
            // half full: then 64 rows and three per CU, whose tail is shorter
            // (Qwen3-8B: 1187 tiles, 292 -> 245 us; at 2048 tiles, Gemma-4,
            // 128 rows stay faster, 252 against 278 us).
            constexpr long kSlots = 2 * 256;
            const long rem = (a.N + 127) / 128 % kSlots;
            if (rem != 0 && rem < kSlots / 2) return launch_dma<32, 64, 1, 2, 4, 64>(a, stream);
            return launch_dma<32, 128, 1, 2, 4, 64>(a, stream);
        }
        if (a.M > 32) return launch_dma<128, 128, 2, 2, 6>(a, stream);
        return launch_dma<32, 128, 1, 2, 6>(a, stream);
    }
    // fp32 hidden states or K not a multiple of 32: register-staged kernel
    if (a.M > 32) return launch_cfg<128, 128, 2, 2>(a, hidden_f32, stream);
    return launch_cfg<32, 128, 1, 4>(a, hidden_f32, stream);
}

}  // namespace dspark
