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
    // XCD-aware order: dispatch sends block i to XCD i % 8; give each XCD a
    // contiguous run of tiles, M fastest, so the M tiles of an N slab share an L2.
    const int sid = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
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
// K advances 32 at a time through an NS-deep ring of LDS stages filled by
// global_load_lds_dwordx4 (each lane's 16 bytes land at LDS slot base + lane,
// no register staging), so NS - 1 stages of loads stay in flight while one is
// multiplied. A stage holds 64-byte rows (4 chunks of 16 B); chunk c of row r
// sits in physical slot c ^ h(r), h(r) = ((r>>1 ^ r>>3) & 1) | ((r>>2 & 1) << 1),
// which spreads the same chunk of any 8 (32-bank view) or 16 (64-bank view)
// consecutive rows over distinct banks. The permutation is applied on the
// global side: the lane that owns slot p fetches the chunk that belongs there.
// Barriers are raw s_barrier with explicit vmcnt waits: a workgroup fence
// would drain every load in flight.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int swz(int row) {
    return (((row >> 1) ^ (row >> 3)) & 1) | (((row >> 2) & 1) << 1);
}


template <int BM, int BN, int WM, int WN, int NS>
__global__ __launch_bounds__(64 * WM * WN) void lmhead_gemm_dma(GemmArgs a) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int IA = BM / 16, IB = BN / 16;     // 1 KB wave-loads per stage
    constexpr int LW = (IA + IB) / NW;            // loads per wave per stage
    constexpr int BKS = 32;
    static_assert((IA + IB) % NW == 0, "stage loads must split evenly over waves");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(NS >= 2 && (NS - 2) * LW < 64, "pipeline depth");

    // One ring for both operands: stage s holds A rows at slots [0, 4*BM) and
    // lm_head rows at [4*BM, 4*(BM+BN)).
    __shared__ u32x4 smem[NS][(BM + BN) * 4];

    const int M = a.M, N = a.N, K = a.K;
    const int nMT = (M + BM - 1) / BM, nNT = (N + BN - 1) / BN, T = nMT * nNT;
    const int bid = blockIdx.x;
    const int sid = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
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
        const int row = slot >> 2, c = (slot & 3) ^ swz(row);
        if (inst < IA) {
            const int m = min(m0 + row, M - 1);
            const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
            src[i] = static_cast<const uint16_t*>(a.hidden) + hrow * K + c * 8;
            dst[i] = (inst * 64);
        } else {
            src[i] = a.lm_head + (long)min(n0 + row, N - 1) * K + c * 8;
            dst[i] = BM * 4 + (inst - IA) * 64;
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
                fa[i] = smem[stage][row * 4 + (ch ^ swz(row))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + lrow;
                fb[j] = smem[stage][(BM + row) * 4 + (ch ^ swz(row))];
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
        block_barrier();  // every wave's part of tile kt is in LDS; stage kt-1 is free
        const int kn = kt + NS - 1;
        if (kn < nK) issue(kn % NS, kn * BKS);
        mma(stage);
        stage = stage + 1 == NS ? 0 : stage + 1;
    }

    store_tile<BM, BN, WM, WN>(a, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Split-ring pipeline for large M (bf16 hidden, K % 64 == 0).
//
// K advances 64 at a time: a stage row is one 128-byte line. The two operands
// get rings sized to their latency: the hidden rows (A) are re-read by every
// lm_head slab and stay in L2, so two stages suffice; the lm_head rows (B) are
// read from HBM once, so they get three stages and two of them are always in
// flight. Per iteration the loads are issued A(kt+1) first, then
// B(kt+NSB-1), so that the in-order vmcnt wait for A(kt) never has to wait
// for the newest B loads. Both rings live in one LDS array: with separate
// arrays the compiler drains every in-flight LDS load before each LDS read.
// ---------------------------------------------------------------------------
template <int CH>
__device__ __forceinline__ int swz_ch(int row) {
    if constexpr (CH == 8) return (row ^ (row >> 3)) & 7;
    else return swz(row);
}

template <int BM, int BN, int WM, int WN, int NSA, int NSB>
__global__ __launch_bounds__(64 * WM * WN) void lmhead_gemm_split(GemmArgs a) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int BKS = 64, CH = BKS / 8;
    constexpr int IA = BM * CH / 64, IB = BN * CH / 64;  // 1 KB wave-loads per stage
    constexpr int LA = IA / NW, LB = IB / NW;
    static_assert(IA % NW == 0 && IB % NW == 0, "stage loads must split evenly over waves");
    static_assert(NSA == 2 && NSB >= 2, "ring depths");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    constexpr int BOFF = NSA * BM * CH;
    __shared__ u32x4 smem[NSA * BM * CH + NSB * BN * CH];

    const int M = a.M, N = a.N, K = a.K;
    const int nMT = (M + BM - 1) / BM, nNT = (N + BN - 1) / BN, T = nMT * nNT;
    const int bid = blockIdx.x;
    const int sid = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
    const int m0 = (sid % nMT) * BM, n0 = (sid / nMT) * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // The lane that owns LDS slot p of a stage fetches the chunk the swizzle
    // puts there; rows past M / N are clamped (their products are not stored).
    const uint16_t* srcA[LA];
    const uint16_t* srcB[LB];
    int dstA[LA], dstB[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int inst = wave + i * NW, slot = inst * 64 + lane;
        const int row = slot / CH, c = (slot % CH) ^ swz_ch<CH>(row);
        const int m = min(m0 + row, M - 1);
        const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
        srcA[i] = static_cast<const uint16_t*>(a.hidden) + hrow * K + c * 8;
        dstA[i] = inst * 64;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int inst = wave + i * NW, slot = inst * 64 + lane;
        const int row = slot / CH, c = (slot % CH) ^ swz_ch<CH>(row);
        srcB[i] = a.lm_head + (long)min(n0 + row, N - 1) * K + c * 8;
        dstB[i] = inst * 64;
    }
    auto issueA = [&](int st, int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(srcA[i] + k0),
                                             (lds_ptr)&smem[st * BM * CH + dstA[i]], 16, 0, 0);
    };
    auto issueB = [&](int st, int k0) {
#pragma unroll
        for (int i = 0; i < LB; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(srcB[i] + k0),
                                             (lds_ptr)&smem[BOFF + st * BN * CH + dstB[i]], 16, 0, 0);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
    const int lrow = lane & 31, lhalf = lane >> 5;
    auto mma = [&](int stA, int stB) {
#pragma unroll
        for (int ks = 0; ks < BKS / 16; ++ks) {
            const int ch = ks * 2 + lhalf;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + lrow;
                fa[i] = smem[stA * BM * CH + row * CH + (ch ^ swz_ch<CH>(row))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + lrow;
                fb[j] = smem[BOFF + stB * BN * CH + row * CH + (ch ^ swz_ch<CH>(row))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        }
    };

    const int nK = K / BKS;
    // Prologue order: B(0 .. NSB-3), A(0), B(NSB-2): at kt = 0 only the newest
    // B stage may still be in flight.
#pragma unroll
    for (int t = 0; t < NSB - 2; ++t)
        if (t < nK) issueB(t, t * BKS);
    issueA(0, 0);
    if (NSB - 2 < nK) issueB(NSB - 2, (NSB - 2) * BKS);

    int sA = 0, sB = 0;
    for (int kt = 0; kt < nK; ++kt) {
        // Loads issued after A(kt): B(kt + NSB - 2) only, when it exists.
        if (kt + NSB - 2 < nK) wait_vmcnt<LB>();
        else wait_vmcnt<0>();
        block_barrier();  // A(kt), B(kt) landed for every wave; stages of kt-1 are free
        if (kt + 1 < nK) issueA(sA ^ 1, (kt + 1) * BKS);
        if (kt + NSB - 1 < nK) issueB((sB + NSB - 1) % NSB, (kt + NSB - 1) * BKS);
        mma(sA, sB);
        sA ^= 1;
        sB = sB + 1 == NSB ? 0 : sB + 1;
    }
    store_tile<BM, BN, WM, WN>(a, acc, m0, n0, wm, wn, lane);
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
    const long tiles = (long)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((lmhead_gemm_dma<BM, BN, WM, WN, NS>), dim3((unsigned)tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, bool f32, hipStream_t s) {
    const long tiles = (long)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
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
        if (a.M > 128 && a.K % 64 == 0) {
            const long tiles = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
            if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
            hipLaunchKernelGGL((lmhead_gemm_split<256, 256, 2, 4, 2, 3>), dim3((unsigned)tiles),
                               dim3(512), 0, stream, a);
            return hipGetLastError();
        }
        if (a.M > 128) return launch_dma<256, 256, 2, 4, 4>(a, stream);
        if (a.M > 32) return launch_dma<128, 128, 2, 2, 6>(a, stream);
        return launch_dma<32, 128, 1, 2, 6>(a, stream);
    }
    // fp32 hidden states or K not a multiple of 32: register-staged kernel
    if (a.M > 32) return launch_cfg<128, 128, 2, 2>(a, hidden_f32, stream);
    return launch_cfg<32, 128, 1, 4>(a, hidden_f32, stream);
}

}  // namespace dspark
