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

template <int BM, int BN, int WM, int WN, bool F32A>
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

    // Global-load descriptors (fixed for the whole K loop).
    long a_off[AC];
    bool a_ok[AC];
    int a_ch[AC], a_slot[AC];
#pragma unroll
    for (int c = 0; c < AC; ++c) {
        const int id = tid + c * NT, row = id >> 3, ch = id & 7;
        const int m = m0 + row;
        a_ok[c] = m < M;
        const int mm = a_ok[c] ? m : 0;
        const long hrow = (long)(mm / a.n_pred) * a.L + a.i_first + mm % a.n_pred;
        a_off[c] = hrow * K + ch * 8;
        a_ch[c] = ch;
        a_slot[c] = row * 8 + (ch ^ (row & 7));
    }
    long b_off[BC];
    bool b_ok[BC];
    int b_ch[BC], b_slot[BC];
#pragma unroll
    for (int c = 0; c < BC; ++c) {
        const int id = tid + c * NT, row = id >> 3, ch = id & 7;
        const int n = n0 + row;
        b_ok[c] = n < N;
        b_off[c] = (long)(b_ok[c] ? n : 0) * K + ch * 8;
        b_ch[c] = ch;
        b_slot[c] = row * 8 + (ch ^ (row & 7));
    }

    u32x4 ra[AC], rb[BC];
    auto gload = [&](int k0) {
#pragma unroll
        for (int c = 0; c < AC; ++c)
            ra[c] = load_a_chunk<F32A>(a.hidden, a_off[c] + k0, a_ok[c] && (k0 + a_ch[c] * 8 < K));
#pragma unroll
        for (int c = 0; c < BC; ++c) {
            const bool ok = b_ok[c] && (k0 + b_ch[c] * 8 < K);
            rb[c] = ok ? *reinterpret_cast<const u32x4*>(a.lm_head + b_off[c] + k0)
                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < AC; ++c) sA[buf][a_slot[c]] = ra[c];
#pragma unroll
        for (int c = 0; c < BC; ++c) sB[buf][b_slot[c]] = rb[c];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int nK = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();

    const int lrow = lane & 31, lhalf = lane >> 5;
    for (int kt = 0; kt < nK; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nK) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + lhalf;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + lrow;
                fa[i] = sA[cur][row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + lrow;
                fb[j] = sB[cur][row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nK) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: + bias, fp32 store. Lanes 0-31 / 32-63 write 32 consecutive
    // columns of two rows per register: two full 128-byte lines per store.
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * TN + j * 32 + lrow;
        if (n >= N) continue;
        const float bn = a.bias ? a.bias[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int m = m0 + wm * TM + i * 32 + acc_row(g, lane);
                if (m < M) a.out[(long)m * N + n] = acc[i][j][g] + bn;
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, bool f32, hipStream_t s) {
    const long tiles = (long)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles), block(64 * WM * WN);
    if (f32)
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((lmhead_gemm<BM, BN, WM, WN, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_gemm(const GemmArgs& a, bool hidden_f32, hipStream_t stream) {
    if (a.M > 128) return launch_cfg<256, 256, 2, 4>(a, hidden_f32, stream);
    if (a.M > 32) return launch_cfg<128, 128, 2, 2>(a, hidden_f32, stream);
    return launch_cfg<32, 128, 1, 4>(a, hidden_f32, stream);
}

}  // namespace dspark
