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
// One launch per slot j. A workgroup owns kChainTileV vocabulary columns for
// up to 64 blocks: it gathers the rank-r rows markov_w1[prev_b] (the MFMA B
// operand, kept in registers), streams markov_w2 rows (the A operand) and
// computes the [v x b] bias tile on the bf16 MFMA, adds the logits of slot j
// and keeps a running top-k per block in registers. The 32x32 accumulator
// layout gives every lane a single block b and 16 vocabulary ids, so the
// per-lane lists see their ids in increasing order. Lists are merged across
// the two lanes that share b, then across the four waves through LDS; the
// workgroup's best key goes to a 64-bit atomicMax on the slot's running
// argmax word (keys order by score, then lower id), and its list to the
// partials used to assemble the candidates after the last slot.
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kWaves = 4;
constexpr int kVBlocksPerWave = kChainTileV / (kWaves * 32);
static_assert(kVBlocksPerWave * kWaves * 32 == kChainTileV, "tile split");

__global__ __launch_bounds__(256) void chain_init(u64* winners, int n, uint32_t* flags) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) winners[i] = 0ull;
    if (i == 0) *flags = 0u;
}

// NB: 32-wide block groups per workgroup; KL: per-lane list length (>= top_k);
// RS: 16-wide k steps covering the rank (r <= 16 * RS, zero padded).
template <int NB, int KL, int RS>
__global__ __launch_bounds__(256) void chain_step(ChainArgs a, int j) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int wg = blockIdx.x;
    const int bbase = blockIdx.y * NB * 32;
    const int B = a.B, V = a.V, r = a.r;

    // Gathered markov_w1 rows of each lane's block: MFMA B operand.
    u32x4 u[NB][RS];
    int bl[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int b = bbase + nb * 32 + lrow;
        bl[nb] = b;
        int prev = 0;
        if (b < B) {
            prev = (j == 0) ? a.anchors[b] : key_id(a.winners[(long)(j - 1) * B + b]);
            if (prev < 0 || prev >= V) {
                if (j == 0) atomicOr(a.flags, 1u);
                prev = 0;
            }
        }
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int k0 = s * 16 + lhalf * 8;
            u[nb][s] = (b < B && k0 < r)
                           ? *reinterpret_cast<const u32x4*>(a.w1 + (long)prev * r + k0)
                           : u32x4{0u, 0u, 0u, 0u};
        }
    }

    u64 list[NB][KL];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < KL; ++i) list[nb][i] = 0ull;

    const bool vec4 = (V & 3) == 0;
    for (int vb = 0; vb < kVBlocksPerWave; ++vb) {
        const int v0 = wg * kChainTileV + (wave * kVBlocksPerWave + vb) * 32;
        if (v0 >= V) break;
        // markov_w2 rows v0 + lrow: MFMA A operand.
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
            f32x16 acc = f32x16{};
            if (r > 0) {
#pragma unroll
                for (int s = 0; s < RS; ++s) acc = mfma32x32x16(w[s], u[nb][s], acc);
            }
            const int b = bl[nb];
            if (b >= B) continue;
            const float* row = a.logits + ((long)b * a.n_pred + j) * V;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int vq = v0 + 8 * q + 4 * lhalf;
                float z[4];
                if (vec4 && vq + 3 < V) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(row + vq);
                    z[0] = x[0]; z[1] = x[1]; z[2] = x[2]; z[3] = x[3];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] = (vq + e < V) ? row[vq + e] : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = vq + e;
                    if (v < V) {
                        const u64 key = make_key(z[e] + acc[4 * q + e], v);
                        if (key > list[nb][KL - 1]) topk_insert<KL>(list[nb], key);
                    }
                }
            }
        }
    }

    // Merge the two lanes that hold the same block (lane, lane ^ 32).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        u64 other[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) other[i] = shfl_xor_u64(list[nb][i], 32);
#pragma unroll
        for (int i = 0; i < KL; ++i) topk_insert<KL>(list[nb], other[i]);
    }

    // Merge across waves through LDS.
    __shared__ u64 s_list[kWaves][NB * 32][KL];
    if (lhalf == 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < KL; ++i) s_list[wave][nb * 32 + lrow][i] = list[nb][i];
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < NB * 32) {
        const int b = bbase + t;
        if (b < B) {
            u64 m[KL];
#pragma unroll
            for (int i = 0; i < KL; ++i) m[i] = s_list[0][t][i];
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2)
#pragma unroll
                for (int i = 0; i < KL; ++i) topk_insert<KL>(m, s_list[w2][t][i]);
            if (a.top_k > 1) {
                u64* p =
                    a.partials + (((long)j * B + b) * a.nwg + wg) * a.top_k;
#pragma unroll
                for (int i = 0; i < KL; ++i)
                    if (i < a.top_k) p[i] = m[i];
            }
            if (m[0] != 0ull) atomicMax(a.winners + (long)j * B + b, m[0]);
        }
    }
}

// Final assembly, one workgroup per block: tokens and candidates of every
// slot, then the confidence head and the prefix cut.
template <int KL>
__global__ __launch_bounds__(256) void finalize(FinalArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int B = a.B, n = a.n_pred, k = a.top_k;

    for (int j = wave; j < n; j += kWaves) {
        const u64 win = a.winners[(long)j * B + b];
        const long o = (long)b * n + j;
        if (k == 1) {
            if (lane == 0) {
                a.tokens[o] = key_id(win);
                a.candidates[o] = key_id(win);
                if (a.cand_logits) a.cand_logits[o] = key_score(win);
            }
            continue;
        }
        u64 list[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) list[i] = 0ull;
        const u64* p = a.partials + ((long)j * B + b) * a.nwg * k;
        const int cnt = a.nwg * k;
        for (int e = lane; e < cnt; e += 64) {
            const u64 key = p[e];
            if (key > list[KL - 1]) topk_insert<KL>(list, key);
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
            a.tokens[o] = key_id(win);
            if (list[0] != win) atomicOr(a.flags, 2u);  // internal consistency check
#pragma unroll
            for (int i = 0; i < KL; ++i) {
                if (i < k) {
                    a.candidates[o * k + i] = key_id(list[i]);
                    if (a.cand_logits) a.cand_logits[o * k + i] = key_score(list[i]);
                }
            }
        }
    }

    // Confidence head: conf = sigmoid(hidden . conf_w); length = first slot
    // with conf < p_min (llama.cpp commit 6fed9f6, "spec: add confidence-based
    // draft pruning for DSpark" and "dspark: fold conf_min into p_min").
    __shared__ int s_len;
    if (threadIdx.x == 0) s_len = n;
    __syncthreads();
    for (int j = wave; j < n; j += kWaves) {
        float c = 1.0f;
        if (a.conf_w) {
            const long row = (long)b * a.L + a.i_first + j;
            float s = 0.0f;
            for (int h = lane * 8; h < a.H; h += 64 * 8) {
                const u32x4 cw = *reinterpret_cast<const u32x4*>(a.conf_w + h);
                float x[8];
                if (a.hidden_f32) {
                    const f32x4* hp = reinterpret_cast<const f32x4*>(
                        static_cast<const float*>(a.hidden) + row * a.H + h);
                    const f32x4 x0 = hp[0], x1 = hp[1];
                    const uint32_t p0 = pack_bf16x2(x0[0], x0[1]), p1 = pack_bf16x2(x0[2], x0[3]);
                    const uint32_t p2 = pack_bf16x2(x1[0], x1[1]), p3 = pack_bf16x2(x1[2], x1[3]);
                    x[0] = bf16_lo(p0); x[1] = bf16_hi(p0); x[2] = bf16_lo(p1); x[3] = bf16_hi(p1);
                    x[4] = bf16_lo(p2); x[5] = bf16_hi(p2); x[6] = bf16_lo(p3); x[7] = bf16_hi(p3);
                } else {
                    const u32x4 hv = *reinterpret_cast<const u32x4*>(
                        static_cast<const uint16_t*>(a.hidden) + row * a.H + h);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        x[2 * q] = bf16_lo(hv[q]);
                        x[2 * q + 1] = bf16_hi(hv[q]);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    s += x[2 * q] * bf16_lo(cw[q]);
                    s += x[2 * q + 1] * bf16_hi(cw[q]);
                }
            }
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, 64);
            c = 1.0f / (1.0f + expf(-s));
            if (lane == 0 && c < a.p_min) atomicMin(&s_len, j);
        }
        if (lane == 0 && a.conf) a.conf[(long)b * n + j] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) a.lengths[b] = s_len;
}

template <int NB, int KL>
hipError_t step_rs(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    const int rs = (a.r + 15) / 16;
    if (rs <= 1) hipLaunchKernelGGL((chain_step<NB, KL, 1>), grid, dim3(256), 0, s, a, j);
    else if (rs <= 2) hipLaunchKernelGGL((chain_step<NB, KL, 2>), grid, dim3(256), 0, s, a, j);
    else if (rs <= 4) hipLaunchKernelGGL((chain_step<NB, KL, 4>), grid, dim3(256), 0, s, a, j);
    else if (rs <= 8) hipLaunchKernelGGL((chain_step<NB, KL, 8>), grid, dim3(256), 0, s, a, j);
    else hipLaunchKernelGGL((chain_step<NB, KL, 16>), grid, dim3(256), 0, s, a, j);
    return hipGetLastError();
}

template <int NB>
hipError_t step_kl(const ChainArgs& a, int j, dim3 grid, hipStream_t s) {
    if (a.top_k == 1) return step_rs<NB, 1>(a, j, grid, s);
    if (a.top_k <= 4) return step_rs<NB, 4>(a, j, grid, s);
    if (a.top_k <= 8) return step_rs<NB, 8>(a, j, grid, s);
    return step_rs<NB, 16>(a, j, grid, s);
}

}  // namespace

hipError_t launch_chain_init(const ChainArgs& a, hipStream_t stream) {
    const int n = a.n_pred * a.B;
    hipLaunchKernelGGL(chain_init, dim3((n + 255) / 256), dim3(256), 0, stream, a.winners, n, a.flags);
    return hipGetLastError();
}

hipError_t launch_chain_step(const ChainArgs& a, int j, hipStream_t stream) {
    // Blocks are taken 64 at a time (two 32-wide MFMA column groups) so that a
    // markov_w2 tile is read once per step for all of them.
    const int nb = a.B > 32 ? 2 : 1;
    dim3 grid(a.nwg, (a.B + 32 * nb - 1) / (32 * nb));
    return nb == 2 ? step_kl<2>(a, j, grid, stream) : step_kl<1>(a, j, grid, stream);
}

hipError_t launch_finalize(const FinalArgs& a, hipStream_t stream) {
    dim3 grid(a.B), block(256);
    if (a.top_k <= 1) hipLaunchKernelGGL(finalize<1>, grid, block, 0, stream, a);
    else if (a.top_k <= 4) hipLaunchKernelGGL(finalize<4>, grid, block, 0, stream, a);
    else if (a.top_k <= 8) hipLaunchKernelGGL(finalize<8>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(finalize<16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace dspark
