// Greedy verification of a proposal against the target's own tokens.
//
// Speculative decoding stays lossless under greedy decoding: the target
// checks the drafted tokens and keeps the longest prefix it would have
// produced itself (llama.cpp commit 6fed9f6 "spec: add DSpark speculative
// decoding", the in-graph chain item: greedy stays lossless, verification is
// unchanged from DFlash). DSpark hands the runtime a candidate lattice of
// top_k ids per slot that the engine walks greedily (onnxruntime-genai PR
// #2490 "Export DSpark block drafters for Qwen 3.5 and 3.8", DFlash 2 and
// DSpark commit messages; lucebox PR #626 description, the tree candidate
// top-k). A block is submitted with its confidence-truncated length, so the
// walk of block b stops at lengths[b], at the latest.
//
// One wave per block: lane j checks slot j (64 slots per round) against the
// slot's candidates, a ballot finds the first slot that fails. A second
// single-workgroup kernel sums the accepted and submitted slots in a fixed
// order, so the outputs are integers, exact and deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kWaves = 4;   // blocks per workgroup of the walk; waves of the sum

__global__ __launch_bounds__(256) void verify_walk(VerifyArgs a) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int len = min(max(a.lengths[b], 0), a.n_pred);
    int m = len;
    for (int j0 = 0; j0 < len; j0 += 64) {
        const int j = j0 + lane;
        bool hit = true;
        if (j < len) {
            const long slot = (long)b * a.n_pred + j;
            const int t = a.target[slot];
            const int32_t* c = a.candidates + slot * a.top_k;
            hit = false;
            for (int i = 0; i < a.width; ++i) hit = hit || c[i] == t;
        }
        const u64 miss = __builtin_amdgcn_ballot_w64(!hit);
        if (miss != 0ull) {
            m = j0 + __builtin_ctzll(miss);
            break;
        }
    }
    if (lane == 0) a.accepted[b] = m;
}

__global__ __launch_bounds__(256) void verify_totals(VerifyArgs a) {
    __shared__ long s_acc[kWaves], s_len[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    long acc_sum = 0, len_sum = 0;
    for (int b = threadIdx.x; b < a.B; b += 256) {
        acc_sum += a.accepted[b];
        len_sum += min(max(a.lengths[b], 0), a.n_pred);
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        acc_sum += __shfl_xor(acc_sum, mask, kWave);
        len_sum += __shfl_xor(len_sum, mask, kWave);
    }
    if (lane == 0) {
        s_acc[wave] = acc_sum;
        s_len[wave] = len_sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        long ta = 0, tl = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            ta += s_acc[w];
            tl += s_len[w];
        }
        a.totals[0] = (int32_t)ta;
        a.totals[1] = (int32_t)tl;
    }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(verify_walk, dim3((a.B + kWaves - 1) / kWaves), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(verify_totals, dim3(1), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dspark
