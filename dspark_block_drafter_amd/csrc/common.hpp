// Shared device helpers for the gfx950 kernels of libdspark.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef unsigned long long u64;

constexpr int kWave = 64;

// 32x32x16 bf16 MFMA (CDNA4). Lane l supplies A[row = l % 32][k = 8 * (l / 32) + i]
// and B[k = 8 * (l / 32) + i][col = l % 32], i = 0..7. The 16 accumulators of
// lane l hold D[row = 8 * (g / 4) + 4 * (l / 32) + g % 4][col = l % 32], g = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator tile held in register g by lane l.
__device__ __forceinline__ int acc_row(int g, int lane) {
    return 8 * (g >> 2) + 4 * (lane >> 5) + (g & 3);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Total order used for every argmax / top-k decision: larger score first,
// then smaller id. A (score, id) pair maps to a 64-bit key whose unsigned
// order is that order: the high word is the score's bits made monotone
// (-0 is folded onto +0 first, so equal scores compare equal), the low word
// is ~id.
__device__ __forceinline__ uint32_t order_f32(float x) {
    uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_f32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
__device__ __forceinline__ u64 make_key(float score, int id) {
    return ((u64)order_f32(score) << 32) | (u64)(~(uint32_t)id);
}
__device__ __forceinline__ int key_id(u64 key) { return (int)(~(uint32_t)key); }
__device__ __forceinline__ float key_score(u64 key) { return unorder_f32((uint32_t)(key >> 32)); }

// Lane exchange within a half wave (ds_swizzle, bitmask mode): the value of
// lane l ^ X, X < 32.
template <int X>
__device__ __forceinline__ float swz_xor(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (X << 10)));
}

// Row maxima of a 32 x 32 accumulator block over its 32 columns: lane l holds
// v[g] for row acc_row(g, l) of column l % 32. A butterfly over the five lane
// bits of the half wave: at the step on bit b every lane keeps the half of
// its rows selected by its own bit b and folds in its partner's (lane ^ 2^b)
// values of those rows, so 16 + 8 + 4 + 2 + 1 exchanges in all. Lane l ends
// with the maximum of row acc_row((l >> 1) & 15, l) (lanes l and l ^ 1 hold
// the same row).
__device__ __forceinline__ float block_row_max(const float (&v)[16], int lane) {
    const bool b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1;
    float w8[8], w4[4], w2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = fmaxf(b4 ? v[k + 8] : v[k], swz_xor<16>(b4 ? v[k] : v[k + 8]));
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = fmaxf(b3 ? w8[k + 4] : w8[k], swz_xor<8>(b3 ? w8[k] : w8[k + 4]));
#pragma unroll
    for (int k = 0; k < 2; ++k) w2[k] = fmaxf(b2 ? w4[k + 2] : w4[k], swz_xor<4>(b2 ? w4[k] : w4[k + 2]));
    const float w1 = fmaxf(b1 ? w2[1] : w2[0], swz_xor<2>(b1 ? w2[0] : w2[1]));
    return fmaxf(w1, swz_xor<1>(w1));
}

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int mask) {
    uint32_t lo = __shfl_xor((uint32_t)v, mask, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, kWave);
    return ((u64)hi << 32) | lo;
}

// Per-lane select (lanes set in `lanes` take if_set). Written as one
// v_cndmask so that a tree of them is not folded back into an indexed array
// access (which the compiler would then place in LDS or scratch).
__device__ __forceinline__ float lane_select(float if_set, float if_clear, u64 lanes) {
    float r;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(lanes));
    return r;
}

// Insert `key` into the descending list `list[0..K)`, keeping the K largest.
template <int K>
__device__ __forceinline__ void topk_insert(u64 (&list)[K], u64 key) {
    // The list is in decreasing order, so key > list[i] implies key > list[i + 1]:
    // all K comparisons are independent, and entry i becomes list[i - 1] (the
    // key went above it), the key (it lands here) or stays. A key not above
    // the last entry (0 among them) changes nothing.
    bool gt[K];
#pragma unroll
    for (int i = 0; i < K; ++i) gt[i] = key > list[i];
#pragma unroll
    for (int i = K - 1; i > 0; --i) list[i] = gt[i - 1] ? list[i - 1] : (gt[i] ? key : list[i]);
    list[0] = gt[0] ? key : list[0];
}

// ---- direct-to-LDS pipelines ----------------------------------------------
// global_load_lds_dwordx4 writes each lane's 16 bytes to LDS slot base + lane;
// completion is tracked by vmcnt, so waits and barriers are explicit (a
// workgroup fence would drain every load in flight).

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `newer` stages of LW loads each are still in flight
// (newer <= D; the immediate has to be a compile-time constant).
template <int LW, int D>
__device__ __forceinline__ void wait_stages(int newer) {
    if constexpr (D == 0) {
        wait_vmcnt<0>();
    } else {
        if (newer >= D) wait_vmcnt<D * LW>();
        else wait_stages<LW, D - 1>(newer);
    }
}

// Wait until every LDS read this wave issued has returned its data.
__device__ __forceinline__ void wait_lds_reads() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Largest squared row norm of a bf16 matrix [rows, r], r a multiple of 8,
// taken by G workgroups (this is group g): a sum of squares of bf16 values in
// fp32 (every square is exact), raised into *out as fp32 bits (the bits of
// non-negative floats order as unsigned integers). When a row is a power of
// two of 16-byte chunks (r = 8, 16, ..., 256) the wave reads the matrix as
// consecutive 16-byte chunks, 16 per lane in flight, and sums each row over
// the aligned group of lanes that hold its chunks; otherwise each thread sums
// whole rows.
__device__ __forceinline__ void row_norm_part(const uint16_t* w, long rows, int r, int g, int G,
                                              uint32_t* out) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int nw = blockDim.x >> 6, wave = tid >> 6;
    const int cpr = r >> 3;   // 16-byte chunks per row
    float best = 0.0f;
    if ((cpr & (cpr - 1)) == 0 && cpr <= 64) {
        constexpr int U = 16;
        const long chunks = rows * cpr;
        const u32x4* p = reinterpret_cast<const u32x4*>(w);
        // wave-steps of 64 U chunks; wave (g, wave) takes steps g * nw + wave + k * G * nw
        for (long base = ((long)g * nw + wave) * 64 * U; base < chunks; base += (long)G * nw * 64 * U) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long c = base + u * 64 + lane;
                x[u] = c < chunks ? p[c] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = bf16_lo(x[u][q]), hi = bf16_hi(x[u][q]);
                    s += lo * lo;
                    s += hi * hi;
                }
                // the row's sum over its cpr lanes (aligned groups of the 64)
                for (int m = 1; m < cpr; m <<= 1) s += __shfl_xor(s, m, kWave);
                best = fmaxf(best, s);
            }
        }
    } else {
        const int nt = blockDim.x;
        for (long row = (long)g * nt + tid; row < rows; row += (long)G * nt) {
            const uint16_t* q0 = w + row * r;
            float s = 0.0f;
            for (int k = 0; k < r; k += 8) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(q0 + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = bf16_lo(x[q]), hi = bf16_hi(x[q]);
                    s += lo * lo;
                    s += hi * hi;
                }
            }
            best = fmaxf(best, s);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) best = fmaxf(best, __shfl_xor(best, m, kWave));
    if (lane == 0) atomicMax(out, __float_as_uint(best));
}

// XCD-aware order of T work units: dispatch sends workgroup i to XCD i % 8,
// so XCD x receives q + (x < rem) of them (T = 8 q + rem); give it that many
// consecutive units, in XCD order, so neighbouring units share an L2. (For
// T % 8 == 0: (i % 8) (T / 8) + i / 8.)
__device__ __forceinline__ int xcd_unit(int i, int T) {
    const int x = i & 7, l = i >> 3, q = T >> 3, rem = T & 7;
    return x * q + (x < rem ? x : rem) + l;
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) char lds_char;
// Cache policy of a load that is read once (non-temporal: gfx950 "nt").
constexpr int kLoadNT = 2;

}  // namespace dspark
