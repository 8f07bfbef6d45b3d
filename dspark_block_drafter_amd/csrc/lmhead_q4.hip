// 4-bit lm_head: packing of the GGUF blocks, per-call preparation of the
// hidden rows, and the projection.
//
// Format (the reading of the requantized 4-bit GGUF drafter that lucebox PR
// #626 "feat(qwen38): add adaptive concurrent DSpark speculation" validates
// on the device, Summary -> Drafter; the pages give no block layout): GGUF's
// plain 4-bit blocks of 32 weights along H, an IEEE binary16 scale d and 16
// code bytes, code byte j holding element j (low nibble) and element j + 16
// (high nibble); a weight is d * (q - 8).
//
// Projection (gfx950): z[m][v] = sum over blocks g of d_vg * sum_e x_me *
// (q_vge - 8), one 16x16x32 bf16 MFMA per block of 16 rows x 16 columns.
//  * B operand: 128 + q, exact in bf16 (the exponent of 128 with the code in
//    the low mantissa bits: one and-or per pair of codes), so the MFMA sums
//    x * (128 + q), every product exact, in fp32.
//  * Its C input is -136 * sum_e x_me, the same MFMA with B = -136 in every
//    slot (exact in bf16, products exact, summed in fp32), so it returns the
//    block's sum_e x_me (q_vge - 8).
//  * Each block's result is scaled by its d in fp32: four FMAs per lane.
// The MFMA pairs A and B by their k slot, so any order of a block's 32
// elements over the slots is correct as long as both operands use it. Lane
// 16 kq + c supplies code bytes 4 kq .. 4 kq + 3 of its column's block, i.e.
// elements 4 kq + {0, 2, 1, 3} (low nibbles, as the and-or pairs bytes 0/2
// and 1/3 of a dword) then 16 + 4 kq + {0, 2, 1, 3} (high nibbles); the
// preparation writes the hidden rows in that same order.
//
// Layout of the packed head: V in tiles of 16 rows, H in quads of 4 blocks.
// Tile t, quad u owns a 1024-byte code record at (t * GQ + u) * 1024 and a
// 128-byte scale record after all code records, at (t * GQ + u) * 128. Lane
// l = 16 kq + c of a wave loads the 16 bytes at 16 l of the code record:
// dword gg holds code bytes 4 kq .. 4 kq + 3 of block 4 u + gg of row
// 16 t + c. Halfword 4 c + gg of the scale record is that block's scale.
// A wave therefore streams every record it needs with one coalesced 1 KB
// load (and one 512-byte scale load), and a tile's records are contiguous.
// At small row counts the projection is bound by HBM: 0.5625 bytes per
// weight against 2 for bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// 16x16x32 bf16 MFMA: lane l supplies A[l % 16][k] and B[k][l % 16] for the
// eight k slots 8 (l / 16) .. 8 (l / 16) + 7, and holds D[4 (l / 16) + i][l % 16],
// i = 0..3.

// Four code bytes c0..c3 -> eight bf16 values 128 + nibble, in the k order
// c0.lo, c2.lo, c1.lo, c3.lo, c0.hi, c2.hi, c1.hi, c3.hi. The constants
// kmask = 0x000F000F and kexp = 0x43004300 (bf16 128.0 in both halves) come
// in registers, so that each pair of codes costs one v_and_or_b32 (a 32-bit
// literal cannot go into a three-operand instruction).
__device__ __forceinline__ u32x4 q4_operand(uint32_t w, uint32_t kmask, uint32_t kexp) {
    return u32x4{(w & kmask) | kexp, ((w >> 8) & kmask) | kexp, ((w >> 4) & kmask) | kexp,
                 ((w >> 12) & kmask) | kexp};
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Element of the block that k slot s (0..7) of lane group kq carries.
__device__ __forceinline__ int q4_elem(int kq, int s) {
    return ((s & 4) ? 16 : 0) + 4 * kq + ((s & 1) << 1) + ((s >> 1) & 1);
}

// ---- packing ------------------------------------------------------------------
// One thread per (record, lane): the lane's 16 code bytes and, for kq = 0,
// its column's four scales.
__global__ __launch_bounds__(256) void q4_pack(Q4PackArgs a) {
    const long id = (long)blockIdx.x * 256 + threadIdx.x;
    const long recs = (long)a.T16 * a.GQ;
    if (id >= recs * 64) return;
    const long rec = id >> 6;
    const int l = (int)(id & 63), kq = l >> 4, c = l & 15;
    const int t = (int)(rec / a.GQ), u = (int)(rec % a.GQ);
    const int v = 16 * t + c;
    uint32_t dw[4], sc[4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
        const int g = 4 * u + gg;
        if (v < a.V && g < a.G) {
            const uint8_t* blk = a.blocks + ((long)v * a.G + g) * kQ4BlockBytes;
            const uint8_t* q = blk + 2 + 4 * kq;
            dw[gg] = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) |
                     ((uint32_t)q[3] << 24);
            sc[gg] = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
        } else {
            dw[gg] = 0x88888888u;   // code 8 with scale 0: weight 0
            sc[gg] = 0u;
        }
    }
    reinterpret_cast<u32x4*>(a.packed)[rec * 64 + l] = u32x4{dw[0], dw[1], dw[2], dw[3]};
    if (kq == 0) {
        uint32_t* s = reinterpret_cast<uint32_t*>(a.packed + (size_t)recs * kQ4CodeRec +
                                                  (size_t)rec * kQ4ScaleRec);
        s[2 * c] = sc[0] | (sc[1] << 16);
        s[2 * c + 1] = sc[2] | (sc[3] << 16);
    }
}

// ---- per-call preparation ----------------------------------------------------------
// One thread per (row m, block g < 4 GQ): the block's 32 hidden values as
// bf16 (fp32 hidden rounded to nearest even) in the k order above. Blocks
// past H/32 are zero.
__global__ __launch_bounds__(256) void q4_prep(Q4Args a) {
    const long id = (long)blockIdx.x * 256 + threadIdx.x;
    const int GP = 4 * a.GQ;
    if (id >= (long)a.M * GP) return;
    const int m = (int)(id / GP), g = (int)(id % GP);
    const long hrow = (long)(m / a.n_pred) * a.L + a.i_first + m % a.n_pred;
    uint32_t x[32];
    if (g < a.G) {
        if (a.hidden_f32) {
            const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.hidden) +
                                                            hrow * a.H + 32 * g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 v = p[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) x[4 * i + k] = bf16_rne(v[k]);
            }
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.hidden) +
                                                            hrow * a.H + 32 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = p[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[8 * i + 2 * k] = v[k] & 0xffffu;
                    x[8 * i + 2 * k + 1] = v[k] >> 16;
                }
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = 0u;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.xp + (size_t)m * 128 * a.GQ + 32 * g);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) w[p] = x[q4_elem(kq, 2 * p)] | (x[q4_elem(kq, 2 * p + 1)] << 16);
        dst[kq] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ---- projection -----------------------------------------------------------------
// A workgroup of four waves owns BM = 16 FM rows and 64 CTW columns (wave w
// owns column tiles CTW w .. CTW w + CTW - 1 of them) over the whole of H,
// one quad of blocks (128 elements) per step, through an NS-stage LDS ring
// filled by global_load_lds (each lane's bytes land at the instruction's LDS
// base + lane * size; completion is counted by vmcnt, so waits and barriers
// are explicit, as in the bf16 projection's direct-to-LDS pipeline). A stage
// holds, for one quad:
//  * the A tile, BM rows x 16 chunks of 16 bytes (chunk 4 gg + kq = the k
//    slots 8 kq .. 8 kq + 7 of block gg); chunk ch of row r sits at
//    ch ^ (r & 15) so that the 16 rows of one operand read fall in distinct
//    banks (the lane that fills a slot fetches the chunk that belongs there);
//    every wave loads FM of its 4 FM 1 KB pieces;
//  * each wave's code records (1 KB per column tile) and scale records
//    (128 bytes per tile, two tiles per 4-byte-per-lane load).
// The 136 sum_e x_me of a block is produced by one more MFMA per row tile
// and block, with B = -136 in every slot (exact in bf16), and enters the
// code MFMAs as their C input: they return sum_e x_me (q - 8) directly.
template <int FM, int CTW, int NS, bool SMAX>
__global__ __launch_bounds__(256) void lmhead_q4(Q4Args a) {
    constexpr int BM = 16 * FM;
    constexpr int AB = BM * 256;                   // A tile bytes per stage
    constexpr int CB = 4 * CTW * kQ4CodeRec;       // code bytes per stage
    constexpr int SB = AB + CB + 4 * CTW * kQ4ScaleRec;
    constexpr int LW = FM + CTW + CTW / 2;         // loads per wave per stage
    static_assert(CTW % 2 == 0, "scale records are loaded two tiles at a time");
    static_assert(NS >= 2 && (NS - 1) * LW < 64, "pipeline depth");
    __shared__ __attribute__((aligned(1024))) char smem[NS * SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, kq = lane >> 4;
    const int M = a.M, V = a.V, GQ = a.GQ;
    const int nrb = (M + BM - 1) / BM;
    const int ncu = (a.T16 + 4 * CTW - 1) / (4 * CTW);
    const int nunits = nrb * ncu;
    if ((int)blockIdx.x >= nunits) {
        // a norm workgroup, in the launch's last, partly filled round
        const int g = blockIdx.x - nunits;
        row_norm_part(a.w2, a.w_rows, a.w_rank, g, a.norm_groups, a.w2n2);
        if (a.w1n2 != nullptr) row_norm_part(a.w1, a.w_rows, a.w_rank, g, a.norm_groups, a.w1n2);
        return;
    }
    // the row blocks of one column unit are consecutive; consecutive
    // workgroups of one XCD (blockIdx % 8) get consecutive units, so a unit's
    // codes come into one L2
    const int bid = xcd_unit(blockIdx.x, nunits);
    const int cu = bid / nrb, rb = bid - cu * nrb;
    const int m0 = rb * BM, t0 = cu * 4 * CTW + wave * CTW;

    // per-lane sources at quad 0 and the LDS offsets (in a stage) of this wave's loads
    const uint8_t* asrc[FM];
    int adst[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int q = wave * FM + i;              // 1 KB piece of the A tile
        const int r = 4 * q + (lane >> 4), ch = (lane & 15) ^ (r & 15);
        asrc[i] = reinterpret_cast<const uint8_t*>(a.xp) + ((size_t)min(m0 + r, M - 1) * 16 * GQ + ch) * 16;
        adst[i] = q * 1024;
    }
    const uint8_t* scale_base = a.packed + (size_t)a.T16 * GQ * kQ4CodeRec;
    const uint8_t* csrc[CTW];
    const uint8_t* ssrc[CTW / 2];
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
        const int t = min(t0 + j, a.T16 - 1);
        csrc[j] = a.packed + (size_t)t * GQ * kQ4CodeRec + 16 * lane;
    }
#pragma unroll
    for (int k = 0; k < CTW / 2; ++k) {
        const int t = min(t0 + 2 * k + (lane >> 5), a.T16 - 1);
        ssrc[k] = scale_base + (size_t)t * GQ * kQ4ScaleRec + 4 * (lane & 31);
    }
    const int cdst = AB + wave * CTW * kQ4CodeRec;
    const int sdst = AB + CB + wave * CTW * kQ4ScaleRec;

    auto issue = [&](int stage, int u) {
        char* base = smem + stage * SB;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + (size_t)u * 256),
                                             (lds_ptr)(base + adst[i]), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < CTW; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(csrc[j] + (size_t)u * kQ4CodeRec),
                                             (lds_ptr)(base + cdst + j * kQ4CodeRec), 16, 0, 0);
#pragma unroll
        for (int k = 0; k < CTW / 2; ++k)
            __builtin_amdgcn_global_load_lds((const void*)(ssrc[k] + (size_t)u * kQ4ScaleRec),
                                             (lds_ptr)(base + sdst + 2 * k * kQ4ScaleRec), 4, 0, 0);
    };

    f32x4 acc[FM][CTW];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int j = 0; j < CTW; ++j) acc[f][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4 neg136 = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
    const f32x4 zero4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // the decoding constants of q4_operand, held in registers
    uint32_t kmask = 0x000F000Fu, kexp = 0x43004300u;
    asm volatile("" : "+v"(kmask), "+v"(kexp));

    auto compute = [&](int stage) {
        const char* base = smem + stage * SB;
        const u32x4* A = reinterpret_cast<const u32x4*>(base);
        // every LDS read of the quad first: one wait for all of them
        u32x4 xa[FM][4], code[CTW];
        u32x2 sc[CTW];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) xa[f][gg] = A[(16 * f + c) * 16 + ((4 * gg + kq) ^ c)];
#pragma unroll
        for (int j = 0; j < CTW; ++j) {
            code[j] = *reinterpret_cast<const u32x4*>(base + cdst + j * kQ4CodeRec + 16 * lane);
            sc[j] = *reinterpret_cast<const u32x2*>(base + sdst + j * kQ4ScaleRec + 8 * c);
        }
        // Block gg's products and block gg - 1's scalings are interleaved: the
        // scalings read the previous block's results, so they can issue while
        // the matrix unit works on the next block's products.
        f32x4 P[2][FM][CTW];
        float D[2][CTW];
        auto products = [&](int gg, f32x4 (&p)[FM][CTW], float (&d)[CTW]) {
            u32x4 bq[CTW];
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                bq[j] = q4_operand(code[j][gg], kmask, kexp);
                const uint32_t pair = gg < 2 ? sc[j].x : sc[j].y;
                d[j] = f16_bits_to_f32((gg & 1) ? (pair >> 16) : (pair & 0xffffu));
            }
            f32x4 corr[FM];
#pragma unroll
            for (int f = 0; f < FM; ++f)
                corr[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, xa[f][gg]), __builtin_bit_cast(bf16x8, neg136), zero4, 0, 0, 0);
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int j = 0; j < CTW; ++j)
                    p[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, xa[f][gg]), __builtin_bit_cast(bf16x8, bq[j]), corr[f], 0, 0, 0);
        };
        auto scale = [&](const f32x4 (&p)[FM][CTW], const float (&d)[CTW]) {
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int j = 0; j < CTW; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(d[j], p[f][j][i], acc[f][j][i]);
        };
        products(0, P[0], D[0]);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            if (gg < 3) products(gg + 1, P[(gg + 1) & 1], D[(gg + 1) & 1]);
            scale(P[gg & 1], D[gg & 1]);
        }
    };

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < GQ) issue(s, s);
    int stage = 0;
    for (int u = 0; u < GQ; ++u) {
        // quad u has landed: at most min(NS - 2, GQ - 1 - u) newer quads may still fly
        wait_stages<LW, NS - 2>(min(NS - 2, GQ - 1 - u));
        // this wave's reads of the previous stage are done before any wave refills it
        wait_lds_reads();
        block_barrier();
        const int un = u + NS - 1;
        if (un < GQ) issue(un % NS, un);
        compute(stage);
        stage = stage + 1 == NS ? 0 : stage + 1;
    }

    // Slab maxima (the chain's top-k bound): per row, the largest logit (bias
    // included) over each slab of kSlabCols = 64 columns. A wave's columns
    // are a whole slab (CTW = 4) or half of one (CTW = 2: waves w and w ^ 1
    // share it). Lane (c, kq) takes the maximum over its CTW columns, then
    // over the 16 lanes of its kq (lane bits 0-3).
    if constexpr (SMAX) {
        static_assert(CTW == 2 || CTW == 4, "a wave holds half a slab or a whole one");
        const int nslab = (V + kSlabCols - 1) / kSlabCols;
        float mx[FM][4];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx[f][i] = -INFINITY;
#pragma unroll
        for (int j = 0; j < CTW; ++j) {
            const int v = 16 * (t0 + j) + c;
            if (v >= V) continue;
            const float b = a.bias ? a.bias[v] : 0.0f;
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx[f][i] = fmaxf(mx[f][i], acc[f][j][i] + b);
        }
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int x = 1; x < 16; x <<= 1) mx[f][i] = fmaxf(mx[f][i], __shfl_xor(mx[f][i], x, kWave));
        bool writer = c == 0;
        if constexpr (CTW == 2) {
            // The pair exchanges its halves through the ring's first bytes,
            // once every wave is past its last read of the ring. (A second
            // LDS array would make the compiler order every ring read after
            // all copies in flight: a vmcnt(0) in the main loop, 20% slower.)
            float* s_half = reinterpret_cast<float*>(smem);
            __syncthreads();
            if (c == 0) {
#pragma unroll
                for (int f = 0; f < FM; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s_half[wave * 16 * FM + 16 * f + 4 * kq + i] = mx[f][i];
            }
            __syncthreads();
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mx[f][i] = fmaxf(mx[f][i], s_half[(wave ^ 1) * 16 * FM + 16 * f + 4 * kq + i]);
            writer = writer && (wave & 1) == 0;   // the even wave of the pair writes the slab
        }
        const int slab = 16 * t0 / kSlabCols;
        if (writer && slab < nslab) {
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * f + 4 * kq + i;
                    if (m < M) a.smax[(size_t)m * nslab + slab] = mx[f][i];
                }
        }
    }

    // + bias, fp32 store (lane (c, kq) holds rows 4 kq + i of column c)
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
        const int v = 16 * (t0 + j) + c;
        if (v >= V) continue;
        const float b = a.bias ? a.bias[v] : 0.0f;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * f + 4 * kq + i;
                if (m < M) __builtin_nontemporal_store(acc[f][j][i] + b, a.out + (size_t)m * V + v);
            }
    }
}

template <int FM, int CTW, int NS>
hipError_t run_q4(const Q4Args& a, hipStream_t stream) {
    const long nrb = (a.M + 16 * FM - 1) / (16 * FM);
    const long ncu = (a.T16 + 4 * CTW - 1) / (4 * CTW);
    const dim3 grid((unsigned)(nrb * ncu + (a.w2n2 ? a.norm_groups : 0)));
    if (a.smax) hipLaunchKernelGGL((lmhead_q4<FM, CTW, NS, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((lmhead_q4<FM, CTW, NS, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_pack(const Q4PackArgs& a, hipStream_t stream) {
    const long threads = (long)a.T16 * a.GQ * 64;
    hipLaunchKernelGGL(q4_pack, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_lmhead_q4(const Q4Args& a, hipStream_t stream) {
    const long threads = (long)a.M * 4 * a.GQ;
    hipLaunchKernelGGL(q4_prep, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Tiles measured on MI355X over (FM, CTW, NS) in {1, 2, 4, 8} x {2, 4} x
    // {2, 3, 4, 6} (prep + projection, us): Qwen3-8B shape (M = 16) 71 with
    // <1, 2, 4> (74 <1, 2, 3>, 81 <1, 2, 6>); Gemma-4 shape (M = 24) 105 with
    // <2, 4, 2> (107 <2, 2, 3>, 109 <2, 4, 3>); B = 8 tree (M = 128) 608 with
    // <4, 2, 2> (643 <2, 4, 2>, 678 <8, 2, 2>); B = 64 (M = 1024) 4199 with
    // <4, 2, 2> (4466 <8, 2, 2>).
    if (a.M <= 16) return run_q4<1, 2, 4>(a, stream);
    if (a.M <= 32) return run_q4<2, 4, 2>(a, stream);
    return run_q4<4, 2, 2>(a, stream);
}

}  // namespace dspark
