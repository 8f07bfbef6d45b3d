/*
 * CPU oracle for the DSpark drafter's proposal step.
 *
 * TEST INFRASTRUCTURE. This library exists only to check the GPU library.
 * Only the test suite, the smoke entry point and the benchmark's CPU-baseline
 * leg may load it. It shares no code, header or table with the GPU path and
 * includes no HIP header.
 *
 * What it computes, one block b at a time, in the order the method states:
 *
 *  1. Projection: every prediction slot j of block b goes through the shared
 *     lm_head, z_j[v] = sum_h x_j[h] * lm_head[v][h] (+ bias[v]). The drafter
 *     owns no output head of its own and borrows the target's
 *     (onnxruntime-genai PR #2490 "Export DSpark block drafters for Qwen 3.5
 *     and 3.8", DSpark commit message; llama.cpp commit 6fed9f6 "spec: add
 *     DSpark speculative decoding", first item). The bias is the -1e9 row
 *     bias of an expanded reduced vocabulary (llama.cpp PR #26275 "dspark:
 *     support speculators-format checkpoints", first commit message).
 *  2. Markov chain: slot j is re-scored with the low-rank bigram bias of the
 *     previous token, z'_j[v] = z_j[v] + sum_k markov_w2[v][k] *
 *     markov_w1[prev_j][k]; prev_0 is the block's anchor and prev_j (j>0) is
 *     the argmax of z'_{j-1} (llama.cpp commit 6fed9f6, item "spec: add DSpark
 *     speculative decoding", the chained-bias formula).
 *  3. Candidates: the top-k of the same biased scores per slot, for the tree /
 *     lattice (lucebox PR #626 description: the tree's candidate top-k also
 *     carries the Markov bias; onnxruntime-genai PR #2490, dspark_top_k).
 *  4. Confidence: one scalar per prediction slot, sigma(sum_h x_j[h] *
 *     conf_w[h]), read as the predicted survival probability; the block is cut
 *     at the first slot below p_min (llama.cpp commit 6fed9f6, items "spec:
 *     add confidence-based draft pruning for DSpark" and "dspark: fold
 *     conf_min into p_min").
 *
 * Reduced draft vocabulary: the draft head scores D draft ids and the int64
 * table d2t gives the absolute target id of each; the draft logits are
 * scattered to those target ids at run time (llama.cpp PR #26275, rework
 * commit message; "Format differences": draft_vocab_size < vocab_size with a
 * d2t table). The chain then runs over the draft ids: the Markov bias of
 * draft id i is markov_w2[i] . markov_w1[prev] with prev a target id, and the
 * chosen draft ids are reported as target ids. Every target id off the table
 * has no score, so it can never be chosen.
 *
 * Adaptive block length: the confidence of every slot is known before the
 * chain runs, so a block cut at slot `length` only drafts its first `length`
 * slots; each block may carry its own threshold and its own number of
 * candidates (lucebox PR #626 description: the confidence-gate adaptive block
 * length and the per-request override).
 *
 * Verification: greedy speculation is lossless because the target keeps only
 * the longest drafted prefix it would have produced itself (llama.cpp commit
 * 6fed9f6, the in-graph chain item: verification unchanged from DFlash); with
 * a candidate lattice the engine walks it greedily, accepting a slot when the
 * target's token is among the slot's candidates (onnxruntime-genai PR #2490,
 * DFlash 2 and DSpark commit messages). A block submits only its
 * confidence-truncated slots.
 *
 * Block layouts: anchor-first (every slot predicts; i_first_pred = 0) and the
 * 1+N bonus-anchor layout (slot 0 holds the bonus token and is never read;
 * i_first_pred = 1) (llama.cpp PR #26275, first commit message and
 * "Format differences").
 *
 * Quantized head (q4): the drafter the pages validate on the device is a
 * requantized GGUF with 4-bit weights (lucebox PR #626, "Drafter"), but they
 * never spell out the block format. The reading taken here is GGUF's plain
 * 4-bit type: every row of lm_head is H/32 blocks of 18 bytes, each an IEEE
 * binary16 scale d (little-endian) followed by 16 bytes of codes; byte j of
 * the codes carries element j of the block in its low nibble and element
 * j + 16 in its high nibble, and an element with code q is worth d * (q - 8).
 * The projection is then the plain one over those exact values (PARITY
 * PINNED by a hand-decoded golden row, numpy, and equality with the bf16
 * path when every decoded weight is a bf16 value).
 *
 * Arithmetic: bf16 operands are decoded exactly, every sum is accumulated in
 * double precision in increasing index order (a bf16*bf16 product is exact in
 * double), and a value is rounded once to float only where the contract hands
 * out a float: the biased scores z' on which argmax / top-k decide, and the
 * confidence compared with p_min. fp32 hidden states are first rounded to
 * bf16 (nearest, ties to even), since the contraction is bf16 x bf16.
 * Argmax ties go to the lowest index; top-k orders by value descending, then
 * index ascending.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR (-1)

/* Value of a bf16 bit pattern: a bf16 is the upper half of a binary32. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even.
 * Written as "pick the nearer of the two neighbouring bf16 values": lo is x
 * truncated toward zero, hi the next bf16 of larger magnitude. */
uint16_t oracle_bf16_round(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(x))
        return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1u);
    double dx = (double)x;
    double dlo = bf16_value(lo);
    double dhi;
    if ((hi & 0x7f80u) == 0x7f80u) /* the next magnitude is past the largest finite bf16 */
        dhi = copysign(ldexp(1.0, 128), dx);
    else
        dhi = bf16_value(hi);
    double elo = fabs(dx - dlo), ehi = fabs(dhi - dx);
    if (elo < ehi)
        return lo;
    if (ehi < elo)
        return hi;
    return (lo & 1u) ? hi : lo;
}

double oracle_bf16_value(uint16_t bits) { return bf16_value(bits); }

/* Row `row` of hidden [B*L, H] as exact doubles of its bf16 values. */
static void load_hidden_row(const void* hidden, int hidden_is_f32, long row, int H, double* x)
{
    if (hidden_is_f32) {
        const float* p = (const float*)hidden + row * (long)H;
        for (int h = 0; h < H; ++h)
            x[h] = bf16_value(oracle_bf16_round(p[h]));
    } else {
        const uint16_t* p = (const uint16_t*)hidden + row * (long)H;
        for (int h = 0; h < H; ++h)
            x[h] = bf16_value(p[h]);
    }
}

/* Projection of the n_pred prediction rows of block b through lm_head.
 * z[j*V + v] = sum_h x_j[h] * lm_head[v*H + h] (+ bias[v]), x_j = hidden row
 * b*L + i_first_pred + j. */
int oracle_block_logits(const void* hidden, int hidden_is_f32, const uint16_t* lm_head,
                        const float* bias, int L, int H, int V, int i_first_pred, int b,
                        double* z)
{
    int n_pred = L - i_first_pred;
    if (n_pred <= 0 || H <= 0 || V <= 0 || b < 0)
        return ORACLE_ERR;
    double* x = (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)H);
    if (!x)
        return ORACLE_ERR;
    for (int j = 0; j < n_pred; ++j)
        load_hidden_row(hidden, hidden_is_f32, (long)b * L + i_first_pred + j, H, x + (size_t)j * H);

#pragma omp parallel for schedule(static)
    for (long v = 0; v < V; ++v) {
        const uint16_t* w = lm_head + v * (long)H;
        for (int j = 0; j < n_pred; ++j) {
            const double* xj = x + (size_t)j * H;
            double s = 0.0;
            for (int h = 0; h < H; ++h)
                s += xj[h] * bf16_value(w[h]);
            if (bias)
                s += (double)bias[v];
            z[(size_t)j * V + v] = s;
        }
    }
    free(x);
    return ORACLE_OK;
}

/* Low-rank bigram bias of token `prev`: m[v] = sum_k w2[v][k] * w1[prev][k]. */
int oracle_markov_bias(const uint16_t* w1, const uint16_t* w2, int V, int r, int prev, double* m)
{
    if (prev < 0 || prev >= V || r < 0)
        return ORACLE_ERR;
    if (r == 0) {
        for (long v = 0; v < V; ++v)
            m[v] = 0.0;
        return ORACLE_OK;
    }
    const uint16_t* u = w1 + (long)prev * r;
#pragma omp parallel for schedule(static)
    for (long v = 0; v < V; ++v) {
        const uint16_t* w = w2 + v * (long)r;
        double s = 0.0;
        for (int k = 0; k < r; ++k)
            s += bf16_value(w[k]) * bf16_value(u[k]);
        m[v] = s;
    }
    return ORACLE_OK;
}

/* Biased scores of one slot under a given previous token, rounded once to
 * float: zp[v] = float(z_row[v] + m[v]). */
int oracle_step_scores(const double* z_row, const uint16_t* w1, const uint16_t* w2, int V, int r,
                       int prev, float* zp)
{
    double* m = (double*)malloc(sizeof(double) * (size_t)V);
    if (!m)
        return ORACLE_ERR;
    int st = oracle_markov_bias(w1, w2, V, r, prev, m);
    if (st == ORACLE_OK)
        for (long v = 0; v < V; ++v)
            zp[v] = (float)(z_row[v] + m[v]);
    free(m);
    return st;
}

/* Scalar argmax, first (lowest) index on ties. */
int oracle_argmax(const float* zp, int V)
{
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (zp[v] > zp[best])
            best = v;
    return best;
}

/* Top-k by k passes of the argmax scan, each skipping the ids already taken;
 * yields value descending, index ascending among equal values. */
int oracle_topk(const float* zp, int V, int k, int32_t* idx, float* val)
{
    if (k < 1 || k > V)
        return ORACLE_ERR;
    for (int t = 0; t < k; ++t) {
        int best = -1;
        for (int v = 0; v < V; ++v) {
            int taken = 0;
            for (int s = 0; s < t; ++s)
                if (idx[s] == v)
                    taken = 1;
            if (taken)
                continue;
            if (best < 0 || zp[v] > zp[best])
                best = v;
        }
        idx[t] = best;
        val[t] = zp[best];
    }
    return ORACLE_OK;
}

/* The chain of one block over precomputed projections z [n_pred][V]. */
int oracle_block_chain(const double* z, const uint16_t* w1, const uint16_t* w2, int V, int r,
                       int anchor, int n_pred, int top_k, int32_t* tokens, int32_t* cand,
                       float* cand_val)
{
    if (anchor < 0 || anchor >= V || n_pred <= 0 || top_k < 1 || top_k > V)
        return ORACLE_ERR;
    float* zp = (float*)malloc(sizeof(float) * (size_t)V);
    if (!zp)
        return ORACLE_ERR;
    int prev = anchor;
    int st = ORACLE_OK;
    for (int j = 0; j < n_pred && st == ORACLE_OK; ++j) {
        st = oracle_step_scores(z + (size_t)j * V, w1, w2, V, r, prev, zp);
        if (st != ORACLE_OK)
            break;
        tokens[j] = oracle_argmax(zp, V);
        st = oracle_topk(zp, V, top_k, cand + (size_t)j * top_k, cand_val + (size_t)j * top_k);
        prev = tokens[j];
    }
    free(zp);
    return st;
}

/* The chain of one block of a reduced draft vocabulary over its draft
 * projections z [n_pred][D]: draft id i scores float(z_j[i] + sum_k
 * w2[i][k] * w1[prev][k]) with w1 [V][r] indexed by the target id prev and
 * w2 [D][r] by draft id; argmax and top-k run over draft ids (lowest draft id
 * on ties) and are reported through d2t; the next prev is d2t[argmax]. */
int oracle_block_chain_d2t(const double* z, const uint16_t* w1, const uint16_t* w2,
                           const int64_t* d2t, int V, int D, int r, int anchor, int n_pred,
                           int top_k, int32_t* tokens, int32_t* cand, float* cand_val)
{
    if (anchor < 0 || anchor >= V || D < 1 || D > V || n_pred <= 0 || top_k < 1 || top_k > D ||
        r < 0)
        return ORACLE_ERR;
    for (int i = 0; i < D; ++i)
        if (d2t[i] < 0 || d2t[i] >= V)
            return ORACLE_ERR;
    float* zp = (float*)malloc(sizeof(float) * (size_t)D);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)top_k);
    if (!zp || !idx) {
        free(zp);
        free(idx);
        return ORACLE_ERR;
    }
    int prev_tok = anchor;   /* a target id */
    for (int j = 0; j < n_pred; ++j) {
        const double* zj = z + (size_t)j * D;
        const uint16_t* u = r > 0 ? w1 + (long)prev_tok * r : NULL;
#pragma omp parallel for schedule(static)
        for (long i = 0; i < D; ++i) {
            double m = 0.0;
            for (int q = 0; q < r; ++q)
                m += bf16_value(w2[i * (long)r + q]) * bf16_value(u[q]);
            zp[i] = (float)(zj[i] + m);
        }
        const int best = oracle_argmax(zp, D);
        oracle_topk(zp, D, top_k, idx, cand_val + (size_t)j * top_k);
        for (int t = 0; t < top_k; ++t)
            cand[(size_t)j * top_k + t] = (int32_t)d2t[idx[t]];
        tokens[j] = (int32_t)d2t[best];
        prev_tok = (int)d2t[best];
    }
    free(zp);
    free(idx);
    return ORACLE_OK;
}

/* Confidence of one prediction slot: float(sigma(sum_h x[h] * conf_w[h])). */
float oracle_conf(const void* hidden, int hidden_is_f32, const uint16_t* conf_w, int L, int H,
                  int i_first_pred, int b, int j)
{
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    if (!x)
        return NAN;
    load_hidden_row(hidden, hidden_is_f32, (long)b * L + i_first_pred + j, H, x);
    double c = 0.0;
    for (int h = 0; h < H; ++h)
        c += x[h] * bf16_value(conf_w[h]);
    free(x);
    return (float)(1.0 / (1.0 + exp(-c)));
}

/* Prefix truncation: the first slot whose confidence is strictly below p_min,
 * or n_pred when there is none. p_min = 0 therefore never truncates. */
int oracle_truncate(const float* conf, int n_pred, float p_min)
{
    for (int j = 0; j < n_pred; ++j)
        if (conf[j] < p_min)
            return j;
    return n_pred;
}

/* Chain, confidence and truncation of block b over its projections z
 * [n_pred][V]; with no conf_w, conf = 1 and length = n_pred. */
static int finish_block(const double* z, const void* hidden, int hidden_is_f32,
                        const uint16_t* w1, const uint16_t* w2, const uint16_t* conf_w,
                        const int32_t* anchors, int L, int H, int V, int r, int i_first_pred,
                        int top_k, float p_min, int b, int32_t* tokens, int32_t* cand,
                        float* cand_val, float* conf, int32_t* length)
{
    const int n_pred = L - i_first_pred;
    int st = oracle_block_chain(z, w1, w2, V, r, anchors[b], n_pred, top_k, tokens, cand, cand_val);
    if (st == ORACLE_OK) {
        for (int j = 0; j < n_pred; ++j)
            conf[j] = conf_w ? oracle_conf(hidden, hidden_is_f32, conf_w, L, H, i_first_pred, b, j)
                             : 1.0f;
        *length = conf_w ? oracle_truncate(conf, n_pred, p_min) : n_pred;
    }
    return st;
}

/* Everything for block b. z (may be NULL) receives the projections
 * [n_pred][V]; with no conf_w, conf = 1 and length = n_pred. */
int oracle_propose_block(const void* hidden, int hidden_is_f32, const uint16_t* lm_head,
                         const float* bias, const uint16_t* w1, const uint16_t* w2,
                         const uint16_t* conf_w, const int32_t* anchors, int L, int H, int V,
                         int r, int i_first_pred, int top_k, float p_min, int b, double* z,
                         int32_t* tokens, int32_t* cand, float* cand_val, float* conf,
                         int32_t* length)
{
    int n_pred = L - i_first_pred;
    double* zz = z ? z : (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)V);
    if (!zz)
        return ORACLE_ERR;
    int st = oracle_block_logits(hidden, hidden_is_f32, lm_head, bias, L, H, V, i_first_pred, b, zz);
    if (st == ORACLE_OK)
        st = finish_block(zz, hidden, hidden_is_f32, w1, w2, conf_w, anchors, L, H, V, r,
                          i_first_pred, top_k, p_min, b, tokens, cand, cand_val, conf, length);
    if (!z)
        free(zz);
    return st;
}

/* ---- quantized head (q4) ------------------------------------------------ */

#define Q4_BLOCK 32
#define Q4_BLOCK_BYTES 18

/* Value of an IEEE binary16 bit pattern: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 holds zero and the subnormals. */
static double f16_value(uint16_t bits)
{
    const int e = (bits >> 10) & 0x1f;
    const int f = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (bits & 0x8000u) ? -v : v;
}

double oracle_f16_value(uint16_t bits) { return f16_value(bits); }

/* Row v of a q4 head as exact doubles w[0..H): block i of the row is bytes
 * [18 i, 18 i + 18) of the row's H/32 * 18 bytes; its scale d is the
 * binary16 in the first two bytes (low byte first), and code byte j (the
 * bytes after the scale) gives element 32 i + j its low nibble and element
 * 32 i + j + 16 its high nibble; an element is d * (code - 8), exact in
 * double (an 11-bit significand times a 4-bit integer). */
int oracle_q4_dequant_row(const uint8_t* q4, int H, long v, double* w)
{
    if (H <= 0 || H % Q4_BLOCK != 0 || v < 0)
        return ORACLE_ERR;
    const int nb = H / Q4_BLOCK;
    const uint8_t* row = q4 + v * (long)nb * Q4_BLOCK_BYTES;
    for (int i = 0; i < nb; ++i) {
        const uint8_t* blk = row + (long)i * Q4_BLOCK_BYTES;
        const double d = f16_value((uint16_t)(blk[0] | (blk[1] << 8)));
        const uint8_t* qs = blk + 2;
        for (int j = 0; j < 16; ++j) {
            w[i * Q4_BLOCK + j] = d * (double)((int)(qs[j] & 0x0f) - 8);
            w[i * Q4_BLOCK + j + 16] = d * (double)((int)(qs[j] >> 4) - 8);
        }
    }
    return ORACLE_OK;
}

/* Projection of the n_pred prediction rows of block b through a q4 head:
 * z[j*V + v] = sum_h x_j[h] * w_v[h] (+ bias[v]) with w_v the decoded row v,
 * summed in increasing h exactly as oracle_block_logits does. */
int oracle_block_logits_q4(const void* hidden, int hidden_is_f32, const uint8_t* q4,
                           const float* bias, int L, int H, int V, int i_first_pred, int b,
                           double* z)
{
    int n_pred = L - i_first_pred;
    if (n_pred <= 0 || H <= 0 || H % Q4_BLOCK != 0 || V <= 0 || b < 0)
        return ORACLE_ERR;
    double* x = (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)H);
    if (!x)
        return ORACLE_ERR;
    const long first_row = (long)b * L + i_first_pred;   /* slot i_first_pred of block b */
    for (int j = 0; j < n_pred; ++j)
        load_hidden_row(hidden, hidden_is_f32, first_row + j, H, x + (size_t)j * H);

    int fail = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
        for (long v = 0; v < V; ++v) {
            if (!w) {
#pragma omp atomic write
                fail = 1;
                continue;
            }
            oracle_q4_dequant_row(q4, H, v, w);
            for (int j = 0; j < n_pred; ++j) {
                const double* xj = x + (size_t)j * H;
                double s = 0.0;
                for (int h = 0; h < H; ++h)
                    s += xj[h] * w[h];
                if (bias)
                    s = s + (double)bias[v];
                z[(size_t)j * V + v] = s;
            }
        }
        free(w);
    }
    free(x);
    return fail ? ORACLE_ERR : ORACLE_OK;
}

/* Everything for block b with a q4 head (as oracle_propose_block). */
int oracle_propose_block_q4(const void* hidden, int hidden_is_f32, const uint8_t* q4,
                            const float* bias, const uint16_t* w1, const uint16_t* w2,
                            const uint16_t* conf_w, const int32_t* anchors, int L, int H, int V,
                            int r, int i_first_pred, int top_k, float p_min, int b, double* z,
                            int32_t* tokens, int32_t* cand, float* cand_val, float* conf,
                            int32_t* length)
{
    int n_pred = L - i_first_pred;
    double* zz = z ? z : (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)V);
    if (!zz)
        return ORACLE_ERR;
    int st = oracle_block_logits_q4(hidden, hidden_is_f32, q4, bias, L, H, V, i_first_pred, b, zz);
    if (st == ORACLE_OK)
        st = finish_block(zz, hidden, hidden_is_f32, w1, w2, conf_w, anchors, L, H, V, r,
                          i_first_pred, top_k, p_min, b, tokens, cand, cand_val, conf, length);
    if (!z)
        free(zz);
    return st;
}

/* Everything for block b of a reduced draft vocabulary: draft projections
 * through lm_head [D][H] (no bias; z may be NULL, else [n_pred][D]), the d2t
 * chain, confidence and truncation as in oracle_propose_block. */
int oracle_propose_block_d2t(const void* hidden, int hidden_is_f32, const uint16_t* lm_head,
                             const int64_t* d2t, const uint16_t* w1, const uint16_t* w2,
                             const uint16_t* conf_w, const int32_t* anchors, int L, int H, int V,
                             int D, int r, int i_first_pred, int top_k, float p_min, int b,
                             double* z, int32_t* tokens, int32_t* cand, float* cand_val,
                             float* conf, int32_t* length)
{
    int n_pred = L - i_first_pred;
    double* zz = z ? z : (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)D);
    if (!zz)
        return ORACLE_ERR;
    int st = oracle_block_logits(hidden, hidden_is_f32, lm_head, NULL, L, H, D, i_first_pred, b, zz);
    if (st == ORACLE_OK)
        st = oracle_block_chain_d2t(zz, w1, w2, d2t, V, D, r, anchors[b], n_pred, top_k, tokens,
                                    cand, cand_val);
    if (st == ORACLE_OK) {
        for (int j = 0; j < n_pred; ++j)
            conf[j] = conf_w ? oracle_conf(hidden, hidden_is_f32, conf_w, L, H, i_first_pred, b, j)
                             : 1.0f;
        *length = conf_w ? oracle_truncate(conf, n_pred, p_min) : n_pred;
    }
    if (!z)
        free(zz);
    return st;
}

/* Greedy verification of B blocks: block b accepts slot j while target[b][j]
 * is one of the first `width` candidates of the slot (width 1: the chain
 * token; width top_k: the lattice), over at most min(max(lengths[b], 0),
 * n_pred) slots. totals[0] = sum of accepted, totals[1] = sum of the clamped
 * lengths. */
int oracle_verify(const int32_t* cand, const int32_t* lengths, const int32_t* target, int B,
                  int n_pred, int top_k, int width, int32_t* accepted, int64_t* totals)
{
    if (B < 1 || n_pred < 1 || top_k < 1 || width < 1 || width > top_k)
        return ORACLE_ERR;
    totals[0] = 0;
    totals[1] = 0;
    for (int b = 0; b < B; ++b) {
        int len = lengths[b] < 0 ? 0 : lengths[b];
        if (len > n_pred)
            len = n_pred;
        int m = 0;
        while (m < len) {
            const int32_t* c = cand + ((size_t)b * n_pred + m) * top_k;
            const int32_t t = target[(size_t)b * n_pred + m];
            int found = 0;
            for (int i = 0; i < width; ++i)
                if (c[i] == t)
                    found = 1;
            if (!found)
                break;
            ++m;
        }
        accepted[b] = m;
        totals[0] += m;
        totals[1] += len;
    }
    return ORACLE_OK;
}

/* Block b under the adaptive gate: its confidences and cut first (threshold
 * p_min of this block), then the chain over the surviving slots only, with kb
 * candidates per slot. Slots past the cut hold token -1 and candidates -1
 * (value -INFINITY), ranks kb .. top_k-1 likewise; z (may be NULL) receives
 * the projections [n_pred][V] of every slot. */
int oracle_propose_block_gated(const void* hidden, int hidden_is_f32, const uint16_t* lm_head,
                               const float* bias, const uint16_t* w1, const uint16_t* w2,
                               const uint16_t* conf_w, const int32_t* anchors, int L, int H, int V,
                               int r, int i_first_pred, int top_k, int kb, float p_min, int b,
                               double* z, int32_t* tokens, int32_t* cand, float* cand_val,
                               float* conf, int32_t* length)
{
    const int n_pred = L - i_first_pred;
    if (!conf_w || kb < 1 || kb > top_k || top_k > V || n_pred < 1)
        return ORACLE_ERR;
    for (int j = 0; j < n_pred; ++j)
        conf[j] = oracle_conf(hidden, hidden_is_f32, conf_w, L, H, i_first_pred, b, j);
    const int len = oracle_truncate(conf, n_pred, p_min);
    *length = len;
    for (int j = 0; j < n_pred; ++j) {
        tokens[j] = -1;
        for (int t = 0; t < top_k; ++t) {
            cand[(size_t)j * top_k + t] = -1;
            cand_val[(size_t)j * top_k + t] = -INFINITY;
        }
    }
    double* zz = z ? z : (double*)malloc(sizeof(double) * (size_t)n_pred * (size_t)V);
    if (!zz)
        return ORACLE_ERR;
    int st = oracle_block_logits(hidden, hidden_is_f32, lm_head, bias, L, H, V, i_first_pred, b, zz);
    if (st == ORACLE_OK && len > 0) {
        int32_t* c = (int32_t*)malloc(sizeof(int32_t) * (size_t)len * kb);
        float* cv = (float*)malloc(sizeof(float) * (size_t)len * kb);
        if (!c || !cv)
            st = ORACLE_ERR;
        else
            st = oracle_block_chain(zz, w1, w2, V, r, anchors[b], len, kb, tokens, c, cv);
        if (st == ORACLE_OK)
            for (int j = 0; j < len; ++j)
                for (int t = 0; t < kb; ++t) {
                    cand[(size_t)j * top_k + t] = c[(size_t)j * kb + t];
                    cand_val[(size_t)j * top_k + t] = cv[(size_t)j * kb + t];
                }
        free(c);
        free(cv);
    }
    if (!z)
        free(zz);
    return st;
}
