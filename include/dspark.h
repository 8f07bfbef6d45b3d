/*
 * dspark.h -- C ABI of libdspark, the DSpark drafter's proposal step on
 * AMD Instinct MI355X (gfx950).
 *
 * The proposal step turns the drafter's hidden states for B blocks of L
 * slots into draft tokens:
 *
 *   1. lm_head projection. Each prediction slot's hidden state goes through
 *      the vocabulary head that the drafter shares with its target model:
 *      logits[b*n_pred + j][v] = sum_h hidden[b][i_first_pred + j][h] *
 *      lm_head[v][h] (+ lm_head_bias[v]).
 *      Sources: onnxruntime-genai PR #2490 "Export DSpark block drafters for
 *      Qwen 3.5 and 3.8" (DSpark commit message: no head of its own, the
 *      target's is shared); llama.cpp PR #26275 "dspark: support
 *      speculators-format checkpoints" (first commit message: the -1e9 bias on
 *      rows a reduced draft vocabulary cannot produce).
 *   2. Markov chain. Slot j's scores get the low-rank bigram bias of the
 *      previous token: z'_j[v] = logits_j[v] + sum_k markov_w2[v][k] *
 *      markov_w1[prev_j][k], with prev_0 = the block's anchor and prev_j =
 *      argmax_v z'_{j-1}[v]; all blocks advance together, one slot at a time.
 *      Source: llama.cpp commit 6fed9f6 "spec: add DSpark speculative
 *      decoding", item of the same name (the chained-bias formula,
 *      vectorised across blocks).
 *   3. Candidates. The top_k ids of z'_j per slot form the candidate lattice
 *      for tree / lattice verification; the Markov bias applies to them too.
 *      Sources: lucebox PR #626 "feat(qwen38): add adaptive concurrent DSpark
 *      speculation" (description); onnxruntime-genai PR #2490 (dspark_top_k).
 *   4. Confidence truncation. conf[b][j] = sigmoid(sum_h hidden[b][i_first_pred
 *      + j][h] * conf_w[h]) is the predicted survival probability of the
 *      slot; lengths[b] is the first slot j with conf < p_min (n_pred if none;
 *      p_min = 0 disables the cut).
 *      Source: llama.cpp commit 6fed9f6, items "spec: add confidence-based
 *      draft pruning for DSpark" and "dspark: fold conf_min into p_min".
 *
 * Block layout (llama.cpp PR #26275, first commit message and "Format
 * differences"): DSPARK_LAYOUT_ANCHOR_FIRST -- every slot predicts
 * (sample_from_anchor = true, i_first_pred = 0, n_pred = L);
 * DSPARK_LAYOUT_BONUS_ANCHOR -- the 1+N fill-in block whose slot 0 carries
 * the bonus token and is never read (sample_from_anchor = false,
 * i_first_pred = 1, n_pred = L - 1).
 *
 * Conventions for every entry point:
 *  - Pointers marked DEVICE are device (HBM) pointers; every array is dense
 *    and row-major. bf16 arrays are passed as their uint16_t bit patterns.
 *  - The caller owns every buffer. The library allocates and frees nothing
 *    and keeps no global mutable state; calls that use distinct workspaces
 *    and outputs may run concurrently.
 *  - `stream` is a hipStream_t (NULL = the default stream). All device work
 *    is enqueued asynchronously on it; outputs are valid once the stream
 *    reaches that point. The host never synchronises inside these calls.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    validation failure nothing is enqueued and the status says why.
 *  - Numerics: hidden and weights are bf16 (fp32 hidden is rounded to bf16,
 *    nearest-even, as it is staged); every product is accumulated in fp32.
 *    Argmax ties go to the lowest id; candidates are ordered by score
 *    descending, then id ascending. Results are bit-for-bit deterministic
 *    for a given input.
 *  - Anchors and previous tokens must lie in [0, V). The kernels never read
 *    out of bounds: an out-of-range anchor is replaced by 0 and raises
 *    DSPARK_FLAG_BAD_ANCHOR in the workspace flags (see dspark_read_flags).
 *    Inputs must be finite; results for NaN / Inf inputs are undefined,
 *    except in the bonus slot, which is never read.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_OK = 0,
    DSPARK_ERR_INVALID_ARG = -1, /* a size, pointer, enum or p_min is not acceptable      */
    DSPARK_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels implement          */
    DSPARK_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than dspark_workspace_bytes */
    DSPARK_ERR_HIP = -4,         /* the HIP runtime reported an error while enqueuing     */
    DSPARK_ERR_SCRATCH = -5      /* dspark_propose_noalloc: sizes exceed its static scratch */
} dspark_status;
/* An error left pending in the HIP runtime by an earlier call outside the
 * library is cleared when an entry point starts enqueuing; only errors of the
 * library's own launches are reported as DSPARK_ERR_HIP. */

typedef enum {
    DSPARK_LAYOUT_ANCHOR_FIRST = 0,
    DSPARK_LAYOUT_BONUS_ANCHOR = 1
} dspark_layout;

typedef enum {
    DSPARK_HIDDEN_BF16 = 0,
    DSPARK_HIDDEN_F32 = 1
} dspark_dtype;

/* Device-side flags accumulated in the workspace by a call. */
#define DSPARK_FLAG_BAD_ANCHOR 1u   /* an anchor was outside [0, V)                      */
#define DSPARK_FLAG_INTERNAL 2u     /* the candidate merge disagreed with the chain's argmax */
#define DSPARK_FLAG_BAD_D2T 4u      /* a d2t entry the chain followed was outside [0, V)  */

/* Limits checked by every entry point. */
#define DSPARK_MAX_TOP_K 16
#define DSPARK_MAX_RANK 256

/*
 * Bytes of device workspace that dspark_propose / dspark_chain need for these
 * sizes (pure host function, no HIP call). Returns 0 if the sizes are invalid.
 * The workspace holds the flags word, the per-slot running argmax words and,
 * for top_k > 1, the per-row slab maxima of the projection and their k-th
 * largest per row (which bound the top-k scores and let the chain skip
 * hopeless columns) and the per-workgroup top-k partial lists. Its contents need no initialisation and
 * are overwritten by every call.
 */
size_t dspark_workspace_bytes(int B, int L, int V, int top_k, int layout);

/*
 * The whole proposal step: projection, Markov chain, candidates, confidence
 * truncation.
 *
 *   hidden        DEVICE [B, L, H], bf16 (hidden_dtype = DSPARK_HIDDEN_BF16)
 *                 or fp32 (DSPARK_HIDDEN_F32). Under the bonus-anchor layout
 *                 slot 0 of every block is not read.
 *   lm_head       DEVICE bf16 [V, H] (one row per vocabulary id).
 *   lm_head_bias  DEVICE fp32 [V], or NULL for no bias.
 *   markov_w1     DEVICE bf16 [V, r]; the row of the previous token is used.
 *   markov_w2     DEVICE bf16 [V, r]; maps the rank-r code to the vocabulary.
 *                 Both NULL iff r == 0 (no Markov head: plain argmax).
 *   conf_w        DEVICE bf16 [H], or NULL: no confidence head, conf = 1 and
 *                 lengths = n_pred.
 *   anchors       DEVICE int32 [B], each in [0, V).
 *   B, L, H, V, r sizes; H and r multiples of 8, r <= DSPARK_MAX_RANK.
 *   layout        dspark_layout.
 *   top_k         candidates per slot, 1 <= top_k <= min(V, DSPARK_MAX_TOP_K).
 *   p_min         truncation threshold (not NaN); 0 never truncates.
 *   logits        DEVICE fp32 [B*n_pred, V] output: the projection (row
 *                 b*n_pred + j), bias included, Markov term excluded.
 *   workspace     DEVICE scratch of at least dspark_workspace_bytes(...)
 *                 bytes, 256-byte aligned.
 *   tokens        DEVICE int32 [B, n_pred] output: the greedy chain.
 *   candidates    DEVICE int32 [B, n_pred, top_k] output; candidates[..., 0]
 *                 equals tokens.
 *   cand_logits   DEVICE fp32 [B, n_pred, top_k] output (z' of each
 *                 candidate), or NULL.
 *   conf          DEVICE fp32 [B, n_pred] output, or NULL.
 *   lengths       DEVICE int32 [B] output. All n_pred slots are always
 *                 drafted; lengths marks how many survive the cut.
 * Returns a dspark_status.
 */
int dspark_propose(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                   const float* lm_head_bias, const uint16_t* markov_w1,
                   const uint16_t* markov_w2, const uint16_t* conf_w, const int32_t* anchors,
                   int B, int L, int H, int V, int r, int layout, int top_k, float p_min,
                   float* logits, void* workspace, size_t workspace_bytes, int32_t* tokens,
                   int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                   void* stream);

/*
 * dspark_propose for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and results, with the workspace taken from a static
 * device array of DSPARK_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on (from the first use until the process ends). The
 * call allocates and frees nothing. The current device's array is used
 * (hipGetDevice; `stream` must belong to that device); its address is taken
 * once per device with hipGetSymbolAddress.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller. Every call clears what must
 * start at zero. Sizes whose workspace (dspark_workspace_bytes) exceeds the
 * array return DSPARK_ERR_SCRATCH with nothing enqueued. The device-side
 * flags (DSPARK_FLAG_*) stay in the array and are not reported.
 * Every other argument is as in dspark_propose. Returns a dspark_status.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES (64u << 20)
int dspark_propose_noalloc(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                           const float* lm_head_bias, const uint16_t* markov_w1,
                           const uint16_t* markov_w2, const uint16_t* conf_w,
                           const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                           int top_k, float p_min, float* logits, int32_t* tokens,
                           int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                           void* stream);

/*
 * dspark_propose with three HIP events (hipEvent_t, each may be NULL)
 * recorded on `stream` between its launches: mark_init after the per-call
 * set-up kernel, mark_projected after the lm_head projection, mark_chained
 * after the last chain step (before the kernel that assembles candidates and
 * confidences). The launches and results are those of dspark_propose; the
 * events let a caller time each phase of the very launches a call makes. A
 * failed event record returns DSPARK_ERR_HIP.
 */
int dspark_propose_marked(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                          const float* lm_head_bias, const uint16_t* markov_w1,
                          const uint16_t* markov_w2, const uint16_t* conf_w,
                          const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                          int top_k, float p_min, float* logits, void* workspace,
                          size_t workspace_bytes, int32_t* tokens, int32_t* candidates,
                          float* cand_logits, float* conf, int32_t* lengths, void* stream,
                          void* mark_init, void* mark_projected, void* mark_chained);

/*
 * Step 1 alone: the lm_head projection into `logits` (same arguments and
 * layout as in dspark_propose). Needs no workspace.
 */
int dspark_logits(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                  const float* lm_head_bias, int B, int L, int H, int V, int layout,
                  float* logits, void* stream);

/*
 * Steps 2-4 on projections the caller provides: `logits` is an INPUT here
 * (DEVICE fp32 [B*n_pred, V], laid out as dspark_propose writes it), and
 * `hidden` is read only by the confidence head (may be NULL when conf_w is
 * NULL). Every other argument is as in dspark_propose.
 */
int dspark_chain(const float* logits, const void* hidden, int hidden_dtype,
                 const uint16_t* markov_w1, const uint16_t* markov_w2, const uint16_t* conf_w,
                 const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                 int top_k, float p_min, void* workspace, size_t workspace_bytes,
                 int32_t* tokens, int32_t* candidates, float* cand_logits, float* conf,
                 int32_t* lengths, void* stream);

/*
 * The proposal step of a draft with a reduced output vocabulary: its head
 * scores D <= V draft ids, and the int64 table d2t gives the absolute target
 * id of each draft id. The projection and the chain run over the D draft
 * ids only; tokens and candidates come out as target ids. This is the
 * run-time scatter of llama.cpp PR #26275 "dspark: support speculators-format
 * checkpoints" (rework commit message: d2t holds I64 absolute target ids, as
 * for EAGLE3, and the draft logits are scattered at run time instead of
 * expanding lm_head / markov_w2 and adding a -1e9 bias at conversion; "Format
 * differences": draft_vocab_size < vocab_size with a d2t table). It computes
 * what dspark_propose computes on the expanded form -- lm_head and markov_w2
 * rows placed at d2t[i], zero rows elsewhere, bias -1e9 off the table --
 * bit for bit on tokens, candidates, cand_logits, conf and lengths.
 *
 *   lm_head       DEVICE bf16 [D, H]: the draft head, one row per draft id.
 *   d2t           DEVICE int64 [D], 8-byte aligned: strictly increasing target
 *                 ids in [0, V) (so ties between draft ids go to the lower
 *                 target id, as in the expanded form). Entries are range
 *                 checked when the chain follows them: an entry outside
 *                 [0, V) is replaced by 0 and raises DSPARK_FLAG_BAD_D2T;
 *                 the order is not checked.
 *   markov_w1     DEVICE bf16 [V, r]: indexed by the previous token, a
 *                 target id (anchors are target ids).
 *   markov_w2     DEVICE bf16 [D, r]: draft rows.
 *   V, D          target and draft vocabulary sizes, 1 <= D <= V;
 *                 top_k <= min(D, DSPARK_MAX_TOP_K).
 *   logits        DEVICE fp32 [B*n_pred, D] output: draft-id projections (no
 *                 bias).
 *   workspace     at least dspark_workspace_bytes(B, L, D, top_k, layout).
 *   tokens, candidates, cand_logits, conf, lengths: as in dspark_propose,
 *                 with target ids.
 * Every other argument is as in dspark_propose. Returns a dspark_status.
 */
int dspark_propose_d2t(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                       const int64_t* d2t, const uint16_t* markov_w1, const uint16_t* markov_w2,
                       const uint16_t* conf_w, const int32_t* anchors, int B, int L, int H, int V,
                       int D, int r, int layout, int top_k, float p_min, float* logits,
                       void* workspace, size_t workspace_bytes, int32_t* tokens,
                       int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                       void* stream);

/*
 * The proposal step with the confidence gate in front of the chain and
 * per-block settings (per-request heterogeneity). The confidence of every
 * slot is computed first and each block is cut at its first slot below its
 * own threshold p_min[b]; the chain then runs only as many slots as the
 * longest surviving block, and slots past a block's cut are reported as not
 * drafted. This wires the adaptive block length that lucebox PR #626
 * "feat(qwen38): add adaptive concurrent DSpark speculation" leaves unwired
 * (description: the confidence-gate adaptive block length, the per-request
 * override of the decode mode), with the threshold semantics of llama.cpp
 * commit 6fed9f6 "spec: add DSpark speculative decoding", items "spec: add
 * confidence-based draft pruning for DSpark" and "dspark: fold conf_min into
 * p_min".
 *
 *   conf_w        DEVICE bf16 [H]; required (the gate needs it).
 *   p_min         DEVICE fp32 [B]: the threshold of each block (not NaN).
 *   block_top_k   DEVICE int32 [B] or NULL: candidates kept per block,
 *                 clamped to [1, top_k]; top_k sizes the candidate arrays.
 *   tokens        slots j >= lengths[b] hold -1.
 *   candidates    slots j >= lengths[b], and ranks >= block_top_k[b], hold -1;
 *   cand_logits   -INFINITY there.
 * Every other argument is as in dspark_propose; on the slots a block keeps,
 * the outputs equal dspark_propose's with that block's p_min and top_k.
 * Returns a dspark_status.
 */
int dspark_propose_adaptive(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                            const float* lm_head_bias, const uint16_t* markov_w1,
                            const uint16_t* markov_w2, const uint16_t* conf_w,
                            const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                            int top_k, const float* p_min, const int32_t* block_top_k,
                            float* logits, void* workspace, size_t workspace_bytes,
                            int32_t* tokens, int32_t* candidates, float* cand_logits, float* conf,
                            int32_t* lengths, void* stream);

/*
 * ---- 4-bit lm_head ---------------------------------------------------------
 * The pages validate the Qwen3.8-27B drafter on the device as a requantized
 * 4-bit GGUF (lucebox PR #626 "feat(qwen38): add adaptive concurrent DSpark
 * speculation", Summary -> Drafter) but do not give its block layout. The
 * reading implemented here is GGUF's plain 4-bit type: each row of lm_head
 * is H/32 blocks of 18 bytes -- an IEEE binary16 scale d (low byte first)
 * and 16 code bytes, code byte j giving element j of the block its low
 * nibble and element j + 16 its high nibble -- and an element with code q is
 * worth d * (q - 8). The projection is computed over those exact weights;
 * every other step is dspark_propose's.
 */

/*
 * Bytes of the packed form of a 4-bit head with V rows and H columns (pure
 * host function); 0 if V <= 0, H <= 0 or H is not a multiple of 32.
 */
size_t dspark_q4_packed_bytes(int V, int H);

/*
 * Rearranges a 4-bit head from its GGUF blocks into the packed form the
 * projection streams (once, when the weights are loaded): rows in tiles of
 * 16, blocks in quads of 4, code bytes interleaved so that one wave-wide
 * 16-byte load brings one quad of blocks of one tile; rows past V and blocks
 * past H/32 are padded with weight 0.
 *
 *   blocks   DEVICE uint8 [V, H/32 * 18]: the GGUF blocks, any alignment.
 *   V, H     rows and columns; H a multiple of 32.
 *   packed   DEVICE, 16-byte aligned, dspark_q4_packed_bytes(V, H) bytes,
 *            owned by the caller, fully overwritten.
 * Returns a dspark_status (DSPARK_ERR_UNSUPPORTED if H % 32 != 0).
 */
int dspark_q4_pack(const void* blocks, int V, int H, void* packed, void* stream);

/*
 * Workspace bytes of dspark_propose_q4 (pure host function; 0 for invalid
 * sizes): dspark_workspace_bytes(B, L, V, top_k, layout) for the chain, at
 * offset 0 (dspark_read_flags reads it as for dspark_propose), followed by the
 * per-call preparation of the hidden rows (bf16 rows in the projection's k
 * order, B*n_pred*128*ceil(H/128)*2 bytes rounded up to 256).
 * dspark_logits_q4 needs this with any valid top_k.
 */
size_t dspark_q4_workspace_bytes(int B, int L, int H, int V, int top_k, int layout);

/*
 * Step 1 alone with a 4-bit head: logits[b*n_pred + j][v] = sum_h
 * hidden[b][i_first_pred + j][h] * w[v][h] (+ lm_head_bias[v]), w the
 * decoded weights, accumulated in fp32 (each block's partial is scaled by its
 * d in fp32).
 *
 *   lm_head_q4  DEVICE: the head as dspark_q4_pack wrote it for (V, H).
 *   H           a multiple of 32.
 *   workspace   DEVICE, 256-byte aligned, dspark_q4_workspace_bytes(B, L, H,
 *               V, 1, layout) bytes.
 * Every other argument is as in dspark_logits. Returns a dspark_status.
 */
int dspark_logits_q4(const void* hidden, int hidden_dtype, const void* lm_head_q4,
                     const float* lm_head_bias, int B, int L, int H, int V, int layout,
                     float* logits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole proposal step with a 4-bit head: dspark_logits_q4, then steps 2-4
 * exactly as dspark_propose runs them on those projections.
 *
 *   lm_head_q4  DEVICE: as dspark_q4_pack wrote it for (V, H); H % 32 == 0.
 *   workspace   DEVICE, 256-byte aligned, at least
 *               dspark_q4_workspace_bytes(B, L, H, V, top_k, layout) bytes.
 * Every other argument is as in dspark_propose. Returns a dspark_status.
 */
int dspark_propose_q4(const void* hidden, int hidden_dtype, const void* lm_head_q4,
                      const float* lm_head_bias, const uint16_t* markov_w1,
                      const uint16_t* markov_w2, const uint16_t* conf_w, const int32_t* anchors,
                      int B, int L, int H, int V, int r, int layout, int top_k, float p_min,
                      float* logits, void* workspace, size_t workspace_bytes, int32_t* tokens,
                      int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                      void* stream);

/*
 * Greedy verification of a proposal against the target's tokens: the target
 * keeps the longest drafted prefix it would have produced itself, so greedy
 * speculation stays lossless (llama.cpp commit 6fed9f6 "spec: add DSpark
 * speculative decoding", the in-graph chain item). With lattice = 0 slot j of
 * block b is accepted when target[b][j] == candidates[b][j][0] (the greedy
 * chain); with lattice = 1 when target[b][j] is any of the slot's top_k
 * candidates, the greedy walk of the candidate lattice (onnxruntime-genai PR
 * #2490 "Export DSpark block drafters for Qwen 3.5 and 3.8", DFlash 2 and
 * DSpark commit messages). The walk of block b stops at the first slot that
 * is not accepted and at lengths[b] (clamped to [0, n_pred]): a truncated
 * block submits only its surviving slots.
 *
 *   candidates    DEVICE int32 [B, n_pred, top_k], as dspark_propose writes it.
 *   lengths       DEVICE int32 [B], as dspark_propose writes it.
 *   target        DEVICE int32 [B, n_pred]: the target's greedy token at each
 *                 slot, given the slots before it.
 *   accepted      DEVICE int32 [B] output: accepted slots per block.
 *   totals        DEVICE int32 [2] output: sum of accepted, sum of the clamped
 *                 lengths (the acceptance rate is their ratio).
 *   B, n_pred, top_k  sizes, 1 <= top_k <= DSPARK_MAX_TOP_K; lattice 0 or 1.
 * Needs no workspace. Returns a dspark_status.
 */
int dspark_verify(const int32_t* candidates, const int32_t* lengths, const int32_t* target, int B,
                  int n_pred, int top_k, int lattice, int32_t* accepted, int32_t* totals,
                  void* stream);

/*
 * Copies the flags word of `workspace` (written by the last dspark_propose /
 * dspark_propose_d2t / dspark_propose_adaptive / dspark_propose_q4 /
 * dspark_chain on it) to *flags after `stream` has drained; this call does
 * synchronise the stream. Returns a dspark_status.
 */
int dspark_read_flags(const void* workspace, uint32_t* flags, void* stream);

/* Static, human-readable text for a status code. */
const char* dspark_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
