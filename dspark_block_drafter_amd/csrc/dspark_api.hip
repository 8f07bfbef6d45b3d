// C ABI of libdspark: argument validation, workspace layout, launch sequence.
//
// Validation runs on the host before any HIP call; a rejected call enqueues
// nothing. The block-uniformity requirement (every block has the same L
// slots, B and L passed explicitly) follows llama.cpp commit 6fed9f6 "spec:
// add DSpark speculative decoding", item "dflash: assert the markov head
// block-uniformity invariant, require the conf head" (a broken layout fails
// loudly instead of silently dropping the bias).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/dspark.h"
#include "kernels.hpp"

using namespace dspark;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kFlagsBytes = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t winners_off, kth_off, smax_off, partials_off, total;
};

// [flags (256 B): flags word, gate's slot count, markov_w2 and markov_w1 norm words]
// [winners: n_pred*kWinnerWays*winners_stride(B) u64]
// [k-th slab maxima: B*n_pred f32]
// [slab maxima: B*n_pred*ceil(V/kSlabCols) f32]
// [partials: n_pred*B*nwg*top_k u64, top_k > 1]
Layout workspace_layout(int B, int n_pred, int V, int top_k) {
    Layout l;
    l.winners_off = kFlagsBytes;
    const size_t win = align_up((size_t)n_pred * kWinnerWays * (size_t)winners_stride(B) * 8u);
    l.kth_off = l.winners_off + win;
    l.smax_off = l.kth_off + align_up((size_t)B * n_pred * 4u);
    const size_t smax = align_up((size_t)B * n_pred * ((V + kSlabCols - 1) / kSlabCols) * 4u);
    l.partials_off = l.smax_off + smax;
    const size_t part =
        top_k > 1 ? align_up((size_t)n_pred * B * (size_t)chain_workgroups_max(V) * top_k * 8u) : 0;
    l.total = l.partials_off + part;
    return l;
}

// Byte offsets of the words in the flags block.
constexpr size_t kStopWord = 4, kW2NormWord = 8, kW1NormWord = 12;
// Extra workgroups of the projection that take the markov_w2 norm for the
// top-k bound (they run in the projection's last, partly filled round).
constexpr int kW2NormGroups = 256;

int first_pred(int layout) { return layout == DSPARK_LAYOUT_BONUS_ANCHOR ? 1 : 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point that runs the chain.
int check_sizes(int B, int L, int H, int V, int layout, int hidden_dtype) {
    if (B <= 0 || L <= 0 || H <= 0 || V <= 0) return DSPARK_ERR_INVALID_ARG;
    if (layout != DSPARK_LAYOUT_ANCHOR_FIRST && layout != DSPARK_LAYOUT_BONUS_ANCHOR)
        return DSPARK_ERR_INVALID_ARG;
    if (hidden_dtype != DSPARK_HIDDEN_BF16 && hidden_dtype != DSPARK_HIDDEN_F32)
        return DSPARK_ERR_INVALID_ARG;
    if (layout == DSPARK_LAYOUT_BONUS_ANCHOR && L < 2) return DSPARK_ERR_INVALID_ARG;
    // every index computed on the device must fit in 32 bits where it is one
    const long n_pred = L - first_pred(layout);
    if ((long)B * L > 0x7fffffffL / 2 || (long)B * n_pred * (long)V > (1L << 53))
        return DSPARK_ERR_UNSUPPORTED;
    if (n_pred * (long)kWinnerWays * winners_stride(B) > 0x7fffffffL) return DSPARK_ERR_UNSUPPORTED;
    if (V >= 0x7fffffff - 1024 || H % 8 != 0) return DSPARK_ERR_UNSUPPORTED;
    return DSPARK_OK;
}

int check_chain_args(int V, int r, int top_k, float p_min, const void* w1, const void* w2) {
    if (top_k < 1 || top_k > DSPARK_MAX_TOP_K || top_k > V) return DSPARK_ERR_INVALID_ARG;
    if (r < 0) return DSPARK_ERR_INVALID_ARG;
    if (r > 0 && (!w1 || !w2)) return DSPARK_ERR_INVALID_ARG;
    if (r == 0 && (w1 || w2)) return DSPARK_ERR_INVALID_ARG;
    if (isnan(p_min)) return DSPARK_ERR_INVALID_ARG;
    if (r % 8 != 0 || r > DSPARK_MAX_RANK) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(w1) || !aligned16(w2)) return DSPARK_ERR_UNSUPPORTED;
    return DSPARK_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

// A call judges its launches by hipGetLastError, so an error left pending by
// an earlier HIP call of the caller (or of another library in the process)
// is cleared first rather than reported as the library's own.
void clear_pending_error() { (void)hipGetLastError(); }

// Options of the chain beyond the plain step.
struct ChainExtras {
    const int64_t* d2t = nullptr;     // reduced draft vocabulary: column c is target id d2t[c]
    int vocab = 0;                    // target vocabulary (rows of markov_w1); 0: V
    const float* p_min_b = nullptr;   // adaptive gate: per-block thresholds, conf before the chain
    const int32_t* top_k_b = nullptr; // adaptive: candidates kept per block
    bool narrow_slabs = false;        // the projection writes kSlabCols-column slab maxima (4-bit head)
};

// Arguments of the chain kernels over V columns. With `bounded` the chain
// reads the bound that the projection of the same call leaves in the
// workspace (bins, slab maxima, row norms).
ChainArgs chain_args(const float* logits, const uint16_t* w1, const uint16_t* w2,
                     const ChainExtras& x, const int32_t* anchors, int B, int L, int H, int V, int r,
                     int layout, int top_k, bool hidden_f32, void* workspace, int32_t* lengths,
                     bool bounded) {
    const int n_pred = L - first_pred(layout);
    const Layout wl = workspace_layout(B, n_pred, V, top_k);
    char* ws = static_cast<char*>(workspace);
    ChainArgs c{};
    c.logits = logits;
    c.w1 = w1;
    c.w2 = w2;
    c.d2t = x.d2t;
    c.vocab = x.vocab > 0 ? x.vocab : V;
    c.stop = x.p_min_b ? reinterpret_cast<const int32_t*>(ws + kStopWord) : nullptr;
    c.anchors = anchors;
    c.winners = reinterpret_cast<unsigned long long*>(ws + wl.winners_off);
    c.partials = top_k > 1 ? reinterpret_cast<unsigned long long*>(ws + wl.partials_off) : nullptr;
    c.flags = reinterpret_cast<uint32_t*>(ws);
    c.lengths = lengths;
    c.B = B;
    c.V = V;
    c.r = r;
    c.n_pred = n_pred;
    c.top_k = top_k;
    // The projection leaves a bound when the chain can use it: the pruned
    // form (one block group, pipelined vocabulary, rank up to 128) uses the
    // slab maxima, their k-th largest per row and both norms; the other forms
    // filter top-k inserts with the k-th largest and the markov_w2 norm.
    bounded = bounded && top_k > 1;
    const bool sparse = bounded && B <= 32 && chain_sparse(V, r);
    c.nwg = sparse ? chain_sparse_workgroups(B, V, r, top_k) : chain_workgroups(B, V, r, top_k);
    c.wstride = winners_stride(B);
    c.kth = bounded ? reinterpret_cast<float*>(ws + wl.kth_off) : nullptr;
    c.smax = bounded ? reinterpret_cast<const float*>(ws + wl.smax_off) : nullptr;
    c.w2n2 = bounded ? reinterpret_cast<uint32_t*>(ws + kW2NormWord) : nullptr;
    c.w1n2 = sparse ? reinterpret_cast<uint32_t*>(ws + kW1NormWord) : nullptr;
    c.sparse = sparse ? 1 : 0;
    // the pruned form reads slabs of kSlabCols; otherwise the four-wave
    // projection takes one wave's columns per slab
    c.slab_cols = !sparse && !x.narrow_slabs && gemm_four_wave(B * n_pred, H, L, n_pred, hidden_f32)
                      ? kSlabColsWide
                      : kSlabCols;
    return c;
}

// The chain over V columns (chain_init already enqueued when `initialised`).
int run_chain(const ChainArgs& c, bool initialised, const void* hidden, int hidden_dtype,
              const ChainExtras& x, const uint16_t* conf_w, int B, int L, int H, int V,
              int layout, int top_k, float p_min, void* workspace, int32_t* tokens,
              int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
              hipStream_t stream, hipEvent_t mark_chained = nullptr) {
    const int i_first = first_pred(layout);
    const int n_pred = L - i_first;
    char* ws = static_cast<char*>(workspace);

    hipError_t e = hipSuccess;
    if (!initialised) {
        clear_pending_error();
        e = launch_chain_init(c, stream);
    }
    if (e == hipSuccess && x.p_min_b) {
        GateArgs g;
        g.hidden = hidden;
        g.conf_w = conf_w;
        g.p_min = x.p_min_b;
        g.conf = conf;
        g.lengths = lengths;
        g.stop = reinterpret_cast<int32_t*>(ws + kStopWord);
        g.B = B;
        g.L = L;
        g.H = H;
        g.n_pred = n_pred;
        g.i_first = i_first;
        g.hidden_f32 = hidden_dtype == DSPARK_HIDDEN_F32;
        e = launch_gate(g, stream);
    }
    if (e == hipSuccess && c.kth) e = launch_row_kth(c, stream);
    for (int j = 0; j < n_pred && e == hipSuccess; ++j) e = launch_chain_step(c, j, stream);
    if (e == hipSuccess && mark_chained) e = hipEventRecord(mark_chained, stream);
    if (e != hipSuccess) return DSPARK_ERR_HIP;

    FinalArgs f;
    f.winners = c.winners;
    f.partials = c.partials;
    f.d2t = x.d2t;
    f.V = V;
    f.gated = x.p_min_b != nullptr;
    f.top_k_b = x.top_k_b;
    f.hidden = hidden;
    f.conf_w = conf_w;
    f.tokens = tokens;
    f.candidates = candidates;
    f.cand_logits = cand_logits;
    f.conf = conf;
    f.lengths = lengths;
    f.flags = c.flags;
    f.B = B;
    f.L = L;
    f.H = H;
    f.n_pred = n_pred;
    f.i_first = i_first;
    f.top_k = top_k;
    f.nwg = c.nwg;
    f.wstride = c.wstride;
    f.hidden_f32 = hidden_dtype == DSPARK_HIDDEN_F32;
    f.p_min = p_min;
    return hip_status(launch_finalize(f, stream));
}

GemmArgs gemm_args(const void* hidden, const uint16_t* lm_head, const float* bias, int B, int L,
                   int H, int V, int layout, float* logits, const ChainArgs* c, int r) {
    GemmArgs g{};
    g.hidden = hidden;
    g.lm_head = lm_head;
    g.bias = bias;
    g.out = logits;
    g.i_first = first_pred(layout);
    g.n_pred = L - g.i_first;
    g.M = B * g.n_pred;
    g.N = V;
    g.K = H;
    g.L = L;
    if (c != nullptr && c->smax != nullptr) {
        g.smax = const_cast<float*>(c->smax);
        g.slab_cols = c->slab_cols;
        if (r > 0) {
            g.w2 = c->w2;
            g.w1 = c->w1;
            g.w2_rows = V;
            g.w1_rows = c->vocab;
            g.w2_rank = r;
            g.w2n2 = c->w2n2;
            g.w1n2 = c->w1n2;   // (nullptr: markov_w2 only)
            g.w2_groups = kW2NormGroups;
        }
    }
    return g;
}

// chain_init (which zeroes the bins and the norm word), then the projection
// with the bound's epilogue when the chain is bounded.
int project(const ChainArgs& c, const void* hidden, int hidden_dtype, const uint16_t* lm_head,
            const float* bias, int B, int L, int H, int V, int layout, float* logits,
            hipStream_t stream, hipEvent_t mark_init = nullptr, hipEvent_t mark_projected = nullptr) {
    clear_pending_error();
    hipError_t e = launch_chain_init(c, stream);
    if (e == hipSuccess && mark_init) e = hipEventRecord(mark_init, stream);
    if (e == hipSuccess)
        e = launch_lmhead_gemm(gemm_args(hidden, lm_head, bias, B, L, H, V, layout, logits, &c, c.r),
                               hidden_dtype == DSPARK_HIDDEN_F32, stream);
    if (e == hipSuccess && mark_projected) e = hipEventRecord(mark_projected, stream);
    return hip_status(e);
}

int propose_impl(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                 const float* lm_head_bias, const uint16_t* markov_w1, const uint16_t* markov_w2,
                 const uint16_t* conf_w, const int32_t* anchors, int B, int L, int H, int V, int r,
                 int layout, int top_k, float p_min, float* logits, void* workspace,
                 size_t workspace_bytes, int32_t* tokens, int32_t* candidates, float* cand_logits,
                 float* conf, int32_t* lengths, hipStream_t s, hipEvent_t mark_init,
                 hipEvent_t mark_projected, hipEvent_t mark_chained) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    st = check_chain_args(V, r, top_k, p_min, markov_w1, markov_w2);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head || !logits || !anchors || !tokens || !candidates || !lengths)
        return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned16(logits) ||
        (conf_w && !aligned16(conf_w)))
        return DSPARK_ERR_UNSUPPORTED;
    if (!workspace) return DSPARK_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return DSPARK_ERR_WORKSPACE;
    const int n_pred = L - first_pred(layout);
    if (workspace_bytes < workspace_layout(B, n_pred, V, top_k).total) return DSPARK_ERR_WORKSPACE;

    const ChainArgs c = chain_args(logits, markov_w1, markov_w2, ChainExtras(), anchors, B, L, H, V, r,
                                   layout, top_k, hidden_dtype == DSPARK_HIDDEN_F32, workspace, lengths,
                                   true);
    st = project(c, hidden, hidden_dtype, lm_head, lm_head_bias, B, L, H, V, layout, logits, s,
                 mark_init, mark_projected);
    if (st != DSPARK_OK) return st;
    return run_chain(c, true, hidden, hidden_dtype, ChainExtras(), conf_w, B, L, H, V, layout, top_k,
                     p_min, workspace, tokens, candidates, cand_logits, conf, lengths, s,
                     mark_chained);
}

// Preparation area of the 4-bit projection: xp, M x 128 GQ bf16, 256-byte
// aligned. dspark_propose_q4 places it after the chain's workspace (so the
// flags word stays at offset 0); dspark_logits_q4 uses it from offset 0.
size_t q4_prep_bytes(int M, int H) { return align_up((size_t)M * 128 * q4_quads(H) * 2); }

// Checks of the 4-bit projection's own arguments.
int check_q4(int B, int L, int H, int V, int layout, const void* lm_head_q4) {
    if (H % kQ4Block != 0) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(lm_head_q4)) return DSPARK_ERR_UNSUPPORTED;
    const long M = (long)B * (L - first_pred(layout));
    // per-thread indices of the preparation and the projection fit in 32 bits
    if (M * 4 * q4_quads(H) > 0x7fffffffL || (long)q4_tiles(V) * q4_quads(H) * 64 > 0x7fffffffL)
        return DSPARK_ERR_UNSUPPORTED;
    return DSPARK_OK;
}

int project_q4(const void* hidden, int hidden_dtype, const void* lm_head_q4, const float* bias,
               int B, int L, int H, int V, int layout, float* logits, void* prep,
               hipStream_t stream, const ChainArgs* c = nullptr) {
    Q4Args q{};
    q.i_first = first_pred(layout);
    q.n_pred = L - q.i_first;
    q.M = B * q.n_pred;
    q.hidden = hidden;
    q.hidden_f32 = hidden_dtype == DSPARK_HIDDEN_F32;
    q.GQ = q4_quads(H);
    q.G = H / kQ4Block;
    q.T16 = q4_tiles(V);
    q.H = H;
    q.V = V;
    q.L = L;
    q.xp = static_cast<uint16_t*>(prep);
    q.packed = static_cast<const uint8_t*>(lm_head_q4);
    q.bias = bias;
    q.out = logits;
    if (c != nullptr && c->smax != nullptr) {
        // the top-k bound: slab maxima, and the norm workgroups when there is a Markov term
        q.smax = const_cast<float*>(c->smax);
        if (c->r > 0) {
            q.w2 = c->w2;
            q.w1 = c->w1;
            q.w_rows = V;
            q.w_rank = c->r;
            q.norm_groups = kW2NormGroups;
            q.w2n2 = c->w2n2;
            q.w1n2 = c->w1n2;   // (nullptr: markov_w2 only)
        }
    }
    return hip_status(launch_lmhead_q4(q, stream));
}

}  // namespace

// Scratch of dspark_propose_noalloc: the workspace of one call in a
// file-scope device array. Every GPU the library runs on holds its own copy
// (DSPARK_NOALLOC_SCRATCH_BYTES) from the first use until the process ends.
// Host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (the array's name on the host is a stand-in).
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // per device: the device address of scratch
std::mutex g_scratch_mu;

// The address of the current device's scratch, taken once per device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return DSPARK_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DSPARK_OK;
}

}  // namespace

extern "C" {

size_t dspark_workspace_bytes(int B, int L, int V, int top_k, int layout) {
    if (B <= 0 || V <= 0 || top_k < 1 || top_k > DSPARK_MAX_TOP_K) return 0;
    if (layout != DSPARK_LAYOUT_ANCHOR_FIRST && layout != DSPARK_LAYOUT_BONUS_ANCHOR) return 0;
    const int n_pred = L - first_pred(layout);
    if (n_pred <= 0) return 0;
    return workspace_layout(B, n_pred, V, top_k).total;
}

int dspark_logits(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                  const float* lm_head_bias, int B, int L, int H, int V, int layout, float* logits,
                  void* stream) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head || !logits) return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head)) return DSPARK_ERR_UNSUPPORTED;
    clear_pending_error();
    return hip_status(launch_lmhead_gemm(gemm_args(hidden, lm_head, lm_head_bias, B, L, H, V, layout,
                                                   logits, nullptr, 0),
                                         hidden_dtype == DSPARK_HIDDEN_F32,
                                         static_cast<hipStream_t>(stream)));
}

int dspark_chain(const float* logits, const void* hidden, int hidden_dtype,
                 const uint16_t* markov_w1, const uint16_t* markov_w2, const uint16_t* conf_w,
                 const int32_t* anchors, int B, int L, int H, int V, int r, int layout, int top_k,
                 float p_min, void* workspace, size_t workspace_bytes, int32_t* tokens,
                 int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                 void* stream) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    st = check_chain_args(V, r, top_k, p_min, markov_w1, markov_w2);
    if (st != DSPARK_OK) return st;
    if (!logits || !anchors || !tokens || !candidates || !lengths) return DSPARK_ERR_INVALID_ARG;
    if (conf_w && !hidden) return DSPARK_ERR_INVALID_ARG;
    if (conf_w && (!aligned16(conf_w) || !aligned16(hidden))) return DSPARK_ERR_UNSUPPORTED;
    if (!workspace) return DSPARK_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return DSPARK_ERR_WORKSPACE;
    if (workspace_bytes < dspark_workspace_bytes(B, L, V, top_k, layout)) return DSPARK_ERR_WORKSPACE;
    if (!aligned16(logits)) return DSPARK_ERR_UNSUPPORTED;
    // caller projections: no bound from a projection of this call
    const ChainArgs c = chain_args(logits, markov_w1, markov_w2, ChainExtras(), anchors, B, L, H, V, r,
                                   layout, top_k, hidden_dtype == DSPARK_HIDDEN_F32, workspace, lengths,
                                   false);
    return run_chain(c, false, hidden, hidden_dtype, ChainExtras(), conf_w, B, L, H, V, layout, top_k,
                     p_min, workspace, tokens, candidates, cand_logits, conf, lengths,
                     static_cast<hipStream_t>(stream));
}

int dspark_propose(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                   const float* lm_head_bias, const uint16_t* markov_w1,
                   const uint16_t* markov_w2, const uint16_t* conf_w, const int32_t* anchors,
                   int B, int L, int H, int V, int r, int layout, int top_k, float p_min,
                   float* logits, void* workspace, size_t workspace_bytes, int32_t* tokens,
                   int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                   void* stream) {
    return propose_impl(hidden, hidden_dtype, lm_head, lm_head_bias, markov_w1, markov_w2, conf_w,
                        anchors, B, L, H, V, r, layout, top_k, p_min, logits, workspace,
                        workspace_bytes, tokens, candidates, cand_logits, conf, lengths,
                        static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr);
}

int dspark_propose_noalloc(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                           const float* lm_head_bias, const uint16_t* markov_w1,
                           const uint16_t* markov_w2, const uint16_t* conf_w,
                           const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                           int top_k, float p_min, float* logits, int32_t* tokens,
                           int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                           void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Validation first (a call without a workspace stops at the workspace
    // check, with nothing enqueued, when every other argument is valid).
    int st = propose_impl(hidden, hidden_dtype, lm_head, lm_head_bias, markov_w1, markov_w2, conf_w,
                          anchors, B, L, H, V, r, layout, top_k, p_min, logits, nullptr, 0, tokens,
                          candidates, cand_logits, conf, lengths, s, nullptr, nullptr, nullptr);
    if (st != DSPARK_ERR_WORKSPACE) return st;
    if (dspark_workspace_bytes(B, L, V, top_k, layout) > (size_t)DSPARK_NOALLOC_SCRATCH_BYTES)
        return DSPARK_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != DSPARK_OK) return st;
    return propose_impl(hidden, hidden_dtype, lm_head, lm_head_bias, markov_w1, markov_w2, conf_w,
                        anchors, B, L, H, V, r, layout, top_k, p_min, logits, ws,
                        (size_t)DSPARK_NOALLOC_SCRATCH_BYTES, tokens, candidates, cand_logits, conf,
                        lengths, s, nullptr, nullptr, nullptr);
}

int dspark_propose_marked(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                          const float* lm_head_bias, const uint16_t* markov_w1,
                          const uint16_t* markov_w2, const uint16_t* conf_w,
                          const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                          int top_k, float p_min, float* logits, void* workspace,
                          size_t workspace_bytes, int32_t* tokens, int32_t* candidates,
                          float* cand_logits, float* conf, int32_t* lengths, void* stream,
                          void* mark_init, void* mark_projected, void* mark_chained) {
    return propose_impl(hidden, hidden_dtype, lm_head, lm_head_bias, markov_w1, markov_w2, conf_w,
                        anchors, B, L, H, V, r, layout, top_k, p_min, logits, workspace,
                        workspace_bytes, tokens, candidates, cand_logits, conf, lengths,
                        static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(mark_init),
                        static_cast<hipEvent_t>(mark_projected), static_cast<hipEvent_t>(mark_chained));
}

int dspark_propose_d2t(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                       const int64_t* d2t, const uint16_t* markov_w1, const uint16_t* markov_w2,
                       const uint16_t* conf_w, const int32_t* anchors, int B, int L, int H, int V,
                       int D, int r, int layout, int top_k, float p_min, float* logits,
                       void* workspace, size_t workspace_bytes, int32_t* tokens,
                       int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                       void* stream) {
    // the projection and the chain run over the D draft ids
    int st = check_sizes(B, L, H, D, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    if (V <= 0 || D > V) return DSPARK_ERR_INVALID_ARG;
    if (V >= 0x7fffffff - 1024) return DSPARK_ERR_UNSUPPORTED;
    st = check_chain_args(D, r, top_k, p_min, markov_w1, markov_w2);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head || !d2t || !logits || !anchors || !tokens || !candidates || !lengths)
        return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned16(logits) ||
        (conf_w && !aligned16(conf_w)) || (reinterpret_cast<uintptr_t>(d2t) & 7u) != 0)
        return DSPARK_ERR_UNSUPPORTED;
    if (!workspace) return DSPARK_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return DSPARK_ERR_WORKSPACE;
    if (workspace_bytes < dspark_workspace_bytes(B, L, D, top_k, layout)) return DSPARK_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    ChainExtras x;
    x.d2t = d2t;
    x.vocab = V;
    const ChainArgs c = chain_args(logits, markov_w1, markov_w2, x, anchors, B, L, H, D, r, layout,
                                   top_k, hidden_dtype == DSPARK_HIDDEN_F32, workspace, lengths, true);
    st = project(c, hidden, hidden_dtype, lm_head, nullptr, B, L, H, D, layout, logits, s);
    if (st != DSPARK_OK) return st;
    return run_chain(c, true, hidden, hidden_dtype, x, conf_w, B, L, H, D, layout, top_k, p_min,
                     workspace, tokens, candidates, cand_logits, conf, lengths, s);
}

int dspark_propose_adaptive(const void* hidden, int hidden_dtype, const uint16_t* lm_head,
                            const float* lm_head_bias, const uint16_t* markov_w1,
                            const uint16_t* markov_w2, const uint16_t* conf_w,
                            const int32_t* anchors, int B, int L, int H, int V, int r, int layout,
                            int top_k, const float* p_min, const int32_t* block_top_k,
                            float* logits, void* workspace, size_t workspace_bytes,
                            int32_t* tokens, int32_t* candidates, float* cand_logits, float* conf,
                            int32_t* lengths, void* stream) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    st = check_chain_args(V, r, top_k, 0.0f, markov_w1, markov_w2);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head || !conf_w || !p_min || !logits || !anchors || !tokens ||
        !candidates || !lengths)
        return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned16(logits) || !aligned16(conf_w))
        return DSPARK_ERR_UNSUPPORTED;
    if (!workspace) return DSPARK_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return DSPARK_ERR_WORKSPACE;
    if (workspace_bytes < dspark_workspace_bytes(B, L, V, top_k, layout)) return DSPARK_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    ChainExtras x;
    x.p_min_b = p_min;
    x.top_k_b = block_top_k;
    const ChainArgs c = chain_args(logits, markov_w1, markov_w2, x, anchors, B, L, H, V, r, layout,
                                   top_k, hidden_dtype == DSPARK_HIDDEN_F32, workspace, lengths, true);
    st = project(c, hidden, hidden_dtype, lm_head, lm_head_bias, B, L, H, V, layout, logits, s);
    if (st != DSPARK_OK) return st;
    return run_chain(c, true, hidden, hidden_dtype, x, conf_w, B, L, H, V, layout, top_k, 0.0f,
                     workspace, tokens, candidates, cand_logits, conf, lengths, s);
}

size_t dspark_q4_packed_bytes(int V, int H) {
    if (V <= 0 || H <= 0 || H % kQ4Block != 0) return 0;
    return q4_packed_bytes(V, H);
}

int dspark_q4_pack(const void* blocks, int V, int H, void* packed, void* stream) {
    if (!blocks || !packed || V <= 0 || H <= 0) return DSPARK_ERR_INVALID_ARG;
    if (H % kQ4Block != 0 || !aligned16(packed)) return DSPARK_ERR_UNSUPPORTED;
    if ((long)q4_tiles(V) * q4_quads(H) * 64 > 0x7fffffffL) return DSPARK_ERR_UNSUPPORTED;
    Q4PackArgs a;
    a.blocks = static_cast<const uint8_t*>(blocks);
    a.packed = static_cast<uint8_t*>(packed);
    a.V = V;
    a.G = H / kQ4Block;
    a.GQ = q4_quads(H);
    a.T16 = q4_tiles(V);
    clear_pending_error();
    return hip_status(launch_q4_pack(a, static_cast<hipStream_t>(stream)));
}

size_t dspark_q4_workspace_bytes(int B, int L, int H, int V, int top_k, int layout) {
    const size_t base = dspark_workspace_bytes(B, L, V, top_k, layout);
    if (base == 0 || H <= 0 || H % kQ4Block != 0) return 0;
    return q4_prep_bytes(B * (L - first_pred(layout)), H) + base;
}

int dspark_logits_q4(const void* hidden, int hidden_dtype, const void* lm_head_q4,
                     const float* lm_head_bias, int B, int L, int H, int V, int layout,
                     float* logits, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head_q4 || !logits) return DSPARK_ERR_INVALID_ARG;
    st = check_q4(B, L, H, V, layout, lm_head_q4);
    if (st != DSPARK_OK) return st;
    if (!aligned16(hidden)) return DSPARK_ERR_UNSUPPORTED;
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
        return DSPARK_ERR_WORKSPACE;
    if (workspace_bytes < q4_prep_bytes(B * (L - first_pred(layout)), H)) return DSPARK_ERR_WORKSPACE;
    clear_pending_error();
    return project_q4(hidden, hidden_dtype, lm_head_q4, lm_head_bias, B, L, H, V, layout, logits,
                      workspace, static_cast<hipStream_t>(stream));
}

int dspark_propose_q4(const void* hidden, int hidden_dtype, const void* lm_head_q4,
                      const float* lm_head_bias, const uint16_t* markov_w1,
                      const uint16_t* markov_w2, const uint16_t* conf_w, const int32_t* anchors,
                      int B, int L, int H, int V, int r, int layout, int top_k, float p_min,
                      float* logits, void* workspace, size_t workspace_bytes, int32_t* tokens,
                      int32_t* candidates, float* cand_logits, float* conf, int32_t* lengths,
                      void* stream) {
    int st = check_sizes(B, L, H, V, layout, hidden_dtype);
    if (st != DSPARK_OK) return st;
    st = check_chain_args(V, r, top_k, p_min, markov_w1, markov_w2);
    if (st != DSPARK_OK) return st;
    if (!hidden || !lm_head_q4 || !logits || !anchors || !tokens || !candidates || !lengths)
        return DSPARK_ERR_INVALID_ARG;
    st = check_q4(B, L, H, V, layout, lm_head_q4);
    if (st != DSPARK_OK) return st;
    if (!aligned16(hidden) || !aligned16(logits) || (conf_w && !aligned16(conf_w)))
        return DSPARK_ERR_UNSUPPORTED;
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
        return DSPARK_ERR_WORKSPACE;
    if (workspace_bytes < dspark_q4_workspace_bytes(B, L, H, V, top_k, layout))
        return DSPARK_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    // [chain workspace][preparation]: the flags word stays at offset 0
    void* prep = static_cast<char*>(workspace) + dspark_workspace_bytes(B, L, V, top_k, layout);
    // With the bound, the 4-bit projection writes 64-column slab maxima and
    // carries the norm workgroups, as the bf16 one does; chain_init (which
    // zeroes the norm words) goes first. Its epilogue pays only where the chain
    // prunes slabs with it (Qwen3.8-27B shape, 64 blocks of 16: 4.52 ms per
    // step unbounded, 4.64 ms with the bound filtering top-k inserts; 8
    // blocks, pruned: 0.889 -> 0.849 ms), so other shapes run unbounded.
    ChainExtras x;
    x.narrow_slabs = true;
    const bool prune = B <= 32 && chain_sparse(V, r);
    const ChainArgs c = chain_args(logits, markov_w1, markov_w2, x, anchors, B, L, H, V, r, layout,
                                   top_k, hidden_dtype == DSPARK_HIDDEN_F32, workspace, lengths, prune);
    clear_pending_error();
    if (launch_chain_init(c, s) != hipSuccess) return DSPARK_ERR_HIP;
    st = project_q4(hidden, hidden_dtype, lm_head_q4, lm_head_bias, B, L, H, V, layout, logits, prep, s,
                    &c);
    if (st != DSPARK_OK) return st;
    return run_chain(c, true, hidden, hidden_dtype, x, conf_w, B, L, H, V, layout, top_k, p_min,
                     workspace, tokens, candidates, cand_logits, conf, lengths, s);
}

int dspark_verify(const int32_t* candidates, const int32_t* lengths, const int32_t* target, int B,
                  int n_pred, int top_k, int lattice, int32_t* accepted, int32_t* totals,
                  void* stream) {
    if (B <= 0 || n_pred <= 0 || top_k < 1 || top_k > DSPARK_MAX_TOP_K) return DSPARK_ERR_INVALID_ARG;
    if (lattice != 0 && lattice != 1) return DSPARK_ERR_INVALID_ARG;
    if (!candidates || !lengths || !target || !accepted || !totals) return DSPARK_ERR_INVALID_ARG;
    if ((long)B * n_pred * top_k > 0x7fffffffL) return DSPARK_ERR_UNSUPPORTED;
    VerifyArgs v;
    v.candidates = candidates;
    v.lengths = lengths;
    v.target = target;
    v.accepted = accepted;
    v.totals = totals;
    v.B = B;
    v.n_pred = n_pred;
    v.top_k = top_k;
    v.width = lattice ? top_k : 1;
    clear_pending_error();
    return hip_status(launch_verify(v, static_cast<hipStream_t>(stream)));
}

int dspark_read_flags(const void* workspace, uint32_t* flags, void* stream) {
    if (!workspace || !flags) return DSPARK_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return DSPARK_ERR_HIP;
    return hip_status(hipStreamSynchronize(s));
}

// Dispatch check (host only: no HIP call, no GPU needed; not part of the
// public header). For every combination of the listed B, V and r, every
// top_k in 1..DSPARK_MAX_TOP_K and both chain modes (with and without the
// projection's bound) that dspark_propose's argument checks accept, the chain
// launcher must reach a compiled kernel with a non-empty grid. Returns the
// number of combinations that do not (the first is written to first_bad[0..4]
// = (B, V, r, top_k, bounded)) and the number checked to *checked.
long dspark_internal_chain_dispatch_walk(const int* Bs, int nB, const int* Vs, int nV, const int* rs,
                                         int nr, int* first_bad, long* checked) {
    if (!Bs || !Vs || !rs || !first_bad || !checked || nB < 0 || nV < 0 || nr < 0) return -1;
    *checked = 0;
    // stand-in addresses: aligned, non-null, never dereferenced
    char* const fake = reinterpret_cast<char*>(uintptr_t(1) << 20);
    const uint16_t* w = reinterpret_cast<const uint16_t*>(fake);
    const int L = 4, H = 64;
    long bad = 0;
    set_chain_dry_dispatch(true);
    for (int ib = 0; ib < nB; ++ib)
        for (int iv = 0; iv < nV; ++iv)
            for (int ir = 0; ir < nr; ++ir)
                for (int k = 1; k <= DSPARK_MAX_TOP_K; ++k)
                    for (int bounded = 0; bounded < 2; ++bounded) {
                        const int B = Bs[ib], V = Vs[iv], r = rs[ir];
                        const uint16_t* w1 = r > 0 ? w : nullptr;
                        if (check_sizes(B, L, H, V, DSPARK_LAYOUT_ANCHOR_FIRST, DSPARK_HIDDEN_BF16) != DSPARK_OK ||
                            check_chain_args(V, r, k, 0.0f, w1, w1) != DSPARK_OK)
                            continue;
                        const ChainArgs c = chain_args(reinterpret_cast<const float*>(fake), w1, w1,
                                                       ChainExtras(), reinterpret_cast<const int32_t*>(fake),
                                                       B, L, H, V, r, DSPARK_LAYOUT_ANCHOR_FIRST, k, false,
                                                       fake, reinterpret_cast<int32_t*>(fake), bounded != 0);
                        ++*checked;
                        const bool ok = c.nwg >= 1 && launch_chain_step(c, 0, nullptr) == hipSuccess;
                        if (!ok && bad++ == 0) {
                            first_bad[0] = B;
                            first_bad[1] = V;
                            first_bad[2] = r;
                            first_bad[3] = k;
                            first_bad[4] = bounded;
                        }
                    }
    set_chain_dry_dispatch(false);
    return bad;
}

const char* dspark_status_string(int status) {
    switch (status) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_INVALID_ARG: return "invalid argument";
        case DSPARK_ERR_UNSUPPORTED: return "unsupported size or alignment";
        case DSPARK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case DSPARK_ERR_HIP: return "HIP runtime error while enqueuing";
        case DSPARK_ERR_SCRATCH:
            return "sizes need more workspace than the allocation-free entry point's static scratch";
        default: return "unknown status";
    }
}

}  // extern "C"
