// sv_api.cpp -- host side of libspecverify: argument checks, the launch
// plan, and the exported C entry points declared in include/specverify.h.
// Every check runs before anything is launched, so an error leaves all
// buffers untouched.
#include "specverify.h"

#include <math.h>
#include <stdint.h>

#include <climits>
#include <initializer_list>

#include "sv_internal.h"

namespace {

// Largest grids: the x-dimension thread count must fit in 32 bits (256
// threads per row-split statistics group, 1024 per sequence-resident group).
constexpr long long kMaxGrid = 16777215LL;
constexpr long long kMaxSeqGrid = 4194303LL;
// Largest vocabulary: keeps every in-row element index and slice bound in int.
constexpr int kMaxV = 1 << 28;

int elem_size(int dtype) { return dtype == SV_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int G, int k, int V, int64_t row_stride) {
    if (B < 0 || G < 1 || k < 0 || V < 1) return SV_ERR_SHAPE;
    if (k > SV_MAX_K || V > kMaxV) return SV_ERR_SHAPE;
    if ((long long)G * (k + 1) > SV_MAX_ROWS_PER_SEQ) return SV_ERR_SHAPE;
    if (row_stride < V) return SV_ERR_SHAPE;
    return SV_OK;
}

struct Plan {
    bool seq;  // sequence-resident layout (no workspace)
    int rows_per_seq;
    int S;
    int slice_len;
    int SD;  // row-split stochastic: draw workgroups per sequence
    bool slice_draw;  // plain sampling: draw from slice statistics
    bool vec;
    size_t ws_bytes;
};

// Layout choice beyond use_seq_resident():
//   ROW_SPLIT  the caller forces the row-split layout (ragged batches of
//              unequal lengths with diagnostics: every row is read, and one
//              workgroup per sequence would wait on the longest sequence);
//   SAMPLE     plain sampling: one pass per row (use_sample_seq()) or
//              row-split with sliced rows (the draw reads one slice again
//              instead of the whole row).
//   SEQ        the caller forces the sequence-resident layout (stochastic
//              calls without diagnostics that take the capped early exit
//              below the usual threshold).
enum PlanFlags { kPlanDefault = 0, kPlanRowSplit = 1, kPlanSample = 2, kPlanSeq = 4 };

int make_plan(int B, int G, int rows_per_seq, int V, int64_t row_stride, int dtype,
              bool stochastic, int flags, const void* const* row_bases, int n_bases,
              Plan* pl) {
    const int es = elem_size(dtype);
    bool vec = ((row_stride * es) % 16) == 0;
    for (int i = 0; i < n_bases; ++i) vec = vec && aligned16(row_bases[i]);
    pl->seq = flags == kPlanDefault && sv::use_seq_resident(B, G);
    if (flags & kPlanSample) pl->seq = sv::use_sample_seq(B, V, vec ? V / (16 / es) : V);
    if (flags & kPlanSeq) pl->seq = true;
    pl->slice_draw = false;
    pl->rows_per_seq = rows_per_seq;
    pl->vec = vec;
    if (pl->seq) {
        pl->S = 1;
        pl->SD = 1;
        pl->slice_len = V;
        pl->ws_bytes = 0;
        return B > kMaxSeqGrid ? SV_ERR_SHAPE : SV_OK;
    }
    const int E = vec ? 16 / es : 1;
    const int S0 = (flags & kPlanSample) ? sv::plan_slices_sample((long long)B * rows_per_seq, V)
                                         : sv::plan_slices((long long)B * rows_per_seq, V);
    // slice length: a whole number of chunks, then drop empty slices
    const int chunks = (V + E - 1) / E;
    int per = (chunks + S0 - 1) / S0;
    if (stochastic && !(flags & kPlanSample)) per = sv::draw_aligned_slice(B, V, E, per);
    const int slice_len = per * E;
    const int S = (V + slice_len - 1) / slice_len;
    // (sampling from slice statistics pads the statistics grid to whole
    // groups of 8 rows)
    const long long Bg = (stochastic && (flags & kPlanSample)) ? (B + 7LL) / 8 * 8 : B;
    if (Bg * rows_per_seq * S > kMaxGrid) return SV_ERR_SHAPE;
    if (B > kMaxSeqGrid) return SV_ERR_SHAPE;  // finishing kernels: one 1024-thread group per sequence
    pl->S = S;
    pl->slice_len = slice_len;
    pl->slice_draw = stochastic && (flags & kPlanSample);
    pl->SD = stochastic ? sv::plan_draw_slices(B, sv::draw_tiles(V / E, V % E)) : 1;
    if ((long long)B * pl->SD > kMaxGrid) return SV_ERR_SHAPE;
    pl->ws_bytes = sv::workspace_bytes_for(B, rows_per_seq, S, stochastic);
    return SV_OK;
}

int check_workspace(const void* ws, size_t bytes, const Plan& pl) {
    if (pl.ws_bytes == 0) return SV_OK;
    if (!ws) return SV_ERR_NULL;
    if (((uintptr_t)ws & 255u) != 0) return SV_ERR_WORKSPACE;
    if (bytes < pl.ws_bytes) return SV_ERR_WORKSPACE;
    return SV_OK;
}

// Workspace bytes of the row-split layout at this shape (an upper bound over
// the load paths: the slice count before rounding to whole chunks).
size_t rowsplit_need(int B, int rows_per_seq, int V, bool stochastic, bool sample) {
    const long long rows = (long long)B * rows_per_seq;
    int S = sample ? sv::plan_slices_sample(rows, V) : sv::plan_slices(rows, V);
    if (stochastic && !sample) {
        // or the slices cut to the draw groups' tiles, for any element size
        // and load path (1, 4 or 8 logits a chunk)
        const int S0 = S;
        for (int E : {1, 4, 8}) {
            const int chunks = (V + E - 1) / E;
            const int per = sv::draw_aligned_slice(B, V, E, (chunks + S0 - 1) / S0);
            const long long len = (long long)per * E;
            const int SE = (int)((V + len - 1) / len);
            if (SE > S) S = SE;
        }
    }
    return sv::workspace_bytes_for(B, rows_per_seq, S, stochastic);
}

// Workspace of the capped early exit (still-accepting flags, then the
// row-split stochastic layout with S slices per row).
size_t exit_need(int B, int k, int S) {
    return sv::exit_flag_bytes(B) + sv::workspace_bytes_for(B, 2 * k + 1, S, true);
}

int exit_slices_max(int V) {
    int s = V / sv::kMinSliceElems;
    if (s > sv::kExitMaxSlices) s = sv::kExitMaxSlices;
    return s < 1 ? 1 : s;
}

}  // namespace

// The library is built with hidden visibility; only the C ABI is exported.
#pragma GCC visibility push(default)
extern "C" {

size_t sv_workspace_bytes(int B, int G, int k, int V) {
    if (check_shape(B, G, k, V, V) != SV_OK) return 0;
    // Enough for every entry point at any B: the stochastic ones (one
    // candidate) may take the row-split layout (sampling outside the one-pass
    // shapes, ragged batches with diagnostics), and so do greedy calls below
    // the sequence-resident threshold and tree verification (G = N, k = 0).
    size_t s = rowsplit_need(B, 2 * k + 1, V, true, k == 0);
    const size_t g = rowsplit_need(B, G * (k + 1), V, false, false);
    // and the capped early exit of dense and ragged stochastic calls, which
    // only sequence-resident batches take
    if (sv::plan_exit_pairs(k) > 0 && B >= sv::kCappedExitMinB && B <= sv::kExitMaxB) {
        const size_t e = exit_need(B, k, exit_slices_max(V));
        if (e > s) s = e;
    }
    return s > g ? s : g;
}

const char* sv_status_string(int status) {
    switch (status) {
        case SV_OK: return "success";
        case SV_ERR_NULL: return "a required pointer is NULL";
        case SV_ERR_SHAPE: return "invalid shape (B, G, k, V or row_stride out of range)";
        case SV_ERR_DTYPE: return "unsupported logit dtype";
        case SV_ERR_TEMPERATURE: return "temperature must be positive and finite";
        case SV_ERR_WORKSPACE: return "workspace smaller than sv_workspace_bytes() or not 256-byte aligned";
        case SV_ERR_HIP: return "the HIP runtime refused the kernel launch";
        case SV_ERR_SCRATCH: return "the shape needs more workspace than the library's own buffer (SV_SCRATCH_BYTES) holds";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Sequence-resident early exit: when the caller's workspace has room, cap
// the first pass at sv::plan_exit_pairs(k) pairs and finish in the row-split
// layout (see sv_internal.h).  Without a workspace (allowed here) the plain
// early exit runs, with the same decisions and tokens.
// Slices per row of the capped early exit's statistics that the workspace
// holds (at most exit_slices_max(V)), or 0 when the capped exit cannot run
// (no usable workspace, too many sequences, no capping at this k).
int capped_exit_slices(int B, int k, int V, const void* workspace, size_t workspace_bytes) {
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || B > sv::kExitMaxB) return 0;
    const int P = sv::plan_exit_pairs(k);
    if (P < 1 || P >= k) return 0;
    int smax = exit_slices_max(V);
    while (smax > 1 && exit_need(B, k, smax) > workspace_bytes) --smax;
    return exit_need(B, k, smax) > workspace_bytes ? 0 : smax;
}

void plan_exit(sv::Params* p, int E, void* workspace, size_t workspace_bytes) {
    const int B = p->B, k = p->k, V = p->V;
    const int smax = capped_exit_slices(B, k, V, workspace, workspace_bytes);
    if (smax == 0) return;
    const int P = sv::plan_exit_pairs(k);
    const int rows = 2 * k + 1;
    char* w = static_cast<char*>(workspace);
    p->active = reinterpret_cast<int*>(w);
    w += sv::exit_flag_bytes(B);
    p->part = reinterpret_cast<float*>(w);
    w += sv::part_bytes(B, rows, smax);
    p->tilesum = reinterpret_cast<float*>(w);
    w += sv::tilesum_bytes(B);
    p->cnt = reinterpret_cast<int*>(w);
    w += sv::cnt_bytes(B);
    p->xl = reinterpret_cast<float*>(w);
    p->exit_pairs = P;
    p->rows_per_seq = rows;
    p->S = smax;
    p->SD = sv::plan_draw_slices(B, sv::draw_tiles(V / E, V % E));
}

// Shared body of the stochastic entry points.  cu == nullptr: dense batch of
// k draft tokens per sequence; else ragged (k is the maximum).  accept_len
// may be null only for internal callers (sv_sample).
int stochastic_impl(const void* target, const void* draft, const int32_t* x, const int32_t* cu,
                    long long total_draft, const float* ua, const float* us, int B, int k, int V,
                    int64_t row_stride, int dtype, float temperature, int32_t* accept_len,
                    int32_t* tokens, float* dbg, void* workspace, size_t workspace_bytes,
                    void* stream) {
    int st = check_shape(B, 1, k, V, row_stride);
    if (st != SV_OK) return st;
    if (cu && (total_draft < 0 || total_draft > INT32_MAX)) return SV_ERR_SHAPE;
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    const double c = 1.4426950408889634 / (double)temperature;
    if (!(temperature > 0.0f) || !isfinite(temperature) || !isfinite((float)c))
        return SV_ERR_TEMPERATURE;
    if (B == 0) return SV_OK;
    const bool drafts = cu ? total_draft > 0 : k > 0;
    if (!target || !us || !tokens) return SV_ERR_NULL;
    if (drafts && (!draft || !x || !ua)) return SV_ERR_NULL;
    const void* bases[2] = {target, drafts ? draft : target};
    int flags = kPlanDefault;
    if (!cu && k == 0) flags = kPlanSample;
    // Unequal ragged lengths (known from the total alone) with every row to
    // be read: balance rows, not sequences, over the GPU.
    if (cu && dbg && total_draft < (long long)B * k) flags = kPlanRowSplit;
    // Without diagnostics, from kCappedExitMinB sequences on: the
    // sequence-resident layout and its capped early exit (see sv_internal.h).
    if (flags == kPlanDefault && !dbg && B >= sv::kCappedExitMinB &&
        !sv::use_seq_resident(B, 1) && capped_exit_slices(B, k, V, workspace, workspace_bytes) > 0)
        flags = kPlanSeq;
    Plan pl;
    st = make_plan(B, 1, 2 * k + 1, V, row_stride, dtype, true, flags, bases, 2, &pl);
    if (st != SV_OK) return st;
    st = check_workspace(workspace, workspace_bytes, pl);
    if (st != SV_OK) return st;

    sv::Params p = {};
    p.target = target;
    p.draft = draft;
    p.tokens_in = x;
    p.u_accept = ua;
    p.u_sample = us;
    p.accept_len = accept_len;
    p.tokens_out = tokens;
    p.best_cand = nullptr;
    p.dbg = dbg;
    p.part = static_cast<float*>(workspace);
    if (!pl.seq) {
        char* w = static_cast<char*>(workspace) + sv::part_bytes(B, pl.rows_per_seq, pl.S);
        p.tilesum = reinterpret_cast<float*>(w);
        w += sv::tilesum_bytes(B);
        p.cnt = reinterpret_cast<int*>(w);
        w += sv::cnt_bytes(B);
        p.xl = reinterpret_cast<float*>(w);
    }
    p.SD = pl.SD;
    p.slice_draw = pl.slice_draw ? 1 : 0;
    p.cu = cu;
    p.total_draft = total_draft;
    p.row_stride = row_stride;
    p.B = B;
    p.G = 1;
    p.k = k;
    p.V = V;
    p.rows_per_seq = pl.rows_per_seq;
    p.S = pl.S;
    p.slice_len = pl.slice_len;
    p.c = (float)c;
    if (pl.seq && !dbg && k >= 2)
        plan_exit(&p, pl.vec ? 16 / elem_size(dtype) : 1, workspace, workspace_bytes);
    return sv::launch_stochastic(p, dtype, pl.vec, pl.seq, stream) == 0 ? SV_OK : SV_ERR_HIP;
}

// Shared body of the greedy entry points (cu as above; ragged means G = 1).
int greedy_impl(const void* target, const int32_t* x, const int32_t* cu, long long total_draft,
                int B, int G, int k, int V, int64_t row_stride, int dtype, int32_t* accept_len,
                int32_t* tokens, int32_t* best_cand, void* workspace, size_t workspace_bytes,
                void* stream) {
    int st = check_shape(B, G, k, V, row_stride);
    if (st != SV_OK) return st;
    if (cu && (G != 1 || total_draft < 0 || total_draft > INT32_MAX)) return SV_ERR_SHAPE;
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (B == 0) return SV_OK;
    const bool drafts = cu ? total_draft > 0 : k > 0;
    if (!target || !tokens || (drafts && !x)) return SV_ERR_NULL;
    const void* bases[1] = {target};
    Plan pl;
    st = make_plan(B, G, G * (k + 1), V, row_stride, dtype, false, kPlanDefault, bases, 1, &pl);
    if (st != SV_OK) return st;
    st = check_workspace(workspace, workspace_bytes, pl);
    if (st != SV_OK) return st;

    sv::Params p = {};
    p.target = target;
    p.draft = nullptr;
    p.tokens_in = x;
    p.accept_len = accept_len;
    p.tokens_out = tokens;
    p.best_cand = best_cand;
    p.part = static_cast<float*>(workspace);
    p.cu = cu;
    p.total_draft = total_draft;
    p.row_stride = row_stride;
    p.B = B;
    p.G = G;
    p.k = k;
    p.V = V;
    p.rows_per_seq = pl.rows_per_seq;
    p.S = pl.S;
    p.slice_len = pl.slice_len;
    p.c = 0.0f;
    return sv::launch_greedy(p, dtype, pl.vec, pl.seq, stream) == 0 ? SV_OK : SV_ERR_HIP;
}

// Greedy draft-tree verification: row statistics (argmax) over all N rows of
// every sequence, then the tree decision per sequence.
int tree_impl(const void* target, const int32_t* node_tokens, const int32_t* parents, int B,
              int N, int V, int64_t row_stride, int dtype, int32_t* accept_len, int32_t* tokens,
              int32_t* path, void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || N < 1 || N > SV_MAX_ROWS_PER_SEQ || V < 1 || V > kMaxV || row_stride < V)
        return SV_ERR_SHAPE;
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (B == 0) return SV_OK;
    if (!target || !node_tokens || !parents || !accept_len || !tokens || !path)
        return SV_ERR_NULL;
    const void* bases[1] = {target};
    Plan pl;
    int st = make_plan(B, 1, N, V, row_stride, dtype, false, kPlanRowSplit, bases, 1, &pl);
    if (st != SV_OK) return st;
    st = check_workspace(workspace, workspace_bytes, pl);
    if (st != SV_OK) return st;

    sv::Params p = {};
    p.target = target;
    p.tokens_in = node_tokens;
    p.parents = parents;
    p.path = path;
    p.accept_len = accept_len;
    p.tokens_out = tokens;
    p.part = static_cast<float*>(workspace);
    p.row_stride = row_stride;
    p.B = B;
    p.G = 1;
    p.k = N - 1;  // rows b*N .. b*N + N - 1, as a dense sequence of N rows
    p.V = V;
    p.rows_per_seq = N;
    p.S = pl.S;
    p.slice_len = pl.slice_len;
    return sv::launch_tree(p, dtype, pl.vec, stream) == 0 ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" {

int sv_verify_greedy_tree(const void* target_logits, const int32_t* node_tokens,
                          const int32_t* parents, int B, int N, int V, int64_t row_stride,
                          int dtype, int32_t* accept_len, int32_t* tokens, int32_t* path,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return tree_impl(target_logits, node_tokens, parents, B, N, V, row_stride, dtype, accept_len,
                     tokens, path, workspace, workspace_bytes, stream);
}

int sv_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W, int32_t* seq_len,
              int32_t* history, int64_t history_stride, int capacity, int32_t* next_token,
              int64_t next_stride, void* stream) {
    if (B < 0 || W < 1 || capacity < 0 || history_stride < capacity || next_stride < 1)
        return SV_ERR_SHAPE;
    if (B > kMaxGrid) return SV_ERR_SHAPE;
    if (B == 0) return SV_OK;
    if (!accept_len || !tokens || !seq_len || !history || !next_token) return SV_ERR_NULL;
    return sv::launch_commit(accept_len, tokens, B, W, seq_len, history, history_stride, capacity,
                             next_token, next_stride, stream) == 0
               ? SV_OK
               : SV_ERR_HIP;
}

int sv_verify_stochastic(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* u_accept,
                         const float* u_sample, int B, int k, int V, int64_t row_stride,
                         int dtype, float temperature, int32_t* accept_len, int32_t* tokens,
                         float* dbg_px_qx, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (B > 0 && !accept_len) return SV_ERR_NULL;
    return stochastic_impl(target_logits, draft_logits, draft_tokens, nullptr, 0, u_accept,
                           u_sample, B, k, V, row_stride, dtype, temperature, accept_len, tokens,
                           dbg_px_qx, workspace, workspace_bytes, stream);
}

int sv_verify_stochastic_ragged(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const int32_t* cu_draft_len,
                                int total_draft, const float* u_accept, const float* u_sample,
                                int B, int k_max, int V, int64_t row_stride, int dtype,
                                float temperature, int32_t* accept_len, int32_t* tokens,
                                float* dbg_px_qx, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (B > 0 && (!accept_len || !cu_draft_len)) return SV_ERR_NULL;
    if (total_draft < 0) return SV_ERR_SHAPE;
    return stochastic_impl(target_logits, draft_logits, draft_tokens, cu_draft_len, total_draft,
                           u_accept, u_sample,
                           B, k_max, V, row_stride, dtype, temperature, accept_len, tokens,
                           dbg_px_qx, workspace, workspace_bytes, stream);
}

int sv_verify_greedy(const void* target_logits, const int32_t* draft_tokens, int B, int G,
                     int k, int V, int64_t row_stride, int dtype, int32_t* accept_len,
                     int32_t* tokens, int32_t* best_cand, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (B > 0 && !accept_len) return SV_ERR_NULL;
    return greedy_impl(target_logits, draft_tokens, nullptr, 0, B, G, k, V, row_stride, dtype,
                       accept_len, tokens, best_cand, workspace, workspace_bytes, stream);
}

int sv_verify_greedy_ragged(const void* target_logits, const int32_t* draft_tokens,
                            const int32_t* cu_draft_len, int total_draft, int B, int k_max,
                            int V, int64_t row_stride, int dtype, int32_t* accept_len,
                            int32_t* tokens, void* workspace, size_t workspace_bytes,
                            void* stream) {
    if (B > 0 && (!accept_len || !cu_draft_len)) return SV_ERR_NULL;
    if (total_draft < 0) return SV_ERR_SHAPE;
    return greedy_impl(target_logits, draft_tokens, cu_draft_len, total_draft, B, 1, k_max, V,
                       row_stride, dtype, accept_len, tokens, nullptr, workspace,
                       workspace_bytes, stream);
}

int sv_sample(const void* logits, const float* u, int B, int V, int64_t row_stride, int dtype,
              float temperature, int greedy, int32_t* tokens, void* workspace,
              size_t workspace_bytes, void* stream) {
    if (greedy)
        return greedy_impl(logits, nullptr, nullptr, 0, B, 1, 0, V, row_stride, dtype, nullptr,
                           tokens, nullptr, workspace, workspace_bytes, stream);
    return stochastic_impl(logits, nullptr, nullptr, nullptr, 0, nullptr, u, B, 0, V, row_stride,
                           dtype, temperature, nullptr, tokens, nullptr, workspace,
                           workspace_bytes, stream);
}

}  // extern "C"
#pragma GCC visibility pop
