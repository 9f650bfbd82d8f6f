// sv_internal.h -- launch plan and kernel parameters shared by the host
// front end (sv_api.cpp) and the kernels (sv_kernels.hip).  Not part of the
// public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

// Each logit row is cut into S slices and every (row, slice) pair is one
// workgroup of the streaming pass.  S is raised above 1 only when the batch
// has too few rows to give every compute unit several workgroups.
constexpr long long kTargetItems = 2048;  // about 8 workgroups per CU (256 CUs)
constexpr int kMinSliceElems = 4096;      // never cut a row finer than this
constexpr int kMaxSlices = 64;
constexpr int kMaxK = 64;
constexpr int kMaxRowsPerSeq = 1024;

// Slices per row for `rows` rows of V logits.
inline int plan_slices(long long rows, int V) {
    long long s = 1;
    if (rows > 0 && rows < kTargetItems) s = (kTargetItems + rows - 1) / rows;
    long long cap = V / kMinSliceElems;
    if (cap < 1) cap = 1;
    if (s > cap) s = cap;
    if (s > kMaxSlices) s = kMaxSlices;
    return (int)s;
}

// Bytes reserved for the per-sequence arrival counters (int32 [B]).
inline size_t counter_bytes(int B) { return ((size_t)B * 4 + 255) / 256 * 256; }

// Bytes of the workspace: counters, then float2 partial statistics
// [B][rows_per_seq][S].
inline size_t workspace_bytes_for(int B, int rows_per_seq, int S) {
    return counter_bytes(B) + (size_t)B * rows_per_seq * S * 8;
}

struct Params {
    const void* target;
    const void* draft;
    const int32_t* tokens_in;
    const float* u_accept;
    const float* u_sample;
    int32_t* accept_len;
    int32_t* tokens_out;
    int32_t* best_cand;
    float* dbg;
    int* counters;        // [B], zero between calls
    float* part;          // [B][rows_per_seq][S][2]
    long long row_stride; // elements
    int B, G, k, V;
    int rows_per_seq;     // stochastic 2k+1, greedy G(k+1)
    int S;                // slices per row
    int slice_len;        // elements per slice
    float c;              // log2(e) / temperature
};

// Launchers (sv_kernels.hip).  dtype: 0 float32, 1 bfloat16; vec: rows start
// on 16-byte boundaries.  Return a hipError_t value (0 = success).
int launch_stochastic(const Params& p, int dtype, bool vec, void* stream);
int launch_greedy(const Params& p, int dtype, bool vec, void* stream);

}  // namespace sv
