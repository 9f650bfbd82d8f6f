// sv_internal.h -- launch plan and kernel parameters shared by the host
// front end (sv_api.cpp) and the kernels (sv_kernels.hip).  Not part of the
// public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxK = 64;
constexpr int kMaxRowsPerSeq = 1024;

// Two ways to lay the work out on the GPU:
//
//  * sequence-resident: one workgroup (kSeqThreads or kSeqWideThreads
//    threads, below) owns one sequence, streams all of its rows and finishes
//    it in place.  Nothing crosses workgroups, so there are no atomics,
//    fences or workspace.  Used when the batch alone fills the machine
//    (single candidate, B >= kSeqResidentMinB).
//
//  * row-split: a statistics kernel gives every (row, slice) its own
//    workgroup and writes 8 bytes per item to the workspace; finishing
//    kernels then merge them per sequence, decide and sample (the
//    stochastic draw spread over several workgroups per sequence for small
//    batches).  The kernel boundary makes the statistics visible.  Used for
//    small batches, several candidates per sequence, draft trees, plain
//    sampling outside the one-pass shapes and ragged batches read in full.
constexpr int kSeqResidentMinB = 192;
// Sequence-resident workgroup size: 1024 threads (one group per CU), or 512
// threads once the sequences outnumber the 256 CUs, so that two or more share
// a CU and the whole batch streams at once instead of in rounds.
constexpr int kSeqThreads = 1024;
constexpr int kSeqWideThreads = 512;
constexpr int kSeqWideMinB = 257;
// Row-split stochastic calls with at least this many sequences (one per CU)
// finish each sequence in one workgroup (kSeqThreads threads, kSeqWideThreads
// from kSeqWideMinB on); smaller batches spread the closing-token draw over SD
// workgroups per sequence instead.
constexpr int kFinishOneGroupMinB = 256;

inline bool use_seq_resident(int B, int G) { return G == 1 && B >= kSeqResidentMinB; }

// Row-split plan: each row is cut into S slices, S raised above 1 only when
// there are too few rows to give every compute unit several workgroups.
constexpr long long kTargetItems = 2048;  // about 8 workgroups per CU (256 CUs)
constexpr int kMinSliceElems = 4096;      // never cut a row finer than this
constexpr int kMaxSlices = 64;

// The statistics kernel runs 512-thread workgroups on slices of at least
// kRowStatsWideChunks chunks (16-byte loads, or single logits on the
// element-wise path), 256-thread ones on shorter slices.  Measured per call
// (256 / 512 threads): B=64, k=4, V=128256 bf16 with 4008 chunks a slice
// 41.1 / 40.7 us, with the draw-aligned 2048 39.7 / 40.3 us; B=128, k=8
// (16032) 108.1 / 105.8 us; greedy B=128, k=4 (4008) 30.3 / 29.6 us; the
// B=32, G=16, k=4, V=32000 f32 lookahead batch (8000) 54.5 / 53.1 us; B=16,
// k=4 (1069) 25.6 / 27.2 us.
constexpr int kRowStatsWideChunks = 3072;

inline int plan_slices(long long rows, int V) {
    long long s = 1;
    if (rows > 0 && rows < kTargetItems) s = (kTargetItems + rows - 1) / rows;
    long long cap = V / kMinSliceElems;
    if (cap < 1) cap = 1;
    if (s > cap) s = cap;
    if (s > kMaxSlices) s = kMaxSlices;
    return (int)s;
}

// Plain sampling (no draft positions) otherwise takes the row-split layout with
// rows cut into slices of at most about kSampleSliceElems logits: the
// statistics kernel then leaves per-slice normalisers, from which the draw
// picks the slice holding r * Z and reads only that slice again.  (The bonus
// token of a verification could be drawn the same way, but a single group
// re-reading a slice measured slower there than the tile sums spread over
// SD groups.)
constexpr int kSampleSliceElems = 16384;
// Short rows, or a batch that fills the GPU with one row per CU, are sampled
// instead in one pass by one workgroup per row, with no workspace.  A row
// then streams through a single CU (about 6 us plus 0.08 ns per logit on
// MI355X, whatever the batch), while slicing spreads it over many.  Measured
// over B in 1..512 and V in 32000..256000 (bf16), one pass is the faster
// layout
//   * with 1024-thread groups, B < kSeqWideMinB: when V <= kSampleSeqBaseElems +
//     kSampleSeqElemsPerRow * B (beyond the 256 CUs a second wave of rows
//     doubles the time);
//   * with 512-thread groups, two per CU, kSeqWideMinB <= B <= 512: when V <=
//     kSampleSeqBaseElems, or B >= kSampleWideMidB and V <=
//     kSampleWideMaxElems.
// Its per-round partial sums sit in registers, which caps a row at
// kSampleSeqRounds rounds of one chunk per thread.
constexpr int kSampleSeqRounds = 32;
// Rows of at most kSampleHeldRounds rounds also keep every chunk they stream
// in registers, so the draw scans its round without reading it again.
constexpr int kSampleHeldRounds = 16;
// The sequence-resident stochastic kernels keep the row pair they have just
// streamed on chip for the closing-token draw, which would otherwise read
// both rows again: each thread's chunks of the first rounds of the target
// row in registers (4 VGPRs per round for 16-byte chunks), and as many
// rounds of the draft row as fit in the LDS left beside the kernel's own
// (kLdsBytesPerCu per CU).  Rounds held: as many as fit in the 128 VGPRs
// that four waves per SIMD allow without spilling, except where holding
// measured slower: the early exit with 512-thread groups on short rows
// (B=300, k=8, V=32000 bf16: 40.2 us without, 48.2 with; B=512, k=8,
// V=32000: 46.6 against 53.9) or below 384 sequences (B=300, k=3,
// V=129280: 101.9 against 102.6), and the capped early exit there.
//
// With 1024-thread groups (up to 256 sequences) the early exit and the full
// read are one kernel that streams the pairs in position order, holding
// each, and draws right after the first rejection, so whichever pair a
// sequence rejects at is on chip; the full read then streams the rest of
// the rows for the diagnostics.  Per call, B=256, k=8, V=128256 bf16, full
// read, against streaming pair 0 last and holding only it: the peaked batch
// (mean accepted length 1.2) 185.4 -> 178.2 us; half the sequences
// accepting every draft (mean 4.0) 185.3 -> 177.4, a quarter (mean 2.0)
// 185.3 -> 179.5; but drafts rejected almost always at position 0 (mean
// 0.1) 185.9 -> 189.3, and every draft accepted 179.8 -> 184.8 (a barrier
// per pair).  With 512-thread groups the early exit holds, and the full
// read runs in position order, only with two groups on most CUs and long
// rows: from kSeqWideLongMinB sequences and kSeqWideLongMinRowBytes per
// row (12 rounds held).  There the full read measured 0.4 us slower to 10
// us faster per call than streaming pair 0 last (B=384..512,
// V=80000..129280 bf16 and 64000 fp32; 9 us faster on B=512, k=3,
// V=129280 bf16), against 3 to 10 us slower on rows of 128 KB or less
// (B=300, k=8, V=32000; B=512, k=6, V=64000 bf16) and below 384 sequences
// (B=320, k=8, V=128256); the early exit 130.1 -> 125.0 us on B=512, k=3,
// V=129280 (with every draft accepted, V=128256: 170.5 -> 156.9; half the
// sequences: 141.1 -> 131.9), within 1 us either way from 384 to 448.
#ifndef SV_HOLD_SEQ_512
#define SV_HOLD_SEQ_512 16
#endif
#ifndef SV_HOLD_EXIT_1024
#define SV_HOLD_EXIT_1024 12
#endif
#ifndef SV_HOLD_EXIT_512
#define SV_HOLD_EXIT_512 0
#endif
constexpr int kPairHeldRounds = 16;  // the most any kernel holds
// Holding limits the full read to two 512-thread workgroups per CU (LDS and
// registers), where up to four fit otherwise: beyond kSeqWideHoldMaxB
// sequences (two per CU) a second round of workgroups would follow, so
// nothing is held there (B=700, k=8, V=32000 bf16: 132.6 us without, 161.1
// with; B=1024, k=3, V=128256: 339.4 without, 334.5 with, two full rounds).
constexpr int kSeqWideHoldMaxB = 512;
constexpr int kSeqWideLongMinB = 384;
constexpr long long kSeqWideLongMinRowBytes = 160000;
#ifndef SV_HOLD_LONG_512
#define SV_HOLD_LONG_512 12
#endif
constexpr int kSeqWideLongHeldRounds = SV_HOLD_LONG_512;
constexpr int kSeqWideHeldRounds = SV_HOLD_SEQ_512;  // full read with pair 0 last, 512 threads
constexpr int held_rounds_exit(int nt) { return nt >= 1024 ? SV_HOLD_EXIT_1024 : SV_HOLD_EXIT_512; }
constexpr size_t kLdsBytesPerCu = 160 * 1024;
constexpr long long kSampleSeqBaseElems = 40960;
constexpr long long kSampleSeqElemsPerRow = 352;
constexpr int kSampleWideMaxB = 512;
constexpr int kSampleWideMidB = 320;
constexpr long long kSampleWideMaxElems = 98304;

inline bool use_sample_seq(int B, int V, int chunks) {
    if (B >= kSeqWideMinB) {  // kSeqWideThreads-thread groups
        return B <= kSampleWideMaxB &&
               (chunks + kSeqWideThreads - 1) / kSeqWideThreads <= kSampleSeqRounds &&
               (V <= kSampleSeqBaseElems || (B >= kSampleWideMidB && V <= kSampleWideMaxElems));
    }
    return (chunks + kSeqThreads - 1) / kSeqThreads <= kSampleSeqRounds &&
           V <= kSampleSeqBaseElems + kSampleSeqElemsPerRow * B;
}

inline int plan_slices_sample(long long rows, int V) {
    int s = plan_slices(rows, V);
    long long need = (V + (long long)kSampleSliceElems - 1) / kSampleSliceElems;
    long long cap = V / kMinSliceElems;
    if (cap < 1) cap = 1;
    if (need > cap) need = cap;
    if (need > kMaxSlices) need = kMaxSlices;
    return s > need ? s : (int)need;
}

// Inverse-CDF tiles: a row's chunks are cut into at most kMaxTiles tiles of
// whole 256-chunk rounds, plus one tile for its trailing logits.
constexpr int kMaxTiles = 256;
constexpr int kDrawRound = 256;  // chunks per round in the row-split draw

inline int draw_tiles(int nch, int rem) {
    const int rounds = (nch + kDrawRound - 1) / kDrawRound;
    int m = (rounds + kMaxTiles - 1) / kMaxTiles;
    if (m < 1) m = 1;
    return (rounds + m - 1) / m + (rem > 0 ? 1 : 0);
}

// The row-split stochastic draw gives every sequence SD workgroups (never
// more than its tiles): 16 up to 32 sequences, 8 up to 256, 4 beyond.  More
// groups per sequence shorten each group's share of the re-read but add
// groups to the hand-over; measured per call on k=4, V=128256 bf16 batches
// (temporal loads for pair 0 and the bonus row), SD = 16 / 8 / 4:
//   B=4  22.1 / 24.3 / 28.9 us (63 groups: 22.1);  B=16 25.5 / 26.4 / 31.1
//   (63: 35.1);  B=32 29.6 / 29.1 / 33.9 (32: 34.8);  B=64 42.4 / 41.1 / 44.2;
//   at B=128 (k=3) every choice within 0.4 us; in the capped early exit at
//   B=256, k=8: 115.1 / 109.9 / 111.4 us (2 groups: 114.4).  With the slices
//   cut to the groups' tiles (draw_aligned_slice), 16 / 8: B=24 24.6 / 25.2
//   us, B=32 27.5 / 27.9 us, B=48 34.2 / 33.9 us, B=64 41.1 / 39.9 us.
inline int plan_draw_slices(int B, int tiles) {
    int sd = B <= 32 ? 16 : (B <= 256 ? 8 : 4);
    if (sd > tiles) sd = tiles;
    if (sd < 1) sd = 1;
    return sd;
}

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Row-split stochastic calls drawn by the spread draw (B <
// kFinishOneGroupMinB) cut every row into the draw groups' shares of tiles
// when there are a multiple of 8 groups per sequence: slice s of a row is
// then read by statistics workgroup ((b * rows + r) * S + s), and its tiles
// by draw workgroup (b * SD + s), both on XCD s mod 8 (workgroups go to the
// 8 XCDs round robin), so the draw's re-read can find the slice in that
// XCD's L2.  Measured per call, k=4, V=128256 bf16, against slices sized
// for about 2048 items: B=4 19.0 -> 16.5 us, B=8 21.1 -> 18.1 us, B=16
// 24.8 -> 22.2 us, B=32 28.9 -> 28.8 us, B=64 unchanged (40.3 us; its rows
// no longer fit the L2s); B=1, k=4, V=32000 fp32 15.5 -> 15.2 us.  Returns
// the chunks per slice (`per` when the rule does not apply).
inline int draw_aligned_slice(int B, int V, int E, int per) {
    if (B >= kFinishOneGroupMinB) return per;
    const int nch = V / E;
    const int rem = V - nch * E;
    const int rounds = (nch + kDrawRound - 1) / kDrawRound;
    int m = (rounds + kMaxTiles - 1) / kMaxTiles;
    if (m < 1) m = 1;
    const int nt_all = (rounds + m - 1) / m + (rem > 0 ? 1 : 0);
    const int sd = plan_draw_slices(B, draw_tiles(nch, rem));
    if (sd % 8 != 0 || nch == 0) return per;
    const int tps = (nt_all + sd - 1) / sd;
    const int aligned = tps * m * kDrawRound;
    return aligned < (V + E - 1) / E ? aligned : per;
}

// Capped early exit with a spread continuation.  A sequence-resident
// early-exit workgroup streams at most plan_exit_pairs(k) pairs, stopping at
// the first rejection, draws the token of a sequence rejected at position 0
// itself, and leaves the statistics of what it streamed in the row-split
// layout.  The sequences that accepted every streamed pair (the few
// that would otherwise keep one CU streaming long after the rest are done)
// have their remaining rows streamed by a persistent row-split kernel spread
// over the whole GPU; then the row-split draw kernels decide and draw every
// other sequence, each closing-token draw spread over several workgroups.  Used when
// the caller passes a workspace (the plain early exit needs none) and B <=
// kExitMaxB.
constexpr int kExitMaxB = 1024;
// Without diagnostics the capped early exit also runs from kCappedExitMinB
// sequences on (below kSeqResidentMinB, where the full read is row-split).
// It reads less only when sequences reject early, so the gain depends on
// the acceptance rate.  Measured per call, k=8, V=128256 bf16, row-split
// full read / capped exit: B=96 81.4 / 75.2 us, B=128 104.2 / 80.7 us,
// B=160 126.8 / 85.3 us on the peaked batch (mean accepted length 1.2);
// with half the sequences accepting every draft (mean 4-5) B=96 79.5 /
// 91.9, B=128 102.1 / 96.6, B=160 123.9 / 108.6 us; with every draft
// accepted B=96 77.7 / 107.6, B=128 99.5 / 124.2, B=160 120.4 / 140.1 us.
// From 128 sequences on it wins unless nearly every draft is accepted.
constexpr int kCappedExitMinB = 128;
constexpr int kExitStatsGrid = 2048;     // persistent statistics groups (8 per CU)
constexpr long long kExitTargetItems = 2048;
// A sequence that the capped pass sees rejected at a position below this
// draws its token in that pass (its CU is free long before the pass ends).
// Measured with the rejected pair held on chip, B=256, k=8, V=128256 bf16:
// 104.5 us drawing after a rejection at position 0 only, 108.2 after
// positions 0 and 1, 116.6 after any of the three capped pairs.
#ifndef SV_EXIT_DRAW_HERE
constexpr int kExitDrawHere = 1;
#else
constexpr int kExitDrawHere = SV_EXIT_DRAW_HERE;
#endif
constexpr int kExitMaxSlices = 16;
// Pairs of the capped pass; 0: no capping.  Measured on B=256, V=128256
// bf16 batches (peaked target, draft noise sigma 1.5), 3 pairs against the
// plain early exit: k=8 118 against 150 us, k=7 113 against 136 us, k=6 110
// against 122 us (2 pairs: 122, 116, 109 us); at k=4 and k=3 the plain early
// exit is faster (95 against 102 us, 140 against 142 us).
#ifndef SV_EXIT_PAIRS
inline int plan_exit_pairs(int k) { return k >= 6 ? 3 : 0; }
#else
inline int plan_exit_pairs(int) { return SV_EXIT_PAIRS; }
#endif
// Its workspace: an int flag per sequence (0: rejected, drawn by the spread
// draw; 1: accepted every pair of the capped pass; 2: finished by the capped
// pass), then the row-split stochastic layout below.
inline size_t exit_flag_bytes(int B) { return round256((size_t)B * 4); }

// Workspace of the row-split layout: float2 statistics [B][rows_per_seq][S],
// then (stochastic only) tile sums float [B][kMaxTiles + 1], the spread
// draw's arrival counter int [B] and the logit at each row's draft token
// float [B][rows_per_seq].
inline size_t part_bytes(int B, int rows_per_seq, int S) {
    return round256((size_t)B * rows_per_seq * S * 8);
}
inline size_t tilesum_bytes(int B) { return round256((size_t)B * (kMaxTiles + 1) * 4); }
inline size_t cnt_bytes(int B) { return round256((size_t)B * 4); }
inline size_t xl_bytes(int B, int rows_per_seq) { return round256((size_t)B * rows_per_seq * 4); }
inline size_t workspace_bytes_for(int B, int rows_per_seq, int S, bool stochastic) {
    size_t n = part_bytes(B, rows_per_seq, S);
    if (stochastic) n += tilesum_bytes(B) + cnt_bytes(B) + xl_bytes(B, rows_per_seq);
    return n;
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
    float* part;          // row-split only: [B][rows_per_seq][S][2]
    float* tilesum;       // row-split stochastic: [B][kMaxTiles + 1]
    int* cnt;             // row-split stochastic: [B] arrival counters of the draw groups
    float* xl;            // row-split stochastic: [B][rows_per_seq] logit at the row's draft token
    int SD;               // row-split stochastic: draw workgroups per sequence
    int slice_draw;       // row-split plain sampling (dense, k = 0): draw from slice statistics
    const int32_t* parents;  // draft trees: parent of every node [B][N], else null
    int32_t* path;        // draft trees: node indices root .. winner [B][N]
    const int32_t* cu;    // ragged batches: cumulative draft lengths [B+1], else null
    long long total_draft;  // ragged batches: draft rows in the buffers
    long long row_stride; // elements
    int B, G, k, V;       // k: draft tokens per sequence (ragged: the maximum)
    int rows_per_seq;     // stochastic 2k+1, greedy G(k+1)
    int S;                // row-split: slices per row
    int slice_len;        // row-split: elements per slice
    float c;              // log2(e) / temperature
    int* active;          // capped early exit: [B] still-accepting flags, else null
    int exit_pairs;       // capped early exit: pairs streamed by the first pass
};

// Launchers (sv_kernels.hip).  dtype: 0 float32, 1 bfloat16; vec: every row
// starts on a 16-byte boundary; seq_resident: which layout (see above).
// Return a hipError_t value (0 = success).
int launch_stochastic(const Params& p, int dtype, bool vec, bool seq_resident, void* stream);
int launch_greedy(const Params& p, int dtype, bool vec, bool seq_resident, void* stream);
// Greedy draft-tree verification (row-split layout; rows_per_seq = N nodes).
int launch_tree(const Params& p, int dtype, bool vec, void* stream);
// Commit of a verified step (see sv_commit in specverify.h).
int launch_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W,
                  int32_t* seq_len, int32_t* history, long long history_stride, int capacity,
                  int32_t* next_token, long long next_stride, void* stream);

}  // namespace sv
