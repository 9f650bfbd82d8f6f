// sv_kernels.hip -- the verification step on gfx950 (MI355X).
//
// Every logit row is streamed from HBM once with 16-byte loads and reduced
// to a few bytes of statistics:
//   stochastic: a reference R and Z = sum_v 2^(x_v*c - R), c = log2(e)/T,
//               with R raised lazily so no exponential overflows (an online
//               softmax normaliser: p(v) = 2^(x_v*c - R) / Z);
//   greedy:     the row maximum and the lowest index holding it.
// From those, one workgroup per sequence computes p_i(x_i) and q_i(x_i),
// runs the acceptance test and the accept-prefix scan, and draws the
// corrective or bonus token by inverse CDF with block-wide LDS scans (the
// only step that reads logits a second time: one or two rows per sequence).
// Nothing is a dense contraction, so no MFMA is used; the stream is bound by
// HBM bandwidth, with VALU/exp issue close behind for bfloat16 stochastic rows.
//
// Two layouts (see sv_internal.h): sequence-resident (one workgroup streams a
// whole sequence; nothing crosses workgroups) and row-split (a statistics
// kernel over (row, slice) items, then a finishing kernel per sequence).
//
// The method (Perplexity, "Accelerating Sonar through speculation", sections
// "Špekulatívne dekódovanie" and "Cieľ-Návrh"): compare complete target and
// draft distributions, keep the longest accepted prefix, sample the closing
// token from the target side.  The exact rule is the lossless one (accept
// when u*q < p, residual max(0, p-q)), as stated in include/specverify.h.
#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {

constexpr int NT_SEQ = kSeqThreads;  // sequence-resident workgroup: 16 wave64s
// More sequences than CUs (B >= kSeqWideMinB): 512-thread workgroups, two or
// more resident per CU (B=512, k=3: 174 against 181 us; at B=256 the
// 1024-thread groups win).
constexpr int NT_SEQ_WIDE = kSeqWideThreads;
constexpr int NT_ROW = 256;    // row-split statistics workgroup: 4 wave64s
constexpr int NT_ROW_WIDE = 512;  // ... 8 wave64s, for slices of kRowStatsWideChunks chunks or more
constexpr int NT_FIN = 1024;   // row-split finishing workgroup
constexpr int UNROLL = 4;      // 16-byte loads in flight per lane while streaming
constexpr int TUNROLL = 4;     // chunk pairs in flight per lane while sampling
constexpr int MAX_TILES = kMaxTiles; // inverse-CDF tiles held in LDS
constexpr int MAX_ROWS_STOCH = 2 * kMaxK + 1;
constexpr int MAX_ROWS_GREEDY_SEQ = kMaxK + 1;
// How far (log2 units) a new maximum may exceed the streaming reference
// before the running sum is rescaled; terms then stay below 2^16.
constexpr float RESCALE_MARGIN = 16.0f;
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-class parts.
constexpr int RSRC_WORD3 = 0x00020000;
// Cache policy of the logit loads: non-temporal.  Every logit is used once
// (the sampling re-read aside), and streaming them with the non-temporal
// hint measured about 13% faster on the B=256, k=8, V=128256 bf16 workload.
constexpr int LOAD_POLICY_NT = 2;
// The full-read kernel streams the pairs of the lowest positions last and
// with ordinary loads, so that the rows a rejection most often lands on are
// the likeliest to be cached when the closing-token draw reads them again
// (measured: a small gain at B=512, none at B=256, where the re-read comes
// from HBM whichever pair it is).
constexpr int KEEP_PAIRS = 1;
// The position-order kernel reads the pairs of positions below this with
// ordinary loads: if such a pair is rejected, what is not held on chip is
// read again right away and part of it is then still cached, while long
// accepted runs keep the non-temporal stream.  Measured per call (B=256,
// k=8, V=128256 bf16; 0 / 1 / 2 / 3 / every position): capped early exit
// 104.9 / 104.2 / 100.8 / 101.1 / 101.4 us; full read 175.1 / 173.9 / 174.5
// / 174.7 / 172.8; full read with every draft accepted 182.8 / 182.6 /
// 181.6 / 186.1 / 197.5; B=512, k=3, V=129280 plain early exit 134.0 /
// 128.9 / 130.7 / 131.1 / 131.0.
constexpr int EXIT_KEEP_PAIRS = 2;
// The same for 512-thread groups (two per CU) that hold the pair on chip,
// where the pair of position 1 kept cached costs more than it saves: full
// read, B=512, k=3, V=129280 bf16, 1 / 2 pairs: 160.0 / 160.5 us (with
// every draft accepted 169.8 / 178.1, measured while the bonus draw still
// took two exponentials per logit); early exit 125.0 / 126.6, with every
// draft accepted (V=128256) 156.9 / 169.8.
constexpr int EXIT_KEEP_PAIRS_WIDE_HELD = 1;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT>
constexpr int elem_bytes() { return DT == 1 ? 2 : 4; }

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int v) {
    if (DT == 1) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[v] << 16);
    return reinterpret_cast<const float*>(row)[v];
}

// ------------------------------------------------------------------------
// Chunks: E consecutive logits.  VEC: 16 bytes (8 bf16 or 4 f32), else one.
template <int DT, bool VEC>
struct Chunk;

template <>
struct Chunk<1, true> {
    static constexpr int E = 8;
    uint32_t w[4];
    __device__ __forceinline__ float get(int j) const {
        const uint32_t x = w[j >> 1];
        return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    }
    __device__ __forceinline__ void set_neg_inf() {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = 0xff80ff80u;
    }
};

template <>
struct Chunk<0, true> {
    static constexpr int E = 4;
    uint32_t w[4];
    __device__ __forceinline__ float get(int j) const { return __uint_as_float(w[j]); }
    __device__ __forceinline__ void set_neg_inf() {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = 0xff800000u;
    }
};

template <int DT>
struct Chunk1 {
    static constexpr int E = 1;
    uint32_t w[1];
    __device__ __forceinline__ float get(int) const { return __uint_as_float(w[0]); }
    __device__ __forceinline__ void set_neg_inf() { w[0] = 0xff800000u; }
};
template <>
struct Chunk<1, false> : Chunk1<1> {};
template <>
struct Chunk<0, false> : Chunk1<0> {};

// n logits at `base` (a row or a slice of one).  VEC rows start on a
// 16-byte boundary and are read through a buffer resource that covers
// exactly their whole chunks, so an index can never leave the row; the
// n % E trailing logits are read one by one.  chunk_at(i, s) is chunk i + s
// with s uniform across the wave (folded into the scalar offset).
template <int DT, bool VEC>
struct Row;

template <int DT>
struct Row<DT, true> {
    using C = Chunk<DT, true>;
    static constexpr int E = C::E;
    __amdgpu_buffer_rsrc_t rs;
    const char* base;
    int n, nch;
    Row() = default;
    __device__ __forceinline__ Row(const char* p, int n_) : base(p), n(n_), nch(n_ / E) {
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, nch * 16,
                                               RSRC_WORD3);
    }
    // KEEP: an ordinary (temporal) load, for rows that will be read again soon.
    template <bool KEEP = false>
    __device__ __forceinline__ C chunk_at(int i, int s) const {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, s * 16,
                                                             KEEP ? 0 : LOAD_POLICY_NT);
        C c;
        c.w[0] = v[0];
        c.w[1] = v[1];
        c.w[2] = v[2];
        c.w[3] = v[3];
        return c;
    }
    __device__ __forceinline__ C chunk(int i) const { return chunk_at(i, 0); }
    __device__ __forceinline__ float elem(int v) const { return load_elem<DT>(base, v); }
};

template <int DT>
struct Row<DT, false> {
    using C = Chunk<DT, false>;
    static constexpr int E = 1;
    const char* base;
    int n, nch;
    Row() = default;
    __device__ __forceinline__ Row(const char* p, int n_) : base(p), n(n_), nch(n_) {}
    template <bool KEEP = false>
    __device__ __forceinline__ C chunk_at(int i, int s) const {
        C c;
        c.w[0] = __float_as_uint(load_elem<DT>(base, i + s));
        return c;
    }
    __device__ __forceinline__ C chunk(int i) const { return chunk_at(i, 0); }
    __device__ __forceinline__ float elem(int v) const { return load_elem<DT>(base, v); }
};

// ------------------------------------------------------------------------
// Wave64 and block reductions.  The wave-level steps move data between
// lanes with DPP (row shifts, mirrors and row broadcasts, GFX9-family
// controls): plain VALU operations, where a shuffle (ds_bpermute) takes an
// LDS round trip per step.  Reductions end in lane 63 and are broadcast
// from it, so every lane gets the same value.
constexpr int DPP_QUAD_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHR1 = 0x111;       // row_shr:n = 0x110 + n
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;    // lane 15 of a row to the next row
constexpr int DPP_ROW_BCAST31 = 0x143;    // lane 31 to rows 2 and 3
constexpr int DPP_WAVE_SHR1 = 0x138;      // the whole wave shifted by one lane

// src from the lane CTRL names; lanes outside ROWM, or whose source lane
// does not exist, get `old`.
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ int dpp_i(int old, int src) {
    return __builtin_amdgcn_update_dpp(old, src, CTRL, ROWM, 0xF, false);
}
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ float dpp_f(float old, float src) {
    return __int_as_float(dpp_i<CTRL, ROWM>(__float_as_int(old), __float_as_int(src)));
}
__device__ __forceinline__ float lane63_f(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Reduction over the wave with op (sum, max, min): within quads, then
// 8- and 16-lane rows, then the rows into lane 63.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
    if constexpr (sizeof(T) == 4 && T(0.5) != T(0)) {  // float
        v = op(v, dpp_f<DPP_QUAD_XOR1>(v, v));
        v = op(v, dpp_f<DPP_QUAD_XOR2>(v, v));
        v = op(v, dpp_f<DPP_ROW_HALF_MIRROR>(v, v));
        v = op(v, dpp_f<DPP_ROW_MIRROR>(v, v));
        v = op(v, dpp_f<DPP_ROW_BCAST15, 0xA>(v, v));
        v = op(v, dpp_f<DPP_ROW_BCAST31, 0xC>(v, v));
        return lane63_f(v);
    } else {
        v = op(v, dpp_i<DPP_QUAD_XOR1>(v, v));
        v = op(v, dpp_i<DPP_QUAD_XOR2>(v, v));
        v = op(v, dpp_i<DPP_ROW_HALF_MIRROR>(v, v));
        v = op(v, dpp_i<DPP_ROW_MIRROR>(v, v));
        v = op(v, dpp_i<DPP_ROW_BCAST15, 0xA>(v, v));
        v = op(v, dpp_i<DPP_ROW_BCAST31, 0xC>(v, v));
        return __builtin_amdgcn_readlane(v, 63);
    }
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ int wave_min_i(int v) {
    return wave_reduce(v, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_max_i(int v) {
    return wave_reduce(v, [](int a, int b) { return max(a, b); });
}
// Inclusive prefix sum over the wave: shifts by 1, 2, 4, 8 within each row
// of 16 lanes, then each row adds the totals of the rows before it.
__device__ __forceinline__ float wave_incl_scan(float v) {
    v += dpp_f<DPP_ROW_SHR1>(0.0f, v);
    v += dpp_f<DPP_ROW_SHR1 + 1>(0.0f, v);
    v += dpp_f<DPP_ROW_SHR1 + 3>(0.0f, v);
    v += dpp_f<DPP_ROW_SHR1 + 7>(0.0f, v);
    v += dpp_f<DPP_ROW_BCAST15, 0xA>(0.0f, v);
    v += dpp_f<DPP_ROW_BCAST31, 0xC>(0.0f, v);
    return v;
}
// The value of the lane below (0 in lane 0).
__device__ __forceinline__ float wave_shift_up1(float v) { return dpp_f<DPP_WAVE_SHR1>(0.0f, v); }
// Larger value wins; equal values go to the lower index.
__device__ __forceinline__ bool argmax_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}
__device__ __forceinline__ void wave_argmax(float& best, int& idx) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o);
        const int oi = __shfl_xor(idx, o);
        if (argmax_better(ob, oi, best, idx)) {
            best = ob;
            idx = oi;
        }
    }
}

template <int NT>
struct Scratch {
    static constexpr int NW = NT / 64;
    float f[NW];
    float g[NW];
    int i[NW];
    int j[NW];
};

// Block-wide operations.  All threads call.  Each publishes per-wave values
// in its own array of sc (f, i or j) behind a barrier; TRAIL adds a second
// barrier after the reads, so that the same array can be written again
// right away.  Without it the caller must order the next write of that
// array after a barrier of its own (as a different operation's first
// barrier does).
//
// Exclusive prefix sum; *total gets the block sum.
template <int NT, bool TRAIL = true>
__device__ __forceinline__ float block_excl_scan(float v, float* total, Scratch<NT>& sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float incl = wave_incl_scan(v);
    const float excl = wave_shift_up1(incl);
    if (lane == 63) sc.f[wave] = incl;
    __syncthreads();
    float off = 0.0f, tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) off += sc.f[w];
        tot += sc.f[w];
    }
    if (TRAIL) __syncthreads();
    *total = tot;
    return off + excl;
}

template <int NT, bool TRAIL = true>
__device__ __forceinline__ int block_min_i(int v, Scratch<NT>& sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_min_i(v);
    if (lane == 0) sc.i[wave] = v;
    __syncthreads();
    int r = sc.i[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = min(r, sc.i[w]);
    if (TRAIL) __syncthreads();
    return r;
}

template <int NT, bool TRAIL = true>
__device__ __forceinline__ int block_max_i(int v, Scratch<NT>& sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_i(v);
    if (lane == 0) sc.j[wave] = v;
    __syncthreads();
    int r = sc.j[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = max(r, sc.j[w]);
    if (TRAIL) __syncthreads();
    return r;
}

// ------------------------------------------------------------------------
// A thread's chunk of rounds 0..N-1 of a row, kept in registers: one member
// per round (no array, which a run-time pick would turn into a scratch
// buffer), set and picked through compile-time indices.  round() also takes
// a run-time round (uniform over the block): it selects among the values of
// every held round without branches, since branches that each read another
// member merge into a read through a pointer picked at run time, which
// keeps the whole object in scratch memory.
template <typename C, int N>
struct HeldRounds : HeldRounds<C, N - 1> {
    static constexpr bool kHeld = true;
    static constexpr int kRounds = N;
    C last;
    template <int J>
    __device__ __forceinline__ C& at() {
        if constexpr (J == N - 1) return last;
        else return HeldRounds<C, N - 1>::template at<J>();
    }
    __device__ __forceinline__ C round(int rd) const {
        C v = HeldRounds<C, N - 1>::round(rd);
        const bool hit = rd == N - 1;
#pragma unroll
        for (int w = 0; w < (int)(sizeof(v.w) / sizeof(v.w[0])); ++w) v.w[w] = hit ? last.w[w] : v.w[w];
        return v;
    }
    template <int NT, typename R>
    __device__ __forceinline__ C tchunk(const R& tr, int rd) const {
        return rd < N ? round(rd) : tr.chunk_at(threadIdx.x, rd * NT);
    }
    template <int NT, typename R>
    __device__ __forceinline__ C dchunk(const R& dr, int rd) const {
        return dr.chunk_at(threadIdx.x, rd * NT);
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const { return dr.elem(v); }
};
template <typename C>
struct HeldRounds<C, 1> {
    static constexpr bool kHeld = true;
    static constexpr int kRounds = 1;
    C last;
    template <int J>
    __device__ __forceinline__ C& at() { return last; }
    __device__ __forceinline__ C round(int) const { return last; }
    template <int NT, typename R>
    __device__ __forceinline__ C tchunk(const R& tr, int rd) const {
        return rd < 1 ? last : tr.chunk_at(threadIdx.x, rd * NT);
    }
    template <int NT, typename R>
    __device__ __forceinline__ C dchunk(const R& dr, int rd) const {
        return dr.chunk_at(threadIdx.x, rd * NT);
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const { return dr.elem(v); }
};

// No round held: everything is read again.
template <typename C>
struct HeldRounds<C, 0> {
    static constexpr bool kHeld = true;
    static constexpr int kRounds = 0;
    __device__ __forceinline__ C round(int) const { return C{}; }
    template <int NT, typename R>
    __device__ __forceinline__ C tchunk(const R& tr, int rd) const {
        return tr.chunk_at(threadIdx.x, rd * NT);
    }
    template <int NT, typename R>
    __device__ __forceinline__ C dchunk(const R& dr, int rd) const {
        return dr.chunk_at(threadIdx.x, rd * NT);
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const { return dr.elem(v); }
};

// held.at<J>() = buf[J - base] for the rounds J < N in [base, base + U)
// (base is a compile-time constant once the caller's loop is unrolled).
template <int J, int N, int U, typename H, typename C>
__device__ __forceinline__ void store_held(H& held, int base, const C* buf) {
    if constexpr (J < N) {
        if (J >= base && J < base + U) held.template at<J>() = buf[J - base];
        store_held<J + 1, N, U>(held, base, buf);
    }
}

// ------------------------------------------------------------------------
// Streaming reductions of one row, per thread.  Thread t visits chunks
// t, t+NT, t+2NT, ... in increasing order, UNROLL loads in flight.

// Softmax normaliser of one thread: sum (s0 + s1) of 2^(x*c - ref).
struct SoftAcc {
    float ref = -FLT_MAX, s0 = 0.0f, s1 = 0.0f;
};

__device__ __forceinline__ void soft_rescale(SoftAcc& a, float newref) {
    const float f = fast_exp2(a.ref - newref);
    a.s0 *= f;
    a.s1 *= f;
    a.ref = newref;
}

// The terms of one step against the reference `ref`, split over two sums.
template <typename C>
__device__ __forceinline__ void soft_terms(const C* buf, float c, float ref, float& s0, float& s1) {
    constexpr int E = C::E;
    const float nref = -ref;
    s0 = fast_exp2(fmaf(buf[0].get(0), c, nref));
    s1 = E > 1 ? fast_exp2(fmaf(buf[0].get(E > 1 ? 1 : 0), c, nref)) : 0.0f;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (u == 0 && e < 2) continue;
            const float t = fast_exp2(fmaf(buf[u].get(e), c, nref));
            if (e & 1) s1 += t;
            else s0 += t;
        }
}

// Add one step of loaded chunks to a thread's normaliser.  The terms are
// taken against the current reference without first looking for a new
// maximum: a logit far above the reference shows up as a step sum of at
// least SUM_GUARD (or inf), and only then is the step redone after raising
// the reference to the step's maximum.  So every term stays below 2^64 (the
// sums far inside float range), and the common path spends no instruction
// on the maximum.  The first step of a thread always takes the slow path
// (its reference starts at -FLT_MAX, so any finite logit overflows).
constexpr float SUM_GUARD = 0x1p64f;

template <typename C>
__device__ __forceinline__ float step_max(const C* buf) {
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
        for (int e = 0; e < C::E; ++e) gm = fmaxf(gm, buf[u].get(e));
    return gm;
}

template <typename C>
__device__ __forceinline__ void soft_consume(const C* buf, float c, SoftAcc& a) {
    float s0, s1;
    soft_terms(buf, c, a.ref, s0, s1);
    if (!(s0 + s1 < SUM_GUARD)) {
        const float gmc = step_max(buf) * c;
        if (gmc > a.ref) soft_rescale(a, gmc);
        soft_terms(buf, c, a.ref, s0, s1);
    }
    a.s0 += s0;
    a.s1 += s1;
}

// A row's first step: the reference is still -FLT_MAX, so it starts at the
// step's maximum directly (the guard would always trip here).
template <typename C>
__device__ __forceinline__ void soft_consume_first(const C* buf, float c, SoftAcc& a) {
    const float gmc = step_max(buf) * c;
    if (gmc > a.ref) soft_rescale(a, gmc);
    float s0, s1;
    soft_terms(buf, c, a.ref, s0, s1);
    a.s0 += s0;
    a.s1 += s1;
}

// Step i0 of a row (chunks i0 + tid + u*NT): whole steps load without
// checks, the row's last step masks chunks past its end with -inf.
template <int DT, bool VEC, int NT, bool KEEP>
__device__ __forceinline__ void load_step(const Row<DT, VEC>& row, int i0, Chunk<DT, VEC>* buf) {
    constexpr int STEP = NT * UNROLL;
    const int i = i0 + threadIdx.x;
    if (i0 + STEP <= row.nch) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) buf[u] = row.template chunk_at<KEEP>(i, u * NT);
    } else {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (i + u * NT < row.nch) buf[u] = row.template chunk_at<KEEP>(i, u * NT);
            else buf[u].set_neg_inf();
        }
    }
}

// The row's last n % E logits (vector rows), one per thread.
template <int DT, bool VEC>
__device__ __forceinline__ void soft_trailing(const Row<DT, VEC>& row, float c, SoftAcc& a) {
    if (VEC) {
        constexpr int E = Chunk<DT, VEC>::E;
        const int rem = row.n - row.nch * E;
        if ((int)threadIdx.x < rem) {
            const float x = row.elem(row.nch * E + threadIdx.x);
            if (x * c > a.ref + RESCALE_MARGIN) soft_rescale(a, x * c);
            a.s0 += fast_exp2(fmaf(x, c, -a.ref));
        }
    }
}

template <int DT, bool VEC, int NT, bool KEEP = false>
__device__ __forceinline__ void stream_softmax(const Row<DT, VEC>& row, float c, SoftAcc& a) {
    using C = Chunk<DT, VEC>;
    constexpr int STEP = NT * UNROLL;
    const int nch = row.nch;
    for (int i0 = 0; i0 < nch; i0 += STEP) {
        C buf[UNROLL];
        load_step<DT, VEC, NT, KEEP>(row, i0, buf);
        if (i0 == 0) soft_consume_first(buf, c, a);
        else soft_consume(buf, c, a);
    }
    soft_trailing(row, c, a);
}

// stream_softmax that also keeps this thread's chunk of rounds 0..N-1 in
// registers (held.at<J>(); chunks past the row's end hold -inf): the first
// N / UNROLL steps are unrolled so that every round has its own register.
// Every held round is written, so nothing held before stays live.
template <int DT, bool VEC, int NT, bool KEEP, int N>
__device__ __forceinline__ void stream_softmax_hold(const Row<DT, VEC>& row, float c, SoftAcc& a,
                                                    HeldRounds<Chunk<DT, VEC>, N>& held) {
    using C = Chunk<DT, VEC>;
    static_assert(N % UNROLL == 0, "whole steps");
    constexpr int STEP = NT * UNROLL;
    const int nch = row.nch;
#pragma unroll
    for (int q = 0; q < N / UNROLL; ++q) {
        C buf[UNROLL];
        if (q * STEP < nch) {  // uniform
            load_step<DT, VEC, NT, KEEP>(row, q * STEP, buf);
            if (q == 0) soft_consume_first(buf, c, a);
            else soft_consume(buf, c, a);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) buf[u].set_neg_inf();
        }
        store_held<0, N, UNROLL>(held, q * UNROLL, buf);
    }
    for (int i0 = N * NT; i0 < nch; i0 += STEP) {
        C buf[UNROLL];
        load_step<DT, VEC, NT, KEEP>(row, i0, buf);
        soft_consume(buf, c, a);
    }
    soft_trailing(row, c, a);
}

// stream_softmax that also stores this thread's chunk of rounds 0..lr-1 in
// LDS (stash[rd * NT + tid]; chunks past the row's end hold -inf).
template <int DT, bool VEC, int NT, bool KEEP = false>
__device__ __forceinline__ void stream_softmax_stash(const Row<DT, VEC>& row, float c, SoftAcc& a,
                                                     Chunk<DT, VEC>* stash, int lr) {
    using C = Chunk<DT, VEC>;
    constexpr int STEP = NT * UNROLL;
    const int nch = row.nch;
    for (int i0 = 0; i0 < nch; i0 += STEP) {
        C buf[UNROLL];
        load_step<DT, VEC, NT, KEEP>(row, i0, buf);
        if (i0 == 0) soft_consume_first(buf, c, a);
        else soft_consume(buf, c, a);
        const int r0 = i0 / NT;
        if (r0 < lr) {  // uniform
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (r0 + u < lr) stash[(r0 + u) * NT + threadIdx.x] = buf[u];
        }
    }
    soft_trailing(row, c, a);
}

// Merge a wave's softmax normalisers into (R, Z) (valid in every lane).
__device__ __forceinline__ void wave_softmax(const SoftAcc& a, float& R, float& Z) {
    R = wave_max(a.ref);
    Z = wave_sum((a.s0 + a.s1) * fast_exp2(a.ref - R));
}

// Argmax of one thread: best value and the element index where a chunk
// holding it starts (or of a single trailing element).
struct ArgAcc {
    float best = -INFINITY;
    int pos = INT_MAX;
};

template <int DT, bool VEC, int NT>
__device__ __forceinline__ void stream_argmax(const Row<DT, VEC>& row, ArgAcc& a) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    constexpr int STEP = NT * UNROLL;
    const int tid = threadIdx.x;
    const int nch = row.nch;
    const int rem = VEC ? row.n - nch * E : 0;
    // An all -inf row still has an argmax: the thread's first element.
    a.pos = tid < nch ? tid * E : (tid < rem ? nch * E + tid : INT_MAX);
    for (int i0 = 0; i0 < nch; i0 += STEP) {
        const int i = i0 + tid;
        C buf[UNROLL];
        if (i0 + STEP <= nch) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) buf[u] = row.chunk_at(i, u * NT);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (i + u * NT < nch) buf[u] = row.chunk_at(i, u * NT);
                else buf[u].set_neg_inf();
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float m = buf[u].get(0);
#pragma unroll
            for (int e = 1; e < E; ++e) m = fmaxf(m, buf[u].get(e));
            if (m > a.best) {
                a.best = m;
                a.pos = (i + u * NT) * E;
            }
        }
    }
    if (VEC && tid < rem) {
        const float x = row.elem(nch * E + tid);
        if (x > a.best) {
            a.best = x;
            a.pos = nch * E + tid;
        }
    }
}

// Lowest index holding `best`, given the lowest chunk (start `pos`) that
// holds it.
template <int DT, bool VEC>
__device__ __forceinline__ int argmax_refine(const Row<DT, VEC>& row, float best, int pos) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    if (pos >= row.nch * E) return pos == INT_MAX ? 0 : pos;
    const C ch = row.chunk(pos / E);
    int idx = pos;
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
        if (ch.get(e) == best) idx = pos + e;
    return idx;
}

// ------------------------------------------------------------------------
// Inverse-CDF draw over one row (or a row pair) with weights W(t[, d]):
// the first index whose cumulative weight exceeds r * total; if rounding
// leaves none, the last index with positive weight (0 if there is none).
//
// The row's whole chunks are cut into tiles of NT*m chunks (m block-wide
// rounds of NT chunks, at most MAX_TILES tiles); the n % E trailing logits
// form one more tile.  Pass A sums every tile into LDS, one slot per wave
// (tile_part[tile * NW + wave]); a block scan over tile sums then finds the
// tile holding r * total and pass B scans inside that tile.

struct TileGeom {
    int nch, rem, rounds, m, ntiles, nt_all;
};

template <int NT>
__device__ __forceinline__ TileGeom tile_geom(int nch, int rem) {
    TileGeom g;
    g.nch = nch;
    g.rem = rem;
    g.rounds = (nch + NT - 1) / NT;
    g.m = max(1, (g.rounds + MAX_TILES - 1) / MAX_TILES);
    g.ntiles = (g.rounds + g.m - 1) / g.m;
    g.nt_all = g.ntiles + (rem > 0 ? 1 : 0);
    return g;
}

// Residual weight max(0, p - q) of one row pair, with each normaliser
// folded into its exponent: p = 2^(t*c - R_t - log2 Z_t).
struct ResidualW {
    float c, nt, nd;  // nt = -(R_t + log2 Z_t), nd likewise for the draft row
    // p, q in [0, 1], so p - q clamped to [0, 1] is max(0, p - q): one
    // subtraction with the output clamp instead of a subtraction and a max
    __device__ __forceinline__ float operator()(float t, float d) const {
        return __builtin_amdgcn_fmed3f(fast_exp2(fmaf(t, c, nt)) - fast_exp2(fmaf(d, c, nd)),
                                       0.0f, 1.0f);
    }
};
// Either weight, chosen at run time (uniform), so that one copy of the held
// draw serves both the residual and the bonus token (each copy of a draw
// over held registers costs registers of its own): pair, max(0, p - q) as
// ResidualW; otherwise 2^(t*c + nt), as TargetW with nt = -R (the draft
// side then reads as -inf and is never loaded).  Each gives exactly the
// value of the weight it stands for.
struct DrawW {
    float c, nt, nd;
    bool pair;
    __device__ __forceinline__ float operator()(float t, float d) const {
        const float pt = fast_exp2(fmaf(t, c, nt));
        return pair ? __builtin_amdgcn_fmed3f(pt - fast_exp2(fmaf(d, c, nd)), 0.0f, 1.0f) : pt;
    }
};
// Unnormalised target weight 2^(t*c - R).
struct TargetW {
    float c, nR;
    __device__ __forceinline__ float operator()(float t, float) const {
        return fast_exp2(fmaf(t, c, nR));
    }
};

template <bool PAIR, typename C, typename Wt>
__device__ __forceinline__ float chunk_weight_sum(const Wt& wf, const C& t, const C& d) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < C::E; ++e) acc += PAIR ? wf(t.get(e), d.get(e)) : wf(t.get(e), 0.0f);
    return acc;
}
// DrawW's mode is the same for the whole block: one branch per chunk, so
// the bonus draw takes one exponential per logit, not the residual's two
// (same terms, same order as the generic sum).
template <bool PAIR, typename C>
__device__ __forceinline__ float chunk_weight_sum(const DrawW& wf, const C& t, const C& d) {
    float acc = 0.0f;
    if (PAIR && wf.pair) {
#pragma unroll
        for (int e = 0; e < C::E; ++e)
            acc += __builtin_amdgcn_fmed3f(fast_exp2(fmaf(t.get(e), wf.c, wf.nt)) -
                                               fast_exp2(fmaf(d.get(e), wf.c, wf.nd)),
                                           0.0f, 1.0f);
    } else {
#pragma unroll
        for (int e = 0; e < C::E; ++e) acc += fast_exp2(fmaf(t.get(e), wf.c, wf.nt));
    }
    return acc;
}

// Where the draw finds a round's chunks (round rd, chunk ci = rd * NT + tid
// of this thread) and the trailing logits (element v): read from the rows
// again (the default), or kept on chip by the kernel that streamed them
// (HeldRounds, PairHold).
struct ReadAgain {
    static constexpr bool kHeld = false;
    template <int NT, typename R>
    __device__ __forceinline__ auto tchunk(const R& tr, int rd) const {
        return tr.chunk_at(threadIdx.x, rd * NT);
    }
    template <int NT, typename R>
    __device__ __forceinline__ auto dchunk(const R& dr, int rd) const {
        return dr.chunk_at(threadIdx.x, rd * NT);
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const { return dr.elem(v); }
};
// Read again, with the draft side switched off at run time (every draft
// logit -inf, nothing loaded), for draws with a DrawW weight.
struct ReadPair {
    static constexpr bool kHeld = false;
    bool dlive = true;
    template <int NT, typename R>
    __device__ __forceinline__ auto tchunk(const R& tr, int rd) const {
        return tr.chunk_at(threadIdx.x, rd * NT);
    }
    template <int NT, typename R>
    __device__ __forceinline__ auto dchunk(const R& dr, int rd) const {
        decltype(dr.chunk(0)) c;
        if (dlive) c = dr.chunk_at(threadIdx.x, rd * NT);
        else c.set_neg_inf();
        return c;
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const {
        return dlive ? dr.elem(v) : -INFINITY;
    }
};

// Pass A over the block-wide rounds [r_begin, r_end) (no barriers;
// tile_part pre-zeroed; tile t is stored at slot (t - tile_base) * NW).
template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename Held = ReadAgain>
__device__ __forceinline__ void cdf_pass_a_rounds(const Row<DT, VEC>& tr, const Row<DT, VEC>& dr,
                                                  const Wt& wf, const TileGeom& g, int r_begin,
                                                  int r_end, int tile_base, float* tile_part,
                                                  const Held& held = Held{}) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int r0 = r_begin; r0 < r_end; r0 += TUNROLL) {
        C tb[TUNROLL], db[TUNROLL];
#pragma unroll
        for (int u = 0; u < TUNROLL; ++u) {
            const int ci = (r0 + u) * NT + tid;
            if (ci < g.nch) {
                tb[u] = held.template tchunk<NT>(tr, r0 + u);
                if (PAIR) db[u] = held.template dchunk<NT>(dr, r0 + u);
            } else {
                tb[u].set_neg_inf();
                if (PAIR) db[u].set_neg_inf();
            }
        }
#pragma unroll
        for (int u = 0; u < TUNROLL; ++u) {
            const int round = r0 + u;
            if (round < r_end) {  // uniform across the block
                const float acc = wave_sum(chunk_weight_sum<PAIR>(wf, tb[u], db[u]));
                if (lane == 0) tile_part[(round / g.m - tile_base) * NW + wave] += acc;
            }
        }
    }
}

// Pass A over a whole row (pair), last round first: a workgroup that has
// just streamed the row finds its tail, read last, still in L2, and reaches
// it before the rest of the pass evicts it (measured per call: B=512, k=3,
// V=129280 bf16 full read 173.7 -> 171.8 us; B=256, k=8: 187.5 -> 187.1 us;
// the capped early exit 110.3 -> 109.5 us).  Each tile is one round here
// unless a row has more than MAX_TILES rounds; the tile sums are the same
// sums either way, in a different order only for such rows.
template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename Held = ReadAgain>
__device__ __forceinline__ void cdf_pass_a_block(const Row<DT, VEC>& tr, const Row<DT, VEC>& dr,
                                                 const Wt& wf, const TileGeom& g,
                                                 float* tile_part, const Held& held = Held{}) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int top = g.rounds; top > 0; top -= TUNROLL) {
        const int r0 = top - TUNROLL;  // rounds r0 .. top-1; those below 0 are skipped
        C tb[TUNROLL], db[TUNROLL];
#pragma unroll
        for (int u = 0; u < TUNROLL; ++u) {
            const int round = r0 + u;
            const int ci = round * NT + tid;
            if (round >= 0 && ci < g.nch) {
                tb[u] = held.template tchunk<NT>(tr, round);
                if (PAIR) db[u] = held.template dchunk<NT>(dr, round);
            } else {
                tb[u].set_neg_inf();
                if (PAIR) db[u].set_neg_inf();
            }
        }
#pragma unroll
        for (int u = TUNROLL - 1; u >= 0; --u) {
            const int round = r0 + u;
            if (round >= 0) {  // uniform across the block
                const float acc = wave_sum(chunk_weight_sum<PAIR>(wf, tb[u], db[u]));
                if (lane == 0) tile_part[(round / g.m) * NW + wave] += acc;
            }
        }
    }
}

// The trailing-logits tile (no barriers; tile_part pre-zeroed).
template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename Held = ReadAgain>
__device__ __forceinline__ void cdf_trailing(const Row<DT, VEC>& tr, const Row<DT, VEC>& dr,
                                             const Wt& wf, const TileGeom& g, float* tile_part,
                                             int tile_base = 0, const Held& held = Held{}) {
    constexpr int NW = NT / 64;
    constexpr int E = Chunk<DT, VEC>::E;
    if (g.rem == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float w = 0.0f;
    if (tid < g.rem) {
        const float tv = held.telem(tr, g.nch * E + tid);
        const float dv = PAIR ? held.delem(dr, g.nch * E + tid) : 0.0f;
        w = wf(tv, dv);
    }
    w = wave_sum(w);
    if (lane == 0) tile_part[(g.ntiles - tile_base) * NW + wave] += w;
}

// The row pair a sequence-resident kernel streamed last, kept on chip for
// the closing-token draw (whose residual weights need both rows again once
// their normalisers are known): this thread's chunks of target rounds
// 0..N-1 in registers, and draft rounds 0..lr-1 in LDS (the chunk of round
// rd for thread tid at stash[rd * NT + tid]).  Later rounds are read again.
// dlive false: the draft side is switched off (as in ReadPair).
template <typename C, int N, int NT>
struct PairHold {
    static constexpr bool kHeld = true;
    static constexpr int kRounds = N;
    HeldRounds<C, N> t;
    C* stash;
    int lr;
    bool dlive;
    template <int, typename R>  // the block size is NT
    __device__ __forceinline__ C tchunk(const R& tr, int rd) const {
        return t.template tchunk<NT>(tr, rd);
    }
    template <int, typename R>
    __device__ __forceinline__ C dchunk(const R& dr, int rd) const {
        C c;
        if (!dlive) c.set_neg_inf();
        else if (rd < lr) c = stash[rd * NT + threadIdx.x];
        else c = dr.chunk_at(threadIdx.x, rd * NT);
        return c;
    }
    template <typename R>
    __device__ __forceinline__ float telem(const R& tr, int v) const { return tr.elem(v); }
    template <typename R>
    __device__ __forceinline__ float delem(const R& dr, int v) const {
        return dlive ? dr.elem(v) : -INFINITY;
    }
};
// The memory side of a held row (pair): what is not held is read again.
template <typename C, int N, int NT>
__device__ __forceinline__ ReadPair read_again_of(const PairHold<C, N, NT>& h) {
    ReadPair r;
    r.dlive = h.dlive;
    return r;
}
template <typename C, int N>
__device__ __forceinline__ ReadAgain read_again_of(const HeldRounds<C, N>&) { return ReadAgain{}; }

// Scan over tile sums, then pass B.  tile_part must be complete (after a
// barrier).  *total_out gets the total weight.  All threads call.

template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename Held = ReadAgain>
__device__ __forceinline__ int cdf_select(const Row<DT, VEC>& tr, const Row<DT, VEC>& dr, const Wt& wf, float r,
                          const TileGeom& g, float* total_out, const float* tile_part,
                          float* tile_excl, Scratch<NT>& sc, const Held& held = Held{}) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    const int nch = g.nch, rem = g.rem;
    // Block scan over tiles (each thread owns a contiguous run of tiles).
    const int tpt = (g.nt_all + NT - 1) / NT;  // tiles per thread, <= 2
    float mine[2] = {0.0f, 0.0f};
    float run = 0.0f;
    for (int j = 0; j < tpt; ++j) {
        const int t = tid * tpt + j;
        float s = 0.0f;
        if (t < g.nt_all) {
#pragma unroll
            for (int w = 0; w < NW; ++w) s += tile_part[t * NW + w];
        }
        mine[j] = s;
        run += s;
    }
    float total;
    const float excl = block_excl_scan<NT, false>(run, &total, sc);
    const float T = r * total;
    int cross = INT_MAX;
    {
        float acc = excl;
        for (int j = 0; j < tpt; ++j) {
            const int t = tid * tpt + j;
            if (t < g.nt_all) {
                tile_excl[t] = acc;
                // Only a tile with weight can hold the draw.  (A later, empty
                // tile's prefix comes from the scan's own association and may
                // exceed the last weighted tile's excl + sum by an ulp; taken
                // as the crossing, its scan would find no token at all.)
                if (cross == INT_MAX && mine[j] > 0.0f && acc + mine[j] > T) cross = t;
                acc += mine[j];
            }
        }
    }
    cross = block_min_i<NT, false>(cross, sc);  // its barrier also publishes tile_excl
    *total_out = total;
    if (cross == INT_MAX) {
        // No cumulative sum exceeds r * total (r = 1, or rounding left r *
        // total at or above the last sum): the draw is the last index with
        // positive weight.  It lies in the last tile with a positive sum
        // (every weight after it is zero), so pass B scans that tile like a
        // crossing tile and, finding no crossing inside it either, returns
        // its last positive index.
        int lt = -1;
        for (int j = 0; j < tpt; ++j) {
            const int t = tid * tpt + j;
            if (t < g.nt_all && mine[j] > 0.0f) lt = t;
        }
        cross = block_max_i<NT, false>(lt, sc);
        if (cross < 0) {  // no positive weight anywhere
            __syncthreads();
            return 0;
        }
    }

    // Pass B: scan inside the crossing tile.
    float cum = tile_excl[cross];
    int found = INT_MAX;
    int tile_last = -1;
    if (cross == g.ntiles) {  // the trailing-logits tile
        float w = 0.0f;
        if (tid < rem) {
            const float tv = held.telem(tr, nch * E + tid);
            const float dv = PAIR ? held.delem(dr, nch * E + tid) : 0.0f;
            w = wf(tv, dv);
            if (w > 0.0f) tile_last = nch * E + tid;
        }
        float tot;
        const float ex = block_excl_scan<NT, false>(w, &tot, sc);
        if (w > 0.0f && cum + (ex + w) > T) found = nch * E + tid;
        found = block_min_i<NT, false>(found, sc);
    } else {
        for (int rd = cross * g.m; rd < min(g.rounds, (cross + 1) * g.m); ++rd) {
            const int ci = rd * NT + tid;
            float wv[E];
            float loc = 0.0f;
            if (ci < nch) {
                const C tc = held.template tchunk<NT>(tr, rd);
                C dc;
                if (PAIR) dc = held.template dchunk<NT>(dr, rd);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    wv[e] = PAIR ? wf(tc.get(e), dc.get(e)) : wf(tc.get(e), 0.0f);
                    loc += wv[e];
                    if (wv[e] > 0.0f) tile_last = ci * E + e;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) wv[e] = 0.0f;
            }
            float tot;
            const float ex = block_excl_scan<NT, false>(loc, &tot, sc);
            int f = INT_MAX;
            float run_e = ex;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                run_e += wv[e];
                if (f == INT_MAX && wv[e] > 0.0f && cum + run_e > T) f = ci * E + e;
            }
            found = block_min_i<NT, false>(f, sc);
            if (found != INT_MAX) break;  // uniform
            cum += tot;
        }
    }
    if (found != INT_MAX) {
        __syncthreads();  // the one trailing barrier (see the block operations)
        return found;
    }
    return max(block_max_i<NT>(tile_last, sc), 0);
}

// The whole draw in one call.  All threads call.
template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename Held = ReadAgain>
__device__ int inverse_cdf_row(const char* trow, const char* drow, int V, const Wt& wf, float r,
                               float* total_out, float* tile_part, float* tile_excl,
                               Scratch<NT>& sc, const Held& held = Held{}) {
    constexpr int NW = NT / 64;
    const Row<DT, VEC> tr(trow, V);
    const Row<DT, VEC> dr(PAIR ? drow : trow, V);
    const int tid = threadIdx.x;
    const TileGeom g = tile_geom<NT>(tr.nch, VEC ? V - tr.nch * Chunk<DT, VEC>::E : 0);
    for (int t = tid; t < g.nt_all * NW; t += NT) tile_part[t] = 0.0f;
    __syncthreads();
    cdf_pass_a_block<DT, VEC, PAIR, NT>(tr, dr, wf, g, tile_part, held);
    cdf_trailing<DT, VEC, PAIR, NT>(tr, dr, wf, g, tile_part, 0, held);
    __syncthreads();
    return cdf_select<DT, VEC, PAIR, NT>(tr, dr, wf, r, g, total_out, tile_part, tile_excl, sc,
                                         held);
}

// inverse_cdf_row for a row (pair) the caller kept on chip (PairHold, or
// HeldRounds for a single row): pass A reads the rounds beyond the held
// ones from memory first, then sums the held rounds (their loads, if any,
// from LDS); pass B scans the crossing tile's chunks from where they are.
// The tile sums are the same sums as inverse_cdf_row's.  All threads call.
template <int DT, bool VEC, bool PAIR, int NT, typename Wt, typename H>
__device__ __forceinline__ int inverse_cdf_held(const char* trow, const char* drow, int V, const Wt& wf, float r,
                                float* total_out, float* tile_part, float* tile_excl,
                                Scratch<NT>& sc, const H& hold) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    constexpr int N = H::kRounds;
    static_assert(N % TUNROLL == 0, "whole steps");
    const Row<DT, VEC> tr(trow, V);
    const Row<DT, VEC> dr(PAIR ? drow : trow, V);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const TileGeom g = tile_geom<NT>(tr.nch, VEC ? V - tr.nch * C::E : 0);
    for (int t = tid; t < g.nt_all * NW; t += NT) tile_part[t] = 0.0f;
    __syncthreads();
    if (g.rounds > N)
        cdf_pass_a_rounds<DT, VEC, PAIR, NT>(tr, dr, wf, g, N, g.rounds, 0, tile_part,
                                             read_again_of(hold));
#pragma unroll
    for (int r0 = 0; r0 < N; r0 += TUNROLL) {
        if (r0 < g.rounds) {  // uniform
            C tb[TUNROLL], db[TUNROLL];
#pragma unroll
            for (int u = 0; u < TUNROLL; ++u) {
                const int rd = r0 + u;
                const int ci = rd * NT + tid;
                if (ci < g.nch) {
                    tb[u] = hold.template tchunk<NT>(tr, rd);
                    if (PAIR) db[u] = hold.template dchunk<NT>(dr, rd);
                } else {
                    tb[u].set_neg_inf();
                    if (PAIR) db[u].set_neg_inf();
                }
            }
#pragma unroll
            for (int u = 0; u < TUNROLL; ++u) {
                const int round = r0 + u;
                if (round < g.rounds) {  // uniform
                    const float acc = wave_sum(chunk_weight_sum<PAIR>(wf, tb[u], db[u]));
                    if (lane == 0) tile_part[(round / g.m) * NW + wave] += acc;
                }
            }
        }
    }
    cdf_trailing<DT, VEC, PAIR, NT>(tr, dr, wf, g, tile_part, 0, read_again_of(hold));
    __syncthreads();
    return cdf_select<DT, VEC, PAIR, NT>(tr, dr, wf, r, g, total_out, tile_part, tile_excl, sc,
                                         hold);
}

// ------------------------------------------------------------------------
// Finishing a sequence.

// A sequence's place in the batch: its draft-token count k, its first
// target row t0 and its first draft row / draft-token index d0.  Dense
// batches: the same k for every sequence (G candidate blocks in greedy
// mode); ragged batches: k_b = cu[b+1] - cu[b] with rows packed (target rows
// cu[b] + b .., draft rows cu[b] ..), clamped so that a malformed cu can
// never address outside buffers of total_draft draft rows.
struct Seq {
    int k;
    long long t0, d0;
    int pos0;  // position of row 0 within the sequence (a continuation's first pair)
};

__device__ __forceinline__ Seq seq_of(const Params& p, int b) {
    Seq s;
    if (p.cu) {
        const long long tot = p.total_draft;
        long long kb = (long long)p.cu[b + 1] - p.cu[b];
        kb = kb < 0 ? 0 : (kb > p.k ? p.k : kb);
        if (kb > tot) kb = tot;
        long long d0 = p.cu[b];
        d0 = d0 < 0 ? 0 : (d0 > tot - kb ? tot - kb : d0);
        s.k = (int)kb;
        s.d0 = d0;
        s.t0 = d0 + b;
    } else {
        s.k = p.k;
        s.d0 = (long long)b * p.G * p.k;
        s.t0 = (long long)b * p.G * (p.k + 1);
    }
    s.pos0 = 0;
    return s;
}

// The rest of sequence b from position pos0 on (pos0 < its k): the same
// rows, tokens and uniforms, starting pos0 pairs later.
__device__ __forceinline__ Seq seq_from(const Params& p, int b, int pos0) {
    Seq s = seq_of(p, b);
    s.pos0 = pos0;
    s.k -= pos0;
    s.t0 += pos0;
    s.d0 += pos0;
    return s;
}

// Row r of a stochastic sequence: target rows 0..k, then draft rows.
template <int DT>
__device__ __forceinline__ const char* stoch_row(const Params& p, const Seq& s, int r) {
    const size_t rb = (size_t)p.row_stride * elem_bytes<DT>();
    if (r <= s.k) return static_cast<const char*>(p.target) + (size_t)(s.t0 + r) * rb;
    return static_cast<const char*>(p.draft) + (size_t)(s.d0 + (r - s.k - 1)) * rb;
}

// Row r of a greedy sequence (candidate c's rows are c(k+1) .. c(k+1)+k).
template <int DT>
__device__ __forceinline__ const char* greedy_row(const Params& p, const Seq& s, int r) {
    return static_cast<const char*>(p.target) +
           (size_t)(s.t0 + r) * (size_t)p.row_stride * elem_bytes<DT>();
}

template <int NT>
struct StochFin {
    Scratch<NT> sc;
    int a;
    float R[MAX_ROWS_STOCH];  // rows 0..k: target, k+1..2k: draft
    float Z[MAX_ROWS_STOCH];
    float px[kMaxK];
    float qx[kMaxK];
    float uv[kMaxK];  // acceptance uniforms
    int xv[kMaxK];    // draft tokens (row-split)
    float tl[kMaxK];  // target / draft logit at the draft token (row-split)
    float dl[kMaxK];
    int js;           // slice draw: the chosen slice, the uniform within it,
    float rf, Rm;     // and the row's reference
    int last;         // spread draw: this group arrived last for its sequence
    float tile_part[(MAX_TILES + 1) * (NT / 64)];
    float tile_excl[MAX_TILES + 1];
};

// Needs R[], Z[] of every row of sequence b in LDS (after a barrier).
// hold (a PairHold, or ReadAgain for none): pair 0 (target row 0 alone when
// k = 0) kept on chip.
template <int DT, bool VEC, int NT, typename H>
__device__ __forceinline__ void finish_stochastic(const Params& p, int b, const Seq& s,
                                                  StochFin<NT>& sm, H& hold) {
    const int tid = threadIdx.x;
    const int k = s.k, V = p.V;
    const int32_t* x = p.tokens_in + s.d0;
    for (int i = tid; i < k; i += NT) {
        const int xi = x[i];
        sm.uv[i] = p.u_accept[s.d0 + i];
        float pi = 0.0f, qi = 0.0f;
        if (xi >= 0 && xi < V) {
            const float tv = load_elem<DT>(stoch_row<DT>(p, s, i), xi);
            const float dv = load_elem<DT>(stoch_row<DT>(p, s, k + 1 + i), xi);
            pi = fast_exp2(fmaf(tv, p.c, -sm.R[i])) / sm.Z[i];
            qi = fast_exp2(fmaf(dv, p.c, -sm.R[k + 1 + i])) / sm.Z[k + 1 + i];
        }
        sm.px[i] = pi;
        sm.qx[i] = qi;
        if (p.dbg) {
            p.dbg[(s.d0 + i) * 2] = pi;
            p.dbg[(s.d0 + i) * 2 + 1] = qi;
        }
    }
    __syncthreads();
    if (tid == 0) {
        // all operands in LDS: no memory round trip per position
        int a = k;
        for (int i = 0; i < k; ++i)
            if (!(sm.uv[i] * sm.qx[i] < sm.px[i])) {
                a = i;
                break;
            }
        sm.a = a;
    }
    __syncthreads();
    const int a = sm.a;
    // a continuation (s.pos0 > 0) writes its own positions only
    int32_t* out = p.tokens_out + (size_t)b * (p.k + 1) + s.pos0;
    for (int i = tid; i <= p.k - s.pos0; i += NT) {
        if (i < a) out[i] = x[i];
        else if (i > a) out[i] = -1;
    }
    const float rr = p.u_sample[b];
    const char* trow = stoch_row<DT>(p, s, a);
    float total = 0.0f;
    int y = 0;
    bool read_again = true;
    if constexpr (H::kHeld) {
        if (a == 0) {
            // pair 0 (or the bonus row when k = 0) kept on chip: one draw
            // code path for either weight
            DrawW w{p.c, -sm.R[k], 0.0f, a < k};
            if (a < k) {
                w.nt = -(sm.R[a] + __log2f(sm.Z[a]));
                w.nd = -(sm.R[k + 1 + a] + __log2f(sm.Z[k + 1 + a]));
            }
            hold.dlive = w.pair;
            y = inverse_cdf_held<DT, VEC, true, NT>(trow, a < k ? stoch_row<DT>(p, s, k + 1) : trow,
                                                    V, w, rr, &total, sm.tile_part, sm.tile_excl,
                                                    sm.sc, hold);
            read_again = false;
            if (w.pair && !(total > 0.0f)) {
                // p == q to float precision: the residual is empty; draw
                // from p_a (read again; this almost never happens).
                const TargetW tw{p.c, -sm.R[a]};
                y = inverse_cdf_row<DT, VEC, false, NT>(trow, nullptr, V, tw, rr, &total,
                                                        sm.tile_part, sm.tile_excl, sm.sc);
            }
        }
    }
    if (read_again) {
        if (a < k) {
            const char* drow = stoch_row<DT>(p, s, k + 1 + a);
            const ResidualW w{p.c, -(sm.R[a] + __log2f(sm.Z[a])),
                              -(sm.R[k + 1 + a] + __log2f(sm.Z[k + 1 + a]))};
            y = inverse_cdf_row<DT, VEC, true, NT>(trow, drow, V, w, rr, &total, sm.tile_part,
                                                   sm.tile_excl, sm.sc);
            if (!(total > 0.0f)) {
                // p == q to float precision: the residual is empty; draw from p_a.
                const TargetW tw{p.c, -sm.R[a]};
                y = inverse_cdf_row<DT, VEC, false, NT>(trow, nullptr, V, tw, rr, &total,
                                                        sm.tile_part, sm.tile_excl, sm.sc);
            }
        } else {
            const TargetW tw{p.c, -sm.R[k]};
            y = inverse_cdf_row<DT, VEC, false, NT>(trow, nullptr, V, tw, rr, &total,
                                                    sm.tile_part, sm.tile_excl, sm.sc);
        }
    }
    if (tid == 0) {
        out[a] = y;
        if (p.accept_len) p.accept_len[b] = s.pos0 + a;
    }
}

template <int NT>
struct GreedyFin {
    Scratch<NT> sc;
    int a;
    int c;
    int g[kMaxRowsPerSeq];           // argmax of every row of the sequence
    int cand_a[kMaxRowsPerSeq];      // G <= kMaxRowsPerSeq / (k+1), k >= 0
};

// Needs g[] of every row of sequence b in LDS (after a barrier).
template <int NT>
__device__ void finish_greedy(const Params& p, int b, const Seq& s, GreedyFin<NT>& sm) {
    const int tid = threadIdx.x;
    const int k = s.k, G = p.G;
    const int32_t* x = p.tokens_in + s.d0;
    for (int c = tid; c < G; c += NT) {
        int a = k;
        for (int i = 0; i < k; ++i)
            if (x[c * k + i] != sm.g[c * (k + 1) + i]) {
                a = i;
                break;
            }
        sm.cand_a[c] = a;
    }
    __syncthreads();
    if (tid == 0) {
        int bc = 0, ba = sm.cand_a[0];
        for (int c = 1; c < G; ++c)
            if (sm.cand_a[c] > ba) {  // lowest candidate wins ties
                ba = sm.cand_a[c];
                bc = c;
            }
        sm.a = ba;
        sm.c = bc;
        if (p.accept_len) p.accept_len[b] = ba;
        if (p.best_cand) p.best_cand[b] = bc;
    }
    __syncthreads();
    const int a = sm.a, bc = sm.c;
    int32_t* out = p.tokens_out + (size_t)b * (p.k + 1);
    for (int i = tid; i <= p.k; i += NT) out[i] = i <= a ? sm.g[bc * (k + 1) + i] : -1;
}

// ------------------------------------------------------------------------
// Sequence-resident kernels: one workgroup per sequence.

// Merge the per-wave partial normalisers of row r: R = max, Z rescaled sum.
template <int NW>
__device__ __forceinline__ void merge_row(const float* wR, const float* wZ, int r, float& R,
                                          float& Z) {
    R = wR[r * NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) R = fmaxf(R, wR[r * NW + w]);
    Z = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Z += wZ[r * NW + w] * fast_exp2(wR[r * NW + w] - R);
}

// Draft rounds of the held pair that a sequence-resident kernel stashes in
// LDS beside `base` bytes of its own shared memory: a 1024-thread workgroup
// has the CU's 160 KB to itself, two 512-thread workgroups share it.
template <int NT>
constexpr int pair_stash_rounds(size_t base) {
    const size_t budget = (NT >= 1024 ? kLdsBytesPerCu : kLdsBytesPerCu / 2) - 512;
    const size_t per_round = (size_t)NT * 16;
    const size_t n = base >= budget ? 0 : (budget - base) / per_round;
    return n < (size_t)kPairHeldRounds ? (int)n : kPairHeldRounds;
}

template <int NT>
struct StochSeqBase {
    StochFin<NT> fin;
    float wR[MAX_ROWS_STOCH * (NT / 64)];  // per-wave partial normalisers
    float wZ[MAX_ROWS_STOCH * (NT / 64)];
};
template <int NT, int NH>
struct StochSeqSmem : StochSeqBase<NT> {
    static constexpr int LR = NH > 0 ? pair_stash_rounds<NT>(sizeof(StochSeqBase<NT>)) : 0;
    static_assert(NH == 0 || LR >= 1, "room for the draft stash");
    uint4 stash[LR > 0 ? LR * NT : 1];
};

// The full read with 512-thread groups (more sequences than CUs), except
// on long rows from 384 to 512 sequences; up to 256 sequences, and there,
// the full read runs in position order in k_stochastic_seq_exit.
// NH: target rounds of pair 0 held in registers (0: nothing held, which
// leaves room for more workgroups per CU).
template <int DT, bool VEC, int NT, int NH>
__global__ __launch_bounds__(NT) void k_stochastic_seq(Params p) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    __shared__ StochSeqSmem<NT, NH> sm;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Seq sq = seq_of(p, b);
    const int k = sq.k;
    const int rows = 2 * k + 1;
    auto put = [&](int r, const SoftAcc& acc) {
        float R, Z;
        wave_softmax(acc, R, Z);
        if (lane == 0) {
            sm.wR[r * NW + wave] = R;
            sm.wZ[r * NW + wave] = Z;
        }
    };
    // Target row k first, then the pairs from position k-1 down to 0, so the
    // pair a rejection most often lands on is read last: its target row
    // stays in registers and the start of its draft row in LDS for the
    // closing-token draw (the bonus row when k = 0).
    PairHold<C, NH, NT> hold;
    hold.stash = reinterpret_cast<C*>(sm.stash);
    hold.lr = StochSeqSmem<NT, NH>::LR;
    const int nlead = NH == 0 ? rows : (k > 0 ? rows - 2 : 0);
    for (int j = 0; j < nlead; ++j) {
        const int i = k - (j + 1) / 2;
        const int r = (j == 0) ? k : ((j & 1) ? k + 1 + i : i);
        const Row<DT, VEC> row(stoch_row<DT>(p, sq, r), p.V);
        SoftAcc acc;
        if (i < KEEP_PAIRS && j > 0) stream_softmax<DT, VEC, NT, true>(row, p.c, acc);
        else stream_softmax<DT, VEC, NT>(row, p.c, acc);
        put(r, acc);
    }
    if constexpr (NH > 0) {
        if (k > 0) {
            const Row<DT, VEC> row(stoch_row<DT>(p, sq, k + 1), p.V);
            SoftAcc acc;
            stream_softmax_stash<DT, VEC, NT, true>(row, p.c, acc, hold.stash, hold.lr);
            put(k + 1, acc);
        }
        const Row<DT, VEC> row(stoch_row<DT>(p, sq, 0), p.V);
        SoftAcc acc;
        stream_softmax_hold<DT, VEC, NT, true, NH>(row, p.c, acc, hold.t);
        put(0, acc);
    }
    __syncthreads();
    for (int r = tid; r < rows; r += NT) {
        float R = sm.wR[r * NW];
#pragma unroll
        for (int w = 1; w < NW; ++w) R = fmaxf(R, sm.wR[r * NW + w]);
        float Z = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) Z += sm.wZ[r * NW + w] * fast_exp2(sm.wR[r * NW + w] - R);
        sm.fin.R[r] = R;
        sm.fin.Z[r] = Z;
    }
    __syncthreads();
    if constexpr (NH > 0) {
        finish_stochastic<DT, VEC, NT>(p, b, sq, sm.fin, hold);
    } else {
        ReadAgain none;
        finish_stochastic<DT, VEC, NT>(p, b, sq, sm.fin, none);
    }
}

// Position-order kernel.  Without per-position diagnostics (the early
// exit) a sequence stops reading at its first rejection, because no later
// row can change accept_len or tokens; its full-read variant (FULL, up to
// 256 sequences) draws there too and then reads the remaining rows for the
// diagnostics.  One block-wide decision per position: after pair i every
// thread merges the pair's per-wave partials from LDS and reaches the same
// verdict.
template <int NT>
struct StochExitBase {
    StochFin<NT> fin;
    float wR[2 * 2 * (NT / 64)];  // [pair parity][target, draft][wave]
    float wZ[2 * 2 * (NT / 64)];
    int xv[kMaxK];    // draft tokens
    float uv[kMaxK];  // acceptance uniforms
    float tv[kMaxK];  // target logit at the draft token (0 if out of range)
    float dv[kMaxK];  // draft logit at the draft token
};
template <int NT, int NH>
struct StochExitSmem : StochExitBase<NT> {
    // no stash where nothing is held (the LDS would limit the groups per CU)
    static constexpr int LR = NH > 0 ? pair_stash_rounds<NT>(sizeof(StochExitBase<NT>)) : 0;
    static_assert(NH == 0 || LR >= 1, "room for the draft stash");
    uint4 stash[LR > 0 ? LR * NT : 1];
};

// NH: target rounds of the pair being streamed held in registers (0: none).
// FULL: the full read (diagnostics asked for): p and q at every position go
// to p.dbg, and once the token is drawn the rest of the rows are streamed
// too, so every row is read once and the draw still finds the pair it needs
// on chip.
template <int DT, bool VEC, int NT, int NH, bool FULL>
__global__ __launch_bounds__(NT) void k_stochastic_seq_exit(Params p) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    __shared__ StochExitSmem<NT, NH> sm;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Seq sq = seq_of(p, b);
    const int k = sq.k, V = p.V;
    const float c = p.c;
    const int32_t* x = p.tokens_in + sq.d0;
    // Wave 0 gathers the tokens, uniforms and the logits at the tokens (lane
    // i: position i) while it streams the first row; the first barrier
    // publishes them.
    const bool gather = wave == 0 && lane < k;
    int gx = -1;
    float gu = 0.0f, gt = 0.0f, gd = 0.0f;
    if (gather) {
        gx = x[lane];
        gu = p.u_accept[sq.d0 + lane];
    }
    int a = k;
    // Capped (p.active set): stream at most p.exit_pairs pairs, leave every
    // streamed row's statistics and the logits at the draft tokens in the
    // row-split layout, and draw only after a rejection at an early position;
    // the continuation kernels finish the rest.
    const bool capped = p.active != nullptr;
    const int npairs = capped ? min(p.exit_pairs, k) : k;
    float* part = capped ? p.part + (size_t)b * p.rows_per_seq * p.S * 2 : nullptr;
    float Rt = 0.0f, Zt = 1.0f, Rd = 0.0f, Zd = 1.0f;
    // The pair streamed last is the one the draw needs (the rejected pair,
    // or the bonus row): with HOLD, each pair's draft row goes through the
    // LDS stash and its target row through registers, overwriting the
    // previous pair's.
    constexpr bool HOLD = NH > 0;
    constexpr bool full = FULL;  // never capped
    PairHold<C, NH, NT> hold;
    hold.stash = reinterpret_cast<C*>(sm.stash);
    hold.lr = StochExitSmem<NT, NH>::LR;
    for (int i = 0; i < npairs; ++i) {
        float* wR = sm.wR + (i & 1) * 2 * NW;
        float* wZ = sm.wZ + (i & 1) * 2 * NW;
        // HOLD: the draft row first (into the stash), then the target row
        // (into registers); otherwise the target row first.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool tgt = HOLD ? h == 1 : h == 0;
            const Row<DT, VEC> row(stoch_row<DT>(p, sq, tgt ? i : k + 1 + i), V);
            SoftAcc acc;
            if (i < (HOLD && NT < 1024 ? EXIT_KEEP_PAIRS_WIDE_HELD : EXIT_KEEP_PAIRS)) {  // uniform
                if constexpr (HOLD) {
                    if (tgt) stream_softmax_hold<DT, VEC, NT, true, NH>(row, c, acc, hold.t);
                    else stream_softmax_stash<DT, VEC, NT, true>(row, c, acc, hold.stash, hold.lr);
                } else {
                    stream_softmax<DT, VEC, NT, true>(row, c, acc);
                }
            } else {
                if constexpr (HOLD) {
                    if (tgt) stream_softmax_hold<DT, VEC, NT, false, NH>(row, c, acc, hold.t);
                    else stream_softmax_stash<DT, VEC, NT>(row, c, acc, hold.stash, hold.lr);
                } else {
                    stream_softmax<DT, VEC, NT>(row, c, acc);
                }
            }
            float R, Z;
            wave_softmax(acc, R, Z);
            if (lane == 0) {
                wR[(tgt ? 0 : NW) + wave] = R;
                wZ[(tgt ? 0 : NW) + wave] = Z;
            }
            if (i == 0 && h == 0 && gather && gx >= 0 && gx < V) {
                gt = load_elem<DT>(stoch_row<DT>(p, sq, lane), gx);
                gd = load_elem<DT>(stoch_row<DT>(p, sq, k + 1 + lane), gx);
            }
        }
        if (i == 0 && gather) {
            sm.xv[lane] = gx;
            sm.uv[lane] = gu;
            sm.tv[lane] = gt;
            sm.dv[lane] = gd;
            if (capped) {
                float* xl = p.xl + (size_t)b * p.rows_per_seq;
                xl[lane] = gt;
                xl[k + 1 + lane] = gd;
            }
        }
        // One barrier per pair; the partials are double-buffered by pair
        // parity, so the next pair never overwrites what is being read.
        __syncthreads();
        merge_row<NW>(wR, wZ, 0, Rt, Zt);
        merge_row<NW>(wR, wZ, 1, Rd, Zd);
        if (capped && tid < 2 * p.S) {
            // slice 0 holds the row's statistics, the other slices merge as empty
            const int half = tid / p.S, j = tid - half * p.S;
            float* d = part + ((size_t)(half == 0 ? i : k + 1 + i) * p.S + j) * 2;
            d[0] = j == 0 ? (half == 0 ? Rt : Rd) : -FLT_MAX;
            d[1] = j == 0 ? (half == 0 ? Zt : Zd) : 0.0f;
        }
        const int xi = sm.xv[i];
        float pi = 0.0f, qi = 0.0f;
        if (xi >= 0 && xi < V) {
            pi = fast_exp2(fmaf(sm.tv[i], c, -Rt)) / Zt;
            qi = fast_exp2(fmaf(sm.dv[i], c, -Rd)) / Zd;
        }
        if (full && tid == 0) {
            p.dbg[(sq.d0 + i) * 2] = pi;
            p.dbg[(sq.d0 + i) * 2 + 1] = qi;
        }
        if (!(sm.uv[i] * qi < pi)) {  // the same verdict in every thread
            a = i;
            break;
        }
    }
    a = __builtin_amdgcn_readfirstlane(a);  // block-uniform: scalar from here on
    if (capped) {
        // 0: rejected, drawn by the spread draw kernels; 1: every streamed
        // pair accepted, the rest of the rows still to read; 2: rejected
        // early enough to draw here, off the critical path (the sequences
        // that stream all the capped pairs take longer)
        const bool here = a < npairs && a < kExitDrawHere;
        if (tid == 0) p.active[b] = here ? 2 : (a < npairs ? 0 : 1);
        if (!here) return;
    }
    int32_t* out = p.tokens_out + (size_t)b * (p.k + 1);
    for (int i = tid; i <= p.k; i += NT) {
        if (i < a) out[i] = x[i];
        else if (i > a) out[i] = -1;
    }
    const float rr = p.u_sample[b];
    int y;
    if constexpr (HOLD) {
        // The row (pair) the draw needs was streamed last and is held on chip:
        // pair a after a rejection, else the bonus row k, streamed here.
        DrawW w{c, -(Rt + __log2f(Zt)), -(Rd + __log2f(Zd)), a < k};
        if (a == k) {
            const Row<DT, VEC> row(stoch_row<DT>(p, sq, k), V);
            SoftAcc acc;
            stream_softmax_hold<DT, VEC, NT, false, NH>(row, c, acc, hold.t);
            float R, Z;
            wave_softmax(acc, R, Z);
            if (lane == 0) {
                sm.wR[(k & 1) * 2 * NW + wave] = R;
                sm.wZ[(k & 1) * 2 * NW + wave] = Z;
            }
            __syncthreads();
            float Rk, Zk;
            merge_row<NW>(sm.wR + (k & 1) * 2 * NW, sm.wZ + (k & 1) * 2 * NW, 0, Rk, Zk);
            (void)Zk;
            w.nt = -Rk;
        }
        const char* trow = stoch_row<DT>(p, sq, a);
        const char* drow = a < k ? stoch_row<DT>(p, sq, k + 1 + a) : trow;
        float total = 0.0f;
        hold.dlive = w.pair;
        y = inverse_cdf_held<DT, VEC, true, NT>(trow, drow, V, w, rr, &total, sm.fin.tile_part,
                                                sm.fin.tile_excl, sm.fin.sc, hold);
        if (w.pair && !(total > 0.0f)) {
            // p == q to float precision: the residual is empty; draw from p_a
            // (read again; this almost never happens).
            w.pair = false;
            w.nt = -Rt;
            ReadPair rd;
            rd.dlive = false;
            y = inverse_cdf_row<DT, VEC, true, NT>(trow, drow, V, w, rr, &total, sm.fin.tile_part,
                                                   sm.fin.tile_excl, sm.fin.sc, rd);
        }
    } else {
        float total = 0.0f;
        if (a < k) {
            const ResidualW w{c, -(Rt + __log2f(Zt)), -(Rd + __log2f(Zd))};
            y = inverse_cdf_row<DT, VEC, true, NT>(stoch_row<DT>(p, sq, a),
                                                   stoch_row<DT>(p, sq, k + 1 + a), V, w, rr,
                                                   &total, sm.fin.tile_part, sm.fin.tile_excl,
                                                   sm.fin.sc);
            if (!(total > 0.0f)) {
                // p == q to float precision: the residual is empty; draw from p_a.
                const TargetW tw{c, -Rt};
                y = inverse_cdf_row<DT, VEC, false, NT>(stoch_row<DT>(p, sq, a), nullptr, V, tw,
                                                        rr, &total, sm.fin.tile_part,
                                                        sm.fin.tile_excl, sm.fin.sc);
            }
        } else {
            // every draft token accepted: the bonus token from row k
            const Row<DT, VEC> row(stoch_row<DT>(p, sq, k), V);
            SoftAcc acc;
            stream_softmax<DT, VEC, NT>(row, c, acc);
            float R, Z;
            wave_softmax(acc, R, Z);
            if (lane == 0) {
                sm.wR[(k & 1) * 2 * NW + wave] = R;
                sm.wZ[(k & 1) * 2 * NW + wave] = Z;
            }
            __syncthreads();
            float Rk, Zk;
            merge_row<NW>(sm.wR + (k & 1) * 2 * NW, sm.wZ + (k & 1) * 2 * NW, 0, Rk, Zk);
            (void)Zk;
            const TargetW tw{c, -Rk};
            y = inverse_cdf_row<DT, VEC, false, NT>(stoch_row<DT>(p, sq, k), nullptr, V, tw, rr,
                                                    &total, sm.fin.tile_part, sm.fin.tile_excl,
                                                    sm.fin.sc);
        }
    }
    if (tid == 0) {
        out[a] = y;
        if (p.accept_len) p.accept_len[b] = a;
    }
    if (full && a < k) {
        // The rows after the rejection, for the diagnostics: p and q at the
        // later positions (one barrier per pair, which measured faster than
        // streaming them all before one merge), then the bonus row, read
        // like every other row.
        for (int i = a + 1; i < k; ++i) {
            float* wR = sm.wR + (i & 1) * 2 * NW;
            float* wZ = sm.wZ + (i & 1) * 2 * NW;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const Row<DT, VEC> row(stoch_row<DT>(p, sq, h == 0 ? i : k + 1 + i), V);
                SoftAcc acc;
                stream_softmax<DT, VEC, NT>(row, c, acc);
                float R, Z;
                wave_softmax(acc, R, Z);
                if (lane == 0) {
                    wR[h * NW + wave] = R;
                    wZ[h * NW + wave] = Z;
                }
            }
            __syncthreads();
            merge_row<NW>(wR, wZ, 0, Rt, Zt);
            merge_row<NW>(wR, wZ, 1, Rd, Zd);
            if (tid == 0) {
                const int xi = sm.xv[i];
                float pi = 0.0f, qi = 0.0f;
                if (xi >= 0 && xi < V) {
                    pi = fast_exp2(fmaf(sm.tv[i], c, -Rt)) / Zt;
                    qi = fast_exp2(fmaf(sm.dv[i], c, -Rd)) / Zd;
                }
                p.dbg[(sq.d0 + i) * 2] = pi;
                p.dbg[(sq.d0 + i) * 2 + 1] = qi;
            }
        }
        const Row<DT, VEC> row(stoch_row<DT>(p, sq, k), V);
        SoftAcc acc;
        stream_softmax<DT, VEC, NT>(row, c, acc);
        float R, Z;
        wave_softmax(acc, R, Z);
        if (lane == 0) {
            sm.wR[(k & 1) * 2 * NW + wave] = R;
            sm.wZ[(k & 1) * 2 * NW + wave] = Z;
        }
    }
}

template <int NT>
struct GreedySeqSmem {
    GreedyFin<NT> fin;
    float wbest[MAX_ROWS_GREEDY_SEQ * (NT / 64)];
    int wpos[MAX_ROWS_GREEDY_SEQ * (NT / 64)];
};

template <int DT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_greedy_seq(Params p) {
    constexpr int NW = NT / 64;
    __shared__ GreedySeqSmem<NT> sm;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Seq sq = seq_of(p, b);
    const int rows = sq.k + 1;  // one candidate
    for (int r = 0; r < rows; ++r) {
        const Row<DT, VEC> row(greedy_row<DT>(p, sq, r), p.V);
        ArgAcc acc;
        stream_argmax<DT, VEC, NT>(row, acc);
        wave_argmax(acc.best, acc.pos);
        if (lane == 0) {
            sm.wbest[r * NW + wave] = acc.best;
            sm.wpos[r * NW + wave] = acc.pos;
        }
    }
    __syncthreads();
    for (int r = tid; r < rows; r += NT) {
        float best = sm.wbest[r * NW];
        int pos = sm.wpos[r * NW];
        for (int w = 1; w < NW; ++w)
            if (argmax_better(sm.wbest[r * NW + w], sm.wpos[r * NW + w], best, pos)) {
                best = sm.wbest[r * NW + w];
                pos = sm.wpos[r * NW + w];
            }
        const Row<DT, VEC> row(greedy_row<DT>(p, sq, r), p.V);
        sm.fin.g[r] = argmax_refine(row, best, pos);
    }
    __syncthreads();
    finish_greedy<NT>(p, b, sq, sm.fin);
}

// ------------------------------------------------------------------------
// Row-split kernels: statistics per (row, slice), then one finishing
// workgroup per sequence.

// Zero the spread draw's arrival counters (kernels that run before
// k_draw_tiles in a call; device-coherent stores, like the counters' updates).
__device__ __forceinline__ void zero_draw_counters(const Params& p) {
    if (p.cnt && blockIdx.x == 0)
        for (int i = threadIdx.x; i < p.B; i += blockDim.x)
            __hip_atomic_store(p.cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, bool VEC, bool STOCH, int NT>
__global__ __launch_bounds__(NT) void k_row_stats(Params p) {
    __shared__ Scratch<NT> sc;
    constexpr int NW = NT / 64;
    if (STOCH) zero_draw_counters(p);
    const int per_seq = p.rows_per_seq * p.S;
    int b, item;
    if (STOCH && p.slice_draw) {
        // Plain sampling from slice statistics: every slice of row b goes to
        // a workgroup on XCD b mod 8 (workgroups are dealt to the 8 XCDs
        // round robin), where k_sample_draw's group for row b runs, so the
        // one slice it reads again is in that XCD's L2 (B=64, V=128256 bf16:
        // 14.0 -> 13.7 us per call; B=300, V=129280: 24.1 -> 23.3 us).  The
        // grid is padded to whole groups of 8 rows.
        const int x = blockIdx.x & 7;
        const int q = blockIdx.x >> 3;
        b = (q / per_seq) * 8 + x;
        item = q - (q / per_seq) * per_seq;
        if (b >= p.B) return;
    } else {
        b = blockIdx.x / per_seq;
        item = blockIdx.x - b * per_seq;
    }
    const int r = item / p.S;
    const int s = item - r * p.S;
    const Seq sq = seq_of(p, b);
    if (r >= (STOCH ? 2 * sq.k + 1 : p.G * (sq.k + 1))) return;  // row absent (ragged)
    const int v0 = s * p.slice_len;
    const int v1 = min(p.V, v0 + p.slice_len);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const char* rp = STOCH ? stoch_row<DT>(p, sq, r) : greedy_row<DT>(p, sq, r);
    const Row<DT, VEC> row(rp + (size_t)v0 * elem_bytes<DT>(), v1 - v0);
    float* dst = p.part + ((size_t)b * per_seq + item) * 2;
    if (STOCH) {
        // The draft token of this row's position (target rows 0..k-1, draft
        // rows k+1..2k); the slice holding it also leaves the logit there,
        // so the finishing kernels need no gather of their own.
        int xi = -1;
        if (p.xl && r != sq.k) xi = p.tokens_in[sq.d0 + (r < sq.k ? r : r - sq.k - 1)];
        // The rows the closing-token draw most often reads again -- pair 0,
        // where a rejection most often lands, and the bonus row -- stream
        // with ordinary loads, so that they are the likeliest to be cached
        // by then (measured on B=64, k=4, V=128256 bf16: 42.4 against
        // 43.6 us per call).
        SoftAcc acc;
        if (r == 0 || r == sq.k || r == sq.k + 1)
            stream_softmax<DT, VEC, NT, true>(row, p.c, acc);
        else
            stream_softmax<DT, VEC, NT>(row, p.c, acc);
        float R, Z;
        wave_softmax(acc, R, Z);
        if (lane == 0) {
            sc.f[wave] = R;
            sc.g[wave] = Z;
        }
        __syncthreads();
        if (tid == 0) {
            float RR = sc.f[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) RR = fmaxf(RR, sc.f[w]);
            float ZZ = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) ZZ += sc.g[w] * fast_exp2(sc.f[w] - RR);
            dst[0] = RR;
            dst[1] = ZZ;
            if (xi >= v0 && xi < v1)
                p.xl[(size_t)b * p.rows_per_seq + r] = load_elem<DT>(rp, xi);
        }
    } else {
        ArgAcc acc;
        stream_argmax<DT, VEC, NT>(row, acc);
        wave_argmax(acc.best, acc.pos);
        if (lane == 0) {
            sc.f[wave] = acc.best;
            sc.i[wave] = acc.pos;
        }
        __syncthreads();
        if (tid == 0) {
            float best = sc.f[0];
            int pos = sc.i[0];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                if (argmax_better(sc.f[w], sc.i[w], best, pos)) {
                    best = sc.f[w];
                    pos = sc.i[w];
                }
            dst[0] = best;
            dst[1] = __int_as_float(v0 + argmax_refine(row, best, pos));
        }
    }
}

// Row-split stochastic finish for batches that fill the GPU on their own:
// one 1024-thread workgroup per sequence merges the slice statistics, takes
// the decisions and draws the closing token, as the sequence-resident kernel
// finishes -- one launch instead of the two below.
template <int DT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_stochastic_finish(Params p) {
    __shared__ StochFin<NT> sm;
    const int b = blockIdx.x;
    const Seq sq = seq_of(p, b);
    const int rows = 2 * sq.k + 1, S = p.S;
    const float* part = p.part + (size_t)b * p.rows_per_seq * S * 2;
    for (int r = threadIdx.x; r < rows; r += NT) {
        float R = -FLT_MAX;
        for (int j = 0; j < S; ++j) R = fmaxf(R, part[(r * S + j) * 2]);
        float Z = 0.0f;
        for (int j = 0; j < S; ++j)
            Z += part[(r * S + j) * 2 + 1] * fast_exp2(part[(r * S + j) * 2] - R);
        sm.R[r] = R;
        sm.Z[r] = Z;
    }
    __syncthreads();
    ReadAgain none;
    finish_stochastic<DT, VEC, NT>(p, b, sq, sm, none);
}

// Continuation of a capped early exit (p.active set by k_stochastic_seq_exit,
// which left the statistics of every row it streamed in p.part, slice 0, and
// the logits at the draft tokens in p.xl): the sequences that accepted every
// streamed pair have the rest of their rows -- the pairs from
// min(exit_pairs, k_b) on and the bonus row -- streamed by this persistent
// row-split kernel, so that a long accepted run is read by many CUs at once
// instead of one.  Then k_draw_tiles decides and draws every
// sequence from the statistics, spreading each closing-token draw over
// several workgroups.  p.part is [B][2k+1][p.S] float2; rows are cut into S2
// <= p.S slices, S2 chosen from the number of still-accepting sequences, and
// slices S2 .. p.S-1 are written empty so the merge over p.S slices is exact.
template <int DT, bool VEC>
__device__ __forceinline__ void exit_slicing(const Params& p, int n_active, int rows2, int& S2,
                                             int& slice_len) {
    constexpr int E = Chunk<DT, VEC>::E;
    const long long items = (long long)n_active * rows2;
    long long s = items > 0 ? (kExitTargetItems + items - 1) / items : 1;
    if (s > p.S) s = p.S;
    if (s < 1) s = 1;
    const int chunks = (p.V + E - 1) / E;
    const int per = (chunks + (int)s - 1) / (int)s;
    slice_len = per * E;
    S2 = (p.V + slice_len - 1) / slice_len;  // no empty slices; S2 <= s
}

// Row-split stochastic finish in one kernel, k_draw_tiles (B*SD groups), so
// that the closing-token draw -- one or two full rows per sequence -- is
// spread over SD workgroups per sequence instead of one: every group merges
// its sequence's statistics and takes the decisions itself (cheap, and it
// saves a launch); group 0 writes everything but the closing token; each
// group sums the draw weights over its share of the tiles and hands the sums
// over; the last group of the sequence to arrive scans the tile sums and the
// one tile holding the draw, and writes the token.
//
// The hand-over needs no cache writeback or invalidation: the tile sums are
// written and read with device-coherent (agent-scope atomic, sc1) stores and
// loads, each thread waits for its stores before the group's barrier, and
// only then is the sequence's arrival counter raised (relaxed agent-scope
// atomic).  The counters are zeroed by the statistics kernel that runs
// before, so a call needs no extra launch to clear them.
constexpr int NT_DRAW = kDrawRound;

// Group sd of the SD groups that draw sequence b (all threads call).
template <int DT, bool VEC>
__device__ void draw_tiles_group(const Params& p, int b, int sd, int SD, StochFin<NT_DRAW>& sm) {
    constexpr int NT = NT_DRAW;
    constexpr int NW = NT / 64;
    constexpr int E = Chunk<DT, VEC>::E;
    const int tid = threadIdx.x;
    const Seq sq = seq_of(p, b);
    const int k = sq.k, V = p.V, S = p.S;
    const float c = p.c;
    const float* part = p.part + (size_t)b * p.rows_per_seq * S * 2;
    const float* xl = p.xl + (size_t)b * p.rows_per_seq;
    const int32_t* x = p.tokens_in + sq.d0;
    // One round of independent loads: the row statistics (one (R, Z) pair
    // per thread, staged in LDS -- tile_part is free until the tile pass --
    // when they fit), the draft tokens, the logits at them (left by the
    // statistics kernel) and the uniforms.  The per-row merge then reads
    // LDS.  (Per thread and row, a chain of loads here waits behind the
    // other groups' tile passes once those start: 3.5-14 us in the capped
    // early exit at 16 slices a row.)
    const int nent = (2 * k + 1) * S;
    const bool staged = 2 * nent <= (MAX_TILES + 1) * NW;  // uniform
    if (staged)
        for (int e = tid; e < nent; e += NT) {
            const float2 v = reinterpret_cast<const float2*>(part)[e];
            sm.tile_part[2 * e] = v.x;
            sm.tile_part[2 * e + 1] = v.y;
        }
    for (int i = tid; i < k; i += NT) {
        sm.xv[i] = x[i];
        sm.uv[i] = p.u_accept[sq.d0 + i];
        sm.tl[i] = xl[i];
        sm.dl[i] = xl[k + 1 + i];
    }
    __syncthreads();
    for (int r = tid; r < 2 * k + 1; r += NT) {
        const float* st = (staged ? sm.tile_part : part) + r * S * 2;
        float R = -FLT_MAX;
        for (int j = 0; j < S; ++j) R = fmaxf(R, st[j * 2]);
        float Z = 0.0f;
        for (int j = 0; j < S; ++j) Z += st[j * 2 + 1] * fast_exp2(st[j * 2] - R);
        sm.R[r] = R;
        sm.Z[r] = Z;
    }
    __syncthreads();
    for (int i = tid; i < k; i += NT) {
        const int xi = sm.xv[i];
        float pi = 0.0f, qi = 0.0f;
        if (xi >= 0 && xi < V) {  // else nothing was left in tl/dl
            pi = fast_exp2(fmaf(sm.tl[i], c, -sm.R[i])) / sm.Z[i];
            qi = fast_exp2(fmaf(sm.dl[i], c, -sm.R[k + 1 + i])) / sm.Z[k + 1 + i];
        }
        sm.px[i] = pi;
        sm.qx[i] = qi;
        if (p.dbg && sd == 0) {
            p.dbg[(sq.d0 + i) * 2] = pi;
            p.dbg[(sq.d0 + i) * 2 + 1] = qi;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int a = k;
        for (int i = 0; i < k; ++i)
            if (!(sm.uv[i] * sm.qx[i] < sm.px[i])) {
                a = i;
                break;
            }
        sm.a = a;
    }
    __syncthreads();
    const int a = sm.a;
    // draw parameters: residual exponents, or the bonus row's reference
    const float w0 = a < k ? -(sm.R[a] + __log2f(sm.Z[a])) : -sm.R[k];
    const float w1 = a < k ? -(sm.R[k + 1 + a] + __log2f(sm.Z[k + 1 + a])) : 0.0f;
    const float w2 = -sm.R[a];  // p_a itself, if the residual turns out empty
    if (sd == 0) {
        int32_t* out = p.tokens_out + (size_t)b * (p.k + 1);
        for (int i = tid; i <= p.k; i += NT) {
            if (i < a) out[i] = x[i];
            else if (i > a) out[i] = -1;
        }
        if (tid == 0 && p.accept_len) p.accept_len[b] = a;
    }
    // this group's tiles of the draw row(s)
    const Row<DT, VEC> tr(stoch_row<DT>(p, sq, a), V);
    const Row<DT, VEC> dr(stoch_row<DT>(p, sq, a < k ? k + 1 + a : a), V);
    const TileGeom g = tile_geom<NT>(tr.nch, VEC ? V - tr.nch * E : 0);
    const int tps = (g.nt_all + SD - 1) / SD;
    const int t0 = sd * tps, t1 = min(g.nt_all, t0 + tps);
    if (t0 >= t1) return;  // uniform: this group has no tiles
    for (int t = tid; t < (t1 - t0) * NW; t += NT) sm.tile_part[t] = 0.0f;
    __syncthreads();
    const int r0 = t0 * g.m, r1 = min(g.rounds, t1 * g.m);
    if (a < k) {
        const ResidualW w{c, w0, w1};
        if (r0 < r1) cdf_pass_a_rounds<DT, VEC, true, NT>(tr, dr, w, g, r0, r1, t0, sm.tile_part);
        if (g.ntiles >= t0 && g.ntiles < t1)
            cdf_trailing<DT, VEC, true, NT>(tr, dr, w, g, sm.tile_part, t0);
    } else {
        const TargetW w{c, w0};
        if (r0 < r1) cdf_pass_a_rounds<DT, VEC, false, NT>(tr, dr, w, g, r0, r1, t0, sm.tile_part);
        if (g.ntiles >= t0 && g.ntiles < t1)
            cdf_trailing<DT, VEC, false, NT>(tr, dr, w, g, sm.tile_part, t0);
    }
    __syncthreads();
    uint32_t* ts = reinterpret_cast<uint32_t*>(p.tilesum) + (size_t)b * (kMaxTiles + 1);
    for (int t = tid; t < t1 - t0; t += NT) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += sm.tile_part[t * NW + w];
        __hip_atomic_store(ts + t0 + t, __float_as_uint(s), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // count this group in; the last of the sequence's groups draws the token
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int groups = (g.nt_all + tps - 1) / tps;  // the groups that have tiles
    if (tid == 0)
        sm.last = __hip_atomic_fetch_add(p.cnt + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  groups - 1;
    __syncthreads();
    if (!sm.last) return;  // uniform
    for (int t = tid; t < g.nt_all * NW; t += NT)
        sm.tile_part[t] = (t % NW) == 0 ? __uint_as_float(__hip_atomic_load(
                                              ts + t / NW, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                                        : 0.0f;
    __syncthreads();
    const float rr = p.u_sample[b];
    float total = 0.0f;
    int y;
    if (a < k) {
        const ResidualW w{c, w0, w1};
        y = cdf_select<DT, VEC, true, NT>(tr, dr, w, rr, g, &total, sm.tile_part, sm.tile_excl,
                                          sm.sc);
        if (!(total > 0.0f)) {
            // p == q to float precision: the residual is empty; draw from p_a.
            const TargetW tw{c, w2};
            y = inverse_cdf_row<DT, VEC, false, NT>(stoch_row<DT>(p, sq, a), nullptr, V, tw, rr,
                                                    &total, sm.tile_part, sm.tile_excl, sm.sc);
        }
    } else {
        const TargetW w{c, w0};
        y = cdf_select<DT, VEC, false, NT>(tr, dr, w, rr, g, &total, sm.tile_part, sm.tile_excl,
                                           sm.sc);
    }
    if (tid == 0) p.tokens_out[(size_t)b * (p.k + 1) + a] = y;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(NT_DRAW) void k_draw_tiles(Params p) {
    __shared__ StochFin<NT_DRAW> sm;
    const int b = blockIdx.x / p.SD;
    const int sd = blockIdx.x - b * p.SD;
    if (p.active && p.active[b] == 2) return;  // drawn by the capped pass
    draw_tiles_group<DT, VEC>(p, b, sd, p.SD, sm);
}

struct ExitStatsSmem {
    Scratch<NT_ROW> sc;
    unsigned long long masks[kExitMaxB / 64];
    int map[kExitMaxB];
};

// Group `group` of `ngroups` persistent statistics groups (all threads call).
template <int DT, bool VEC>
__device__ void exit_stats_groups(const Params& p, int group, int ngroups, ExitStatsSmem& es) {
    constexpr int NW = NT_ROW / 64;
    Scratch<NT_ROW>& sc = es.sc;
    unsigned long long* masks = es.masks;
    int* map = es.map;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Compact the still-accepting sequences, in index order (the same map in
    // every workgroup): one ballot per 64 flags, then popcount prefixes.
    const int ng = (p.B + 63) / 64;
    for (int g = wave; g < ng; g += NW) {
        const int bb = g * 64 + lane;
        const unsigned long long m = __ballot(bb < p.B && p.active[bb] == 1);
        if (lane == 0) masks[g] = m;
    }
    __syncthreads();
    int n_active = 0;
    for (int g = 0; g < ng; ++g) n_active += __popcll(masks[g]);
    for (int g = wave; g < ng; g += NW) {
        int pre = 0;
        for (int h = 0; h < g; ++h) pre += __popcll(masks[h]);
        const unsigned long long m = masks[g];
        if ((m >> lane) & 1ull) map[pre + __popcll(m & ((1ull << lane) - 1ull))] = g * 64 + lane;
    }
    // rows left per sequence: at most 2 (k - min(exit_pairs, k)) + 1
    const int rows2 = 2 * (p.k - min(p.exit_pairs, p.k)) + 1;
    int S2, slice_len;
    exit_slicing<DT, VEC>(p, n_active, rows2, S2, slice_len);
    __syncthreads();
    const int per_seq = rows2 * S2;
    const long long items = (long long)n_active * per_seq;
    for (long long it = group; it < items; it += ngroups) {
        const int j = (int)(it / per_seq);
        const int rem = (int)(it - (long long)j * per_seq);
        const int r = rem / S2;
        const int sl = rem - r * S2;
        const int b = map[j];
        const int kb = seq_of(p, b).k;
        const Seq sq = seq_from(p, b, min(p.exit_pairs, kb));
        if (r >= 2 * sq.k + 1) continue;  // row absent (ragged): uniform in the group
        // the row's index in the sequence's full layout (draft rows after k_b + 1)
        const int ra = r <= sq.k ? sq.pos0 + r : kb + 1 + sq.pos0 + (r - sq.k - 1);
        const int v0 = sl * slice_len;
        const int v1 = min(p.V, v0 + slice_len);
        const Row<DT, VEC> row(stoch_row<DT>(p, sq, r) + (size_t)v0 * elem_bytes<DT>(), v1 - v0);
        SoftAcc acc;
        stream_softmax<DT, VEC, NT_ROW>(row, p.c, acc);
        float R, Z;
        wave_softmax(acc, R, Z);
        if (lane == 0) {
            sc.f[wave] = R;
            sc.g[wave] = Z;
        }
        __syncthreads();
        float* dst = p.part + ((size_t)b * p.rows_per_seq + ra) * p.S * 2;
        if (tid == 0) {
            float RR = sc.f[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) RR = fmaxf(RR, sc.f[w]);
            float ZZ = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) ZZ += sc.g[w] * fast_exp2(sc.f[w] - RR);
            dst[sl * 2] = RR;
            dst[sl * 2 + 1] = ZZ;
        }
        if (sl == 0)
            for (int e = S2 + tid; e < p.S; e += NT_ROW) {
                dst[e * 2] = -FLT_MAX;
                dst[e * 2 + 1] = 0.0f;
            }
        __syncthreads();  // sc is reused by the next item
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(NT_ROW) void k_exit_stats(Params p) {
    __shared__ ExitStatsSmem es;
    zero_draw_counters(p);
    exit_stats_groups<DT, VEC>(p, blockIdx.x, gridDim.x, es);
}

// Plain sampling of row r from the statistics kernel's slice normalisers:
// the slice whose cumulative weight first exceeds u * total, then the inverse
// CDF inside that slice at the uniform's position within the slice's weight.
// Only the slice is read again.  All threads call.
template <int DT, bool VEC, int NT>
__device__ int slice_draw(const Params& p, const Seq& sq, int b, int r, float u,
                          StochFin<NT>& sm) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int S = p.S;  // <= kMaxSlices = 64: one wave holds every slice
    const float* ps = p.part + ((size_t)b * p.rows_per_seq + r) * S * 2;
    if (tid < 64) {
        const float Rj = lane < S ? ps[2 * lane] : -FLT_MAX;
        const float Zj = lane < S ? ps[2 * lane + 1] : 0.0f;
        const float Rm = wave_max(Rj);
        const float Wj = lane < S ? Zj * fast_exp2(Rj - Rm) : 0.0f;
        const float incl = wave_incl_scan(Wj);
        const float T = u * __shfl(incl, 63);
        const unsigned long long hit = __ballot(lane < S && Wj > 0.0f && incl > T);
        int js;
        float rf;
        if (hit) {
            js = __ffsll(hit) - 1;
            const float w = __shfl(Wj, js);
            rf = fmaxf(0.0f, (T - (__shfl(incl, js) - w)) / w);
        } else {
            // rounding left u * total at or above the last sum: the last
            // slice with weight (whose own draw then falls back to its last
            // positive-weight index)
            const unsigned long long pos = __ballot(lane < S && Wj > 0.0f);
            js = pos ? 63 - __clzll(pos) : -1;
            rf = 1.0f;
        }
        if (lane == 0) {
            sm.js = js;
            sm.rf = rf;
            sm.Rm = Rm;
        }
    }
    __syncthreads();
    const int js = sm.js;
    if (js < 0) return 0;
    const int v0 = js * p.slice_len;
    const int v1 = min(p.V, v0 + p.slice_len);
    const char* base = stoch_row<DT>(p, sq, r) + (size_t)v0 * elem_bytes<DT>();
    const TargetW tw{p.c, -sm.Rm};
    float total;
    return v0 + inverse_cdf_row<DT, VEC, false, NT>(base, nullptr, v1 - v0, tw, sm.rf, &total,
                                                   sm.tile_part, sm.tile_excl, sm.sc);
}

// Plain sampling in one pass, one row per 1024-thread workgroup: while the
// row streams, every thread keeps -- besides its running normaliser -- the
// sum it added in each round of NT chunks (relative to its current
// reference, rescaled with it), so the per-round sums the inverse CDF scans
// come from registers instead of a second pass over the row; only the round
// holding the draw is read again.  Rows of at most SAMPLE_ROUNDS rounds.
constexpr int SAMPLE_ROUNDS = kSampleSeqRounds;
constexpr int SAMPLE_UNROLL = 4;  // rounds loaded per step (SAMPLE_ROUNDS a multiple)

// HOLD (rows of at most kSampleHeldRounds rounds): every thread also keeps
// the chunks it streamed, so the round holding the draw is scanned from
// registers instead of being read again.
template <int DT, bool VEC, int NT, bool HOLD>
__global__ __launch_bounds__(NT) void k_sample_seq(Params p) {
    using C = Chunk<DT, VEC>;
    constexpr int NW = NT / 64;
    constexpr int E = C::E;
    constexpr int RMAX = HOLD ? kSampleHeldRounds : SAMPLE_ROUNDS;
    static_assert(RMAX % SAMPLE_UNROLL == 0, "whole steps");
    __shared__ StochFin<NT> sm;
    __shared__ float wref[NW];
    const int b = blockIdx.x;
    const Seq sq = seq_of(p, b);
    const int V = p.V;
    const float c = p.c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Row<DT, VEC> row(stoch_row<DT>(p, sq, 0), V);
    const TileGeom g = tile_geom<NT>(row.nch, VEC ? V - row.nch * E : 0);
    float rs[RMAX];  // this thread's sum in each round
    HeldRounds<C, HOLD ? RMAX : 1> held;
    SoftAcc acc;
#pragma unroll
    for (int q = 0; q < RMAX / SAMPLE_UNROLL; ++q) {
        if (q * SAMPLE_UNROLL < g.rounds) {  // uniform
            C buf[SAMPLE_UNROLL];
#pragma unroll
            for (int u = 0; u < SAMPLE_UNROLL; ++u) {
                const int ci = (q * SAMPLE_UNROLL + u) * NT + tid;
                if (ci < g.nch) buf[u] = row.chunk(ci);
                else buf[u].set_neg_inf();
            }
            float gm = -INFINITY;
#pragma unroll
            for (int u = 0; u < SAMPLE_UNROLL; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) gm = fmaxf(gm, buf[u].get(e));
            const float gmc = gm * c;
            if (gmc > acc.ref + RESCALE_MARGIN) {
                const float f = fast_exp2(acc.ref - gmc);
                acc.s0 *= f;
#pragma unroll
                for (int j = 0; j < q * SAMPLE_UNROLL; ++j) rs[j] *= f;
                acc.ref = gmc;
            }
            const float nref = -acc.ref;
#pragma unroll
            for (int u = 0; u < SAMPLE_UNROLL; ++u) {
                float su = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) su += fast_exp2(fmaf(buf[u].get(e), c, nref));
                rs[q * SAMPLE_UNROLL + u] = su;
                acc.s0 += su;
            }
            if constexpr (HOLD) store_held<0, RMAX, SAMPLE_UNROLL>(held, q * SAMPLE_UNROLL, buf);
        } else {
#pragma unroll
            for (int u = 0; u < SAMPLE_UNROLL; ++u) rs[q * SAMPLE_UNROLL + u] = 0.0f;
        }
    }
    float trail = 0.0f;
    if (tid < g.rem) {  // the row's last V mod E logits
        const float x = row.elem(g.nch * E + tid);
        if (x * c > acc.ref + RESCALE_MARGIN) {
            const float f = fast_exp2(acc.ref - x * c);
#pragma unroll
            for (int j = 0; j < RMAX; ++j) rs[j] *= f;
            acc.ref = x * c;
        }
        trail = fast_exp2(fmaf(x, c, -acc.ref));
    }
    // the row's reference R (block max of the thread references)
    const float wr = wave_max(acc.ref);
    if (lane == 0) wref[wave] = wr;
    for (int t = tid; t < g.nt_all * NW; t += NT) sm.tile_part[t] = 0.0f;
    __syncthreads();
    float R = wref[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) R = fmaxf(R, wref[w]);
    const float f = fast_exp2(acc.ref - R);
    // per-round sums relative to R: the inverse CDF's tiles (one round each)
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
        if (j < g.rounds) {  // uniform
            const float w = wave_sum(rs[j] * f);
            if (lane == 0) sm.tile_part[j * NW + wave] = w;
        }
    }
    if (g.rem > 0) {
        const float w = wave_sum(trail * f);
        if (lane == 0) sm.tile_part[g.ntiles * NW + wave] = w;
    }
    __syncthreads();
    const TargetW tw{c, -R};
    float total;
    int y;
    if constexpr (HOLD)
        y = cdf_select<DT, VEC, false, NT>(row, row, tw, p.u_sample[b], g, &total, sm.tile_part,
                                           sm.tile_excl, sm.sc, held);
    else
        y = cdf_select<DT, VEC, false, NT>(row, row, tw, p.u_sample[b], g, &total, sm.tile_part,
                                           sm.tile_excl, sm.sc);
    if (tid == 0) {
        p.tokens_out[b] = y;
        if (p.accept_len) p.accept_len[b] = 0;
    }
}

// Plain sampling after the statistics kernel (no decisions to take): one
// workgroup per row draws from its slice statistics.
constexpr int NT_SAMPLE = 512;

template <int DT, bool VEC>
__global__ __launch_bounds__(NT_SAMPLE) void k_sample_draw(Params p) {
    __shared__ StochFin<NT_SAMPLE> sm;
    const int b = blockIdx.x;
    const Seq sq = seq_of(p, b);
    const int y = slice_draw<DT, VEC, NT_SAMPLE>(p, sq, b, 0, p.u_sample[b], sm);
    if (threadIdx.x == 0) {
        p.tokens_out[b] = y;
        if (p.accept_len) p.accept_len[b] = 0;
    }
}

__global__ __launch_bounds__(NT_FIN) void k_greedy_finish(Params p) {
    __shared__ GreedyFin<NT_FIN> sm;
    const int b = blockIdx.x;
    const int S = p.S;
    const Seq sq = seq_of(p, b);
    const float* part = p.part + (size_t)b * p.rows_per_seq * S * 2;
    for (int r = threadIdx.x; r < p.G * (sq.k + 1); r += NT_FIN) {
        float best = part[(r * S) * 2];
        int idx = __float_as_int(part[(r * S) * 2 + 1]);
        for (int j = 1; j < S; ++j) {
            const float m = part[(r * S + j) * 2];
            if (m > best) {  // earlier slices hold lower indices: they win ties
                best = m;
                idx = __float_as_int(part[(r * S + j) * 2 + 1]);
            }
        }
        sm.g[r] = idx;
    }
    __syncthreads();
    finish_greedy<NT_FIN>(p, b, sq, sm);
}

// ------------------------------------------------------------------------
// Greedy verification of a draft tree per sequence (N nodes; node 0 is the
// root, parents[j] < j).  After the row statistics give the argmax g of every
// node's row, one workgroup per sequence (one thread per node) decides:
// node j is accepted when every edge on its root path matches (the child's
// token equals the argmax of the parent's row).  Pointer jumping folds the
// path in ceil(log2 N) rounds: anc[j] is the node the fold has reached,
// ok[j] and dep[j] the AND of the edge tests and the edge count from j up to
// anc[j].  The deepest accepted node wins, lowest index on ties.  A parent
// outside [0, j) (a malformed tree) makes the node unaccepted.
constexpr int kMaxTreeNodes = kMaxRowsPerSeq;

struct TreeSmem {
    int g[kMaxTreeNodes];
    int par[kMaxTreeNodes];
    int tok[kMaxTreeNodes];
    int anc[kMaxTreeNodes];
    int ok[kMaxTreeNodes];
    int dep[kMaxTreeNodes];
    Scratch<NT_FIN> sc;
};

__global__ __launch_bounds__(NT_FIN) void k_tree_finish(Params p) {
    __shared__ TreeSmem sm;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int N = p.rows_per_seq, S = p.S;
    const float* part = p.part + (size_t)b * N * S * 2;
    const int32_t* par = p.parents + (size_t)b * N;
    const int32_t* tok = p.tokens_in + (size_t)b * N;
    for (int j = tid; j < N; j += NT_FIN) {
        float best = part[(j * S) * 2];
        int idx = __float_as_int(part[(j * S) * 2 + 1]);
        for (int s = 1; s < S; ++s) {
            const float m = part[(j * S + s) * 2];
            if (m > best) {  // earlier slices hold lower indices: they win ties
                best = m;
                idx = __float_as_int(part[(j * S + s) * 2 + 1]);
            }
        }
        sm.g[j] = idx;
        sm.par[j] = par[j];
        sm.tok[j] = tok[j];
    }
    __syncthreads();
    for (int j = tid; j < N; j += NT_FIN) {
        const int pj = sm.par[j];
        const bool valid = j > 0 && pj >= 0 && pj < j;
        sm.anc[j] = valid ? pj : 0;
        sm.ok[j] = j == 0 ? 1 : (valid && sm.tok[j] == sm.g[pj]);
        sm.dep[j] = j == 0 ? 0 : 1;
    }
    __syncthreads();
    for (int span = 1; span < N; span <<= 1) {
        int o[kMaxTreeNodes / NT_FIN], d[kMaxTreeNodes / NT_FIN], a2[kMaxTreeNodes / NT_FIN];
#pragma unroll
        for (int u = 0; u < kMaxTreeNodes / NT_FIN; ++u) {
            const int j = tid + u * NT_FIN;
            if (j < N) {
                const int a = sm.anc[j];
                o[u] = sm.ok[a];
                d[u] = sm.dep[a];
                a2[u] = sm.anc[a];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kMaxTreeNodes / NT_FIN; ++u) {
            const int j = tid + u * NT_FIN;
            if (j < N) {
                sm.ok[j] &= o[u];
                sm.dep[j] += d[u];
                sm.anc[j] = a2[u];
            }
        }
        __syncthreads();
    }
    // deepest accepted node, lowest index on ties: maximise dep * 2048 + (2047 - j)
    int key = -1;
    for (int j = tid; j < N; j += NT_FIN)
        if (sm.ok[j]) key = max(key, sm.dep[j] * 2048 + (2047 - j));
    {
        const int lane = tid & 63, wave = tid >> 6;
        key = wave_max_i(key);
        if (lane == 0) sm.sc.j[wave] = key;
        __syncthreads();
        key = sm.sc.j[0];
#pragma unroll
        for (int w = 1; w < NT_FIN / 64; ++w) key = max(key, sm.sc.j[w]);
    }
    const int best = 2047 - (key & 2047);  // the root (key 2047) is always accepted
    const int d = key >> 11;
    int32_t* out_t = p.tokens_out + (size_t)b * N;
    int32_t* out_p = p.path + (size_t)b * N;
    for (int i = tid; i < N; i += NT_FIN)
        if (i > d) {
            out_t[i] = -1;
            out_p[i] = -1;
        }
    if (tid == 0) {
        // walk back from the winner: its ancestors are all accepted, so the
        // parents on the way are valid and strictly decreasing
        int j = best;
        for (int i = d; i >= 0; --i) {
            out_p[i] = j;
            if (i > 0) out_t[i - 1] = sm.tok[j];
            j = i > 0 ? sm.par[j] : 0;
        }
        out_t[d] = sm.g[best];
        p.accept_len[b] = d;
    }
}

// Commit of a verified step: one thread per sequence appends its emitted
// tokens to its history (up to the capacity), advances its length and writes
// the last emitted token into the next step's input slot.
__global__ __launch_bounds__(256) void k_commit(const int32_t* __restrict__ accept_len,
                                                const int32_t* __restrict__ tokens, int B, int W,
                                                int32_t* seq_len, int32_t* history,
                                                long long history_stride, int capacity,
                                                int32_t* next_token, long long next_stride) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= B) return;
    int a = accept_len[b];
    a = a < 0 ? 0 : (a >= W ? W - 1 : a);  // keeps a malformed value inside the row
    const int32_t* t = tokens + (size_t)b * W;
    int L = seq_len[b];
    if (L < 0) L = 0;
    int32_t* h = history + (size_t)b * history_stride;
    for (int j = 0; j <= a && L < capacity; ++j) h[L++] = t[j];
    seq_len[b] = L;
    next_token[(size_t)b * next_stride] = t[a];
}

// ------------------------------------------------------------------------
template <typename K>
static int launch1(K kernel, const Params& p, long long grid, int block, void* stream) {
    Params pc = p;
    void* args[] = {&pc};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                dim3(block), args, 0, static_cast<hipStream_t>(stream));
}

// The row-split statistics kernel, in workgroups of NT_ROW_WIDE threads when
// a slice has kRowStatsWideChunks chunks or more, else NT_ROW.
template <int DT, bool VEC, bool STOCH>
static int launch_row_stats(const Params& p, void* stream) {
    const long long rows = STOCH && p.slice_draw ? (p.B + 7LL) / 8 * 8 : p.B;  // see k_row_stats
    const long long items = rows * p.rows_per_seq * p.S;
    const int chunks = p.slice_len / Chunk<DT, VEC>::E;
    return chunks >= kRowStatsWideChunks
               ? launch1(k_row_stats<DT, VEC, STOCH, NT_ROW_WIDE>, p, items, NT_ROW_WIDE, stream)
               : launch1(k_row_stats<DT, VEC, STOCH, NT_ROW>, p, items, NT_ROW, stream);
}

template <int DT, bool VEC>
static int launch_stochastic_t(const Params& p, bool seq, void* stream) {
    if (seq && p.k == 0 && !p.cu) {  // plain sampling in one pass
        const int nch = p.V / Chunk<DT, VEC>::E;
        const bool wide = p.B >= kSeqWideMinB;
        const bool hold = (nch + (wide ? NT_SEQ_WIDE : NT_SEQ) - 1) / (wide ? NT_SEQ_WIDE : NT_SEQ) <=
                          kSampleHeldRounds;
        if (wide)
            return hold ? launch1(k_sample_seq<DT, VEC, NT_SEQ_WIDE, true>, p, p.B, NT_SEQ_WIDE, stream)
                        : launch1(k_sample_seq<DT, VEC, NT_SEQ_WIDE, false>, p, p.B, NT_SEQ_WIDE,
                                  stream);
        return hold ? launch1(k_sample_seq<DT, VEC, NT_SEQ, true>, p, p.B, NT_SEQ, stream)
                    : launch1(k_sample_seq<DT, VEC, NT_SEQ, false>, p, p.B, NT_SEQ, stream);
    }
    constexpr int NHX = held_rounds_exit(NT_SEQ), NHXW = held_rounds_exit(NT_SEQ_WIDE);
    if (seq && p.active) {  // capped early exit, then the spread continuation
        const bool wide = p.B >= kSeqWideMinB;
        int e = wide ? launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ_WIDE, NHXW, false>, p, p.B,
                               NT_SEQ_WIDE, stream)
                     : launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ, NHX, false>, p, p.B, NT_SEQ,
                               stream);
        if (e) return e;
        e = launch1(k_exit_stats<DT, VEC>, p, kExitStatsGrid, NT_ROW, stream);
        if (e) return e;
        return launch1(k_draw_tiles<DT, VEC>, p, (long long)p.B * p.SD, NT_DRAW, stream);
    }
    if (seq && p.B >= kSeqWideMinB) {
        // long rows, two groups on most CUs: the pair streamed last held on
        // chip, in the early exit and in the full read in position order
        constexpr int NHL = kSeqWideLongHeldRounds;
        const long long row_bytes = (long long)p.V * elem_bytes<DT>();
        const bool held = p.B >= kSeqWideLongMinB && p.B <= kSeqWideHoldMaxB &&
                          row_bytes >= kSeqWideLongMinRowBytes;
        if (!p.dbg)
            return held ? launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ_WIDE, NHL, false>, p, p.B,
                                  NT_SEQ_WIDE, stream)
                        : launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ_WIDE, NHXW, false>, p, p.B,
                                  NT_SEQ_WIDE, stream);
        if (held)
            return launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ_WIDE, NHL, true>, p, p.B,
                           NT_SEQ_WIDE, stream);
        if (p.B > kSeqWideHoldMaxB)
            return launch1(k_stochastic_seq<DT, VEC, NT_SEQ_WIDE, 0>, p, p.B, NT_SEQ_WIDE, stream);
        constexpr int NH = kSeqWideHeldRounds;
        return launch1(k_stochastic_seq<DT, VEC, NT_SEQ_WIDE, NH>, p, p.B, NT_SEQ_WIDE, stream);
    }
    // one group per sequence, up to 256: the early exit, and the full read
    // in position order (the same kernel, with p.dbg)
    if (seq)
        return p.dbg ? launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ, NHX, true>, p, p.B, NT_SEQ,
                               stream)
                     : launch1(k_stochastic_seq_exit<DT, VEC, NT_SEQ, NHX, false>, p, p.B, NT_SEQ,
                               stream);
    int e = launch_row_stats<DT, VEC, true>(p, stream);
    if (e) return e;
    if (p.slice_draw) return launch1(k_sample_draw<DT, VEC>, p, p.B, NT_SAMPLE, stream);
    if (p.B >= kSeqWideMinB)
        return launch1(k_stochastic_finish<DT, VEC, NT_SEQ_WIDE>, p, p.B, NT_SEQ_WIDE, stream);
    if (p.B >= kFinishOneGroupMinB)
        return launch1(k_stochastic_finish<DT, VEC, NT_SEQ>, p, p.B, NT_SEQ, stream);
    return launch1(k_draw_tiles<DT, VEC>, p, (long long)p.B * p.SD, NT_DRAW, stream);
}

template <int DT, bool VEC>
static int launch_greedy_t(const Params& p, bool seq, void* stream) {
    if (seq && p.B >= kSeqWideMinB)
        return launch1(k_greedy_seq<DT, VEC, NT_SEQ_WIDE>, p, p.B, NT_SEQ_WIDE, stream);
    if (seq) return launch1(k_greedy_seq<DT, VEC, NT_SEQ>, p, p.B, NT_SEQ, stream);
    int e = launch_row_stats<DT, VEC, false>(p, stream);
    if (e) return e;
    return launch1(k_greedy_finish, p, p.B, NT_FIN, stream);
}

int launch_stochastic(const Params& p, int dtype, bool vec, bool seq, void* stream) {
    if (dtype == 1)
        return vec ? launch_stochastic_t<1, true>(p, seq, stream)
                   : launch_stochastic_t<1, false>(p, seq, stream);
    return vec ? launch_stochastic_t<0, true>(p, seq, stream)
               : launch_stochastic_t<0, false>(p, seq, stream);
}

int launch_greedy(const Params& p, int dtype, bool vec, bool seq, void* stream) {
    if (dtype == 1)
        return vec ? launch_greedy_t<1, true>(p, seq, stream) : launch_greedy_t<1, false>(p, seq, stream);
    return vec ? launch_greedy_t<0, true>(p, seq, stream) : launch_greedy_t<0, false>(p, seq, stream);
}

template <int DT, bool VEC>
static int launch_tree_t(const Params& p, void* stream) {
    int e = launch_row_stats<DT, VEC, false>(p, stream);
    if (e) return e;
    return launch1(k_tree_finish, p, p.B, NT_FIN, stream);
}

int launch_tree(const Params& p, int dtype, bool vec, void* stream) {
    if (dtype == 1) return vec ? launch_tree_t<1, true>(p, stream) : launch_tree_t<1, false>(p, stream);
    return vec ? launch_tree_t<0, true>(p, stream) : launch_tree_t<0, false>(p, stream);
}

int launch_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W,
                  int32_t* seq_len, int32_t* history, long long history_stride, int capacity,
                  int32_t* next_token, long long next_stride, void* stream) {
    // The launch's own status: an error left by the caller's earlier HIP work
    // is neither reported here nor cleared.
    void* args[] = {&accept_len, &tokens, &B, &W, &seq_len, &history, &history_stride,
                    &capacity, &next_token, &next_stride};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(k_commit),
                                dim3((unsigned)((B + 255) / 256)), dim3(256), args, 0,
                                static_cast<hipStream_t>(stream));
}

}  // namespace sv
