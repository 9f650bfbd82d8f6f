// sv_kernels.hip -- the verification step on gfx950 (MI355X).
//
// One kernel per decision rule.  Every workgroup first streams one slice of
// one logit row from HBM once, with 16-byte loads, and reduces it to 8 bytes
// of statistics:
//   stochastic: a reference R and Z = sum_v 2^(x_v*c - R), c = log2(e)/T,
//               kept with a lazily raised R so the exponentials never
//               overflow (an online softmax normaliser);
//   greedy:     the slice maximum and the lowest index holding it.
// The workgroup then bumps its sequence's arrival counter; the one that
// arrives last merges the sequence's statistics and finishes the sequence on
// the spot: acceptance test, accept-prefix scan, the extra token, outputs.
// Nothing is a dense contraction, so no MFMA is used; the pass is bound by
// HBM bandwidth (and, for bfloat16 stochastic rows, by VALU/exp issue).
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

constexpr int NT = 256;        // threads per workgroup: four wave64s
constexpr int NW = NT / 64;    // waves per workgroup
constexpr int UNROLL = 8;      // 16-byte loads in flight per lane (stream)
constexpr int TUNROLL = 4;     // row pairs in flight per lane (tail)
constexpr int MAX_TILES = 256; // inverse-CDF tiles held in LDS
// How far (in log2 units) the streaming reference may sit below a new
// maximum before the running sum is rescaled.  Terms then stay <= 2^16.
constexpr float RESCALE_MARGIN = 16.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------
// Element access.  DT 0 = float32, 1 = bfloat16.  VEC: 16-byte chunks
// (8 bf16 or 4 f32), else one element per load.
template <int DT, bool VEC>
struct Chunk;

template <>
struct Chunk<1, true> {
    static constexpr int E = 8;
    uint4 w;
    __device__ __forceinline__ static Chunk load(const char* row, int i) {
        Chunk c;
        c.w = reinterpret_cast<const uint4*>(row)[i];
        return c;
    }
    __device__ __forceinline__ static Chunk neg_inf() {
        Chunk c;
        c.w = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
        return c;
    }
    __device__ __forceinline__ float get(int j) const {
        uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
        return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    }
};

template <>
struct Chunk<0, true> {
    static constexpr int E = 4;
    float4 w;
    __device__ __forceinline__ static Chunk load(const char* row, int i) {
        Chunk c;
        c.w = reinterpret_cast<const float4*>(row)[i];
        return c;
    }
    __device__ __forceinline__ static Chunk neg_inf() {
        Chunk c;
        c.w = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        return c;
    }
    __device__ __forceinline__ float get(int j) const {
        return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
    }
};

template <>
struct Chunk<1, false> {
    static constexpr int E = 1;
    uint32_t w;
    __device__ __forceinline__ static Chunk load(const char* row, int i) {
        Chunk c;
        c.w = (uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16;
        return c;
    }
    __device__ __forceinline__ static Chunk neg_inf() {
        Chunk c;
        c.w = 0xff800000u;
        return c;
    }
    __device__ __forceinline__ float get(int) const { return __uint_as_float(w); }
};

template <>
struct Chunk<0, false> {
    static constexpr int E = 1;
    float w;
    __device__ __forceinline__ static Chunk load(const char* row, int i) {
        Chunk c;
        c.w = reinterpret_cast<const float*>(row)[i];
        return c;
    }
    __device__ __forceinline__ static Chunk neg_inf() {
        Chunk c;
        c.w = -INFINITY;
        return c;
    }
    __device__ __forceinline__ float get(int) const { return w; }
};

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int v) {
    if (DT == 1) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[v] << 16);
    return reinterpret_cast<const float*>(row)[v];
}

template <int DT>
constexpr int elem_bytes() { return DT == 1 ? 2 : 4; }

// ------------------------------------------------------------------------
// Wave / block reductions (wave64).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float n = __shfl_up(v, o);
        if (lane >= o) v += n;
    }
    return v;
}

struct BlockScratch {
    float f[NW];
    float g[NW];
    int i[NW];
    int j[NW];
};

// Block-wide exclusive prefix sum; *total receives the block sum.  All
// threads must call.
__device__ __forceinline__ float block_excl_scan(float v, float* total, BlockScratch& sc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float incl = wave_incl_scan(v);
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0f;
    if (lane == 63) sc.f[wave] = incl;
    __syncthreads();
    float off = 0.0f, tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) off += sc.f[w];
        tot += sc.f[w];
    }
    __syncthreads();
    *total = tot;
    return off + excl;
}

__device__ __forceinline__ int block_min_i(int v, BlockScratch& sc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_min_i(v);
    if (lane == 0) sc.i[wave] = v;
    __syncthreads();
    int r = sc.i[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = min(r, sc.i[w]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ int block_max_i(int v, BlockScratch& sc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_i(v);
    if (lane == 0) sc.j[wave] = v;
    __syncthreads();
    int r = sc.j[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = max(r, sc.j[w]);
    __syncthreads();
    return r;
}

// ------------------------------------------------------------------------
// Streaming pass, stochastic: (R, Z) of elements [v0, v1) of one row with
// Z = sum 2^(x*c - R).  Result valid in thread 0.
template <int DT, bool VEC>
__device__ __forceinline__ void stream_softmax_stats(const char* row, int v0, int v1, float c,
                                                     float* R_out, float* Z_out, BlockScratch& sc) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    const char* base = row + (size_t)v0 * elem_bytes<DT>();
    const int n = v1 - v0;
    const int nch = n / E;
    const int tid = threadIdx.x;
    float ref = -FLT_MAX, s0 = 0.0f, s1 = 0.0f;

    auto consume = [&](const C* buf, int cnt) {
        float gm = -INFINITY;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (u < cnt) {
#pragma unroll
                for (int e = 0; e < E; ++e) gm = fmaxf(gm, buf[u].get(e));
            }
        }
        const float gmc = gm * c;
        if (gmc > ref + RESCALE_MARGIN) {
            const float sc_ = fast_exp2(ref - gmc);
            s0 *= sc_;
            s1 *= sc_;
            ref = gmc;
        }
        const float nref = -ref;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (u < cnt) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float t = fast_exp2(fmaf(buf[u].get(e), c, nref));
                    if (e & 1) s1 += t;
                    else s0 += t;
                }
            }
        }
    };

    const int step = NT * UNROLL;
    const int full_end = (nch / step) * step;
    for (int i = tid; i < full_end; i += step) {
        C buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) buf[u] = C::load(base, i + u * NT);
        consume(buf, UNROLL);
    }
    if (full_end < nch) {
        C buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = full_end + tid + u * NT;
            buf[u] = idx < nch ? C::load(base, idx) : C::neg_inf();
        }
        consume(buf, UNROLL);
    }
    // Elements past the last whole chunk (vector path only).
    if (VEC) {
        const int rem = n - nch * E;
        if (tid < rem) {
            const float x = load_elem<DT>(base, nch * E + tid);
            const float xc = x * c;
            if (xc > ref + RESCALE_MARGIN) {
                const float sc_ = fast_exp2(ref - xc);
                s0 *= sc_;
                s1 *= sc_;
                ref = xc;
            }
            s0 += fast_exp2(fmaf(x, c, -ref));
        }
    }
    // Merge (ref, sum) across the block.
    const int lane = tid & 63, wave = tid >> 6;
    float R = wave_max(ref);
    float S = wave_sum((s0 + s1) * fast_exp2(ref - R));
    if (lane == 0) {
        sc.f[wave] = R;
        sc.g[wave] = S;
    }
    __syncthreads();
    if (tid == 0) {
        float RR = sc.f[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) RR = fmaxf(RR, sc.f[w]);
        float SS = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) SS += sc.g[w] * fast_exp2(sc.f[w] - RR);
        *R_out = RR;
        *Z_out = SS;
    }
}

// Streaming pass, greedy: maximum of elements [v0, v1) and the lowest
// (absolute) index holding it.  Result valid in thread 0.
template <int DT, bool VEC>
__device__ __forceinline__ void stream_argmax(const char* row, int v0, int v1, float* M_out,
                                              int* I_out, BlockScratch& sc) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    const char* base = row + (size_t)v0 * elem_bytes<DT>();
    const int n = v1 - v0;
    const int nch = n / E;
    const int rem = VEC ? n - nch * E : 0;
    const int tid = threadIdx.x;
    // best: this thread's maximum; bpos: element offset (from v0) of the
    // chunk that first reached it, or of a single trailing element when
    // bpos >= nch*E.
    float best = -INFINITY;
    int bpos = tid < nch ? tid * E : (tid < rem ? nch * E + tid : INT_MAX);

    const int step = NT * UNROLL;
    const int full_end = (nch / step) * step;
    for (int i = tid; i < full_end; i += step) {
        C buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) buf[u] = C::load(base, i + u * NT);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float m = buf[u].get(0);
#pragma unroll
            for (int e = 1; e < E; ++e) m = fmaxf(m, buf[u].get(e));
            if (m > best) {
                best = m;
                bpos = (i + u * NT) * E;
            }
        }
    }
    if (full_end < nch) {
        C buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = full_end + tid + u * NT;
            buf[u] = idx < nch ? C::load(base, idx) : C::neg_inf();
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float m = buf[u].get(0);
#pragma unroll
            for (int e = 1; e < E; ++e) m = fmaxf(m, buf[u].get(e));
            if (m > best) {
                best = m;
                bpos = (full_end + tid + u * NT) * E;
            }
        }
    }
    if (VEC && tid < rem) {
        const float x = load_elem<DT>(base, nch * E + tid);
        if (x > best) {
            best = x;
            bpos = nch * E + tid;
        }
    }
    // Lowest index inside the winning chunk.
    int idx = INT_MAX;
    if (bpos < nch * E) {
        const C ch = C::load(base, bpos / E);
#pragma unroll
        for (int e = E - 1; e >= 0; --e)
            if (ch.get(e) == best) idx = bpos + e;
    } else if (bpos != INT_MAX) {
        idx = bpos;
    }
    // Block argmax: larger value wins, lower index on equal values.
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o);
        const int oi = __shfl_xor(idx, o);
        if (ob > best || (ob == best && oi < idx)) {
            best = ob;
            idx = oi;
        }
    }
    if (lane == 0) {
        sc.f[wave] = best;
        sc.i[wave] = idx;
    }
    __syncthreads();
    if (tid == 0) {
        float bb = sc.f[0];
        int ii = sc.i[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            if (sc.f[w] > bb || (sc.f[w] == bb && sc.i[w] < ii)) {
                bb = sc.f[w];
                ii = sc.i[w];
            }
        *M_out = bb;
        *I_out = ii == INT_MAX ? v0 : v0 + ii;
    }
}

// ------------------------------------------------------------------------
// Arrival: thread 0 publishes this workgroup's statistics and counts in; the
// workgroup that completes its sequence returns true (in every thread).
__device__ __forceinline__ bool arrive(const Params& p, int b, int item, float a, float bv,
                                       int* flag) {
    const int per_seq = p.rows_per_seq * p.S;
    if (threadIdx.x == 0) {
        float* dst = p.part + ((size_t)b * per_seq + item) * 2;
        dst[0] = a;
        dst[1] = bv;
        __threadfence();
        const int old = atomicAdd(&p.counters[b], 1);
        *flag = (old == per_seq - 1);
        if (*flag) __threadfence();
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (last) __threadfence();
    return last;
}

// The finishing workgroup has read its sequence's statistics; zero them so
// the whole workspace is zero again when the call completes (the counter is
// reset separately).  A later call with another shape may place its counters
// where these statistics were.
__device__ __forceinline__ void clear_partials(const Params& p, int b) {
    const int n = p.rows_per_seq * p.S * 2;
    float* dst = p.part + (size_t)b * n;
    for (int j = threadIdx.x; j < n; j += NT) dst[j] = 0.0f;
}

// ------------------------------------------------------------------------
// Inverse-CDF draw over one row (or a row pair) with weights W(t[, d]):
// the first index whose cumulative weight exceeds r * total; if rounding
// leaves none, the last index with positive weight (0 if there is none).
// The row is cut into tiles of NT*m chunks; pass A sums each tile, a block
// scan over tile sums finds the tile holding the draw, pass B scans inside
// that tile.  *total receives the total weight.  All threads must call.
template <int DT, bool VEC, bool PAIR, typename W>
__device__ int inverse_cdf_row(const char* trow, const char* drow, int V, const W& wf, float r,
                               float* total_out, float* tile_part, float* tile_excl,
                               BlockScratch& sc) {
    using C = Chunk<DT, VEC>;
    constexpr int E = C::E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = V / E;
    const int rem = VEC ? V - nch * E : 0;
    const int rounds = (nch + NT - 1) / NT;         // block-wide rounds of chunks
    const int m = max(1, (rounds + MAX_TILES - 1) / MAX_TILES);  // rounds per tile
    const int ntiles = (rounds + m - 1) / m;
    const int nt_all = ntiles + (rem > 0 ? 1 : 0);  // trailing elements = last tile

    for (int t = tid; t < nt_all * NW; t += NT) tile_part[t] = 0.0f;
    __syncthreads();

    // Pass A: per-tile partial sums, per wave.
    int lastpos = -1;
    for (int r0 = 0; r0 < rounds; r0 += TUNROLL) {
        C tb[TUNROLL], db[TUNROLL];
#pragma unroll
        for (int u = 0; u < TUNROLL; ++u) {
            const int ci = (r0 + u) * NT + tid;
            if (ci < nch) {
                tb[u] = C::load(trow, ci);
                if (PAIR) db[u] = C::load(drow, ci);
            } else {
                tb[u] = C::neg_inf();
                if (PAIR) db[u] = C::neg_inf();
            }
        }
#pragma unroll
        for (int u = 0; u < TUNROLL; ++u) {
            const int round = r0 + u;
            if (round < rounds) {  // uniform across the block
                const int ci = round * NT + tid;
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float w = PAIR ? wf(tb[u].get(e), db[u].get(e)) : wf(tb[u].get(e), 0.0f);
                    acc += w;
                    if (w > 0.0f && ci < nch) lastpos = ci * E + e;
                }
                acc = wave_sum(acc);
                if (lane == 0) tile_part[(round / m) * NW + wave] += acc;
            }
        }
    }
    if (rem > 0) {
        float w = 0.0f;
        if (tid < rem) {
            const float tv = load_elem<DT>(trow, nch * E + tid);
            const float dv = PAIR ? load_elem<DT>(drow, nch * E + tid) : 0.0f;
            w = wf(tv, dv);
            if (w > 0.0f) lastpos = nch * E + tid;
        }
        w = wave_sum(w);
        if (lane == 0) tile_part[ntiles * NW + wave] += w;
    }
    __syncthreads();

    // Block scan over tiles (each thread owns a contiguous run of tiles).
    const int tpt = (nt_all + NT - 1) / NT;  // tiles per thread, <= 2
    float mine[2] = {0.0f, 0.0f};
    float run = 0.0f;
    for (int j = 0; j < tpt; ++j) {
        const int t = tid * tpt + j;
        float s = 0.0f;
        if (t < nt_all) {
#pragma unroll
            for (int w = 0; w < NW; ++w) s += tile_part[t * NW + w];
        }
        mine[j] = s;
        run += s;
    }
    float total;
    const float excl = block_excl_scan(run, &total, sc);
    const float T = r * total;
    int cross = INT_MAX;
    {
        float acc = excl;
        for (int j = 0; j < tpt; ++j) {
            const int t = tid * tpt + j;
            if (t < nt_all) {
                tile_excl[t] = acc;
                if (cross == INT_MAX && acc + mine[j] > T) cross = t;
                acc += mine[j];
            }
        }
    }
    cross = block_min_i(cross, sc);  // barrier also publishes tile_excl
    *total_out = total;

    if (cross == INT_MAX) return max(block_max_i(lastpos, sc), 0);

    // Pass B: scan inside the crossing tile.
    float cum = tile_excl[cross];
    int found = INT_MAX;
    int tile_last = -1;
    if (cross == ntiles) {  // the trailing-elements tile
        float w = 0.0f;
        if (tid < rem) {
            const float tv = load_elem<DT>(trow, nch * E + tid);
            const float dv = PAIR ? load_elem<DT>(drow, nch * E + tid) : 0.0f;
            w = wf(tv, dv);
            if (w > 0.0f) tile_last = nch * E + tid;
        }
        float tot;
        const float ex = block_excl_scan(w, &tot, sc);
        if (w > 0.0f && cum + (ex + w) > T) found = nch * E + tid;
        found = block_min_i(found, sc);
    } else {
        for (int rd = cross * m; rd < min(rounds, (cross + 1) * m); ++rd) {
            const int ci = rd * NT + tid;
            float wv[E];
            float loc = 0.0f;
            if (ci < nch) {
                const C tc = C::load(trow, ci);
                C dc;
                if (PAIR) dc = C::load(drow, ci);
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
            const float ex = block_excl_scan(loc, &tot, sc);
            int f = INT_MAX;
            float run_e = ex;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                run_e += wv[e];
                if (f == INT_MAX && wv[e] > 0.0f && cum + run_e > T) f = ci * E + e;
            }
            found = block_min_i(f, sc);
            if (found != INT_MAX) break;
            cum += tot;
        }
    }
    if (found != INT_MAX) return found;
    return max(block_max_i(tile_last, sc), 0);
}

// Residual weight max(0, p - q) of one row pair.
struct ResidualW {
    float c, nRt, iZt, nRd, iZd;
    __device__ __forceinline__ float operator()(float t, float d) const {
        const float pt = fast_exp2(fmaf(t, c, nRt)) * iZt;
        const float qd = fast_exp2(fmaf(d, c, nRd)) * iZd;
        return fmaxf(pt - qd, 0.0f);
    }
};
// Unnormalised target weight 2^(t*c - R).
struct TargetW {
    float c, nR;
    __device__ __forceinline__ float operator()(float t, float) const {
        return fast_exp2(fmaf(t, c, nR));
    }
};

// ------------------------------------------------------------------------
constexpr int MAX_ROWS_STOCH = 2 * kMaxK + 1;

struct StochSmem {
    BlockScratch sc;
    int flag;
    int a;
    float R[MAX_ROWS_STOCH];
    float Z[MAX_ROWS_STOCH];
    float px[kMaxK];
    float qx[kMaxK];
    float tile_part[(MAX_TILES + 1) * NW];
    float tile_excl[MAX_TILES + 1];
};

template <int DT>
__device__ __forceinline__ const char* stoch_row(const Params& p, int b, int r) {
    const size_t eb = elem_bytes<DT>();
    if (r <= p.k)
        return static_cast<const char*>(p.target) +
               ((size_t)b * (p.k + 1) + r) * (size_t)p.row_stride * eb;
    return static_cast<const char*>(p.draft) +
           ((size_t)b * p.k + (r - p.k - 1)) * (size_t)p.row_stride * eb;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(NT) void k_verify_stochastic(Params p) {
    __shared__ StochSmem sm;
    const int per_seq = p.rows_per_seq * p.S;
    const int b = blockIdx.x / per_seq;
    const int item = blockIdx.x - b * per_seq;
    const int r = item / p.S;
    const int s = item - r * p.S;
    const int v0 = s * p.slice_len;
    const int v1 = min(p.V, v0 + p.slice_len);

    float R = 0.0f, Z = 0.0f;
    stream_softmax_stats<DT, VEC>(stoch_row<DT>(p, b, r), v0, v1, p.c, &R, &Z, sm.sc);
    if (!arrive(p, b, item, R, Z, &sm.flag)) return;

    // ---- last workgroup of sequence b ----
    const int tid = threadIdx.x;
    const int k = p.k, V = p.V;
    const float* part = p.part + (size_t)b * per_seq * 2;
    for (int row = tid; row < p.rows_per_seq; row += NT) {
        float RR = -FLT_MAX;
        for (int j = 0; j < p.S; ++j) RR = fmaxf(RR, part[(row * p.S + j) * 2]);
        float ZZ = 0.0f;
        for (int j = 0; j < p.S; ++j)
            ZZ += part[(row * p.S + j) * 2 + 1] * fast_exp2(part[(row * p.S + j) * 2] - RR);
        sm.R[row] = RR;
        sm.Z[row] = ZZ;
    }
    __syncthreads();
    clear_partials(p, b);
    const int32_t* x = p.tokens_in + (size_t)b * k;
    for (int i = tid; i < k; i += NT) {
        const int xi = x[i];
        float pi = 0.0f, qi = 0.0f;
        if (xi >= 0 && xi < V) {
            const float tv = load_elem<DT>(stoch_row<DT>(p, b, i), xi);
            const float dv = load_elem<DT>(stoch_row<DT>(p, b, k + 1 + i), xi);
            pi = fast_exp2(fmaf(tv, p.c, -sm.R[i])) / sm.Z[i];
            qi = fast_exp2(fmaf(dv, p.c, -sm.R[k + 1 + i])) / sm.Z[k + 1 + i];
        }
        sm.px[i] = pi;
        sm.qx[i] = qi;
        if (p.dbg) {
            p.dbg[((size_t)b * k + i) * 2] = pi;
            p.dbg[((size_t)b * k + i) * 2 + 1] = qi;
        }
    }
    __syncthreads();
    if (tid == 0) {
        const float* u = p.u_accept + (size_t)b * k;
        int a = k;
        for (int i = 0; i < k; ++i)
            if (!(u[i] * sm.qx[i] < sm.px[i])) {
                a = i;
                break;
            }
        sm.a = a;
    }
    __syncthreads();
    const int a = sm.a;
    int32_t* out = p.tokens_out + (size_t)b * (k + 1);
    for (int i = tid; i <= k; i += NT) {
        if (i < a) out[i] = x[i];
        else if (i > a) out[i] = -1;
    }
    const float rr = p.u_sample[b];
    const char* trow = stoch_row<DT>(p, b, a);
    float total;
    int y;
    if (a < k) {
        const char* drow = stoch_row<DT>(p, b, k + 1 + a);
        ResidualW w{p.c, -sm.R[a], 1.0f / sm.Z[a], -sm.R[k + 1 + a], 1.0f / sm.Z[k + 1 + a]};
        y = inverse_cdf_row<DT, VEC, true>(trow, drow, V, w, rr, &total, sm.tile_part,
                                           sm.tile_excl, sm.sc);
        if (!(total > 0.0f)) {
            // p == q to float precision: the residual is empty; draw from p_a.
            TargetW tw{p.c, -sm.R[a]};
            y = inverse_cdf_row<DT, VEC, false>(trow, nullptr, V, tw, rr, &total, sm.tile_part,
                                                sm.tile_excl, sm.sc);
        }
    } else {
        TargetW tw{p.c, -sm.R[k]};
        y = inverse_cdf_row<DT, VEC, false>(trow, nullptr, V, tw, rr, &total, sm.tile_part,
                                            sm.tile_excl, sm.sc);
    }
    if (tid == 0) {
        out[a] = y;
        p.accept_len[b] = a;
        p.counters[b] = 0;  // leave the workspace zeroed for the next call
    }
}

// ------------------------------------------------------------------------
struct GreedySmem {
    BlockScratch sc;
    int flag;
    int a;
    int c;
    int g[kMaxRowsPerSeq];
    int cand_a[kMaxRowsPerSeq / 2];  // G <= kMaxRowsPerSeq / (k+1), k >= 1
};

template <int DT, bool VEC>
__global__ __launch_bounds__(NT) void k_verify_greedy(Params p) {
    __shared__ GreedySmem sm;
    const int per_seq = p.rows_per_seq * p.S;
    const int b = blockIdx.x / per_seq;
    const int item = blockIdx.x - b * per_seq;
    const int r = item / p.S;
    const int s = item - r * p.S;
    const int v0 = s * p.slice_len;
    const int v1 = min(p.V, v0 + p.slice_len);
    const char* row = static_cast<const char*>(p.target) +
                      ((size_t)b * p.rows_per_seq + r) * (size_t)p.row_stride * elem_bytes<DT>();

    float M = 0.0f;
    int I = 0;
    stream_argmax<DT, VEC>(row, v0, v1, &M, &I, sm.sc);
    if (!arrive(p, b, item, M, __int_as_float(I), &sm.flag)) return;

    // ---- last workgroup of sequence b ----
    const int tid = threadIdx.x;
    const int k = p.k, G = p.G;
    const float* part = p.part + (size_t)b * per_seq * 2;
    for (int rw = tid; rw < p.rows_per_seq; rw += NT) {
        float bm = part[(rw * p.S) * 2];
        int bi = __float_as_int(part[(rw * p.S) * 2 + 1]);
        for (int j = 1; j < p.S; ++j) {
            const float mj = part[(rw * p.S + j) * 2];
            if (mj > bm) {  // earlier slices win ties: lowest index
                bm = mj;
                bi = __float_as_int(part[(rw * p.S + j) * 2 + 1]);
            }
        }
        sm.g[rw] = bi;
    }
    __syncthreads();
    clear_partials(p, b);
    const int32_t* x = p.tokens_in + (size_t)b * G * k;
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
            if (sm.cand_a[c] > ba) {
                ba = sm.cand_a[c];
                bc = c;
            }
        sm.a = ba;
        sm.c = bc;
        p.accept_len[b] = ba;
        if (p.best_cand) p.best_cand[b] = bc;
        p.counters[b] = 0;
    }
    __syncthreads();
    const int a = sm.a, bc = sm.c;
    int32_t* out = p.tokens_out + (size_t)b * (k + 1);
    for (int i = tid; i <= k; i += NT) out[i] = i <= a ? sm.g[bc * (k + 1) + i] : -1;
}

// ------------------------------------------------------------------------
template <typename K>
static int launch(K kernel, const Params& p, void* stream) {
    const long long grid = (long long)p.B * p.rows_per_seq * p.S;
    Params pc = p;
    void* args[] = {&pc};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                dim3(NT), args, 0, static_cast<hipStream_t>(stream));
}

int launch_stochastic(const Params& p, int dtype, bool vec, void* stream) {
    if (dtype == 1)
        return vec ? launch(k_verify_stochastic<1, true>, p, stream)
                   : launch(k_verify_stochastic<1, false>, p, stream);
    return vec ? launch(k_verify_stochastic<0, true>, p, stream)
               : launch(k_verify_stochastic<0, false>, p, stream);
}

int launch_greedy(const Params& p, int dtype, bool vec, void* stream) {
    if (dtype == 1)
        return vec ? launch(k_verify_greedy<1, true>, p, stream)
                   : launch(k_verify_greedy<1, false>, p, stream);
    return vec ? launch(k_verify_greedy<0, true>, p, stream)
               : launch(k_verify_greedy<0, false>, p, stream);
}

}  // namespace sv
