/*
 * svo.c -- plain float64 CPU oracle for the speculative-decoding verification
 * step.  TEST INFRASTRUCTURE ONLY (see svo.h for the method, its sources and
 * the layouts).  Deliberately slow and literal: every row is turned into a
 * full float64 probability vector before anything is decided, and sampling
 * walks the cumulative distribution from token 0 upwards.
 */
#include "svo.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One logit as float64.  bf16 is the top half of an IEEE float32, so the
 * conversion is exact; so is float32 -> float64. */
static double logit(const void* base, int dtype, int64_t idx) {
    if (dtype == SVO_F32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* prob[v] = exp((x_v - M)/tau) / sum_w exp((x_w - M)/tau), M = max_v x_v.
 * A -inf logit gets probability 0.  (Perplexity, "Accelerating Sonar through
 * speculation", section "Cieľ-Návrh": full distributions are compared.) */
static void softmax_row(const void* base, int dtype, int64_t row_off, int V,
                        double tau, double* prob) {
    double M = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double x = logit(base, dtype, row_off + v);
        if (x > M) M = x;
    }
    double Z = 0.0;
    for (int v = 0; v < V; ++v) {
        prob[v] = exp((logit(base, dtype, row_off + v) - M) / tau);
        Z += prob[v];
    }
    for (int v = 0; v < V; ++v) prob[v] /= Z;
}

/* Inverse-CDF draw from the distribution proportional to w[0..V-1] (w >= 0):
 * the first token whose cumulative normalised mass exceeds r.  If no token
 * qualifies (r = 1, where the total mass 1 does not exceed r, or a sum that
 * rounds below r), the last token with positive weight.  Tokens of zero
 * weight are never returned.  lo/hi receive the cumulative mass before and
 * through the returned token. */
static int inverse_cdf(const double* w, int V, double r, double* lo,
                       double* hi) {
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += w[v];
    double C = 0.0;
    for (int v = 0; v < V; ++v) {
        double prev = C;
        C += w[v] / S;
        if (w[v] > 0.0 && C > r) {
            if (lo) *lo = prev;
            if (hi) *hi = C;
            return v;
        }
    }
    int last = 0;
    for (int v = 0; v < V; ++v)
        if (w[v] > 0.0) last = v;
    if (lo) *lo = C - w[last] / S;
    if (hi) *hi = C;
    return last;
}

/* The distribution the extra token is drawn from when the first rejection is
 * at position a (a < k): max(0, p_a - q_a), or p_a itself if that is zero
 * everywhere (rejection then had probability zero).  When every draft token
 * was accepted (a == k): the target distribution p_k (the bonus token).
 * (Perplexity, "Accelerating Sonar through speculation", section
 * "Špekulatívne dekódovanie", target-generation stage: the target's logits at
 * the mismatch or after the last draft token give the closing token.) */
static void emit_distribution(const double* pa, const double* qa, int V,
                              int a, int k, double* w) {
    if (a == k) {
        for (int v = 0; v < V; ++v) w[v] = pa[v];
        return;
    }
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        double d = pa[v] - qa[v];
        w[v] = d > 0.0 ? d : 0.0;
        S += w[v];
    }
    if (S == 0.0)
        for (int v = 0; v < V; ++v) w[v] = pa[v];
}

static int64_t t_row(int b, int k, int i, int64_t stride) {
    return ((int64_t)b * (k + 1) + i) * stride;
}
static int64_t d_row(int b, int k, int i, int64_t stride) {
    return ((int64_t)b * k + i) * stride;
}

static void stochastic_one(const void* target, const void* draft,
                           const int32_t* x, const float* u, float r, int b,
                           int k, int V, int64_t stride, int dtype, double tau,
                           const int8_t* force, int32_t* accept_len,
                           int32_t* tok, double* px, double* qx, double* lo,
                           double* hi, double* p, double* q, double* w) {
    int a = k;
    for (int i = 0; i < k; ++i) {
        softmax_row(target, dtype, t_row(b, k, i, stride), V, tau, p);
        softmax_row(draft, dtype, d_row(b, k, i, stride), V, tau, q);
        int xi = x[i];
        double pi = (xi >= 0 && xi < V) ? p[xi] : 0.0;
        double qi = (xi >= 0 && xi < V) ? q[xi] : 0.0;
        if (px) px[i] = pi;
        if (qx) qx[i] = qi;
        int accept = (double)u[i] * qi < pi;
        if (force && force[i] == SVO_FORCE_ACCEPT) accept = 1;
        if (force && force[i] == SVO_FORCE_REJECT) accept = 0;
        if (!accept) {
            a = i;
            break;
        }
    }
    /* Diagnostics for positions after the first rejection are still filled
     * in, so callers can compare every position. */
    for (int i = a + 1; i < k && (px || qx); ++i) {
        softmax_row(target, dtype, t_row(b, k, i, stride), V, tau, p);
        softmax_row(draft, dtype, d_row(b, k, i, stride), V, tau, q);
        int xi = x[i];
        if (px) px[i] = (xi >= 0 && xi < V) ? p[xi] : 0.0;
        if (qx) qx[i] = (xi >= 0 && xi < V) ? q[xi] : 0.0;
    }
    softmax_row(target, dtype, t_row(b, k, a, stride), V, tau, p);
    if (a < k) softmax_row(draft, dtype, d_row(b, k, a, stride), V, tau, q);
    emit_distribution(p, q, V, a, k, w);
    double l = 0.0, h = 0.0;
    int y = inverse_cdf(w, V, (double)r, &l, &h);
    *accept_len = a;
    for (int i = 0; i < a; ++i) tok[i] = x[i];
    tok[a] = y;
    for (int i = a + 1; i <= k; ++i) tok[i] = -1;
    if (lo) *lo = l;
    if (hi) *hi = h;
}

int svo_verify_stochastic(const void* target, const void* draft,
                          const int32_t* draft_tokens, const float* u_accept,
                          const float* u_sample, int B, int k, int V,
                          int64_t row_stride, int dtype, double temperature,
                          const int8_t* force, int32_t* accept_len,
                          int32_t* tokens, double* px, double* qx,
                          double* cdf_lo, double* cdf_hi) {
    if (!target || !draft || !draft_tokens || !u_accept || !u_sample ||
        !accept_len || !tokens)
        return -1;
    if (B < 0 || k < 1 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
    if (!(temperature > 0.0) || !isfinite(temperature)) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* q = (double*)malloc(sizeof(double) * (size_t)V);
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        if (!p || !q || !w) {
#pragma omp atomic write
            bad = 1;
        } else {
            stochastic_one(target, draft, draft_tokens + (int64_t)b * k,
                           u_accept + (int64_t)b * k, u_sample[b], b, k, V,
                           row_stride, dtype, temperature,
                           force ? force + (int64_t)b * k : NULL,
                           accept_len + b, tokens + (int64_t)b * (k + 1),
                           px ? px + (int64_t)b * k : NULL,
                           qx ? qx + (int64_t)b * k : NULL,
                           cdf_lo ? cdf_lo + b : NULL,
                           cdf_hi ? cdf_hi + b : NULL, p, q, w);
        }
        free(p);
        free(q);
        free(w);
    }
    return bad ? -1 : 0;
}

int svo_emit_cdf(const void* target, const void* draft, int b, int k, int V,
                 int64_t row_stride, int dtype, double temperature, int a,
                 int y, double* lo, double* hi) {
    if (!target || !draft || !lo || !hi) return -1;
    if (b < 0 || k < 1 || V < 1 || row_stride < V || a < 0 || a > k) return -1;
    if (y < 0 || y >= V) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !w) {
        free(p);
        free(q);
        free(w);
        return -1;
    }
    softmax_row(target, dtype, t_row(b, k, a, row_stride), V, temperature, p);
    if (a < k)
        softmax_row(draft, dtype, d_row(b, k, a, row_stride), V, temperature,
                    q);
    emit_distribution(p, q, V, a, k, w);
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += w[v];
    double C = 0.0;
    for (int v = 0; v < y; ++v) C += w[v] / S;
    *lo = C;
    *hi = C + w[y] / S;
    free(p);
    free(q);
    free(w);
    return 0;
}

/* Index of the largest logit, lowest index among equal maxima. */
static int argmax_row(const void* base, int dtype, int64_t row_off, int V) {
    int best = 0;
    double bv = logit(base, dtype, row_off);
    for (int v = 1; v < V; ++v) {
        double x = logit(base, dtype, row_off + v);
        if (x > bv) {
            bv = x;
            best = v;
        }
    }
    return best;
}

/* Greedy verification of one sequence whose first candidate row is at
 * element offset `base`: G candidates of k+1 rows each (k may be 0: then the
 * emitted token is just the argmax of row 0). */
static void greedy_one(const void* target, const int32_t* x, int G, int k, int V,
                       int64_t stride, int dtype, int64_t base, int32_t* accept_len,
                       int32_t* out, int32_t* best_cand, int32_t* cand_accept) {
    int best_c = 0, best_a = -1;
    for (int c = 0; c < G; ++c) {
        const int32_t* xc = x + (int64_t)c * k;
        int64_t row0 = base + (int64_t)c * (k + 1) * stride;
        int a = k;
        for (int i = 0; i < k; ++i) {
            int g = argmax_row(target, dtype, row0 + i * stride, V);
            if (xc[i] != g) {
                a = i;
                break;
            }
        }
        if (cand_accept) cand_accept[c] = a;
        if (a > best_a) {
            best_a = a;
            best_c = c;
        }
    }
    int64_t row0 = base + (int64_t)best_c * (k + 1) * stride;
    for (int i = 0; i <= best_a; ++i) out[i] = argmax_row(target, dtype, row0 + i * stride, V);
    for (int i = best_a + 1; i <= k; ++i) out[i] = -1;
    *accept_len = best_a;
    if (best_cand) *best_cand = best_c;
}

int svo_verify_greedy(const void* target, const int32_t* draft_tokens, int B,
                      int G, int k, int V, int64_t row_stride, int dtype,
                      int32_t* accept_len, int32_t* tokens, int32_t* best_cand,
                      int32_t* cand_accept) {
    if (!target || !draft_tokens || !accept_len || !tokens) return -1;
    if (B < 0 || G < 1 || k < 1 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        greedy_one(target, draft_tokens + (int64_t)b * G * k, G, k, V, row_stride, dtype,
                   (int64_t)b * G * (k + 1) * row_stride, accept_len + b,
                   tokens + (int64_t)b * (k + 1), best_cand ? best_cand + b : NULL,
                   cand_accept ? cand_accept + (int64_t)b * G : NULL);
    return 0;
}

/* Ragged batches: sequence b has k_b = cu[b+1] - cu[b] draft tokens (0 <= k_b
 * <= k_max) and its rows are packed: target rows cu[b] + b .. cu[b] + b + k_b,
 * draft rows cu[b] .. cu[b] + k_b - 1; draft tokens and acceptance uniforms
 * at cu[b] ..; outputs padded to k_max + 1 per sequence.  Each sequence is
 * verified exactly as a batch of one with its own k (k_b = 0 samples the
 * first target row). */
static int ragged_ok(const int32_t* cu, int B, int k_max) {
    if (cu[0] != 0) return 0;
    for (int b = 0; b < B; ++b) {
        int kb = cu[b + 1] - cu[b];
        if (kb < 0 || kb > k_max) return 0;
    }
    return 1;
}

static size_t elem_size(int dtype) { return dtype == SVO_F32 ? 4 : 2; }

int svo_verify_stochastic_ragged(const void* target, const void* draft,
                                 const int32_t* draft_tokens, const int32_t* cu,
                                 const float* u_accept, const float* u_sample,
                                 int B, int k_max, int V, int64_t row_stride,
                                 int dtype, double temperature,
                                 int32_t* accept_len, int32_t* tokens,
                                 double* px, double* qx) {
    if (!target || !draft || !draft_tokens || !cu || !u_accept || !u_sample ||
        !accept_len || !tokens)
        return -1;
    if (B < 0 || k_max < 0 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
    if (!(temperature > 0.0) || !isfinite(temperature)) return -1;
    if (!ragged_ok(cu, B, k_max)) return -1;
    const size_t es = elem_size(dtype);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int kb = cu[b + 1] - cu[b];
        const int64_t t0 = (int64_t)cu[b] + b, d0 = cu[b];
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* q = (double*)malloc(sizeof(double) * (size_t)V);
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        if (!p || !q || !w) {
#pragma omp atomic write
            bad = 1;
        } else {
            int32_t* out = tokens + (int64_t)b * (k_max + 1);
            stochastic_one((const char*)target + t0 * row_stride * es,
                           (const char*)draft + d0 * row_stride * es, draft_tokens + d0,
                           u_accept + d0, u_sample[b], 0, kb, V, row_stride, dtype,
                           temperature, NULL, accept_len + b, out, px ? px + d0 : NULL,
                           qx ? qx + d0 : NULL, NULL, NULL, p, q, w);
            for (int i = kb + 1; i <= k_max; ++i) out[i] = -1;
        }
        free(p);
        free(q);
        free(w);
    }
    return bad ? -1 : 0;
}

int svo_verify_greedy_ragged(const void* target, const int32_t* draft_tokens,
                             const int32_t* cu, int B, int k_max, int V,
                             int64_t row_stride, int dtype, int32_t* accept_len,
                             int32_t* tokens) {
    if (!target || !draft_tokens || !cu || !accept_len || !tokens) return -1;
    if (B < 0 || k_max < 0 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
    if (!ragged_ok(cu, B, k_max)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int kb = cu[b + 1] - cu[b];
        int32_t* out = tokens + (int64_t)b * (k_max + 1);
        greedy_one(target, draft_tokens + cu[b], 1, kb, V, row_stride, dtype,
                   ((int64_t)cu[b] + b) * row_stride, accept_len + b, out, NULL, NULL);
        for (int i = kb + 1; i <= k_max; ++i) out[i] = -1;
    }
    return 0;
}

/* Plain sampling of one token per row: the first token whose cumulative
 * softmax(row / T) mass exceeds u[b], or (greedy) the row's argmax, lowest
 * index on ties. */
int svo_sample(const void* logits, const float* u, int B, int V,
               int64_t row_stride, int dtype, double temperature, int greedy,
               int32_t* tokens) {
    if (!logits || !tokens || (!greedy && !u)) return -1;
    if (B < 0 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
    if (!greedy && (!(temperature > 0.0) || !isfinite(temperature))) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        if (greedy) {
            tokens[b] = argmax_row(logits, dtype, (int64_t)b * row_stride, V);
            continue;
        }
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        if (!p) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        softmax_row(logits, dtype, (int64_t)b * row_stride, V, temperature, p);
        tokens[b] = inverse_cdf(p, V, (double)u[b], NULL, NULL);
        free(p);
    }
    return bad ? -1 : 0;
}

/* Greedy tree verification: per node, in index order (a parent always
 * precedes its children), accepted = parent accepted and token == argmax of
 * the parent's row; then the deepest accepted node, lowest index on ties,
 * and the walk back to the root. */
int svo_verify_greedy_tree(const void* target, const int32_t* node_tokens,
                           const int32_t* parents, int B, int N, int V,
                           int64_t row_stride, int dtype, int32_t* accept_len,
                           int32_t* tokens, int32_t* path) {
    if (!target || !node_tokens || !parents || !accept_len || !tokens || !path) return -1;
    if (B < 0 || N < 1 || V < 1 || row_stride < V) return -1;
    if (dtype != SVO_F32 && dtype != SVO_BF16) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parents + (int64_t)b * N;
        if (par[0] != -1) return -1;
        for (int j = 1; j < N; ++j)
            if (par[j] < 0 || par[j] >= j) return -1;
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parents + (int64_t)b * N;
        const int32_t* tok = node_tokens + (int64_t)b * N;
        int* acc = (int*)malloc(sizeof(int) * (size_t)N);
        int* depth = (int*)malloc(sizeof(int) * (size_t)N);
        if (!acc || !depth) {
#pragma omp atomic write
            bad = 1;
            free(acc);
            free(depth);
            continue;
        }
        acc[0] = 1;
        depth[0] = 0;
        int best = 0;
        for (int j = 1; j < N; ++j) {
            const int pj = par[j];
            depth[j] = depth[pj] + 1;
            acc[j] = 0;
            if (acc[pj]) {
                const int g = argmax_row(target, dtype, ((int64_t)b * N + pj) * row_stride, V);
                acc[j] = tok[j] == g;
            }
            if (acc[j] && depth[j] > depth[best]) best = j;
        }
        const int d = depth[best];
        int32_t* out_t = tokens + (int64_t)b * N;
        int32_t* out_p = path + (int64_t)b * N;
        for (int i = 0; i < N; ++i) {
            out_t[i] = -1;
            out_p[i] = -1;
        }
        for (int j = best, i = d; i >= 0; j = par[j], --i) out_p[i] = j;
        for (int i = 0; i < d; ++i) out_t[i] = tok[out_p[i + 1]];
        out_t[d] = argmax_row(target, dtype, ((int64_t)b * N + best) * row_stride, V);
        accept_len[b] = d;
        free(acc);
        free(depth);
    }
    return bad ? -1 : 0;
}

/* Commit of a verified step: append the emitted tokens, advance the length,
 * hand the last emitted token to the next step. */
int svo_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W,
               int32_t* seq_len, int32_t* history, int64_t history_stride,
               int capacity, int32_t* next_token, int64_t next_stride) {
    if (!accept_len || !tokens || !seq_len || !history || !next_token) return -1;
    if (B < 0 || W < 1 || capacity < 0 || history_stride < capacity || next_stride < 1)
        return -1;
    for (int b = 0; b < B; ++b)
        if (accept_len[b] < 0 || accept_len[b] >= W || seq_len[b] < 0) return -1;
    for (int b = 0; b < B; ++b) {
        const int a = accept_len[b];
        const int32_t* t = tokens + (int64_t)b * W;
        int32_t* h = history + (int64_t)b * history_stride;
        int L = seq_len[b];
        for (int j = 0; j <= a && L < capacity; ++j) h[L++] = t[j];
        seq_len[b] = L;
        next_token[(int64_t)b * next_stride] = t[a];
    }
    return 0;
}

int svo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void svo_set_num_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
