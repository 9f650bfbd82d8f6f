/* The CPU oracle (oracle/svo.c) under AddressSanitizer and UBSan: every
 * entry point on small seeded cases -- both logit types, padded rows, -inf
 * entries, out-of-range draft tokens, ragged lengths with empty sequences,
 * several candidates, draft trees and commits -- with the output invariants
 * checked (accepted length in range, -1 after the emitted token).  Built and
 * run by tests/test_host_sanitizers.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "svo.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
    st ^= st >> 12;
    st ^= st << 25;
    st ^= st >> 27;
    return (uint32_t)((st * 2685821657736338717ull) >> 32);
}
static double unif(void) { return (rnd() >> 8) * (1.0 / 16777216.0); }
static float unif_f(void) { return (float)((rnd() >> 8) * (1.0 / 16777216.0)); }
static double normal(void) { return sqrt(-2.0 * log(1.0 - unif())) * cos(6.283185307179586 * unif()); }

static uint16_t to_bf16(float x) { /* round to nearest even */
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* rows x (V + pad) logits, either float or bf16 bits; pad entries NaN */
static void* logits(int rows, int V, int pad, int dtype, double scale, int neginf) {
    const int W = V + pad;
    void* p = malloc((size_t)rows * W * (dtype == SVO_BF16 ? 2 : 4));
    for (int r = 0; r < rows; ++r)
        for (int v = 0; v < W; ++v) {
            float x = v >= V ? NAN : (float)(normal() * scale);
            if (v < V && v > 0 && neginf && unif() < 0.2) x = -INFINITY;
            if (dtype == SVO_BF16) ((uint16_t*)p)[(size_t)r * W + v] = to_bf16(x);
            else ((float*)p)[(size_t)r * W + v] = x;
        }
    return p;
}

static int fails = 0;
#define CHECK(c)                                                           \
    do {                                                                   \
        if (!(c)) {                                                        \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                                       \
        }                                                                  \
    } while (0)

static void check_tokens(const int32_t* a, const int32_t* tok, int B, int k) {
    for (int b = 0; b < B; ++b) {
        CHECK(a[b] >= 0 && a[b] <= k);
        if (a[b] < 0 || a[b] > k) continue; /* counted; do not index with it */
        for (int i = a[b] + 1; i <= k; ++i) CHECK(tok[b * (k + 1) + i] == -1);
        CHECK(tok[b * (k + 1) + a[b]] >= 0);
    }
}

int main(void) {
    for (int it = 0; it < 60; ++it) {
        const int dtype = it & 1;
        const int B = 1 + (int)(rnd() % 5), k = 1 + (int)(rnd() % 4), V = 1 + (int)(rnd() % 70);
        const int pad = (int)(rnd() % 3), W = V + pad, neginf = it % 3 == 0;
        const double tau = 0.5 + unif();
        void* t = logits(B * (k + 1), V, pad, dtype, 2.0, neginf);
        void* d = logits(B * k, V, pad, dtype, 2.0, neginf);
        int32_t* x = malloc(sizeof(int32_t) * (B * k + 1));
        float* ua = malloc(sizeof(float) * (B * k + 1));
        float* us = malloc(sizeof(float) * B);
        for (int i = 0; i < B * k; ++i) {
            x[i] = (int32_t)(rnd() % (V + 2)) - (it % 4 == 0 ? 1 : 0); /* some out of range */
            ua[i] = unif_f();
        }
        for (int b = 0; b < B; ++b) us[b] = unif_f();
        int32_t* a = calloc(B, sizeof(int32_t));
        int32_t* tok = calloc((size_t)B * (k + 1), sizeof(int32_t));
        double* px = malloc(sizeof(double) * (B * k + 1));
        double* qx = malloc(sizeof(double) * (B * k + 1));
        double* lo = malloc(sizeof(double) * B);
        double* hi = malloc(sizeof(double) * B);
        CHECK(svo_verify_stochastic(t, d, x, ua, us, B, k, V, W, dtype, tau, NULL, a, tok, px, qx,
                                    lo, hi) == 0);
        check_tokens(a, tok, B, k);
        for (int b = 0; b < B; ++b) {
            double l2, h2;
            CHECK(svo_emit_cdf(t, d, b, k, V, W, dtype, tau, a[b], tok[b * (k + 1) + a[b]], &l2,
                               &h2) == 0);
            CHECK(l2 <= h2);
        }
        /* greedy, several candidates: target rows [B][G][k+1] */
        const int G = 1 + (int)(rnd() % 3);
        void* tg = logits(B * G * (k + 1), V, pad, dtype, 1.0, 0);
        int32_t* xg = malloc(sizeof(int32_t) * (B * G * k + 1));
        for (int i = 0; i < B * G * k; ++i) xg[i] = (int32_t)(rnd() % V);
        int32_t* best = malloc(sizeof(int32_t) * B);
        int32_t* ca = malloc(sizeof(int32_t) * B * G);
        CHECK(svo_verify_greedy(tg, xg, B, G, k, V, W, dtype, a, tok, best, ca) == 0);
        check_tokens(a, tok, B, k);
        for (int b = 0; b < B; ++b) CHECK(best[b] >= 0 && best[b] < G);
        /* ragged: k_b in 0..k, some empty */
        int32_t* cu = malloc(sizeof(int32_t) * (B + 1));
        cu[0] = 0;
        for (int b = 0; b < B; ++b) cu[b + 1] = cu[b] + (int)(rnd() % (k + 1));
        const int n = cu[B];
        void* tr = logits(n + B, V, pad, dtype, 2.0, neginf);
        void* dr = logits(n > 0 ? n : 1, V, pad, dtype, 2.0, neginf);
        int32_t* xr = malloc(sizeof(int32_t) * (n + 1));
        float* uar = malloc(sizeof(float) * (n + 1));
        for (int i = 0; i < n; ++i) {
            xr[i] = (int32_t)(rnd() % V);
            uar[i] = unif_f();
        }
        CHECK(svo_verify_stochastic_ragged(tr, dr, xr, cu, uar, us, B, k, V, W, dtype, tau, a, tok,
                                           NULL, NULL) == 0);
        check_tokens(a, tok, B, k);
        CHECK(svo_verify_greedy_ragged(tr, xr, cu, B, k, V, W, dtype, a, tok) == 0);
        check_tokens(a, tok, B, k);
        /* plain sampling and argmax of B rows */
        CHECK(svo_sample(t, us, B, V, W, dtype, tau, 0, a) == 0);
        for (int b = 0; b < B; ++b) CHECK(a[b] >= 0 && a[b] < V);
        CHECK(svo_sample(t, NULL, B, V, W, dtype, tau, 1, a) == 0);
        /* a draft tree of N nodes per sequence: node j's parent in [0, j) */
        const int N = 1 + (int)(rnd() % 6);
        void* tt = logits(B * N, V, pad, dtype, 1.0, 0);
        int32_t* nt = malloc(sizeof(int32_t) * B * N);
        int32_t* par = malloc(sizeof(int32_t) * B * N);
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < N; ++j) {
                nt[b * N + j] = (int32_t)(rnd() % V);
                par[b * N + j] = j == 0 ? -1 : (int32_t)(rnd() % j);
            }
        int32_t* ttok = malloc(sizeof(int32_t) * B * N);
        int32_t* path = malloc(sizeof(int32_t) * B * N);
        CHECK(svo_verify_greedy_tree(tt, nt, par, B, N, V, W, dtype, a, ttok, path) == 0);
        for (int b = 0; b < B; ++b) CHECK(a[b] >= 0 && a[b] < N && path[b * N] == 0);
        /* commit the stochastic step into short histories */
        CHECK(svo_verify_stochastic(t, d, x, ua, us, B, k, V, W, dtype, tau, NULL, a, tok, NULL,
                                    NULL, NULL, NULL) == 0);
        const int cap = 1 + (int)(rnd() % 8);
        int32_t* len = malloc(sizeof(int32_t) * B);
        int32_t* hist = malloc(sizeof(int32_t) * B * cap);
        int32_t* next = malloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b) len[b] = (int)(rnd() % (cap + 1));
        CHECK(svo_commit(a, tok, B, k + 1, len, hist, cap, cap, next, 1) == 0);
        for (int b = 0; b < B; ++b) CHECK(len[b] >= 0 && len[b] <= cap);
        free(t), free(d), free(x), free(ua), free(us), free(a), free(tok), free(px), free(qx);
        free(lo), free(hi), free(tg), free(xg), free(best), free(ca), free(cu), free(tr), free(dr);
        free(xr), free(uar), free(tt), free(nt), free(par), free(ttok), free(path), free(len);
        free(hist), free(next);
    }
    /* bad arguments are refused */
    CHECK(svo_verify_stochastic(NULL, NULL, NULL, NULL, NULL, 2, 1, 4, 4, 0, 1.0, NULL, NULL, NULL,
                                NULL, NULL, NULL, NULL) == -1);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer checks ok\n");
    return 0;
}
