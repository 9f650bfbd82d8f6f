/*
 * svo.h -- plain CPU oracle for the speculative-decoding verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two only see the same
 * seeded inputs.
 *
 * Everything is computed in IEEE float64 with scalar loops, one sequence at a
 * time, in the order the method states its steps:
 *
 *   1. full softmax of every target row and every draft row, divided by the
 *      temperature (Perplexity, "Accelerating Sonar through speculation",
 *      section "Cieľ-Návrh": acceptance compares the complete draft and target
 *      distributions);
 *   2. accept/reject of each draft token in order, keeping the longest accepted
 *      prefix (same page, section "Špekulatívne dekódovanie", the acceptance stage);
 *   3. one more token sampled from the target side at the first rejection
 *      (the residual distribution) or after the last draft token (the bonus
 *      token), so n drafts yield up to n+1 tokens (same page and section, the
 *      "target generation" stage and the n -> n+1 remark).
 *
 * The exact acceptance rule is the lossless speculative-sampling rule: accept
 * draft token x at position i when u_i * q_i(x) < p_i(x) (that is,
 * u_i < min(1, p_i(x)/q_i(x))); on rejection sample from max(0, p_a - q_a)
 * renormalised.  This is the plainest rule that keeps the original model's
 * output distribution, which aidevelopers.cz, "Zkoumání spekulativního
 * dekódování v vLLM na AMD GPU", section "Základní autoregresivní dekódování",
 * names as the point of the method.
 *
 * Greedy mode accepts while the draft token equals the target argmax (lowest
 * index among equal maxima) and emits the target argmax at the first mismatch
 * or after the last draft token.  With G > 1 candidates per sequence (the
 * n-gram verification of the Lookahead decoding page, gateex.cc, section
 * "A descodificação avançada quebra a dependência da ordem", items 2 and 4)
 * the candidate with the longest accepted prefix wins, lowest index on ties.
 *
 * Layouts (row_stride in elements, >= V):
 *   stochastic target row i of sequence b: target + (b*(k+1) + i) * row_stride
 *   stochastic draft  row i of sequence b: draft  + (b*k     + i) * row_stride
 *   greedy target row i of candidate c of sequence b:
 *                                          target + ((b*G + c)*(k+1) + i) * row_stride
 *   draft tokens: int32 [B][k] (stochastic), [B][G][k] (greedy)
 *   u_accept: float [B][k]; u_sample: float [B]
 *   outputs: accept_len int32 [B], tokens int32 [B][k+1] (-1 after the
 *   emitted token), best_cand int32 [B] (greedy).
 *
 * A draft token outside [0, V) has probability 0 under both distributions
 * and is therefore rejected (greedy: it never equals the argmax).
 *
 * Parity pins: every function here is pinned by tests (exact enumeration of
 * the emitted-token law on tiny vocabularies, library special cases,
 * invariants, brute force); none is "parity unpinned".
 */
#ifndef SVO_ORACLE_H
#define SVO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SVO_F32 = 0, SVO_BF16 = 1 };
enum { SVO_FORCE_NONE = 0, SVO_FORCE_ACCEPT = 1, SVO_FORCE_REJECT = 2 };

/* Stochastic verification of B sequences.  force (nullable, int8 [B][k])
 * overrides individual accept/reject decisions; it exists so a caller can
 * follow another implementation's decision at a position where the two are
 * within rounding of the threshold.  px, qx (nullable, [B][k]) receive
 * p_i(x_i), q_i(x_i); cdf_lo, cdf_hi (nullable, [B]) receive the cumulative
 * probability just before and at the emitted token under the distribution it
 * was sampled from.  Returns 0, or -1 on a bad argument. */
int svo_verify_stochastic(const void* target, const void* draft,
                          const int32_t* draft_tokens, const float* u_accept,
                          const float* u_sample, int B, int k, int V,
                          int64_t row_stride, int dtype, double temperature,
                          const int8_t* force, int32_t* accept_len,
                          int32_t* tokens, double* px, double* qx,
                          double* cdf_lo, double* cdf_hi);

/* For sequence b, given that position a is where the extra token is drawn
 * (a < k: residual of row pair a; a == k: target row k), return the
 * cumulative probability before token y (lo) and through token y (hi). */
int svo_emit_cdf(const void* target, const void* draft, int b, int k, int V,
                 int64_t row_stride, int dtype, double temperature, int a,
                 int y, double* lo, double* hi);

/* Greedy verification, G >= 1 candidates per sequence.  cand_accept
 * (nullable, [B][G]) receives each candidate's accepted length. */
int svo_verify_greedy(const void* target, const int32_t* draft_tokens, int B,
                      int G, int k, int V, int64_t row_stride, int dtype,
                      int32_t* accept_len, int32_t* tokens, int32_t* best_cand,
                      int32_t* cand_accept);

/* Ragged batches (sequence b has k_b = cu[b+1] - cu[b] draft tokens,
 * 0 <= k_b <= k_max, cu[0] = 0): target rows of sequence b are rows
 * cu[b] + b .. cu[b] + b + k_b, its draft rows cu[b] .. cu[b] + k_b - 1, its
 * draft tokens and acceptance uniforms entries cu[b] ..; px/qx (nullable)
 * are [cu[B]]; tokens are [B][k_max + 1].  k_b = 0 samples the first target
 * row (plain sampling).  Returns -1 on a bad argument or malformed cu. */
int svo_verify_stochastic_ragged(const void* target, const void* draft,
                                 const int32_t* draft_tokens, const int32_t* cu,
                                 const float* u_accept, const float* u_sample,
                                 int B, int k_max, int V, int64_t row_stride,
                                 int dtype, double temperature,
                                 int32_t* accept_len, int32_t* tokens,
                                 double* px, double* qx);

int svo_verify_greedy_ragged(const void* target, const int32_t* draft_tokens,
                             const int32_t* cu, int B, int k_max, int V,
                             int64_t row_stride, int dtype, int32_t* accept_len,
                             int32_t* tokens);

/* Plain sampling, one token per row b of logits: inverse CDF of
 * softmax(row / temperature) at u[b], or the argmax when greedy != 0. */
int svo_sample(const void* logits, const float* u, int B, int V,
               int64_t row_stride, int dtype, double temperature, int greedy,
               int32_t* tokens);

/* Greedy verification of a draft tree per sequence (the Top-K tree of the
 * EAGLE scheme: Perplexity, "Accelerating Sonar through speculation", section
 * "EAGLE").  Sequence b has N nodes; node 0 is the root (the last committed
 * token, never verified), node j >= 1 carries draft token node_tokens[b][j]
 * and parent parents[b][j] in [0, j) (parents[b][0] = -1).  Target row j of
 * sequence b, at (b*N + j) * row_stride, is the target's output at node j (it
 * predicts the token that follows node j's path).  Node j >= 1 is accepted
 * when its parent is accepted and its token equals the argmax (lowest index)
 * of its parent's row; the root is accepted.  The deepest accepted node wins,
 * lowest node index among equal depths.  Outputs, each [B][N] with -1 after
 * the used entries: tokens = the draft tokens along the root-to-winner path,
 * then the argmax of the winner's row (so d accepted drafts give d + 1
 * tokens); path = the node indices root, ..., winner.  accept_len [B] = the
 * winner's depth.  Returns -1 on a bad argument or a malformed tree. */
int svo_verify_greedy_tree(const void* target, const int32_t* node_tokens,
                           const int32_t* parents, int B, int N, int V,
                           int64_t row_stride, int dtype, int32_t* accept_len,
                           int32_t* tokens, int32_t* path);

/* Commit of a verified step (Perplexity, same page, sections "MTP" and
 * "Plánovanie MTP pre Jediný Token": the accepted tokens are put in place for
 * the next step on the GPU, without waiting for the host).  For sequence b,
 * with a = accept_len[b] and L = seq_len[b]: the a + 1 emitted tokens
 * tokens[b][0..a] (row width W) are appended to history[b] (row stride
 * history_stride) at positions L, L+1, ... as far as position capacity - 1,
 * seq_len[b] becomes min(L + a + 1, capacity) (unchanged when L >= capacity),
 * and next_token[b * next_stride] receives tokens[b][a], the token the next
 * step starts from.  Returns -1 on a bad argument or an accept_len outside
 * [0, W - 1]. */
int svo_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W,
               int32_t* seq_len, int32_t* history, int64_t history_stride,
               int capacity, int32_t* next_token, int64_t next_stride);

/* Number of OpenMP threads the batched entry points use. */
int svo_num_threads(void);
void svo_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif
