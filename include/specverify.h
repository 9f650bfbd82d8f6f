/*
 * specverify.h -- C ABI of libspecverify, the speculative-decoding
 * verification step on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  A draft model proposes k tokens per sequence; the target
 * model produces logits for the k draft positions plus one more.  The
 * verification step decides how many draft tokens the target accepts and
 * emits one further token, so k drafts yield between 1 and k+1 tokens
 * (Perplexity, "Accelerating Sonar through speculation", section
 * "Špekulatívne dekódovanie": the acceptance stage keeps the longest
 * acceptable draft prefix and the target-generation stage samples the closing
 * token from the target's logits at the first mismatch or after the last
 * draft token).  Acceptance compares the full target and draft distributions
 * (same page, section "Cieľ-Návrh"), and one verifier serves every drafting
 * scheme -- draft model, MTP head, n-gram candidates -- since all of them only
 * change how the logits are produced (same page, section "MTP").
 *
 * Two entry points, one per decision rule:
 *
 *   sv_verify_stochastic -- lossless speculative sampling.  With
 *     p_i = softmax(target_i / T) and q_i = softmax(draft_i / T) over the whole
 *     vocabulary, draft token x_i is accepted when u_i * q_i(x_i) < p_i(x_i)
 *     (u_i < min(1, p_i/q_i)); a is the first rejected position (k if none).
 *     At a < k the extra token is drawn from max(0, p_a - q_a) renormalised
 *     (from p_a if that is zero everywhere); at a == k it is drawn from p_k.
 *     Drawing is by inverse CDF over ascending token index with the caller's
 *     uniform r: the first token whose cumulative mass exceeds r.  This rule
 *     is the one that keeps the target model's output distribution unchanged,
 *     which is the aim the pages set (aidevelopers.cz, "Zkoumání
 *     spekulativního dekódování v vLLM na AMD GPU", section "Základní
 *     autoregresivní dekódování").
 *
 *   sv_verify_greedy -- accept while the draft token equals the target
 *     argmax (lowest index among equal maxima); the extra token is the target
 *     argmax at the first mismatch or at position k.  With G > 1 candidate
 *     token sequences per sequence (n-gram verification of Lookahead decoding,
 *     gateex.cc, section "A descodificação avançada quebra a dependência da
 *     ordem", items 2 and 4: many guessed n-grams are checked in one step and
 *     the longest verified one is kept) the candidate with the longest
 *     accepted prefix wins, lowest candidate index on ties.
 *
 * Memory and ownership.  Every pointer is a device pointer owned by the
 * caller (u_accept, u_sample, tokens, outputs and workspace included).  The
 * library allocates nothing and keeps no state between calls, apart from the
 * fixed per-GPU buffer of sv_verify_stochastic_noalloc (below).  Logits are
 * float32 or bfloat16, row-major, one row of V entries every row_stride
 * elements (row_stride >= V; padding entries are never read).  Rows:
 *   stochastic: target row i of sequence b at (b*(k+1) + i) * row_stride,
 *               draft  row i of sequence b at (b*k     + i) * row_stride;
 *   greedy:     target row i of candidate c of sequence b at
 *               ((b*G + c)*(k+1) + i) * row_stride.
 * Rows whose start is 16-byte aligned (base pointer 16-byte aligned and
 * row_stride * element size a multiple of 16) take the vector path; others
 * are read element by element (correct, slower).
 *
 * Ordering.  Calls are asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream) and never synchronise with the host: accept_len and tokens are
 * valid once the stream reaches the end of the call.  Reading them on the
 * host is the one GPU-to-CPU crossing of a decoding step (Perplexity, same
 * page, section "Inferencia so špekulatívnym dekódovaním": the accepted
 * length decides the next step's shape).
 *
 * Workspace.  sv_workspace_bytes() gives a scratch size that suffices for
 * every entry point at a shape: room for 8 bytes of statistics per row slice
 * plus a few bytes per row and per sequence.  Pass at least that many bytes,
 * 256-byte aligned.  Dense verification calls with k >= 1 need none when the
 * batch fills the GPU on its own (one candidate and B >= 192: every sequence
 * is then verified by a single workgroup), and accept NULL with size 0 there
 * (stochastic calls without diagnostics are faster with one, see below);
 * so does sv_sample with u when it samples each row in one pass (see
 * sv_sample).  Any
 * other call given NULL returns SV_ERR_NULL, and one given too few or
 * misaligned bytes SV_ERR_WORKSPACE, before launching anything.  Its
 * contents on entry do not matter and are unspecified on return.  Two calls
 * that overlap in time on the same workspace race.
 *
 * Errors.  Arguments are checked on the host before anything is launched; on
 * an error nothing is written and a negative SV_ERR_* status is returned.
 * Values inside device buffers are not checked: acceptance uniforms u in
 * [0,1), sampling uniforms r (u_sample, sv_sample's u) in [0,1], logits
 * finite or -inf with at least one finite entry per row (NaN and +inf are
 * undefined).  At r = 1 no token's cumulative mass exceeds r, and the draw
 * returns the last token with positive mass (the rule's own fallback, which
 * also covers a float32 cumulative sum that rounds below r * total).  A draft token outside [0, V) is defined behaviour: it has
 * probability 0 under both distributions and is rejected (greedy: it never
 * matches).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SV_OK 0
#define SV_ERR_NULL (-1)        /* a required pointer is NULL               */
#define SV_ERR_SHAPE (-2)       /* B < 0, k < 0, G/V < 1, k > SV_MAX_K, G*(k+1) > */
                                /* SV_MAX_ROWS_PER_SEQ, row_stride < V, or   */
                                /* the launch grid would be too large        */
#define SV_ERR_DTYPE (-3)       /* dtype is not SV_DTYPE_F32/SV_DTYPE_BF16  */
#define SV_ERR_TEMPERATURE (-4) /* temperature <= 0 or not finite           */
#define SV_ERR_WORKSPACE (-5)   /* workspace smaller than required or not   */
                                /* 256-byte aligned                         */
#define SV_ERR_HIP (-6)         /* the HIP runtime refused the launch       */
#define SV_ERR_SCRATCH (-7)     /* sv_verify_stochastic_noalloc: the shape  */
                                /* needs more than SV_SCRATCH_BYTES         */

/* Logit element types. */
#define SV_DTYPE_F32 0
#define SV_DTYPE_BF16 1

/* Limits. */
#define SV_MAX_K 64               /* draft tokens per sequence (candidate)   */
#define SV_MAX_ROWS_PER_SEQ 1024  /* G*(k+1) in greedy mode                 */
/* Device memory the library holds on each GPU it runs on, for
 * sv_verify_stochastic_noalloc: 8 MiB. */
#define SV_SCRATCH_BYTES 8388608u

/*
 * Stochastic verification of B sequences.
 *   target_logits  [B][k+1] rows of V logits (see layout above)
 *   draft_logits   [B][k]   rows, same dtype and row_stride as the target
 *   draft_tokens   int32 [B][k]
 *   u_accept       float [B][k]  acceptance uniforms, one per position
 *   u_sample       float [B]     one uniform per sequence for the extra token
 *   temperature    divides target and draft logits alike
 *   accept_len     out int32 [B]: accepted draft tokens a in [0, k]
 *   tokens         out int32 [B][k+1]: x_0..x_{a-1}, the extra token, then -1
 *   dbg_px_qx      optional out float [B][k][2]: p_i(x_i), q_i(x_i) for every
 *                  position (NULL to skip)
 * B == 0 is a no-op that returns SV_OK.  k = 0 is allowed (no draft tokens:
 * the one emitted token is sampled from target row 0; draft_logits,
 * draft_tokens and u_accept may then be NULL).
 *
 * Rows after a sequence's first rejection cannot change accept_len or
 * tokens.  Without dbg_px_qx, a batch large enough to give every sequence its
 * own workgroup (B >= 192) stops reading a sequence at its first rejection
 * (the "early termination" of Novita's verification strategy, read as
 * stopping at the first mismatch); with dbg_px_qx every position of every
 * sequence is evaluated.  The outputs are the same either way.  Given a
 * workspace of sv_workspace_bytes(B, 1, k, V) bytes, batches with 128 <= B
 * <= 1024 and k >= 6 use it to keep the few sequences that accept a long run
 * from holding the GPU: each sequence's own workgroup streams at most its
 * first few pairs, stopping at the first rejection, and the rows of the
 * sequences still accepting after them are then spread over all compute
 * units (with NULL, 0 the single-workgroup early exit runs instead for
 * B >= 192, with the same decisions and tokens; below 192 the workspace is
 * required).
 */
int sv_verify_stochastic(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* u_accept,
                         const float* u_sample, int B, int k, int V,
                         int64_t row_stride, int dtype, float temperature,
                         int32_t* accept_len, int32_t* tokens,
                         float* dbg_px_qx, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Greedy verification of B sequences with G >= 1 candidates each.
 *   target_logits  [B][G][k+1] rows of V logits
 *   draft_tokens   int32 [B][G][k]
 *   accept_len     out int32 [B]: accepted tokens of the winning candidate
 *   tokens         out int32 [B][k+1]: its tokens, the target argmax after
 *                  them, then -1
 *   best_cand      optional out int32 [B]: index of the winning candidate
 * B == 0 is a no-op that returns SV_OK.
 */
int sv_verify_greedy(const void* target_logits, const int32_t* draft_tokens,
                     int B, int G, int k, int V, int64_t row_stride, int dtype,
                     int32_t* accept_len, int32_t* tokens, int32_t* best_cand,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged batches: sequence b carries k_b = cu_draft_len[b+1] - cu_draft_len[b]
 * draft tokens, 0 <= k_b <= k_max, cu_draft_len[0] = 0 (cumulative lengths,
 * int32 [B+1], device memory), total_draft = cu_draft_len[B] (known to the
 * caller, who sized the buffers).  Rows are packed: target rows of sequence b
 * are rows cu[b] + b .. cu[b] + b + k_b of target_logits (total_draft + B
 * rows), its draft rows cu[b] .. cu[b] + k_b - 1 of draft_logits
 * (total_draft rows); draft_tokens and u_accept hold total_draft entries at
 * cu[b] ..; dbg_px_qx is [total_draft][2].  Outputs keep the dense shapes:
 * accept_len [B], tokens [B][k_max + 1] (-1 after each sequence's extra
 * token).  A sequence with k_b = 0 just samples its one target row.  Draft
 * lengths that change per sequence and per step are what Novita's blog
 * describes in its section "Метод реализации" (the number of candidates is
 * steered by an adaptive probability threshold; its Fig. 1 shows the draft
 * length varying), and aidevelopers.cz reports that the gain depends on the
 * draft length.  Each sequence is verified exactly as a dense batch of one with its
 * own k would be.  Malformed cu_draft_len values cannot make the library
 * read outside buffers of the stated sizes (they are clamped on the device),
 * but give undefined results.  draft_logits, draft_tokens and u_accept may
 * be NULL when total_draft == 0.  Workspace: sv_workspace_bytes(B, 1, k_max, V)
 * (the capped early exit of sv_verify_stochastic applies with k_max for k).
 */
int sv_verify_stochastic_ragged(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const int32_t* cu_draft_len,
                                int total_draft, const float* u_accept,
                                const float* u_sample, int B, int k_max, int V,
                                int64_t row_stride, int dtype, float temperature,
                                int32_t* accept_len, int32_t* tokens, float* dbg_px_qx,
                                void* workspace, size_t workspace_bytes, void* stream);

int sv_verify_greedy_ragged(const void* target_logits, const int32_t* draft_tokens,
                            const int32_t* cu_draft_len, int total_draft, int B, int k_max,
                            int V, int64_t row_stride, int dtype, int32_t* accept_len,
                            int32_t* tokens, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Plain sampling of one token per row -- the step the drafter and the prefill
 * take before verification (Perplexity, section "Cieľ-Návrh": at prefill the
 * target logits are sampled at once; the draft samples one token per step).
 *   logits   [B] rows of V logits (row_stride, dtype as above)
 *   u        float [B]: the uniform of each row (unused, may be NULL, when greedy)
 *   greedy   nonzero: the argmax of each row (lowest index on ties);
 *            zero: inverse CDF of softmax(row / temperature) at u[b]
 *   tokens   out int32 [B]
 * It is the verification of sequences with no draft tokens.  Workspace:
 * sv_workspace_bytes(B, 1, 0, V); none (NULL, 0) where each row is sampled
 * in one pass by one workgroup (the faster layout there): not greedy, and
 * B <= 256 with V <= 40960 + 352 B, or 256 < B <= 512 with V <= 40960 or
 * (B >= 320 and) V <= 98304 -- with V at most 32768 (B <= 256) or 16384
 * (B > 256) unless logits and the row stride are 16-byte aligned.
 */
int sv_sample(const void* logits, const float* u, int B, int V, int64_t row_stride, int dtype,
              float temperature, int greedy, int32_t* tokens, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * Greedy verification of a draft tree per sequence: the Top-K tree of the
 * EAGLE scheme (Perplexity, "Accelerating Sonar through speculation", section
 * "EAGLE": several draft continuations are explored as a tree, the longest
 * acceptable one is kept and the target adds one more token).
 *   target_logits [B][N] rows: row j of sequence b (at (b*N + j) * row_stride)
 *                 is the target's output at node j, i.e. its prediction of
 *                 the token that follows node j's path (tree attention mask
 *                 on the model side)
 *   node_tokens   int32 [B][N]: the draft token of node j (node 0, the root,
 *                 is the last committed token and is not verified)
 *   parents       int32 [B][N]: parent of node j, in [0, j) for j >= 1;
 *                 parents[b][0] = -1
 *   accept_len    out int32 [B]: depth d of the winning node
 *   tokens        out int32 [B][N]: the draft tokens along the root-to-winner
 *                 path, then the argmax of the winner's row; -1 after
 *   path          out int32 [B][N]: node indices root, ..., winner; -1 after
 * Node j is accepted when its parent is and its token equals the argmax
 * (lowest index on ties) of the parent's row; the deepest accepted node wins,
 * lowest node index among equal depths.  A chain (parents[j] = j - 1) is
 * sv_verify_greedy with k = N - 1.  1 <= N <= SV_MAX_ROWS_PER_SEQ.  A parent
 * outside [0, j) is not checked on the host: that node is never accepted.
 * Workspace: sv_workspace_bytes(B, N, 0, V).
 */
int sv_verify_greedy_tree(const void* target_logits, const int32_t* node_tokens,
                          const int32_t* parents, int B, int N, int V, int64_t row_stride,
                          int dtype, int32_t* accept_len, int32_t* tokens, int32_t* path,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Commit of a verified step on the GPU, so that the next step can be launched
 * without the host reading accept_len first (Perplexity, same page, sections
 * "MTP" and "Plánovanie MTP pre Jediný Token": the accepted tokens are shifted
 * into place by kernels and the next draft runs on the same batch, the host
 * learns the lengths in parallel).  For sequence b, with a = accept_len[b]
 * and L = seq_len[b]:
 *   history[b][L + j] = tokens[b][j] for j = 0..a while L + j < capacity
 *   seq_len[b]        = min(L + a + 1, capacity)   (unchanged if L >= capacity)
 *   next_token[b * next_stride] = tokens[b][a]     (the token the next step
 *                                                    starts from)
 *   accept_len [B], tokens [B][W] as the verification calls write them (W =
 *   k + 1, k_max + 1 or N); seq_len int32 [B] in/out; history int32 rows of
 *   history_stride >= capacity entries.  An accept_len outside [0, W - 1] or
 *   a negative seq_len is clamped into range (undefined result, no
 *   out-of-bounds access).  No workspace.
 */
int sv_commit(const int32_t* accept_len, const int32_t* tokens, int B, int W, int32_t* seq_len,
              int32_t* history, int64_t history_stride, int capacity, int32_t* next_token,
              int64_t next_stride, void* stream);

/*
 * sv_verify_stochastic without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * hosts that forbid hipMalloc.  Arguments, outputs and results are exactly
 * those of sv_verify_stochastic given a workspace of sv_workspace_bytes(B, 1,
 * k, V) bytes (same kernels, bit-identical outputs).  The workspace is a
 * buffer of SV_SCRATCH_BYTES that the library holds on each GPU from the
 * first call there until the process ends; this call allocates nothing.
 * Shapes whose sv_workspace_bytes(B, 1, k, V) exceeds SV_SCRATCH_BYTES return
 * SV_ERR_SCRATCH before anything is launched.  Every call on one GPU shares
 * that GPU's buffer: calls that overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race.  The stream decides the
 * GPU; NULL means the current device.
 */
int sv_verify_stochastic_noalloc(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* u_accept,
                                 const float* u_sample, int B, int k, int V,
                                 int64_t row_stride, int dtype, float temperature,
                                 int32_t* accept_len, int32_t* tokens, float* dbg_px_qx,
                                 void* stream);

/* Workspace bytes that suffice for any entry point at this shape (G = 1 for
 * stochastic, ragged (k = k_max) and sampling (k = 0) calls; G = N, k = 0 for
 * tree verification).  Returns 0 for an invalid shape. */
size_t sv_workspace_bytes(int B, int G, int k, int V);

/* Static, human-readable text for a status code. */
const char* sv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
