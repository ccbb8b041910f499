/*
 * specverify.h - C ABI of the MI355X (gfx950) greedy speculative-decoding verify path.
 *
 * One verify round, all on the device, no host synchronisation inside it:
 *   specverify_propose  n-gram prompt-lookup drafter over the committed token stream
 *   specverify_verify   int8 per-block-32 head matmul of the S = K+1 window + per-row argmax
 *   specverify_accept   greedy longest-prefix acceptance, commits 1 + j tokens
 *   specverify_round    the three fused: verify -> accept -> the next drafts
 *   specverify_*_sample sampling verify at temperature > 0 (probabilities, residual redraw)
 *   specverify_*_tree   tree drafts (merged n-gram matches) and the greedy walk down the tree
 *   specverify_*_q4b32  the same head with int4 per-block-32 codes
 *   specverify_generate[_sample|_tree]  many rounds back to back on the device, window rows
 *                       gathered from a token-indexed stand-in model (specverify_gather_window)
 * plus the dense weight-bound stack in front of the head (rmsnorm, gate/up + SiLU*mul,
 * down + residual) built on the same int8 matmul core.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers (hipMalloc'd, or torch CUDA tensors), owned by the caller
 *     and valid until the work enqueued on `stream` has completed.  `stream` is a
 *     hipStream_t; NULL means the default stream.
 *   - A call validates its arguments, then enqueues kernels on `stream` and returns.  It
 *     never allocates, frees, synchronises, prints, aborts or throws.
 *   - The return value is an sv_status.  Argument errors are detected on the host before any
 *     HIP call is made and nothing is enqueued.  SV_ERR_HIP reports a launch failure; the
 *     detail is in specverify_last_error() (thread-local).
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - Calls on one stream are ordered; calls that share output buffers on different streams
 *     race unless the caller orders them.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_NULL = 1,       /* a required pointer is NULL                                  */
    SV_ERR_SHAPE = 2,      /* a size is out of range or inconsistent                      */
    SV_ERR_ALIGN = 3,      /* a pointer is not aligned as documented                      */
    SV_ERR_WORKSPACE = 4,  /* workspace smaller than the *_workspace_bytes() answer       */
    SV_ERR_CAPACITY = 5,   /* token buffer capacity too small for the call                */
    SV_ERR_HIP = 6,        /* a HIP call failed (see specverify_last_error)               */
    SV_ERR_DEVICE = 7      /* the current device is not gfx950                            */
} sv_status;

/* Limits. */
#define SV_MAX_S 64        /* rows of one verify window (K <= 63)                          */
#define SV_MAX_NGRAM 8     /* largest n-gram order of the drafter                          */
#define SV_BLOCK 32        /* quantization block length along the hidden axis             */

/*
 * Round state: int32_t[SV_STATE_WORDS] on the device, zero-filled by the caller before the
 * first call, then owned by the library's kernels.
 *   [0] len      committed tokens in `tokens`; tokens[len-1] is the pending anchor a0
 *   [1] j        drafts accepted by the last specverify_accept
 *   [2] n_valid  non-pad drafts written by the last specverify_propose
 *   [3] n_used   n-gram order that matched in the last propose (0 = no match)
 *   [4] flags    sticky error bits: bit 0 = a call would have overflowed `cap` or found
 *                len outside [0, cap] (that call wrote no token); bit 1 = a gathered token
 *                id was outside [0, V); bit 2 = the id an accept would commit after the
 *                accepted drafts was -1, i.e. that window row had no argmax or draw (every
 *                logit NaN, e.g. from an overflowed activation): that call wrote no token
 *                and recorded no round
 *   [5] rounds   number of accept calls that committed tokens
 *   [6] sum_j    sum of j over those calls
 *   [7] reserved
 *   [8 + j]      histogram of j, j = 0 .. SV_MAX_S-1
 *   [72] gate_after  hit-rate gate, set by the caller (0 = off): once this many consecutive
 *                    rounds have accepted no draft, the drafter emits only pads for the rest
 *                    of the stream ("Stream C - Speculative decoding", the shipped app note:
 *                    the drafter is dropped after gateAfter zero-accept rounds)
 *   [73] zero_run    consecutive rounds with j = 0, kept by the accept step
 *   [74] gated       0, or the round count at which the gate fired (sticky)
 */
#define SV_STATE_WORDS 80
#define SV_STATE_LEN 0
#define SV_STATE_J 1
#define SV_STATE_NVALID 2
#define SV_STATE_NUSED 3
#define SV_STATE_FLAGS 4
#define SV_STATE_ROUNDS 5
#define SV_STATE_SUMJ 6
#define SV_STATE_HIST 8
#define SV_STATE_GATE_AFTER 72
#define SV_STATE_ZERO_RUN 73
#define SV_STATE_GATED 74
#define SV_FLAG_CAPACITY 1
#define SV_FLAG_TOKEN 2    /* a token id outside [0, V) was gathered (its row read as zeros) */
#define SV_FLAG_ARGMAX 4   /* the row whose id would be committed had no argmax (all NaN)    */

/*
 * specverify_propose - n-gram prompt-lookup drafter.
 * Page: "Stream C - Speculative decoding: feasibility verdict + implementation plan",
 * section "The delta" (a hashtable over the prompt+generated stream maps the last m tokens
 * to their most recent continuation; draft cost is nil) and the handoff's n-gram order /
 * draft length knobs; "Spec-decode on GDN hybrids - static-S verify design", harness
 * lessons (the stream ends in the pending anchor, drafts continue past it).
 *
 * Once the hit-rate gate has fired (state[74] != 0) every draft is -1 and nothing is read.
 * Otherwise reads tokens[0 .. len) with len = state[0].  For n = ngram_max, ..., 1 the first n whose
 * last-n suffix occurs earlier wins; among its occurrences the one ending latest (end
 * position e <= len-2, overlap with the suffix allowed) is used, and
 *   drafts[i] = tokens[e+1+i]  for e+1+i <= len-1,  else -1,   i = 0 .. K-1.
 * No match: all K drafts are -1.  Writes state[2] (non-pad drafts) and state[3] (n used).
 *   tokens    int32 [cap], 4-byte aligned; ids are compared, never range-checked
 *   cap       capacity of `tokens`; a state with len outside [0, cap] sets bit 0 of
 *             state[4] and is treated as an empty stream (all pads)
 *   ngram_max 1 .. SV_MAX_NGRAM (3 in the reference workloads)
 *   K         1 .. SV_MAX_S-1
 *   drafts    int32 [K] output
 */
int specverify_propose(const int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max,
                       int32_t K, int32_t* drafts, hipStream_t stream);

/*
 * specverify_verify - q8b32 head matmul of the verify window with a fused per-row argmax.
 * Pages: "Riding Apple's pipelined GPU engine", section "Quantization on the GPU delegate"
 * (linear per-block-32 int8 head with absmax symmetric scales) and section "Why hand-rolled
 * per-token loops lose" (sample on the GPU, only the sampled ids leave it);
 * "Stream C - Speculative decoding", sections "C1 - Engine substrate map" and "The delta"
 * (one verify forward gives logits for every window position; a batched [K, vocab] -> [K]
 * argmax replaces the full-logits readback); "Spec-decode on GDN hybrids", verify graph
 * (static S = K+1 window, all-position logits).
 *
 *   L[s, v]   = sum_b f32(wscale[v, b]) * sum_{k in block b} f32(wq[v, k]) * f32(hidden[s, k])
 *   argmax[s] = min { v : L[s, v] = max_v' L[s, v'] }   (largest logit, lowest id on ties)
 * Products are exact, accumulation is fp32.  A NaN logit never wins; a row whose logits are
 * all NaN gets argmax -1, which the accept steps refuse to commit (flag bit 2).
 *   wq        int8 [V][H] row-major (vocab row contiguous), 16-byte aligned
 *   wscale    fp16 [V][H/32] row-major (block b of row v at v*H/32 + b), 16-byte aligned
 *   V         1 .. 2^30;   H: multiple of 32, 32 .. 65536
 *   hidden    fp16 [S][H] row-major, 16-byte aligned;   S: 1 .. SV_MAX_S
 *   argmax    int32 [S] output
 *   logits    fp32 [S][V] output, or NULL (the timed path writes no logits)
 *   workspace device scratch of at least specverify_verify_workspace_bytes(V, H, S) bytes,
 *             16-byte aligned; its contents need no initialisation and are clobbered, so
 *             calls that share a workspace must be ordered (one stream)
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_ALIGN, SV_ERR_WORKSPACE, SV_ERR_DEVICE, SV_ERR_HIP.
 */
size_t specverify_verify_workspace_bytes(int32_t V, int32_t H, int32_t S);
int specverify_verify(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                      const uint16_t* hidden, int32_t S, int32_t* argmax, float* logits,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * specverify_round - one whole verify round in as few launches as the shape allows:
 *   specverify_verify(hidden, S = K+1) -> specverify_accept(argmax, drafts_in)
 *   -> specverify_propose(next drafts into drafts_out)
 * with the same results as the three calls in that order, in two launches: the matmul, then
 * one workgroup that reduces the argmax, accepts and drafts from LDS ("Riding Apple's
 * pipelined GPU engine", section "Why hand-rolled per-token loops lose": per-step
 * dispatches and host round trips are what a pipelined engine removes).
 *   hidden     fp16 [K+1][H], the rows of the window [a0, d_1 .. d_K]
 *   drafts_in  int32 [K] drafts being verified; drafts_out int32 [K] the next round's drafts
 *              (may alias drafts_in: the accept reads them before the drafter writes)
 *   other arguments as for specverify_verify / _accept / _propose; K in 1 .. SV_MAX_S-1.
 */
int specverify_round(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                     const uint16_t* hidden, int32_t K, const int32_t* drafts_in, int32_t* tokens,
                     int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts_out,
                     int32_t* argmax, float* logits, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * specverify_round_noalloc - specverify_round for callers that cannot allocate device memory
 * or hand the library a workspace: code under HIP graph capture that must not allocate,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, results and errors
 * as specverify_round, minus the workspace: its scratch (the head's per-workgroup argmax
 * partials) is a library-held static device array of 2 MiB, one per GPU, kept until the
 * process ends.  The call allocates nothing.  Every call on one GPU shares that GPU's array,
 * and nothing in it needs to start at zero: calls on one stream are ordered, but calls that
 * overlap on one GPU (streams not ordered against each other) race and must not be made.
 * The array holds the argmax partials of any window (S <= SV_MAX_S), and the split sums of a
 * hidden axis split across workgroups when they fit: a shape whose specverify_verify_
 * workspace_bytes answer exceeds 2 MiB (a split hidden axis over a large vocabulary, e.g.
 * V = 30000 at H = 16384) fails with SV_ERR_SHAPE before anything is enqueued.
 */
int specverify_round_noalloc(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                             const uint16_t* hidden, int32_t K, const int32_t* drafts_in, int32_t* tokens,
                             int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts_out,
                             int32_t* argmax, float* logits, hipStream_t stream);

/*
 * specverify_verify_q4b32 / specverify_round_q4b32 - the int4 per-block-32 head: the same
 * contract as specverify_verify / specverify_round with half the weight bytes.
 * Page: "Riding Apple's pipelined GPU engine", sections "Quantization on the GPU delegate"
 * (int4 linear per-block-32, the int4 class that ships) and "Numerics gating" (QAT q4_0
 * weights follow the per-block-32 absmax grid).
 *   L[s, v] = sum_b f32(wscale[v, b]) * sum_{k in block b} code[v, k] * f32(hidden[s, k])
 *   wq      uint8 [V][H/2]: per 32-block 16 bytes, byte i = (element i + 8) | (element i+16 + 8) << 4,
 *           codes -8 .. 7 (the library's quantizer writes -7 .. 7); 16-byte aligned
 *   wscale  fp16 [V][H/32], 16-byte aligned;   H: multiple of 256 in [256, 65536] that 8 or
 *           16 blocks per wave cover with 1 .. 16 waves (e.g. 512, 1024, 2048, 2560, 3072,
 *           4096, 5120 ...);   S = K+1: 1 .. 16
 *   workspace  at least specverify_verify_workspace_bytes(V, H, S) bytes
 * Other arguments and errors as for specverify_verify / specverify_round.
 */
int specverify_verify_q4b32(const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                            const uint16_t* hidden, int32_t S, int32_t* argmax, float* logits,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
int specverify_round_q4b32(const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                           const uint16_t* hidden, int32_t K, const int32_t* drafts_in,
                           int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max,
                           int32_t* drafts_out, int32_t* argmax, float* logits, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Sampling verify (temperature > 0): specverify_verify_sample, specverify_accept_sample and
 * the fused specverify_round_sample.
 * Page: "Stream C - Speculative decoding", the deferred list (sampling stays lossless only if
 * verify uses the target's probabilities and redraws a rejected position from the residual
 * distribution).  The rule is standard speculative sampling for a drafter that proposes one
 * token per position (the n-gram drafter, q = point mass at d):
 *   z_s = L[s, :] / T,  p_s = softmax(z_s),  lse_s = log sum_v exp(z_s[v])
 *   draft d_{s+1} is kept iff it is a vocabulary id and u_s < p_s(d_{s+1}) = exp(z_s[d] - lse_s)
 *   at the first draft not kept (j), row j's token is drawn from max(0, p_j - e_d) renormalised
 *   (the ids other than d_{j+1}); if all K are kept, row K's token is drawn from p_K;
 *   the round appends d_1..d_j and that draw (len += 1 + j), as the greedy round does.
 * Random numbers are Philox4x32-10 (Salmon et al., SC'11) with key = seed (low word first); a
 * round that starts at len = state[0] = P0 uses for the draw of row s, id v the counter
 * (v, P0, s/4, 0), word s%4, and for the test of d_{s+1} the counter (0, P0, s/4, 1), word
 * s%4; a word w becomes u = (floor(w / 2^9) + 0.5) / 2^23.  Draws use Gumbel-max: the id of
 * the largest z_s[v] - log(-log u), lowest id on equal keys.  Window rows S = K+1 <= 16.
 *
 * specverify_verify_sample - the head matmul with the sampling epilogue:
 *   sample[s]  int32 [S]: row s's draw from its residual against d_{s+1} (row S-1: from p)
 *   lse[s]     fp32 [S]:  lse_s;   zd[s] fp32 [S]: z_s[d_{s+1}] for rows with a vocabulary-id
 *              draft (other entries are not written);   logits fp32 [S][V] or NULL (L, not z)
 *   drafts     int32 [S-1] (NULL when S = 1);  state: state[0] gives P0 (read only)
 *   temperature > 0, finite, with a finite inverse;  workspace: specverify_sample_workspace_bytes
 * specverify_accept_sample - the accept step from those outputs (one wave); K in 0 .. 15, K = 0
 *   commits sample[0] (the bootstrap draw of the anchor) and is not counted as a round.
 * specverify_round_sample - verify_sample -> accept_sample -> specverify_propose in two
 *   launches; sample / lse (may be NULL) receive the per-row draws and log-normalisers.
 * Errors as for specverify_verify / specverify_round; SV_ERR_SHAPE for a temperature out of
 * range or S > 16.
 */
size_t specverify_sample_workspace_bytes(int32_t V, int32_t H, int32_t S);
int specverify_verify_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                             const uint16_t* hidden, int32_t S, const int32_t* drafts,
                             float temperature, uint64_t seed, const int32_t* state,
                             int32_t* sample, float* lse, float* zd, float* logits,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
int specverify_accept_sample(const int32_t* sample, const float* lse, const float* zd,
                             const int32_t* drafts, int32_t K, int32_t V, uint64_t seed,
                             int32_t* tokens, int32_t cap, int32_t* state, hipStream_t stream);
int specverify_round_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                            const uint16_t* hidden, int32_t K, const int32_t* drafts_in,
                            float temperature, uint64_t seed, int32_t* tokens, int32_t cap,
                            int32_t* state, int32_t ngram_max, int32_t* drafts_out,
                            int32_t* sample, float* lse, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Tree verify (greedy): specverify_propose_tree, specverify_accept_tree and the fused
 * specverify_round_tree.
 * Page: "Stream C - Speculative decoding", the EAGLE-3 + tree handoff and the deferred list
 * (the drafter proposes a tree; one verify forward covers every node under a tree attention
 * mask; the linear accept becomes a walk down the tree).
 * Tree: K draft nodes (1 .. 15) under the anchor a0 (node 0); node i (1..K) has parent
 * parents[i-1] (0 <= parents[i-1] < i) and token drafts[i-1] (-1 = a pad, never matched).
 * Window row i is the row after the path root -> i, S = K+1 <= 16 rows (for a token-indexed
 * model, specverify_gather_window of `drafts` gives them).
 *   accept:  from node c = 0, move to the lowest-index child of c whose token is argmax[c];
 *            repeat until none matches; append the path's tokens and argmax of the last node
 *            (len += 1 + j, j = path length); statistics and the hit-rate gate as the linear
 *            accept.  Children listed with a parent index >= their own index are ignored.
 *   drafter: the `branches` (1 .. 4) best earlier end positions of the stream's suffix, ranked
 *            as specverify_propose ranks them (longer match up to ngram_max, then more recent),
 *            each continued for up to `depth` (1 .. K) tokens, inserted into a prefix tree in
 *            rank order (a node is reused when its parent already has a child with that
 *            token) until K nodes exist; free slots become pads under the root.  state[2]
 *            = real nodes, state[3] = match length of the best position.  One branch of depth
 *            K gives specverify_propose's drafts as a chain (parents 0, 1, 2, ...).
 *   specverify_round_tree = specverify_verify(hidden, S = K+1) -> accept_tree -> propose_tree
 *            in two launches; parents_out / drafts_out may alias parents_in / drafts_in.
 * Arguments not listed are as for specverify_verify / specverify_round / specverify_propose.
 * Errors: SV_ERR_SHAPE for K, branches, depth or ngram_max out of range; otherwise as those.
 */
int specverify_propose_tree(const int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max,
                            int32_t K, int32_t branches, int32_t depth, int32_t* parents,
                            int32_t* drafts, hipStream_t stream);
int specverify_accept_tree(const int32_t* argmax, const int32_t* parents, const int32_t* drafts,
                           int32_t K, int32_t* tokens, int32_t cap, int32_t* state,
                           hipStream_t stream);
int specverify_round_tree(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                          const uint16_t* hidden, int32_t K, const int32_t* parents_in,
                          const int32_t* drafts_in, int32_t* tokens, int32_t cap, int32_t* state,
                          int32_t ngram_max, int32_t branches, int32_t depth,
                          int32_t* parents_out, int32_t* drafts_out, int32_t* argmax,
                          float* logits, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * specverify_gather_window - the window rows of a token-indexed stand-in model:
 *   window[0] = table[tokens[len-1]] (the anchor a0, len = state[0]),
 *   window[i] = table[drafts[i-1]] for i = 1 .. K, a pad (-1) reading token 0's row,
 * so a whole generation loop stays on the device (the model body is a per-token table, the
 * "Markov" stand-in of the control-logic proof in "Stream C - Speculative decoding"; pads
 * feed token 0 as in the static-S window of "Spec-decode on GDN hybrids").
 *   table   fp16 [V][H], 16-byte aligned;  window fp16 [K+1][H] output, 16-byte aligned
 *   K       0 .. SV_MAX_S-1 (drafts may be NULL when K = 0)
 * An id outside [0, V) writes a zero row and sets bit 1 (SV_FLAG_TOKEN) of state[4]; a
 * length outside [1, cap] writes zero rows and sets bit 0.
 */
int specverify_gather_window(const int32_t* tokens, int32_t cap, int32_t* state,
                             const int32_t* drafts, int32_t K, const uint16_t* table, int32_t V,
                             int32_t H, uint16_t* window, hipStream_t stream);

/*
 * specverify_gather_positions - the window rows of a position-indexed stand-in model, whose
 * row after a prefix of p + 1 ids is rows[p] whatever the ids (a target whose greedy
 * continuation is fixed in advance, e.g. a recorded trajectory):
 *   window[i] = rows[len - 1 + i] for i = 0 .. K, len = state[0]
 * so rounds over such a target stay on the device.  Rows after a rejected draft are never used
 * by an accept, so this is a valid target for speculative decoding ("Stream C - Speculative
 * decoding", control-logic proof: the committed stream is the target's greedy stream).
 *   rows    fp16 [nrows][H], 16-byte aligned;  window fp16 [K+1][H] output, 16-byte aligned
 *   K       0 .. SV_MAX_S-1;  cap: capacity of the caller's token buffer (len is checked against it)
 * A position outside [0, nrows) or a length outside [1, cap] writes a zero row and sets bit 0
 * of state[4].
 */
int specverify_gather_positions(int32_t* state, int32_t cap, const uint16_t* rows, int32_t nrows, int32_t H,
                                int32_t K, uint16_t* window, hipStream_t stream);

/*
 * specverify_generate - `rounds` speculative-decoding rounds enqueued back to back with no
 * host synchronisation ("Riding Apple's pipelined GPU engine", "Why hand-rolled per-token
 * loops lose": encode and return, only sampled ids leave the GPU).  Each round is
 *   specverify_gather_window(table) -> specverify_round(window, drafts -> drafts)
 * i.e. verify [a0, d_1 .. d_K], accept, draft the next round, with the hit-rate gate of the
 * state word.  Before the first call the stream must hold its anchor (the bootstrap:
 * specverify_verify at S = 1 and specverify_accept with K = 0) and `drafts` the first
 * drafts (specverify_propose).  A round that would overflow `cap` commits nothing and sets
 * the capacity flag; later rounds then repeat the same window.  Capturable in a HIP graph
 * (no allocation, no memset, no synchronisation).
 *   table   fp16 [V][H] (the stand-in model);  window fp16 [K+1][H] scratch;  argmax int32 [K+1]
 *   drafts  int32 [K], read and rewritten by every round;  rounds >= 0
 *   other arguments as for specverify_round; logits are not written.
 */
int specverify_generate(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                        const uint16_t* table, int32_t K, int32_t rounds, int32_t* tokens,
                        int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts,
                        uint16_t* window, int32_t* argmax, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * specverify_generate_sample / specverify_generate_tree - the same device-resident loop for
 * sampling verify and for tree verify ("Riding Apple's pipelined GPU engine", "Why hand-rolled
 * per-token loops lose"; "Stream C - Speculative decoding", the deferred list: sampling and
 * tree proposals).  Each round is
 *   specverify_gather_window(table, drafts) -> specverify_round_sample(window, drafts -> drafts)
 *   specverify_gather_window(table, drafts) -> specverify_round_tree(window, tree -> tree)
 * For a tree, window row i is the table row of node i's own token: under the token-indexed
 * model that is the row after the path root -> i.  The sampling noise is keyed by `seed` and
 * the stream position, so one seed serves every round of a stream.  Before the first call the
 * stream must hold its anchor and `drafts` (and `parents`) the first proposal
 * (specverify_propose / specverify_propose_tree).  Capacity: as specverify_generate.
 * Capturable in a HIP graph.
 *   table  fp16 [V][H];  window fp16 [K+1][H] scratch;  K 1 .. 15;  rounds >= 0
 *   drafts int32 [K] (and parents int32 [K]), read and rewritten by every round
 *   other arguments as for specverify_round_sample / specverify_round_tree; the sampling loop
 *   writes no per-row draws or log-normalisers, the tree loop no logits.
 * Errors: as specverify_generate, and as the round entry points.
 */
int specverify_generate_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                               const uint16_t* table, int32_t K, int32_t rounds, float temperature,
                               uint64_t seed, int32_t* tokens, int32_t cap, int32_t* state,
                               int32_t ngram_max, int32_t* drafts, uint16_t* window,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
int specverify_generate_tree(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                             const uint16_t* table, int32_t K, int32_t rounds, int32_t* tokens,
                             int32_t cap, int32_t* state, int32_t ngram_max, int32_t branches,
                             int32_t depth, int32_t* parents, int32_t* drafts, uint16_t* window,
                             int32_t* argmax, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * specverify_accept - greedy longest-prefix acceptance with the fused anchor.
 * Pages: "Stream C - Speculative decoding", sections "The delta" and "Control-logic proof"
 * (draft i is accepted iff it equals the greedy id of its position and every earlier draft
 * was accepted; the first miss emits the correction, all-accept emits the bonus) and
 * "Implementation status" (fused scheme: the anchor a0 is always correct; a round commits
 * what was accepted); "Spec-decode on GDN hybrids", hybrid state discipline (the row after
 * the last accepted token is the next anchor: correction and bonus are one rule).
 *
 * argmax[0..K] are the greedy ids of the window [a0, d_1 .. d_K]; drafts[0..K-1] = d_1..d_K.
 *   j = max { i in [0, K] : drafts[m-1] == argmax[m-1] for all 1 <= m <= i }
 * Writes tokens[len .. len+j] = d_1 .. d_j, argmax[j] and sets len += 1 + j (state[0]);
 * records j in state[1], state[5], state[6] and the histogram, and advances the hit-rate
 * gate (state[73], state[74]).  K = 0 appends argmax[0]: the anchor bootstrap of a fresh
 * stream (it records nothing else).
 * If len + K + 1 > cap the call writes no token and sets bit 0 of state[4] (sticky).
 *   argmax    int32 [K+1];  drafts int32 [K] (may be NULL when K = 0); -1 = pad
 *   K         0 .. SV_MAX_S-1;  tokens int32 [cap]
 */
int specverify_accept(const int32_t* argmax, const int32_t* drafts, int32_t K, int32_t* tokens,
                      int32_t cap, int32_t* state, hipStream_t stream);

/*
 * Weight-bound dense stack in front of the head (all projections q8b32, same layout and
 * matmul core as specverify_verify).  Page: "Flagship dramatic-speedup plan - the full
 * stackable tuning set", sections "Baseline byte model" (decode reads every weight byte
 * once per forward) and "Axis 4" (fused RMSNorm and SwiGLU).  The pages do not fix the
 * block; the library implements the weightless pre-norm residual MLP block:
 *
 * specverify_rmsnorm: y[s, :] = fp16(x[s, :] / sqrt(mean_k x[s, k]^2 + eps)), fp32 math.
 *   x, y fp16 [S][H] (may alias), S 1 .. SV_MAX_S, H multiple of 32, 16-byte aligned.
 *
 * specverify_gateup_silu_q8b32: m[s, n] = fp16(silu(g) * u) with
 *   g = sum_k x[s, k] Wg[n, k] and u = sum_k x[s, k] Wu[n, k] (fp32), silu(g) = g/(1+e^-g).
 *   wg, wu int8 [N][Kin]; sg, su fp16 [N][Kin/32]; x fp16 [S][Kin]; m fp16 [S][N].
 *
 * specverify_linear_q8b32: y[s, n] = fp16(sum_k x[s, k] W[n, k] + residual[s, n]) with
 *   residual fp16 [S][N] or NULL (then no add).  y may alias residual, never x.
 *   w int8 [N][Kin]; scale fp16 [N][Kin/32]; x fp16 [S][Kin]; y fp16 [S][N].
 *
 * specverify_linear_residual_rmsnorm_q8b32: specverify_linear_q8b32, then
 *   norm_out = specverify_rmsnorm(y, eps): the end of one block and the input norm of the
 *   next ("Axis 4": the norm fused into the neighbouring kernel).  When the hidden axis is
 *   split, one row pass sums the split partials, adds the residual, writes y and the norm.
 *   norm_out fp16 [S][N] must not alias x, y or residual (SV_ERR_SHAPE); eps >= 0.
 *
 * Both matmuls take S = 1 .. 16 and the alignment rules of specverify_verify (N plays V,
 * Kin plays H).  Very long Kin splits the hidden axis across workgroups and then needs a
 * scratch `workspace` of specverify_stack_workspace_bytes(N, Kin, S, gateup) bytes
 * (16-byte aligned, no initialisation); when that is 0, workspace may be NULL.
 */
int specverify_rmsnorm(const uint16_t* x, int32_t S, int32_t H, float eps, uint16_t* y,
                       hipStream_t stream);
size_t specverify_stack_workspace_bytes(int32_t N, int32_t Kin, int32_t S, int32_t gateup);
int specverify_gateup_silu_q8b32(const int8_t* wg, const uint16_t* sg, const int8_t* wu,
                                 const uint16_t* su, int32_t N, int32_t Kin,
                                 const uint16_t* x, int32_t S, uint16_t* m,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
int specverify_linear_q8b32(const int8_t* w, const uint16_t* scale, int32_t N, int32_t Kin,
                            const uint16_t* x, int32_t S, const uint16_t* residual, uint16_t* y,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
int specverify_linear_residual_rmsnorm_q8b32(const int8_t* w, const uint16_t* scale, int32_t N,
                                             int32_t Kin, const uint16_t* x, int32_t S,
                                             const uint16_t* residual, uint16_t* y, float eps,
                                             uint16_t* norm_out, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/*
 * specverify_stack - the whole weight-bound dense stack in front of the head, one call:
 * L blocks of [n = rmsnorm(x); m = fp16(silu(n Wg^T) * (n Wu^T)); x = fp16(x + m Wd^T)],
 * then norm_out = rmsnorm(x) (the head's input).  Pages: "Flagship dramatic-speedup plan -
 * the full stackable tuning set", "Baseline byte model" (every weight byte read once per
 * forward) and "Axis 4" (RMSNorm fused into the neighbouring kernels; SwiGLU in the
 * projection's epilogue).  Block as for the per-op calls above; rmsnorm(x) =
 * fp16(x / sqrt(mean(x^2) + eps)) with the sum of squares in fp32 over the fp16 values.
 *
 * Two launches per block: gate/up (normalising its window rows on the fly) and down (adding
 * the residual, storing x and the per-tile sums of squares the next norm needs).
 *   wg, wu  int8 [L][F][H] (layer l at l*F*H);  sg, su fp16 [L][F][H/32]
 *   wd      int8 [L][H][F];                      sd     fp16 [L][H][F/32]
 *   H, F    multiples of 512 in [512, 65536] with H * F < 2^31;   S 1 .. 16;   L 1 .. 4096;
 *           eps >= 0
 *   x       fp16 [S][H]: the stack's input; overwritten with the output of block L-1 when
 *           x_layers is NULL, else left unchanged
 *   x_layers fp16 [L][S][H] or NULL: the output of every block (for per-block checks)
 *   norm_out fp16 [S][H]: rmsnorm of the last block's output; must not overlap x or x_layers
 *   workspace  at least specverify_stack_forward_workspace_bytes(H, F, S) bytes, no
 *           initialisation; calls that share it must be ordered (one stream)
 * All pointers 16-byte aligned.  Errors: SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_ALIGN,
 * SV_ERR_WORKSPACE, SV_ERR_DEVICE, SV_ERR_HIP.  Returns 0 bytes for unsupported shapes.
 */
size_t specverify_stack_forward_workspace_bytes(int32_t H, int32_t F, int32_t S);
int specverify_stack(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                     const int8_t* wd, const uint16_t* sd, int32_t L, int32_t H, int32_t F,
                     uint16_t* x, int32_t S, float eps, uint16_t* x_layers, uint16_t* norm_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Launch-shape override of the q8b32 matmuls, for tuning sweeps: waves per workgroup
 * (4, 8 or 16; 0 = automatic), an upper bound on workgroups per launch (1 .. 4096;
 * 0 = automatic) and, for the chunked stack kernels, load units in flight per wave (2 .. 4;
 * 0 = automatic; a depth that has no kernel for a shape falls back to the automatic one),
 * and the head matmul kernel family (0 = automatic, 1 = one pass per 16-row item, 2 = the
 * chunked ring kernel where the shape allows it, S <= 16, 3 = automatic except that a
 * 17-row window uses two 16-row tiles instead of one tile plus the 17th row's dot
 * products), and the split of specverify_stack's down projection (0 or 1 = unsplit, the
 * automatic choice; 2 .. 8 = its hidden axis split that many ways across workgroups where a
 * held-row shape for the slices exists, else unsplit).  Waves that do not divide a chunked shape make specverify_stack
 * fail with SV_ERR_SHAPE.  The override belongs to the calling thread: it affects only calls
 * made from that thread (including its *_workspace_bytes answers, so query them after
 * changing it), and other threads keep the automatic choice.  (0, 0, 0, 0, 0) restores it.
 */
void specverify_set_tuning(int32_t waves_per_group, int32_t max_groups, int32_t depth,
                           int32_t head_kernel, int32_t split);

/*
 * Timing hook for the dominant kernel.  The next int8 or int4 matmul that this thread
 * enqueues through any entry point (the head matmul of specverify_verify / _round / the
 * sampling, tree and int4 variants, a per-op projection, or the first projection of
 * specverify_stack: block 0's gate/up) is launched with `before` and `after` attached to its
 * dispatch: they take the kernel's own start and end timestamps (the end of its
 * split-combine pass when the hidden axis is split across workgroups), the clock a kernel
 * trace reads; the hook is then cleared.  The events are the caller's (created on the
 * current device, timing enabled).  (NULL, NULL) clears a pending hook; one NULL alone is
 * SV_ERR_NULL.  Not for use under stream capture.
 */
int specverify_profile_next_matmul(hipEvent_t before, hipEvent_t after);

/* Static description of a status code. */
const char* specverify_status_string(int status);
/* Detail of the last failure on this thread ("" if none). */
const char* specverify_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
