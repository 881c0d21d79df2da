/*
 * specv -- batched speculative-sampling verification for AMD MI355X (gfx950).
 *
 * C ABI of libspecv.so. Every pointer argument documented as "device" is a
 * device pointer owned by the caller; the library never allocates, frees or
 * synchronises. Every call is asynchronous on the given HIP stream
 * (hipStream_t, passed as void*; NULL = the null stream) and returns after
 * enqueueing its kernels. Arguments are validated on the host before any
 * launch; on a non-OK status nothing was launched (except SPECV_ERR_HIP, which
 * reports a launch failure) and specv_last_error() describes the problem.
 * No C++ exception crosses this interface.
 *
 * Sources, by page title and section:
 *  [L5]  Lecture 5: Speculative Decoding and SpecInfer -- sec. 2.1 (tempered
 *        softmax), 2.2 (accept iff u <= p(x)/q(x); resample from
 *        norm(max(0, p - q))), 2.7 (greedy), 3.1 (one iteration: first
 *        rejection, residual or a free token from p_{gamma+1}), 6.4
 *        (VerifyGreedy and multi-step speculative sampling on token trees).
 *  [DLN] Speculative Decoding (dl-note) -- sec. 2.2-2.3, Appendix
 *        "Implementation Details" (vLLM: zero draft probability rejects).
 *  [SSD] Speculative Speculative Decoding -- sec. 2.1 (outcome (k, t*)),
 *        sec. 4.1.1 (top-F bonus candidates excluding the drafted token; the
 *        speculation cache and its fan-out), sec. 4.1.2 and Appendix A.2
 *        (geometric fan-out), sec. 4.2.1 (Saguaro sampling).
 *  [L5 sec. 2.8] the lenient rule.
 *
 * Random numbers: uniforms come from Philox4x32-10 (Salmon et al., SC'11) with
 * key = (seed mod 2^32, seed >> 32), counter = (offset mod 2^32, offset >> 32,
 * sequence b, (tag << 24) | (j >> 2)), word = output[j & 3], mapped to
 * ((word >> 8) + 1) * 2^-24 in (0, 1]. Chain verification uses tag 0 with
 * j = i for the accept test at position i and j = gamma for the bonus; tree
 * verification uses tag 1 with j = child node id for its test and j = N for
 * the bonus. A call is fully determined by its inputs, seed and offset.
 */
#ifndef SPECV_H
#define SPECV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPECV_OK = 0,
    SPECV_ERR_INVALID_ARG = 1, /* bad size, null pointer, misaligned pointer */
    SPECV_ERR_WORKSPACE = 2,   /* workspace missing, too small or misaligned */
    SPECV_ERR_UNSUPPORTED = 3, /* dtype or combination not built */
    SPECV_ERR_HIP = 4          /* a HIP launch failed */
} specv_status;

typedef enum {
    SPECV_F32 = 0,  /* IEEE binary32 logits */
    SPECV_BF16 = 1  /* bfloat16 logits (upper 16 bits of binary32) */
} specv_dtype;

/* A strided 3-D view of logits [batch][row][vocab] in device memory.
 * `data` points at element [0][0][0] and must be aligned to the element size.
 * Strides are in elements (not bytes), may be 0 (broadcast) and must be >= 0;
 * the vocabulary dimension is contiguous. Rows whose start is 16-byte aligned
 * are read with 16-byte vector loads, others element by element. Logits may
 * be -inf but never NaN (results are unspecified for NaN logits). A caller
 * that holds probabilities rather than logits passes their natural logarithms
 * (log 0 = -inf) with temperature 1: softmax(log p) = p. */
typedef struct {
    const void* data;
    int32_t dtype;        /* specv_dtype */
    int64_t stride_seq;   /* elements between [b][.][.] and [b+1][.][.] */
    int64_t stride_row;   /* elements between [.][r][.] and [.][r+1][.] */
} specv_logits;

/* Limits checked by the validators. */
#define SPECV_MAX_GAMMA 64
#define SPECV_MAX_VOCAB 1048576
#define SPECV_MAX_TOPF 31
#define SPECV_MAX_TREE_NODES 4096

/* Bytes of workspace specv_verify needs for (batch, gamma, vocab). */
specv_status specv_verify_workspace_size(int32_t batch, int32_t gamma,
                                         int32_t vocab, size_t* bytes);

/*
 * Chain verification [L5 sec. 2.2, 3.1; DLN sec. 2.2-2.3; SSD sec. 2.1].
 *
 * For each sequence b with temperature T = temperature[b]:
 *  T > 0: p_t = softmax(target[b][i]/T), p_d = softmax(draft[b][i]/T).
 *         Position i < gamma accepts draft_tokens[b][i] = x iff p_d(x) > 0 and
 *         u_i <= p_t(x)/p_d(x). k = the first rejected position (gamma if none).
 *         If k < gamma the bonus is drawn from w = max(p_t - p_d, 0) of row k;
 *         otherwise from w = p_t of row gamma. Drawing: the smallest index j
 *         with w_0 + ... + w_j >= v * (w_0 + ... + w_{V-1}). If the residual
 *         has zero total mass (rounding only) the bonus is drawn from p_t of
 *         row k and out_bonus_mass reports 0.
 *  T == 0 (greedy, [L5 sec. 2.7]): x is accepted iff it equals the target
 *         argmax of row i (lowest index on ties); the bonus is the target
 *         argmax of row k. Draft logits are not read.
 *  A draft token outside [0, vocab) is rejected (it has probability 0).
 *
 * target: [batch][gamma+1][vocab]; draft: [batch][>= gamma][vocab] (row i is
 * read for i < gamma, only when T > 0); both with the same dtype.
 * draft_tokens: device int32 [batch][gamma], contiguous.
 * temperature:  device float [batch]; must be >= 0 and finite. Every row read
 *               must contain at least one finite logit.
 * Outputs (device, contiguous):
 *  out_tokens       int32 [batch][gamma+1]: x_0..x_{k-1}, the bonus, then -1.
 *  out_num_accepted int32 [batch]: k.
 *  out_probs        float [batch][gamma][2] or NULL: (p_t(x_i), p_d(x_i)) for
 *                   every i < gamma; for greedy sequences (1 or 0, 1).
 *  out_bonus_mass   float [batch] or NULL: total mass of the weights the bonus
 *                   was drawn from (1 - alpha of row k after a rejection, ~1
 *                   when every token was accepted, 1 for greedy, 0 on the
 *                   zero-residual fallback).
 * workspace: device memory of at least specv_verify_workspace_size() bytes,
 *            256-byte aligned. It must be zero-filled before its first use;
 *            every call leaves it zero-filled again (but for word 1 of its
 *            256-byte header, below), so one workspace can be reused by calls
 *            that are ordered on one stream. Calls that may run concurrently
 *            need separate workspaces. Workgroups of one call exchange
 *            statistics through it, every word tagged with the call's own
 *            epoch (so a word another call left never counts). Enqueues two
 *            kernels: the verification, and a finisher. A bonus workgroup
 *            waits for the row workgroups of its sequence, which the map of
 *            workgroups puts before it, for at most about 1.3 ms; if that
 *            runs out it marks the sequence deferred and the finisher, which
 *            starts once every workgroup of the first kernel has finished,
 *            completes it with the same arithmetic (the outcome is the same).
 *            So the call drains whatever the order in which the GPU starts
 *            workgroups and whatever else runs on it. Header word 1 (uint64)
 *            counts the sequences completed by finishers: a statistic, never
 *            read by the library, that only grows (0 in normal operation).
 */
specv_status specv_verify(specv_logits target, specv_logits draft,
                          const int32_t* draft_tokens, const float* temperature,
                          int32_t batch, int32_t gamma, int32_t vocab,
                          uint64_t seed, uint64_t offset,
                          int32_t* out_tokens, int32_t* out_num_accepted,
                          float* out_probs, float* out_bonus_mass,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * SSD/Saguaro bonus-token candidates [SSD sec. 4.1.1; Appendix A.3, Thm 19].
 *
 * For every sequence b and lookahead position k in [0, gamma]: the F token ids
 * with the largest draft logits of row draft[b][k], ordered by logit
 * (descending) then id (ascending), -0 equal to +0, after removing
 * draft_tokens[b][k] when k < gamma (the token sent for verification cannot
 * be the bonus). Position gamma excludes nothing. Temperature plays no part.
 *
 * draft: [batch][gamma+1][vocab]. draft_tokens: device int32 [batch][gamma] or
 * NULL (no exclusion anywhere). 1 <= F <= min(SPECV_MAX_TOPF, vocab - 1).
 * Outputs (device, contiguous): out_topk int32 [batch][gamma+1][F];
 * out_topk_logits float [batch][gamma+1][F] or NULL (the candidates' logits).
 * No workspace.
 */
specv_status specv_bonus_topk(specv_logits draft, const int32_t* draft_tokens,
                              int32_t batch, int32_t gamma, int32_t vocab,
                              int32_t F, int32_t* out_topk,
                              float* out_topk_logits, void* stream);

/* Bytes of workspace specv_verify_topk needs for (batch, gamma, vocab). */
specv_status specv_verify_topk_workspace_size(int32_t batch, int32_t gamma,
                                              int32_t vocab, size_t* bytes);

/*
 * specv_verify and specv_bonus_topk(draft, draft_tokens, ...) in one call,
 * with the same outputs as the two calls. One kernel streams every draft row
 * once for both the softmax statistics and the top-F candidates (in small
 * batches each row in chunks, whose top-F keys are merged through the
 * workspace). draft must have gamma + 1 rows per sequence. Arguments and outputs
 * as for specv_verify and specv_bonus_topk (draft_tokens is required here and
 * serves both); workspace as for specv_verify, sized by
 * specv_verify_topk_workspace_size.
 */
specv_status specv_verify_topk(specv_logits target, specv_logits draft,
                               const int32_t* draft_tokens, const float* temperature,
                               int32_t batch, int32_t gamma, int32_t vocab, int32_t F,
                               uint64_t seed, uint64_t offset,
                               int32_t* out_tokens, int32_t* out_num_accepted,
                               float* out_probs, float* out_bonus_mass,
                               int32_t* out_topk, float* out_topk_logits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * specv_verify_topk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument; the workspace is a static array of
 * 4 MiB in the library, one per GPU, held until the process ends. Shapes whose
 * specv_verify_topk_workspace_size exceeds 4 MiB are refused with
 * SPECV_ERR_WORKSPACE (B = 256, gamma = 8, vocab = 128256 needs about 2.1
 * MiB). Allocates nothing: the first call on a device looks up the array's
 * address and enqueues a clear of it on `stream`; every call leaves it
 * zero-filled (but for the statistic word of specv_verify's workspace
 * header). All calls on one GPU share the array: calls that overlap in time
 * on one GPU (different streams, or threads) race and must not be made.
 * Everything else as for specv_verify_topk, outputs identical.
 */
specv_status specv_verify_topk_noalloc(specv_logits target, specv_logits draft,
                                       const int32_t* draft_tokens, const float* temperature,
                                       int32_t batch, int32_t gamma, int32_t vocab, int32_t F,
                                       uint64_t seed, uint64_t offset,
                                       int32_t* out_tokens, int32_t* out_num_accepted,
                                       float* out_probs, float* out_bonus_mass,
                                       int32_t* out_topk, float* out_topk_logits, void* stream);

/* Bytes of workspace specv_verify_cache needs for (batch, gamma, vocab). */
specv_status specv_verify_cache_workspace_size(int32_t batch, int32_t gamma,
                                               int32_t vocab, size_t* bytes);

/*
 * Chain verification for SSD's speculation cache [SSD sec. 4.1.1, 4.2.1;
 * L5 sec. 2.8]: specv_verify_topk generalised in three ways.
 *
 *  fanout: HOST int32 [gamma+1]. Position k has F_k = fanout[k] cache
 *          candidates (0 <= F_k <= min(SPECV_MAX_TOPF, vocab - 1), at least
 *          one F_k >= 1): the F_k largest draft logits of row k, without
 *          draft_tokens[b][k] (k < gamma). out_topk / out_topk_logits are
 *          [batch][gamma+1][Fmax], Fmax = max F_k; row k holds F_k entries, then
 *          -1 (-inf). See specv_geometric_fanout for a budgeted choice.
 *  saguaro_C: in [0, 1]. The draft tokens of T > 0 sequences were sampled from
 *          Saguaro sampling sigma_{F_k,C}(draft[b][k] / T): weight
 *          C * exp(z_t / T) on the F_k largest logits of the row (ties: lower
 *          index first), exp(z_t / T) elsewhere. That distribution is the q of
 *          the accept test and of the residual. 1 = plain softmax. (If the
 *          total weight is 0, the plain softmax is used.)
 *  lenience: l in (0, 1]. Accept iff q(x) > 0 and u <= p_t(x) / (l q(x));
 *          1 = the exact rule. The residual stays max(p_t - q, 0).
 *  out_hit: device int32 [batch] or NULL: 1 iff the outcome (k, bonus) is in
 *          the cache, i.e. the bonus is one of the F_k candidates at k.
 *
 * Greedy sequences (T == 0) verify as in specv_verify; C and l do not apply.
 * Other arguments, outputs and the workspace as for specv_verify_topk. One
 * kernel streams every target and draft row once at every batch size.
 */
specv_status specv_verify_cache(specv_logits target, specv_logits draft,
                                const int32_t* draft_tokens, const float* temperature,
                                int32_t batch, int32_t gamma, int32_t vocab,
                                const int32_t* fanout, float saguaro_C, float lenience,
                                uint64_t seed, uint64_t offset,
                                int32_t* out_tokens, int32_t* out_num_accepted,
                                float* out_probs, float* out_bonus_mass,
                                int32_t* out_topk, float* out_topk_logits,
                                int32_t* out_hit, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Saguaro's geometric fan-out [SSD sec. 4.1.2, Appendix A.2, Theorem 12]
 * (host only, no GPU): for acceptance rate a in (0, 1) and a power-law hit
 * rate 1 - F^-r (r > 0), the fan-outs F_k = F_0 a^(k/(1+r)) for k < K and
 * F_K = F_0 a^(K/(1+r)) (1-a)^(-1/(1+r)), with F_0 such that they sum to
 * `budget`, rounded to integers by largest remainder (floors first, then +1
 * to the largest fractional parts, lower k first on equal parts) so that the
 * K + 1 entries of out (HOST int32) sum to budget. 0 <= K <= SPECV_MAX_GAMMA.
 */
specv_status specv_geometric_fanout(int32_t K, double accept_rate, double r,
                                    int32_t budget, int32_t* out);

/* Bytes of workspace specv_verify_ragged needs for (batch, max_gamma, vocab)
 * with (has_draft != 0) or without draft logits. */
specv_status specv_verify_ragged_workspace_size(int32_t batch, int32_t max_gamma,
                                                int32_t vocab, int32_t has_draft,
                                                size_t* bytes);

/*
 * Chain verification of a ragged batch [L5 sec. 2.2, 3.1; DLN sec. 2.2-2.3,
 * Appendix "Implementation Details"]: sequence b drafts gamma_b tokens,
 * draft_tokens[draft_offsets[b] .. draft_offsets[b+1]) (0 <= gamma_b <=
 * max_gamma), and the rule is that of specv_verify with gamma = gamma_b (the
 * bonus uniform uses j = gamma_b, so a batch with every gamma_b = gamma gives
 * specv_verify's results).
 *
 * Rows are packed, addressed by stride_row (stride_seq is ignored):
 *  target: num_draft + batch rows; sequence b's target rows 0..gamma_b are
 *          rows draft_offsets[b] + b + i.
 *  draft:  num_draft rows; sequence b's row i is row draft_offsets[b] + i.
 *          draft.data == NULL: the drafts have no probabilities (an n-gram or
 *          prompt-lookup proposer): q is the point mass at the drafted token,
 *          so x is accepted iff u <= p_t(x), and the bonus after a rejection
 *          is drawn from p_t with x removed.
 * draft_offsets: device int32 [batch + 1], nondecreasing, draft_offsets[0]
 *          = 0, draft_offsets[batch] = num_draft. A sequence whose offsets
 *          break this (or exceed max_gamma tokens) reads nothing and reports
 *          out_num_accepted = -2.
 * draft_tokens: device int32 [num_draft] (may be NULL when num_draft == 0).
 * Outputs: out_tokens int32 [batch][max_gamma+1] (accepted tokens, the bonus,
 *          then -1), out_num_accepted [batch], out_probs float [num_draft][2]
 *          or NULL ((p_t(x), 1) without draft probabilities), out_bonus_mass
 *          [batch] or NULL. Workspace as for specv_verify, sized by
 *          specv_verify_ragged_workspace_size.
 */
specv_status specv_verify_ragged(specv_logits target, specv_logits draft,
                                 const int32_t* draft_offsets, const int32_t* draft_tokens,
                                 const float* temperature, int32_t batch, int32_t max_gamma,
                                 int32_t num_draft, int32_t vocab, uint64_t seed,
                                 uint64_t offset, int32_t* out_tokens,
                                 int32_t* out_num_accepted, float* out_probs,
                                 float* out_bonus_mass, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Bytes of workspace specv_tree_verify needs for (batch, nodes, vocab). */
specv_status specv_tree_verify_workspace_size(int32_t batch, int32_t nodes,
                                              int32_t vocab, size_t* bytes);

/*
 * Token-tree verification: VerifyGreedy (T == 0) and multi-step speculative
 * sampling (T > 0) [L5 sec. 6.2, 6.4].
 *
 * A tree has `nodes` = N nodes in topological order: parent[b][0] = -1 and
 * 0 <= parent[b][n] < n for n >= 1 (an entry breaking this is treated as
 * "no parent": the node is never visited). tokens[b][n] is node n's token.
 * target[b][n] holds the target logits after the path to node n; draft[b][n]
 * holds the draft logits at node n, the distribution q its children were
 * drawn from (children must be independent draws for MSS to be exact).
 * Walk from the root: at node n with children c_1 < c_2 < ... (by id),
 *  T > 0: r = p_n; child c with token t is accepted iff q(t) > 0 and
 *         u_c <= r(t)/q(t); on acceptance the walk moves to c; on rejection
 *         r <- norm(max(0, r - q)) (kept if that mass is 0). If every child is
 *         rejected the bonus is drawn from r; at a leaf, from p of the leaf.
 *  T == 0: move to the lowest-id child whose token is the target argmax of n;
 *         if none, the bonus is that argmax.
 *
 * parent, tokens: device int32 [batch][N], contiguous. temperature: device
 * float [batch]. target, draft: [batch][N][vocab] (draft rows are read only
 * for nodes that have children, only when T > 0).
 * Outputs (device, contiguous): out_path int32 [batch][N]: accepted node ids
 * in walk order, then -1; out_num_accepted int32 [batch]; out_bonus int32
 * [batch]. Workspace as for specv_verify (zero-filled before first use, left
 * zero-filled by every call).
 * Enqueues one kernel for trees of up to 256 nodes (the row statistics, and
 * each tree's walk, which follows its tree's rows node by node) and two
 * beyond (the row statistics, then the walks). A walk's passes over a node's
 * rows are shared by up to 16 workgroups per tree that wait for each other
 * and for the tree's rows. Each workgroup takes its task number from a
 * ticket counter in the workspace header (word 0, zero at rest) when it
 * starts, so tasks are numbered in the order workgroups actually start; a
 * task waits only for tasks with smaller numbers or for the other walkers of
 * its tree, whose numbers are consecutive, so every wait is on a task a
 * running workgroup holds or the next one to start will take. A wait that
 * still times out (about 1.3 s; not expected) makes that tree report -1.
 */
specv_status specv_tree_verify(specv_logits target, specv_logits draft,
                               const int32_t* parent, const int32_t* tokens,
                               const float* temperature, int32_t batch,
                               int32_t nodes, int32_t vocab, uint64_t seed,
                               uint64_t offset, int32_t* out_path,
                               int32_t* out_num_accepted, int32_t* out_bonus,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* The uniforms the kernels draw: out[b][j] = U(seed, offset, b, tag, j) for
 * b < batch, j < count (device float [batch][count]). For tests and replay. */
specv_status specv_uniforms(uint64_t seed, uint64_t offset, int32_t tag,
                            int32_t batch, int32_t count, float* out,
                            void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* specv_last_error(void);

/*
 * For tests of the bounded waits. The kernels' workgroups wait for each
 * other's published words (row statistics, tile sums, top-F keys, a tree's
 * pass totals); every wait is bounded in ticks of the GPU's 100 MHz constant
 * clock: a chain call's (specv_verify, specv_verify_topk, specv_verify_cache,
 * specv_verify_ragged) by min(bound, 2^17), after which the sequence is left
 * to the call's finisher (same outcome), a tree call's by the bound itself,
 * by default 2^27 (about 1.3 s), after which the tree reports -1. This sets
 * the bound for later calls from any thread (0 restores the default) and
 * returns the previous one. Every call leaves its workspace zero-filled
 * whether or not its waits ran out. Not for production use.
 */
uint64_t specv_debug_set_wait_bound(uint64_t ticks);

/* Library version string. */
const char* specv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECV_H */
