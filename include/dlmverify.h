/*
 * libdlmverify: the per-position verification pass of masked diffusion
 * language-model decoding, for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [DualDiffusion] "DualDiffusion: A Speculative Decoding Strategy for Masked
 *       Diffusion Models" (gist.science summary of arXiv 2604.05250).
 *   [SPOT] "On the SPOT: Enhancing Speculative Decoding for Diffusion Language
 *       Models via Commit-Order Prediction" (paper review, blog.secrett2633.cloud).
 *   [COVER] "Stop the Flip-Flop: Context-Preserving Verification for Fast
 *       Revocable Diffusion Decoding" (gist.science summary of arXiv 2602.06161).
 *
 * Conventions shared by every call:
 *   - Every array pointer is a caller-owned DEVICE pointer (hipMalloc'd or a
 *     torch tensor's data_ptr()). The library allocates nothing; scratch
 *     memory, where a call needs it, is passed in. The one exception is
 *     dv_verify_rows_noalloc, whose scratch is a fixed array in device memory
 *     (one per GPU, held until the process ends) that every call of it on
 *     that GPU shares; no other call keeps state between calls.
 *   - Calls validate their arguments on the host first. An invalid argument
 *     returns a status != DV_OK synchronously, before any HIP call, with no
 *     side effect. Valid calls enqueue kernels on `stream` and return without
 *     waiting: inputs must stay alive and outputs are valid only once the
 *     stream has reached that point. A launch failure returns DV_ERR_HIP.
 *   - dv_last_error() gives a message for the last failing call of the calling
 *     thread. Nothing throws across this interface and nothing aborts.
 *   - Rows are independent; indices are int32, so rows and vocab are < 2^31.
 *   - Calls on one stream run in order; calls on different streams that share
 *     output buffers race, as with any kernel.
 */
#ifndef DLMVERIFY_H
#define DLMVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DV_VERSION 1

typedef enum dv_status {
  DV_OK = 0,
  DV_ERR_NULL = 1,        /* a required pointer is NULL */
  DV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  DV_ERR_DTYPE = 3,       /* unknown element type */
  DV_ERR_ALIGN = 4,       /* a pointer or row pitch is not 16-byte aligned */
  DV_ERR_ARG = 5,         /* a scalar argument is out of range (T, tau, theta, k, rule, ...) */
  DV_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  DV_ERR_UNSUPPORTED = 7, /* a valid request the library cannot serve (e.g. seq_len too long) */
  DV_ERR_HIP = 8          /* a HIP launch or runtime call failed */
} dv_status;

typedef enum dv_dtype { DV_FP32 = 0, DV_BF16 = 1 } dv_dtype;

/* Decision codes written by dv_decide. */
typedef enum dv_decision { DV_NONE = 0, DV_KEEP = 1, DV_REPLACE = 2, DV_REMASK = 3 } dv_decision;

/* Verifier and drafter logits of `rows` positions over a vocabulary of `vocab`.
 * Layout: row-major [rows][ld] elements of `dtype` (fp32 values or bfloat16
 * bit patterns); element (r, i) sits at base + r*ld + i, and each buffer spans
 * rows*ld elements. Only the first `vocab` entries of a row are read as
 * logits; the padding up to the next 16-byte boundary is read and ignored.
 * Requirements: both base pointers 16-byte aligned, ld*elt a multiple of 16,
 * vocab <= ld, all logits finite with |x| <= 1e8 (larger magnitudes overflow
 * the running sums), or also -inf with DV_LOGITS_NEG_INF. */
#define DV_LOGITS_NEG_INF 1  /* logits may be -inf: vocabulary entries masked out of the
                                distribution (probability 0). Each row keeps a finite logit in
                                each model. Values at or below -2^100 count as -inf. A divergence
                                is reported +inf when it exceeds 2^64, which it does when one
                                model puts more than about 1e-11 of its mass where the other has
                                -inf. */
typedef struct dv_logits {
  const void *verifier;
  const void *drafter;
  int32_t dtype;   /* dv_dtype */
  int32_t flags;   /* 0 or DV_LOGITS_NEG_INF */
  int64_t rows;
  int64_t vocab;
  int64_t ld;
} dv_logits;

/* Shared Gumbel noise ([SPOT] §1 and §3, coupled-noise verification): at
 * temperature > 0 both models draw token argmax_i(x_i / T + g_i) with the SAME
 * standard Gumbel g_i, which depends only on (seed, position, vocabulary index)
 * and, for the indices of a partial last group, on the vocabulary size. The g_i are drawn from counter hash words (DV_HASH_V1: MurmurHash3's 32-bit
 * finalizer over (seed, position, index)), in groups of 8 consecutive indices
 * largest first (DV_NOISE_V2): a full group's maximum, Gumbel shifted by ln 8,
 * sits at a place given by the group's own hash word, and the other seven are
 * Gumbel truncated below it at their index words' uniforms; the indices of a
 * partial last group draw on their own. In law these are i.i.d. standard
 * Gumbel values, so the tokens are exact samples of softmax(x / T).
 * temperature == 0 means greedy decoding (token = argmax, no noise).
 * Position of row r: pos[r] when pos != NULL (device int32 [rows]); else
 * r % pos_period when pos_period > 0; else r. Rows with equal positions see
 * equal noise (e.g. the candidates of one tree level). */
typedef struct dv_noise {
  float temperature;
  int32_t reserved;
  uint64_t seed;
  const int32_t *pos;
  int64_t pos_period;
} dv_noise;

/* Per-row statistics, structure of arrays of length rows (device). Any member
 * may be NULL to skip that output. Definitions ([DualDiffusion] §2,
 * "Verification algorithms" items 2-3; [COVER] §2, uncertainty u):
 *   lse_v, lse_d   log sum_i exp(x_i) of the verifier / drafter logits
 *   kl             KL(p_verifier || p_drafter), nats
 *   entropy        -sum_i p_v,i ln p_v,i, nats
 *   conf           max_i p_v,i
 *   argmax_v/_d    lowest index of the row maximum
 *   tok_v/_d       Gumbel-max token under the shared noise (argmax at T = 0)
 *   kl_rev         KL(p_drafter || p_verifier), nats (asking for it, like
 *                  DV_LOGITS_NEG_INF, selects the extended pass: one more
 *                  multiply-add per logit pair)
 *   p_tok_d        p_v of the drafter's token tok_d: the verifier's confidence
 *                  for the drafted token ([DualDiffusion] §2 item 3, the other
 *                  reading of "confidence for the token") */
typedef struct dv_row_stats {
  float *lse_v;
  float *lse_d;
  float *kl;
  float *entropy;
  float *conf;
  int32_t *argmax_v;
  int32_t *argmax_d;
  int32_t *tok_v;
  int32_t *tok_d;
  float *kl_rev;
  float *p_tok_d;
} dv_row_stats;

/* Optional launch-shape override for dv_verify_rows (NULL = automatic). A
 * zero field keeps its automatic value. Results do not depend on it beyond
 * float rounding: integer outputs are identical for every shape.
 *   split         vocabulary slices per row (1..16), each one wavefront; the
 *                 slices of a row run in one workgroup
 *   shared_noise  1: rows share positions (needs temperature > 0, pos == NULL
 *                 and pos_period > 0): a table of the largest noise value of
 *                 each (position, 16-byte chunk), built in the workspace,
 *                 bounds the Gumbel scores of each chunk;
 *                 0: the bound comes from each chunk's own hash words;
 *                 -1: automatic (the table when rows >= 2 * pos_period)
 *   reserved      must be zero */
typedef struct dv_tuning {
  int32_t split;
  int32_t shared_noise;
  int32_t reserved[2];
} dv_tuning;

/* Bytes of device workspace dv_verify_rows needs for these arguments (may be
 * 0). Validates like dv_verify_rows does, but does not look at pointers. */
dv_status dv_verify_workspace_bytes(const dv_logits *logits, const dv_noise *noise,
                                    const dv_tuning *tuning, size_t *bytes);

/* One fused pass over both logit matrices ([DualDiffusion] §2 "Core process":
 * the verifier's distributions are compared with the drafter's predictions;
 * [SPOT] §3: all candidate states are verified in one batched pass). Writes
 * the non-NULL members of `out`. `workspace` (device, 256-byte aligned) must
 * hold dv_verify_workspace_bytes() bytes; it may be NULL when that is 0.
 * Errors: DV_ERR_NULL (logits, noise or out NULL; verifier/drafter NULL),
 * DV_ERR_SHAPE (rows < 0, vocab < 1, vocab > ld, sizes >= 2^31, pos_period < 0),
 * DV_ERR_DTYPE, DV_ERR_ALIGN, DV_ERR_ARG (temperature < 0 or not finite, bad
 * tuning), DV_ERR_WORKSPACE, DV_ERR_HIP. rows == 0 is a no-op. */
dv_status dv_verify_rows(const dv_logits *logits, const dv_noise *noise, const dv_tuning *tuning,
                         const dv_row_stats *out, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same as
 * dv_verify_rows (same kernels, launch shape and results, bit for bit) but
 * with no workspace argument: the noise table dv_verify_rows builds in its
 * workspace when rows share positions goes into a fixed scratch array of
 * DV_NOALLOC_SCRATCH_BYTES that the library holds on each device (resolved on
 * the first call on that device and kept until the process ends). The call
 * allocates nothing. Every call on one device shares that scratch and
 * overwrites it, so calls that overlap on one device (concurrent streams,
 * threads) race; calls ordered on one stream do not. Errors: those of
 * dv_verify_rows, except DV_ERR_WORKSPACE; DV_ERR_UNSUPPORTED when the table
 * would exceed DV_NOALLOC_SCRATCH_BYTES (pass tuning.shared_noise = 0, which
 * needs no table, or call dv_verify_rows with a workspace); DV_ERR_HIP when
 * the scratch address cannot be resolved. */
#define DV_NOALLOC_SCRATCH_BYTES (8u << 20)
dv_status dv_verify_rows_noalloc(const dv_logits *logits, const dv_noise *noise, const dv_tuning *tuning,
                                 const dv_row_stats *out, hipStream_t stream);

typedef enum dv_rule {
  DV_RULE_TRUST = 0,          /* [DualDiffusion] §2 verification item 1: accept all */
  DV_RULE_KL = 1,             /* item 2: REMASK iff kl > tau_kl */
  DV_RULE_CONF = 2,           /* item 3: REMASK iff conf < conf_thr */
  DV_RULE_KL_OR_CONF = 3,     /* REMASK iff either holds */
  DV_RULE_COVER = 4,          /* [COVER] §3: KEEP if tok_v == current; else REPLACE if
                                 conf >= conf_thr; else REMASK */
  DV_RULE_COUPLED_ACCEPT = 5, /* [SPOT] §1/§3: per candidate of group_len rows, KEEP the
                                 leading rows whose tok_v equals the current token,
                                 REPLACE the first disagreeing row with tok_v, REMASK
                                 the rows after it */
  DV_RULE_CONF_DRAFT = 6,     /* [DualDiffusion] §2 item 3 read as the verifier's confidence
                                 in the drafted token: REMASK iff p_tok_d < conf_thr */
  DV_RULE_KL_STOCHASTIC = 7   /* [DualDiffusion] §2 item 2 with its second, probabilistic
                                 remask condition, read as one Bernoulli draw per row remasking with
                                 probability min(1, kl / tau_kl): REMASK iff the float32
                                 product u * tau_kl < kl, where u = (2 (h >> 9) + 1) 2^-24
                                 and h is the noise hash word (DV_HASH_V1, as in dv_noise)
                                 of (seed, the row's position) at index 2^32 - 1, which no
                                 vocabulary entry uses. kl > tau_kl always remasks; kl = 0
                                 never does. Needs tau_kl > 0. */
} dv_rule;

typedef struct dv_decide_args {
  int32_t rule;        /* dv_rule */
  float tau_kl;        /* finite */
  float conf_thr;      /* finite */
  int32_t mask_token;  /* token id written for REMASK rows ([COVER] problem statement:
                          a remasked position holds [MASK]) */
  int64_t rows;
  int64_t group_len;   /* rows per candidate (consecutive rows, commit order); 0 = none.
                          Required (> 0, dividing rows) for COUPLED_ACCEPT and for
                          prefix_len / best_group. */
  /* KL_STOCHASTIC only: the draws are keyed like dv_noise (seed; position pos[r]
     when pos is non-NULL, device int32 [rows]; else r % pos_period when
     pos_period > 0; else r). */
  uint64_t seed;
  const int32_t *pos;
  int64_t pos_period;  /* >= 0 */
} dv_decide_args;

/* Per-position decision ([DualDiffusion] §2 verification items 1-3;
 * [COVER] §3 adaptive revision outcomes; [SPOT] §1/§3 coupled-noise check).
 * Reads from `stats` only the members the rule needs (kl; conf; tok_v;
 * p_tok_d), plus tok_d when cur_tok is NULL. subject: device uint8 [rows] or NULL (all
 * rows); rows with subject == 0 get DV_NONE and keep their current token.
 * cur_tok: device int32 [rows], the current token assignment, or NULL to use
 * tok_d. Outputs: decision uint8 [rows], out_tok int32 [rows] (current token
 * for KEEP/NONE, tok_v for REPLACE, mask_token for REMASK); prefix_len int32
 * [rows/group_len] (offset of the first decided row of each group that is not
 * KEEP, group_len if none) or NULL; best_group int32 [1] (group with the
 * longest prefix, lowest index on ties) or NULL; best_group requires
 * prefix_len. decision and out_tok may be NULL to skip them.
 * Errors: DV_ERR_NULL, DV_ERR_SHAPE (rows < 0, group_len < 0, group_len not
 * dividing rows, pos_period < 0), DV_ERR_ARG (unknown rule, non-finite
 * thresholds, tau_kl <= 0 for KL_STOCHASTIC). */
dv_status dv_decide(const dv_decide_args *args, const dv_row_stats *stats, const uint8_t *subject,
                    const int32_t *cur_tok, uint8_t *decision, int32_t *out_tok,
                    int32_t *prefix_len, int32_t *best_group, hipStream_t stream);

/* COVER stability-aware seed score ([COVER] §2, the Score equation):
 * score = u * (1 + d_in) / (1 + d_out) where eligible (or everywhere when
 * eligible is NULL), -inf elsewhere. All arrays device [rows]; u, d_in, d_out
 * float32 (u is normally the verifier entropy from dv_verify_rows).
 * Errors: DV_ERR_NULL, DV_ERR_SHAPE (rows < 0). */
dv_status dv_seed_score(int64_t rows, const float *u, const float *d_in, const float *d_out,
                        const uint8_t *eligible, float *score, hipStream_t stream);

/* Per-sequence selection ([COVER] §2: a small set of top-scoring positions
 * becomes the seeds; [SPOT] §3: threshold decoding with SPOT-Sets).
 * score: device float32 [nseq][seq_len]; eligible: uint8 [nseq][seq_len] or
 * NULL. Picks, per sequence, the k eligible positions with the largest
 * (largest != 0) or smallest scores, equal scores to the lower index, sorted;
 * with use_thr != 0 keeps of those only score > thr (largest) or score < thr
 * (smallest). Outputs: out_idx int32 [nseq][k] and out_val float32 [nseq][k]
 * (padded with -1 / NaN after the count), out_count int32 [nseq], out_mask
 * uint8 [nseq][seq_len] (1 at kept positions) — each may be NULL. Scores must
 * not be NaN. Errors: DV_ERR_NULL, DV_ERR_SHAPE (nseq < 0, seq_len < 1),
 * DV_ERR_ARG (k < 1 or k > seq_len, thr not finite), DV_ERR_UNSUPPORTED
 * (seq_len > 16384). */
dv_status dv_select_topk(int64_t nseq, int64_t seq_len, const float *score, const uint8_t *eligible,
                         int32_t k, int32_t largest, int32_t use_thr, float thr, int32_t *out_idx,
                         float *out_val, int32_t *out_count, uint8_t *out_mask, hipStream_t stream);

/* The seed score and the per-sequence selection of it in one call ([COVER] §2:
 * every position's seed score, then the top-scoring positions become the
 * seeds). Output for output the same as dv_seed_score(nseq * seq_len, u, d_in,
 * d_out, seed_eligible, score) followed by dv_select_topk(nseq, seq_len,
 * score, select_eligible, k, largest, use_thr, thr, ...): u, d_in, d_out are
 * device float32 [nseq][seq_len]; seed_eligible and select_eligible uint8
 * [nseq][seq_len] or NULL; score (required) receives the seed scores; the
 * selection outputs are dv_select_topk's. Up to 2048 positions per sequence
 * it is one launch (the selection computes the scores it ranks); longer
 * sequences take the two launches. Errors: DV_ERR_NULL (u, d_in, d_out or
 * score NULL), DV_ERR_SHAPE (nseq < 0, seq_len < 1), DV_ERR_ARG (k < 1 or
 * k > seq_len, thr not finite), DV_ERR_UNSUPPORTED (seq_len > 16384). */
dv_status dv_seed_select(int64_t nseq, int64_t seq_len, const float *u, const float *d_in, const float *d_out,
                         const uint8_t *seed_eligible, float *score, const uint8_t *select_eligible,
                         int32_t k, int32_t largest, int32_t use_thr, float thr, int32_t *out_idx,
                         float *out_val, int32_t *out_count, uint8_t *out_mask, hipStream_t stream);

/* dv_decide and dv_seed_select of one decoding step in one launch ([COVER] §2
 * and §3: the seeds are chosen by the Score equation while the positions are
 * decided; [SPOT] §3: the coupled check and the threshold selection of one
 * step). Arguments: dv_decide's (a .. best_group), then dv_seed_select's
 * (nseq .. out_mask), then the stream; each means what it means there, and the
 * outputs are those of dv_decide followed by dv_seed_select. The two calls run
 * together, so they may share no memory that either writes: a decision output
 * overlapping a seed-selection input or output, or a seed-selection output
 * overlapping a decision input, is DV_ERR_ARG (so a selection's out_mask cannot
 * be the subject of the decisions in the same call). One launch when the
 * selection takes at most 2048 positions per sequence (nseq >= 1) and the
 * decision is the one-workgroup path (group_len > 0, rows <= 16384, at most 1024
 * groups) or needs no best_group; otherwise the calls' own launches, in order.
 * Errors: those of dv_decide, then those of dv_seed_select, then DV_ERR_ARG
 * for shared memory; nothing is launched when any check fails. */
dv_status dv_decide_seed_select(const dv_decide_args *a, const dv_row_stats *stats, const uint8_t *subject,
                                const int32_t *cur_tok, uint8_t *decision, int32_t *out_tok, int32_t *prefix_len,
                                int32_t *best_group, int64_t nseq, int64_t seq_len, const float *u, const float *d_in,
                                const float *d_out, const uint8_t *seed_eligible, float *score,
                                const uint8_t *select_eligible, int32_t k, int32_t largest, int32_t use_thr, float thr,
                                int32_t *out_idx, float *out_val, int32_t *out_count, uint8_t *out_mask,
                                hipStream_t stream);

/* COVER's seed step in one launch ([COVER] §2: the top-scoring positions by
 * the Score equation become the seeds; §3: the seeds are re-verified, KEEP,
 * REPLACE or REMASK): dv_seed_select, then dv_decide over the same rows with
 * the selection as its subject. Arguments: dv_seed_select's (nseq .. out_mask;
 * out_mask is required here), then dv_decide's without subject, prefix_len and
 * best_group (a, stats, cur_tok, decision, out_tok), then the stream. The
 * outputs are those of dv_seed_select(...) followed by dv_decide(a, stats,
 * out_mask, cur_tok, decision, out_tok, NULL, NULL): rows not selected get
 * DV_NONE and keep their current token. a->rows must be nseq * seq_len, and
 * the rule one of single rows (not COUPLED_ACCEPT). No buffer that one part
 * writes may overlap one the other reads or writes. One launch up to 2048
 * positions per sequence (the selection's workgroups decide their own
 * positions); longer sequences take the selection's launches and then the
 * decisions'. Errors: those of dv_seed_select; DV_ERR_NULL (out_mask NULL);
 * those of dv_decide; DV_ERR_SHAPE (a->rows != nseq * seq_len); DV_ERR_ARG
 * (COUPLED_ACCEPT, or shared memory). Nothing is launched when a check fails. */
dv_status dv_seed_select_decide(int64_t nseq, int64_t seq_len, const float *u, const float *d_in, const float *d_out,
                                const uint8_t *seed_eligible, float *score, const uint8_t *select_eligible,
                                int32_t k, int32_t largest, int32_t use_thr, float thr, int32_t *out_idx,
                                float *out_val, int32_t *out_count, uint8_t *out_mask, const dv_decide_args *a,
                                const dv_row_stats *stats, const int32_t *cur_tok, uint8_t *decision,
                                int32_t *out_tok, hipStream_t stream);

/* Shape of dv_tree_accept's input: ntrees independent trees of `nodes` nodes
 * each over blocks of `block_len` positions. */
typedef struct dv_tree_args {
  int64_t ntrees;     /* >= 0 */
  int64_t nodes;      /* 1..1024 per tree; node 0 is the root */
  int64_t block_len;  /* 1..1024 positions per block state */
} dv_tree_args;

/* Acceptance over trees of candidate block states and the commit it yields
 * ([SPOT] §1 "Key Terms & Definitions" and §3 "Method & Key Results": the
 * drafter proposes a multi-level tree of block states, the target verifies
 * all of them in one batched pass, and under coupled noise a proposed child is
 * right exactly when it equals the target's own transition).
 * Inputs, all device, trees consecutive:
 *   parent      int32 [ntrees][nodes], 0 <= parent[i] < i for i >= 1 (the
 *               root's entry is ignored); node i >= 1 commits node_tok[i] at
 *               block position node_pos[i] on top of its parent's state
 *   node_pos, node_tok  int32 [ntrees][nodes]
 *   root_masked uint8 [ntrees][block_len], nonzero = masked in the root state
 *   conf, tok_v float32 / int32 [ntrees][nodes][block_len]: the verifier's
 *               confidence and shared-noise token of every position of every
 *               node's state (the dv_row_stats of those rows, row index
 *               (tree * nodes + node) * block_len + position); conf not NaN
 * The target's transition from a state commits its masked position (the
 * root's masked positions minus those committed on the path) of highest conf,
 * lowest position on ties, with that position's tok_v. A node is accepted
 * when its parent is and (node_pos, node_tok) equals the parent's transition;
 * the root is accepted. A node whose parent breaks the order, or whose path
 * is longer than block_len, is not accepted.
 * Outputs, each may be NULL: accepted uint8 [ntrees][nodes]; depth int32
 * [ntrees][nodes] (commits from the root, -1 if not accepted); best_node
 * int32 [ntrees] (deepest accepted node, lowest index on ties); commit_pos /
 * commit_tok int32 [ntrees][block_len] (the path's commits in order, then the
 * target's transition at the best node if it has one; padded with -1);
 * commit_len int32 [ntrees]; block_tokens int32 [ntrees][block_len] (in/out:
 * committed positions take their tokens); out_masked uint8
 * [ntrees][block_len] (root_masked with committed positions cleared; may be
 * the root_masked buffer itself).
 * Errors: DV_ERR_NULL (args or a required input NULL), DV_ERR_SHAPE (sizes out
 * of range). */
dv_status dv_tree_accept(const dv_tree_args *args, const int32_t *parent, const int32_t *node_pos,
                         const int32_t *node_tok, const uint8_t *root_masked, const float *conf,
                         const int32_t *tok_v, uint8_t *accepted, int32_t *depth, int32_t *best_node,
                         int32_t *commit_pos, int32_t *commit_tok, int32_t *commit_len,
                         int32_t *block_tokens, uint8_t *out_masked, hipStream_t stream);

/* Attention probabilities of nseq sequences: `heads` maps of [len][len] each,
 * row-major [nseq][heads][len][ld] of `dtype` (rows sum to one; row i holds the
 * attention of query i over the keys). Requirements as for dv_logits: 16-byte
 * aligned base, ld*elt a multiple of 16, len <= ld. */
typedef struct dv_attention {
  const void *probs;
  int32_t dtype;     /* dv_dtype */
  int32_t reserved;
  int64_t nseq;      /* 0..65535 */
  int64_t heads;     /* 1..65535: heads (of one or several layers) averaged with equal weight */
  int64_t len;       /* 1..4096 positions */
  int64_t ld;
} dv_attention;

/* Bytes of device workspace dv_influence_drift needs (never 0 for nseq > 0). */
dv_status dv_influence_drift_workspace_bytes(const dv_attention *att, size_t *bytes);

/* COVER's influence and drift sensitivity of every position ([COVER] "Method:
 * COVER" part 2, Stability-Aware Seed Selection: d_in measures how much the
 * positions that are still masked rely on a token as context, d_out how
 * strongly the token attends to the newly written positions):
 *   d_in[b][j]  = (1/heads) sum_h sum_{i: query_masked[b][i]} A[b][h][i][j]
 *   d_out[b][i] = (1/heads) sum_h sum_{k: new_cols[b][k]}     A[b][h][i][k]
 * query_masked, new_cols: device uint8 [nseq][len] (nonzero = set); d_in,
 * d_out: device float32 [nseq][len] (either may be NULL). The result does not
 * depend on scheduling (fixed summation order). `workspace` (device, 256-byte
 * aligned) holds dv_influence_drift_workspace_bytes() bytes.
 * Errors: DV_ERR_NULL, DV_ERR_SHAPE, DV_ERR_DTYPE, DV_ERR_ALIGN,
 * DV_ERR_WORKSPACE, DV_ERR_HIP. */
dv_status dv_influence_drift(const dv_attention *att, const uint8_t *query_masked, const uint8_t *new_cols,
                             float *d_in, float *d_out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Shape of dv_dual_view_attention's input. */
typedef struct dv_dual_view_args {
  int64_t nseq;      /* 0..65535 */
  int64_t heads;     /* query heads, 1..65535 */
  int64_t kv_heads;  /* key/value heads, dividing heads (grouped-query attention) */
  int64_t len;       /* positions, a multiple of 32, 32..65536 */
  int64_t head_dim;  /* 64 or 128 */
  float scale;       /* score scale, finite (usually 1/sqrt(head_dim)) */
  int32_t reserved;
} dv_dual_view_args;

/* COVER's dual-view attention ([COVER] "Method: COVER" part 1, Dual-View Feed
 * Forward through KV cache override): queries, keys and values come from the
 * input with the seed positions masked; every seed column is read from the KV
 * cache of the previous step (k_prev, v_prev), except by the seed's own query,
 * whose diagonal reads the current key and value (leave-one-out, no self
 * leakage); the softmax renormalizes over the corrected row:
 *   k_eff(i, j) = k_prev[j] if seed[j] and j != i, else k_cur[j] (likewise v)
 *   out_i = sum_j softmax_j(scale <q_i, k_eff(i, j)>) v_eff(i, j)
 * Bidirectional (no causal mask). Query head h reads key/value head
 * h / (heads / kv_heads).
 * q: device bf16 [nseq][heads][len][head_dim]; k_cur, v_cur, k_prev, v_prev:
 * device bf16 [nseq][kv_heads][len][head_dim]; seed: device uint8 [nseq][len]
 * (nonzero = seed); out: device float32 [nseq][heads][len][head_dim]. All
 * contiguous and 16-byte aligned. Products on the matrix cores in bf16 with
 * float32 accumulation; the probabilities are rounded to bf16 for the second
 * product (relative error of the output about 2^-9 of the values' scale).
 * Inputs must be finite, and values below 2^100 in magnitude (the float32
 * accumulator holds up to 2^24 weighted values). DV_ERR_SHAPE also when nseq * heads * ceil(len /
 * 128) exceeds 2^24 (one workgroup per 128 queries of a head).
 * Errors: DV_ERR_NULL, DV_ERR_SHAPE, DV_ERR_ALIGN, DV_ERR_ARG, DV_ERR_HIP. */
dv_status dv_dual_view_attention(const dv_dual_view_args *args, const void *q, const void *k_cur,
                                 const void *v_cur, const void *k_prev, const void *v_prev,
                                 const uint8_t *seed, float *out, hipStream_t stream);

/* The index hash words h[r][i] (uint32, device [rows][vocab], DV_HASH_V1)
 * for the positions described as in dv_noise. For testing the noise generator
 * bit for bit; the same as dv_debug_noise with DV_DEBUG_INDEX_WORDS.
 * Errors: DV_ERR_NULL, DV_ERR_SHAPE. */
dv_status dv_debug_hash(uint64_t seed, const int32_t *pos, int64_t pos_period, int64_t rows,
                        int64_t vocab, uint32_t *out, hipStream_t stream);

/* What dv_debug_noise writes, per row r (positions as in dv_noise). Every
 * mode is computed by the same device functions the verification kernels use.
 *   DV_DEBUG_INDEX_WORDS  uint32 [rows][vocab]: index word h of each index
 *   DV_DEBUG_GROUP_WORDS  uint32 [rows][vocab / 8]: group word w_c of each
 *                         full group of 8 indices (DV_NOISE_V2, see dv_noise)
 *   DV_DEBUG_NOISE_LOG2   float32 [rows][vocab]: the Gumbel value of each
 *                         index in log2 units, G = g log2(e) + log2(ln 2)
 *                         for the standard Gumbel g the definition gives
 *   DV_DEBUG_CHUNK_BOUND  float32 [rows][ceil(vocab / chunk_elems)]: the
 *                         upper bound of a 16-byte chunk's noise that the
 *                         streaming pass computes in registers (+inf for a
 *                         partly filled last chunk, which is never bounded)
 *   DV_DEBUG_TABLE_BOUND  float32 [rows][ceil(vocab / chunk_elems)]: the
 *                         noise table dv_verify_rows builds in its workspace
 *                         when rows share positions, over positions
 *                         0 .. rows-1 (needs pos == NULL, pos_period == 0)
 * chunk_elems: elements per 16-byte chunk, 8 (bf16 logits) or 4 (fp32). */
typedef enum dv_debug_noise_mode {
  DV_DEBUG_INDEX_WORDS = 0,
  DV_DEBUG_GROUP_WORDS = 1,
  DV_DEBUG_NOISE_LOG2 = 2,
  DV_DEBUG_CHUNK_BOUND = 3,
  DV_DEBUG_TABLE_BOUND = 4
} dv_debug_noise_mode;

/* Test-only dump of the shared noise and of the bounds the Gumbel pruning
 * takes from it (modes above), so that the noise can be checked word for word
 * and the bounds against every value they cover. out: device, the mode's
 * element type and shape. Errors: DV_ERR_NULL (out NULL with a non-empty
 * result), DV_ERR_SHAPE (sizes out of range), DV_ERR_ARG (unknown mode,
 * chunk_elems not 4 or 8, pos or pos_period given with DV_DEBUG_TABLE_BOUND),
 * DV_ERR_HIP. */
dv_status dv_debug_noise(uint64_t seed, const int32_t *pos, int64_t pos_period, int64_t rows,
                         int64_t vocab, int32_t mode, int32_t chunk_elems, void *out,
                         hipStream_t stream);

/* Measurement-only: a read-only streaming probe over both logit matrices in
 * dv_verify_rows's launch shape for these sizes (and tuning.split, if given):
 * the same 16-byte non-temporal loads and wave-per-(row, slice) layout, with
 * no arithmetic but an xor fold, so that its rate is the read ceiling of the
 * verify pass's access pattern on the device. Writes an xor of what each wave
 * read to sink (device uint32 [rows][16], entry [r][slice]; entries of slices
 * past the row's split are left as they are). Errors: as dv_verify_rows for
 * the logits; DV_ERR_ARG for tuning.shared_noise = 1; DV_ERR_NULL (sink NULL
 * with rows > 0). */
dv_status dv_debug_read_probe(const dv_logits *logits, const dv_tuning *tuning, uint32_t *sink,
                              hipStream_t stream);

const char *dv_status_str(dv_status status);
const char *dv_last_error(void);
int dv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLMVERIFY_H */
