// Host side of libdlmverify: argument validation, launch geometry, status
// codes and error text. Every check runs before any HIP call, so a rejected
// call has no side effect.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dv_internal.h"

namespace {

thread_local char g_err[512] = "";

dv_status fail(dv_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

dv_status ok() {
  g_err[0] = '\0';
  return DV_OK;
}

dv_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(DV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch shape of dv_verify_rows, decided from the sizes alone.
struct Geometry {
  int32_t split = 1;
  int32_t pruned = 0;       // chunk-max noise table (rows share positions)
  int32_t slice_chunks = 0;
  int32_t rows_per_block = 1;
  int64_t cmax_rows = 0;
  int64_t cmax_ld = 0;
  size_t cmax_bytes = 0;    // at the start of the workspace, 256-byte aligned size
  size_t workspace = 0;
};

constexpr size_t kMaxTableBytes = size_t(1) << 30;
constexpr int32_t kMaxSplit = 16;  // waves of one workgroup

dv_status check_logits(const dv_logits *x, bool need_ptrs) {
  if (!x) return fail(DV_ERR_NULL, "logits descriptor is NULL");
  if (x->dtype != DV_FP32 && x->dtype != DV_BF16) return fail(DV_ERR_DTYPE, "unknown dtype %d", x->dtype);
  if ((x->flags & ~DV_LOGITS_NEG_INF) != 0) return fail(DV_ERR_ARG, "unknown logits flags 0x%x", x->flags);
  if (x->rows < 0 || x->rows > kMaxIndex) return fail(DV_ERR_SHAPE, "rows %lld out of range", (long long)x->rows);
  if (x->vocab < 1 || x->vocab > kMaxIndex) return fail(DV_ERR_SHAPE, "vocab %lld out of range", (long long)x->vocab);
  if (x->ld < x->vocab) return fail(DV_ERR_SHAPE, "ld %lld < vocab %lld", (long long)x->ld, (long long)x->vocab);
  const int64_t elt = x->dtype == DV_BF16 ? 2 : 4;
  if (x->ld > (int64_t(1) << 40) / elt) return fail(DV_ERR_SHAPE, "ld %lld too large", (long long)x->ld);
  if ((x->ld * elt) % 16 != 0) return fail(DV_ERR_ALIGN, "row pitch ld*elt = %lld bytes is not a multiple of 16", (long long)(x->ld * elt));
  if (need_ptrs && x->rows > 0) {
    if (!x->verifier || !x->drafter) return fail(DV_ERR_NULL, "verifier or drafter pointer is NULL");
    if (!aligned16(x->verifier) || !aligned16(x->drafter)) return fail(DV_ERR_ALIGN, "logit pointers must be 16-byte aligned");
  }
  return DV_OK;
}

dv_status check_noise(const dv_noise *n) {
  if (!n) return fail(DV_ERR_NULL, "noise descriptor is NULL");
  if (!std::isfinite(n->temperature) || n->temperature < 0.0f)
    return fail(DV_ERR_ARG, "temperature must be finite and >= 0");
  if (n->temperature > 0.0f && !std::isfinite(1.44269504088896340736f / n->temperature))
    return fail(DV_ERR_ARG, "temperature too small");
  if (n->pos_period < 0 || n->pos_period > kMaxIndex) return fail(DV_ERR_SHAPE, "pos_period out of range");
  return DV_OK;
}

dv_status choose_geometry(const dv_logits *x, const dv_noise *n, const dv_tuning *t, Geometry &g) {
  const int64_t N = x->dtype == DV_BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int64_t nch = (x->vocab + N - 1) / N;
  const bool greedy = n->temperature == 0.0f;
  const bool can_share = !greedy && n->pos == nullptr && n->pos_period > 0;
  const int32_t want_shared = t ? t->shared_noise : -1;
  if (t) {
    if (t->split < 0 || t->split > kMaxSplit) return fail(DV_ERR_ARG, "tuning.split must be 0..%d", kMaxSplit);
    if (t->reserved[0] != 0 || t->reserved[1] != 0) return fail(DV_ERR_ARG, "tuning.reserved must be zero");
    if (want_shared < -1 || want_shared > 1) return fail(DV_ERR_ARG, "tuning.shared_noise must be -1, 0 or 1");
    if (want_shared == 1 && !can_share)
      return fail(DV_ERR_ARG, "shared noise needs temperature > 0, pos == NULL and pos_period > 0");
  }
  const int64_t npos = can_share ? (n->pos_period < x->rows ? n->pos_period : x->rows) : 0;
  const size_t cmax_bytes = can_share ? ((static_cast<size_t>(npos) * nch * 4 + 255) / 256) * 256 : 0;
  if (want_shared == 1) {
    if (cmax_bytes > kMaxTableBytes) return fail(DV_ERR_ARG, "noise table of %zu bytes is too large", cmax_bytes);
    g.pruned = 1;
  } else if (want_shared == -1) {
    // positions carrying several rows amortize the table
    g.pruned = can_share && x->rows >= 2 * n->pos_period && cmax_bytes <= kMaxTableBytes ? 1 : 0;
  }
  if (g.pruned) {
    g.cmax_rows = npos;
    g.cmax_ld = nch;
    g.cmax_bytes = cmax_bytes;
  }
  // aim for ~2048 waves (two per SIMD), each slice at least 256 chunks: fewer, longer slices
  // stream faster than 4096 waves at every measured size (512 and 2048 rows, 126k-152k vocabularies)
  int64_t split = x->rows > 0 ? (2048 + x->rows - 1) / x->rows : 1;
  const int64_t max_by_len = nch / 256 > 0 ? nch / 256 : 1;
  if (split > max_by_len) split = max_by_len;
  if (t && t->split > 0) split = t->split;
  if (split > kMaxSplit) split = kMaxSplit;
  if (split > nch) split = nch;
  if (split < 1) split = 1;
  // a slice is read through a buffer resource, whose byte range is 32 bits: at most 2^28 - 1 chunks
  const int64_t max_slice = (int64_t(1) << 28) - 1;
  if (split < (nch + max_slice - 1) / max_slice) split = (nch + max_slice - 1) / max_slice;
  g.split = static_cast<int32_t>(split);
  g.slice_chunks = static_cast<int32_t>((nch + split - 1) / split);
  // a workgroup holds whole rows: 4 waves when split divides 4, else one row
  g.rows_per_block = 4 % split == 0 ? static_cast<int32_t>(4 / split) : 1;
  g.workspace = g.cmax_bytes;
  return DV_OK;
}

bool finite(float v) { return std::isfinite(v); }

dv_status influence_geometry(const dv_attention *a, bool need_ptrs, dv::InfluenceLaunch &p, size_t &ws) {
  if (!a) return fail(DV_ERR_NULL, "attention descriptor is NULL");
  if (a->dtype != DV_FP32 && a->dtype != DV_BF16) return fail(DV_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->nseq < 0 || a->nseq > 65535) return fail(DV_ERR_SHAPE, "nseq must be 0..65535");
  if (a->heads < 1 || a->heads > 65535) return fail(DV_ERR_SHAPE, "heads must be 1..65535");
  if (a->len < 1 || a->len > dv::kMaxInfluenceLen) return fail(DV_ERR_SHAPE, "len must be 1..%d", dv::kMaxInfluenceLen);
  if (a->ld < a->len) return fail(DV_ERR_SHAPE, "ld %lld < len %lld", (long long)a->ld, (long long)a->len);
  const int64_t elt = a->dtype == DV_BF16 ? 2 : 4;
  if (a->ld > (int64_t(1) << 30)) return fail(DV_ERR_SHAPE, "ld too large");
  if ((a->ld * elt) % 16 != 0) return fail(DV_ERR_ALIGN, "row pitch ld*elt is not a multiple of 16 bytes");
  if (need_ptrs && a->nseq > 0) {
    if (!a->probs) return fail(DV_ERR_NULL, "probs is NULL");
    if (!aligned16(a->probs)) return fail(DV_ERR_ALIGN, "probs must be 16-byte aligned");
  }
  // about 512 workgroups: split each head's rows into tiles of a multiple of 8 rows
  const int64_t maps = a->nseq * a->heads;
  int64_t tiles = maps > 0 ? (512 + maps - 1) / maps : 1;
  const int64_t max_tiles = (a->len + 63) / 64;
  if (tiles > max_tiles) tiles = max_tiles;
  if (tiles < 1) tiles = 1;
  int64_t tile_rows = (a->len + tiles - 1) / tiles;
  tile_rows = (tile_rows + 7) / 8 * 8;
  tiles = (a->len + tile_rows - 1) / tile_rows;
  p.bf16 = a->dtype == DV_BF16;
  p.tiles = static_cast<int32_t>(tiles);
  p.tile_rows = static_cast<int32_t>(tile_rows);
  p.nseq = a->nseq;
  p.heads = a->heads;
  p.len = a->len;
  p.ld = a->ld;
  p.probs = a->probs;
  ws = static_cast<size_t>(maps) * tiles * ((a->len + 7) / 8) * 16 * sizeof(float);
  return DV_OK;
}

// The launch of a validated dv_verify_rows call, with its noise table (if any) at `table`.
dv_status launch_verify_rows(const dv_logits *logits, const dv_noise *noise, const Geometry &g, const dv_row_stats *out,
                             void *table, hipStream_t stream) {
  dv::VerifyLaunch p{};
  p.va = logits->verifier;
  p.vb = logits->drafter;
  p.rows = logits->rows;
  p.vocab = logits->vocab;
  p.ld = logits->ld;
  p.bf16 = logits->dtype == DV_BF16;
  p.greedy = noise->temperature == 0.0f;
  p.neg_inf = (logits->flags & DV_LOGITS_NEG_INF) != 0;
  p.cT = p.greedy ? 0.0f : 1.44269504088896340736f / noise->temperature;
  if (!p.greedy && !std::isfinite(p.cT)) return fail(DV_ERR_ARG, "temperature too small");
  p.seed_b = dv::seed_word(noise->seed);
  p.pos = noise->pos;
  p.pos_period = noise->pos_period;
  p.split = g.split;
  p.slice_chunks = g.slice_chunks;
  p.rows_per_block = g.rows_per_block;
  p.noise_cmax = g.pruned ? static_cast<float *>(table) : nullptr;
  p.cmax_rows = g.cmax_rows;
  p.cmax_ld = g.cmax_ld;
  p.out = *out;
  return hip_status(dv::launch_verify(p, stream), "dv_verify_rows launch");
}

}  // namespace

extern "C" {

dv_status dv_verify_workspace_bytes(const dv_logits *logits, const dv_noise *noise, const dv_tuning *tuning,
                                    size_t *bytes) {
  if (!bytes) return fail(DV_ERR_NULL, "bytes is NULL");
  dv_status s = check_logits(logits, false);
  if (s != DV_OK) return s;
  if ((s = check_noise(noise)) != DV_OK) return s;
  Geometry g;
  if ((s = choose_geometry(logits, noise, tuning, g)) != DV_OK) return s;
  *bytes = g.workspace;
  return ok();
}

dv_status dv_verify_rows(const dv_logits *logits, const dv_noise *noise, const dv_tuning *tuning,
                         const dv_row_stats *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  dv_status s = check_logits(logits, true);
  if (s != DV_OK) return s;
  if ((s = check_noise(noise)) != DV_OK) return s;
  if (!out) return fail(DV_ERR_NULL, "output descriptor is NULL");
  Geometry g;
  if ((s = choose_geometry(logits, noise, tuning, g)) != DV_OK) return s;
  if (g.workspace > 0) {
    if (!workspace) return fail(DV_ERR_WORKSPACE, "workspace of %zu bytes required", g.workspace);
    if (workspace_bytes < g.workspace)
      return fail(DV_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", g.workspace, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DV_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  if (logits->rows == 0) return ok();
  return launch_verify_rows(logits, noise, g, out, workspace, stream);
}

dv_status dv_verify_rows_noalloc(const dv_logits *logits, const dv_noise *noise, const dv_tuning *tuning,
                                 const dv_row_stats *out, hipStream_t stream) {
  dv_status s = check_logits(logits, true);
  if (s != DV_OK) return s;
  if ((s = check_noise(noise)) != DV_OK) return s;
  if (!out) return fail(DV_ERR_NULL, "output descriptor is NULL");
  Geometry g;
  if ((s = choose_geometry(logits, noise, tuning, g)) != DV_OK) return s;
  if (g.workspace > DV_NOALLOC_SCRATCH_BYTES)
    return fail(DV_ERR_UNSUPPORTED,
                "the noise table needs %zu bytes, more than the library's fixed scratch of %zu bytes: pass "
                "tuning.shared_noise = 0 (no table) or call dv_verify_rows with a workspace",
                g.workspace, static_cast<size_t>(DV_NOALLOC_SCRATCH_BYTES));
  if (logits->rows == 0) return ok();
  void *table = nullptr;
  if (g.workspace > 0) {
    const hipError_t e = dv::noalloc_scratch(stream, &table);
    if (e != hipSuccess) return hip_status(e, "dv_verify_rows_noalloc scratch address");
  }
  return launch_verify_rows(logits, noise, g, out, table, stream);
}

// dv_decide's checks and launch parameters; `launch` is false when the call has nothing to do.
static dv_status decide_launch_of(const dv_decide_args *a, const dv_row_stats *stats, const uint8_t *subject,
                                  const int32_t *cur_tok, uint8_t *decision, int32_t *out_tok, int32_t *prefix_len,
                                  int32_t *best_group, dv::DecideLaunch &p, bool &launch) {
  launch = false;
  p = dv::DecideLaunch{};
  if (!a || !stats) return fail(DV_ERR_NULL, "args or stats is NULL");
  if (a->rows < 0 || a->rows > kMaxIndex) return fail(DV_ERR_SHAPE, "rows out of range");
  if (a->group_len < 0 || a->group_len > kMaxIndex) return fail(DV_ERR_SHAPE, "group_len out of range");
  if (a->rule < DV_RULE_TRUST || a->rule > DV_RULE_KL_STOCHASTIC) return fail(DV_ERR_ARG, "unknown rule %d", a->rule);
  if (!finite(a->tau_kl) || !finite(a->conf_thr)) return fail(DV_ERR_ARG, "thresholds must be finite");
  if (a->rule == DV_RULE_KL_STOCHASTIC && !(a->tau_kl > 0.0f)) return fail(DV_ERR_ARG, "KL_STOCHASTIC needs tau_kl > 0");
  if (a->pos_period < 0) return fail(DV_ERR_SHAPE, "pos_period must be >= 0");
  const bool need_groups = a->rule == DV_RULE_COUPLED_ACCEPT || prefix_len || best_group;
  if (need_groups) {
    if (a->group_len <= 0) return fail(DV_ERR_SHAPE, "group_len must be > 0 for this request");
    if (a->rows % a->group_len != 0) return fail(DV_ERR_SHAPE, "group_len must divide rows");
  }
  if (best_group && !prefix_len) return fail(DV_ERR_NULL, "best_group needs prefix_len");
  if (a->rows > 0) {
    if (!cur_tok && !stats->tok_d) return fail(DV_ERR_NULL, "cur_tok and stats.tok_d are both NULL");
    switch (a->rule) {
      case DV_RULE_KL:
      case DV_RULE_KL_STOCHASTIC:
        if (!stats->kl) return fail(DV_ERR_NULL, "this KL rule needs stats.kl");
        break;
      case DV_RULE_CONF:
        if (!stats->conf) return fail(DV_ERR_NULL, "rule CONF needs stats.conf");
        break;
      case DV_RULE_KL_OR_CONF:
        if (!stats->kl || !stats->conf) return fail(DV_ERR_NULL, "rule KL_OR_CONF needs stats.kl and stats.conf");
        break;
      case DV_RULE_COVER:
        if (!stats->conf || !stats->tok_v) return fail(DV_ERR_NULL, "rule COVER needs stats.conf and stats.tok_v");
        break;
      case DV_RULE_COUPLED_ACCEPT:
        if (!stats->tok_v) return fail(DV_ERR_NULL, "rule COUPLED_ACCEPT needs stats.tok_v");
        break;
      case DV_RULE_CONF_DRAFT:
        if (!stats->p_tok_d) return fail(DV_ERR_NULL, "rule CONF_DRAFT needs stats.p_tok_d");
        break;
      default:
        break;
    }
  }
  if (a->rows == 0) {
    if (best_group) {
      // no groups: the answer is -1, written by the reduction kernel
      p.rows = 0;
      p.best_group = best_group;
      p.prefix_len = prefix_len;
      launch = true;
    }
    return ok();
  }
  p.rule = a->rule;
  p.tau_kl = a->tau_kl;
  p.conf_thr = a->conf_thr;
  p.mask_token = a->mask_token;
  p.rows = a->rows;
  p.group_len = a->group_len;
  p.kl = stats->kl;
  p.conf = stats->conf;
  p.p_tok = stats->p_tok_d;
  p.tok_v = stats->tok_v;
  p.tok_d = stats->tok_d;
  p.subject = subject;
  p.cur_tok = cur_tok;
  p.decision = decision;
  p.out_tok = out_tok;
  p.prefix_len = prefix_len;
  p.best_group = best_group;
  p.seed_b = dv::seed_word(a->seed);
  p.pos = a->pos;
  p.pos_period = a->pos_period;
  launch = true;
  return ok();
}

dv_status dv_decide(const dv_decide_args *a, const dv_row_stats *stats, const uint8_t *subject, const int32_t *cur_tok,
                    uint8_t *decision, int32_t *out_tok, int32_t *prefix_len, int32_t *best_group, hipStream_t stream) {
  dv::DecideLaunch p;
  bool launch;
  const dv_status s = decide_launch_of(a, stats, subject, cur_tok, decision, out_tok, prefix_len, best_group, p, launch);
  if (s != DV_OK || !launch) return s;
  return hip_status(dv::launch_decide(p, stream), "dv_decide launch");
}

dv_status dv_seed_score(int64_t rows, const float *u, const float *d_in, const float *d_out, const uint8_t *eligible,
                        float *score, hipStream_t stream) {
  if (rows < 0 || rows > kMaxIndex) return fail(DV_ERR_SHAPE, "rows out of range");
  if (rows > 0 && (!u || !d_in || !d_out || !score)) return fail(DV_ERR_NULL, "u, d_in, d_out and score are required");
  return hip_status(dv::launch_seed_score(rows, u, d_in, d_out, eligible, score, stream), "dv_seed_score launch");
}

dv_status dv_select_topk(int64_t nseq, int64_t seq_len, const float *score, const uint8_t *eligible, int32_t k,
                         int32_t largest, int32_t use_thr, float thr, int32_t *out_idx, float *out_val,
                         int32_t *out_count, uint8_t *out_mask, hipStream_t stream) {
  if (nseq < 0 || nseq > kMaxIndex) return fail(DV_ERR_SHAPE, "nseq out of range");
  if (seq_len < 1) return fail(DV_ERR_SHAPE, "seq_len must be >= 1");
  if (seq_len > dv::kMaxSelectLen)
    return fail(DV_ERR_UNSUPPORTED, "seq_len %lld exceeds %lld", (long long)seq_len, (long long)dv::kMaxSelectLen);
  if (k < 1 || k > seq_len) return fail(DV_ERR_ARG, "k must be in [1, seq_len]");
  if (use_thr && !finite(thr)) return fail(DV_ERR_ARG, "thr must be finite");
  if (nseq > 0 && !score) return fail(DV_ERR_NULL, "score is NULL");
  dv::SelectLaunch p{};
  p.nseq = nseq;
  p.seq_len = seq_len;
  p.score = score;
  p.eligible = eligible;
  p.k = k;
  p.largest = largest != 0;
  p.use_thr = use_thr != 0;
  p.thr = thr;
  p.out_idx = out_idx;
  p.out_val = out_val;
  p.out_count = out_count;
  p.out_mask = out_mask;
  return hip_status(dv::launch_select_topk(p, stream), "dv_select_topk launch");
}

// dv_seed_select's checks and launch parameters.
static dv_status seed_select_launch_of(int64_t nseq, int64_t seq_len, const float *u, const float *d_in,
                                       const float *d_out, const uint8_t *seed_eligible, float *score,
                                       const uint8_t *select_eligible, int32_t k, int32_t largest, int32_t use_thr,
                                       float thr, int32_t *out_idx, float *out_val, int32_t *out_count,
                                       uint8_t *out_mask, dv::SelectLaunch &p) {
  p = dv::SelectLaunch{};
  if (nseq < 0 || nseq > kMaxIndex) return fail(DV_ERR_SHAPE, "nseq out of range");
  if (seq_len < 1) return fail(DV_ERR_SHAPE, "seq_len must be >= 1");
  if (seq_len > dv::kMaxSelectLen)
    return fail(DV_ERR_UNSUPPORTED, "seq_len %lld exceeds %lld", (long long)seq_len, (long long)dv::kMaxSelectLen);
  if (nseq > kMaxIndex / seq_len) return fail(DV_ERR_SHAPE, "nseq * seq_len out of range");
  if (k < 1 || k > seq_len) return fail(DV_ERR_ARG, "k must be in [1, seq_len]");
  if (use_thr && !finite(thr)) return fail(DV_ERR_ARG, "thr must be finite");
  if (nseq > 0 && (!u || !d_in || !d_out || !score)) return fail(DV_ERR_NULL, "u, d_in, d_out and score are required");
  p.nseq = nseq;
  p.seq_len = seq_len;
  p.eligible = select_eligible;
  p.k = k;
  p.largest = largest != 0;
  p.use_thr = use_thr != 0;
  p.thr = thr;
  p.out_idx = out_idx;
  p.out_val = out_val;
  p.out_count = out_count;
  p.out_mask = out_mask;
  p.u = u;
  p.d_in = d_in;
  p.d_out = d_out;
  p.seed_eligible = seed_eligible;
  p.score_out = score;
  return ok();
}

dv_status dv_seed_select(int64_t nseq, int64_t seq_len, const float *u, const float *d_in, const float *d_out,
                         const uint8_t *seed_eligible, float *score, const uint8_t *select_eligible, int32_t k,
                         int32_t largest, int32_t use_thr, float thr, int32_t *out_idx, float *out_val,
                         int32_t *out_count, uint8_t *out_mask, hipStream_t stream) {
  dv::SelectLaunch p;
  const dv_status s = seed_select_launch_of(nseq, seq_len, u, d_in, d_out, seed_eligible, score, select_eligible, k,
                                            largest, use_thr, thr, out_idx, out_val, out_count, out_mask, p);
  if (s != DV_OK) return s;
  return hip_status(dv::launch_seed_select(p, stream), "dv_seed_select launch");
}

namespace {
// A device byte range [lo, lo + bytes); null or empty ranges overlap nothing.
struct Span {
  uintptr_t lo;
  size_t bytes;
};
Span span_of(const void *p, int64_t n, size_t elem) {
  return Span{reinterpret_cast<uintptr_t>(p), p && n > 0 ? static_cast<size_t>(n) * elem : 0u};
}
bool overlap(const Span &x, const Span &y) {
  return x.bytes && y.bytes && x.lo < y.lo + y.bytes && y.lo < x.lo + x.bytes;
}

// A decision and a seed selection that run in one launch: no buffer one of them writes may be
// one the other reads or writes (the decisions' inputs as the rule reads them).
dv_status check_no_shared_writes(const dv::DecideLaunch &pd, const dv::SelectLaunch &ps) {
  const int64_t R = pd.rows, n = ps.nseq * ps.seq_len, ng = pd.group_len > 0 ? R / pd.group_len : 0;
  const int32_t *tok_d_read = pd.cur_tok ? nullptr : pd.tok_d;
  const Span d_in_spans[] = {span_of(pd.kl, R, 4), span_of(pd.conf, R, 4), span_of(pd.p_tok, R, 4),
                             span_of(pd.tok_v, R, 4), span_of(tok_d_read, R, 4), span_of(pd.subject, R, 1),
                             span_of(pd.cur_tok, R, 4), span_of(pd.pos, R, 4)};
  const Span d_out_spans[] = {span_of(pd.decision, R, 1), span_of(pd.out_tok, R, 4), span_of(pd.prefix_len, ng, 4),
                              span_of(pd.best_group, 1, 4)};
  const Span s_in_spans[] = {span_of(ps.u, n, 4), span_of(ps.d_in, n, 4), span_of(ps.d_out, n, 4),
                             span_of(ps.seed_eligible, n, 1), span_of(ps.eligible, n, 1)};
  const Span s_out_spans[] = {span_of(ps.score_out, n, 4), span_of(ps.out_idx, ps.nseq * ps.k, 4),
                              span_of(ps.out_val, ps.nseq * ps.k, 4), span_of(ps.out_count, ps.nseq, 4),
                              span_of(ps.out_mask, n, 1)};
  for (const Span &x : d_out_spans) {
    for (const Span &y : s_in_spans)
      if (overlap(x, y)) return fail(DV_ERR_ARG, "a decision output overlaps a seed-selection input");
    for (const Span &y : s_out_spans)
      if (overlap(x, y)) return fail(DV_ERR_ARG, "a decision output overlaps a seed-selection output");
  }
  for (const Span &x : s_out_spans)
    for (const Span &y : d_in_spans)
      if (overlap(x, y)) return fail(DV_ERR_ARG, "a seed-selection output overlaps a decision input");
  return ok();
}
}  // namespace

dv_status dv_decide_seed_select(const dv_decide_args *a, const dv_row_stats *stats, const uint8_t *subject,
                                const int32_t *cur_tok, uint8_t *decision, int32_t *out_tok, int32_t *prefix_len,
                                int32_t *best_group, int64_t nseq, int64_t seq_len, const float *u, const float *d_in,
                                const float *d_out, const uint8_t *seed_eligible, float *score,
                                const uint8_t *select_eligible, int32_t k, int32_t largest, int32_t use_thr, float thr,
                                int32_t *out_idx, float *out_val, int32_t *out_count, uint8_t *out_mask,
                                hipStream_t stream) {
  dv::DecideLaunch pd;
  bool decide;
  dv_status s = decide_launch_of(a, stats, subject, cur_tok, decision, out_tok, prefix_len, best_group, pd, decide);
  if (s != DV_OK) return s;
  dv::SelectLaunch ps;
  s = seed_select_launch_of(nseq, seq_len, u, d_in, d_out, seed_eligible, score, select_eligible, k, largest, use_thr,
                            thr, out_idx, out_val, out_count, out_mask, ps);
  if (s != DV_OK) return s;
  s = check_no_shared_writes(pd, ps);
  if (s != DV_OK) return s;
  return hip_status(dv::launch_decide_seed_select(pd, decide, ps, stream), "dv_decide_seed_select launch");
}

dv_status dv_seed_select_decide(int64_t nseq, int64_t seq_len, const float *u, const float *d_in, const float *d_out,
                                const uint8_t *seed_eligible, float *score, const uint8_t *select_eligible, int32_t k,
                                int32_t largest, int32_t use_thr, float thr, int32_t *out_idx, float *out_val,
                                int32_t *out_count, uint8_t *out_mask, const dv_decide_args *a,
                                const dv_row_stats *stats, const int32_t *cur_tok, uint8_t *decision,
                                int32_t *out_tok, hipStream_t stream) {
  dv::SelectLaunch ps;
  dv_status s = seed_select_launch_of(nseq, seq_len, u, d_in, d_out, seed_eligible, score, select_eligible, k, largest,
                                      use_thr, thr, out_idx, out_val, out_count, out_mask, ps);
  if (s != DV_OK) return s;
  if (!out_mask) return fail(DV_ERR_NULL, "out_mask is required: the selection is the decisions' subject");
  dv::DecideLaunch pd;
  bool decide;
  s = decide_launch_of(a, stats, nullptr, cur_tok, decision, out_tok, nullptr, nullptr, pd, decide);
  if (s != DV_OK) return s;
  if (a->rows != nseq * seq_len) return fail(DV_ERR_SHAPE, "the decisions' rows must be nseq * seq_len");
  if (a->rule == DV_RULE_COUPLED_ACCEPT)
    return fail(DV_ERR_ARG, "the decisions over the selected seeds take a rule of single rows");
  s = check_no_shared_writes(pd, ps);
  if (s != DV_OK) return s;
  return hip_status(dv::launch_seed_select_decide(ps, pd, stream), "dv_seed_select_decide launch");
}

dv_status dv_influence_drift_workspace_bytes(const dv_attention *att, size_t *bytes) {
  if (!bytes) return fail(DV_ERR_NULL, "bytes is NULL");
  dv::InfluenceLaunch p{};
  size_t ws = 0;
  dv_status s = influence_geometry(att, false, p, ws);
  if (s != DV_OK) return s;
  *bytes = ws;
  return ok();
}

dv_status dv_influence_drift(const dv_attention *att, const uint8_t *query_masked, const uint8_t *new_cols,
                             float *d_in, float *d_out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  dv::InfluenceLaunch p{};
  size_t ws = 0;
  dv_status s = influence_geometry(att, true, p, ws);
  if (s != DV_OK) return s;
  if (att->nseq == 0) return ok();
  if (!query_masked || !new_cols) return fail(DV_ERR_NULL, "query_masked or new_cols is NULL");
  if (!workspace) return fail(DV_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
  if (workspace_bytes < ws) return fail(DV_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", ws, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DV_ERR_ALIGN, "workspace must be 256-byte aligned");
  p.query_masked = query_masked;
  p.new_cols = new_cols;
  p.d_in = d_in;
  p.d_out = d_out;
  p.part = static_cast<float *>(workspace);
  return hip_status(dv::launch_influence(p, stream), "dv_influence_drift launch");
}

dv_status dv_dual_view_attention(const dv_dual_view_args *a, const void *q, const void *k_cur, const void *v_cur,
                                 const void *k_prev, const void *v_prev, const uint8_t *seed, float *out,
                                 hipStream_t stream) {
  if (!a) return fail(DV_ERR_NULL, "args is NULL");
  if (a->nseq < 0 || a->nseq > 65535) return fail(DV_ERR_SHAPE, "nseq must be 0..65535");
  if (a->heads < 1 || a->heads > 65535) return fail(DV_ERR_SHAPE, "heads must be 1..65535");
  if (a->kv_heads < 1 || a->heads % a->kv_heads != 0) return fail(DV_ERR_SHAPE, "kv_heads must divide heads");
  if (a->len < 32 || a->len > 65536 || a->len % 32 != 0) return fail(DV_ERR_SHAPE, "len must be a multiple of 32 in 32..65536");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(DV_ERR_SHAPE, "head_dim must be 64 or 128");
  if (!std::isfinite(a->scale)) return fail(DV_ERR_ARG, "scale must be finite");
  if ((a->len + 127) / 128 * a->heads * a->nseq > (int64_t{1} << 24))
    return fail(DV_ERR_SHAPE, "nseq * heads * ceil(len / 128) must be at most 2^24");
  if (a->nseq == 0) return ok();
  const void *ptrs[] = {q, k_cur, v_cur, k_prev, v_prev, out};
  for (const void *ptr : ptrs) {
    if (!ptr) return fail(DV_ERR_NULL, "an input or the output is NULL");
    if (!aligned16(ptr)) return fail(DV_ERR_ALIGN, "tensors must be 16-byte aligned");
  }
  if (!seed) return fail(DV_ERR_NULL, "seed is NULL");
  dv::DualViewLaunch p{};
  p.q = static_cast<const uint16_t *>(q);
  p.k_cur = static_cast<const uint16_t *>(k_cur);
  p.v_cur = static_cast<const uint16_t *>(v_cur);
  p.k_prev = static_cast<const uint16_t *>(k_prev);
  p.v_prev = static_cast<const uint16_t *>(v_prev);
  p.seed = seed;
  p.out = out;
  p.scale = a->scale;
  p.head_dim = static_cast<int32_t>(a->head_dim);
  p.nseq = a->nseq;
  p.heads = a->heads;
  p.kv_heads = a->kv_heads;
  p.len = a->len;
  return hip_status(dv::launch_dual_view(p, stream), "dv_dual_view_attention launch");
}

dv_status dv_tree_accept(const dv_tree_args *a, const int32_t *parent, const int32_t *node_pos,
                         const int32_t *node_tok, const uint8_t *root_masked, const float *conf,
                         const int32_t *tok_v, uint8_t *accepted, int32_t *depth, int32_t *best_node,
                         int32_t *commit_pos, int32_t *commit_tok, int32_t *commit_len, int32_t *block_tokens,
                         uint8_t *out_masked, hipStream_t stream) {
  if (!a) return fail(DV_ERR_NULL, "args is NULL");
  if (a->ntrees < 0 || a->ntrees > kMaxIndex) return fail(DV_ERR_SHAPE, "ntrees out of range");
  if (a->nodes < 1 || a->nodes > dv::kMaxTreeNodes)
    return fail(DV_ERR_SHAPE, "nodes must be 1..%d", dv::kMaxTreeNodes);
  if (a->block_len < 1 || a->block_len > dv::kMaxTreeBlockLen)
    return fail(DV_ERR_SHAPE, "block_len must be 1..%d", dv::kMaxTreeBlockLen);
  if (a->ntrees > 0 && (!parent || !node_pos || !node_tok || !root_masked || !conf || !tok_v))
    return fail(DV_ERR_NULL, "an input array is NULL");
  dv::TreeLaunch p{};
  p.ntrees = a->ntrees;
  p.nodes = a->nodes;
  p.block_len = a->block_len;
  p.parent = parent;
  p.node_pos = node_pos;
  p.node_tok = node_tok;
  p.root_masked = root_masked;
  p.conf = conf;
  p.tok_v = tok_v;
  p.accepted = accepted;
  p.depth = depth;
  p.best_node = best_node;
  p.commit_pos = commit_pos;
  p.commit_tok = commit_tok;
  p.commit_len = commit_len;
  p.block_tokens = block_tokens;
  p.out_masked = out_masked;
  return hip_status(dv::launch_tree_accept(p, stream), "dv_tree_accept launch");
}

dv_status dv_debug_hash(uint64_t seed, const int32_t *pos, int64_t pos_period, int64_t rows, int64_t vocab,
                        uint32_t *out, hipStream_t stream) {
  if (rows < 0 || rows > kMaxIndex || vocab < 0 || vocab > kMaxIndex) return fail(DV_ERR_SHAPE, "size out of range");
  if (pos_period < 0 || pos_period > kMaxIndex) return fail(DV_ERR_SHAPE, "pos_period out of range");
  if (rows > 0 && vocab > 0 && !out) return fail(DV_ERR_NULL, "out is NULL");
  return hip_status(dv::launch_debug_noise(dv::seed_word(seed), pos, pos_period, rows, vocab, DV_DEBUG_INDEX_WORDS, 8,
                                           out, stream),
                    "dv_debug_hash launch");
}

dv_status dv_debug_noise(uint64_t seed, const int32_t *pos, int64_t pos_period, int64_t rows, int64_t vocab,
                         int32_t mode, int32_t chunk_elems, void *out, hipStream_t stream) {
  if (rows < 0 || rows > kMaxIndex || vocab < 0 || vocab > kMaxIndex) return fail(DV_ERR_SHAPE, "size out of range");
  if (pos_period < 0 || pos_period > kMaxIndex) return fail(DV_ERR_SHAPE, "pos_period out of range");
  if (mode < DV_DEBUG_INDEX_WORDS || mode > DV_DEBUG_TABLE_BOUND) return fail(DV_ERR_ARG, "unknown mode %d", mode);
  if (chunk_elems != 4 && chunk_elems != 8) return fail(DV_ERR_ARG, "chunk_elems must be 4 or 8");
  if (mode == DV_DEBUG_TABLE_BOUND) {
    if (pos || pos_period) return fail(DV_ERR_ARG, "the table covers positions 0 .. rows-1: pos must be NULL, pos_period 0");
    if (rows * ((vocab + chunk_elems - 1) / chunk_elems) >= (int64_t{1} << 28)) return fail(DV_ERR_SHAPE, "table too large");
  }
  const int64_t width = mode == DV_DEBUG_GROUP_WORDS ? vocab / 8
                        : (mode == DV_DEBUG_CHUNK_BOUND || mode == DV_DEBUG_TABLE_BOUND) ? (vocab + chunk_elems - 1) / chunk_elems
                                                                                        : vocab;
  if (rows > 0 && width > 0 && !out) return fail(DV_ERR_NULL, "out is NULL");
  return hip_status(dv::launch_debug_noise(dv::seed_word(seed), pos, pos_period, rows, vocab, mode, chunk_elems, out,
                                           stream),
                    "dv_debug_noise launch");
}

dv_status dv_debug_read_probe(const dv_logits *logits, const dv_tuning *tuning, uint32_t *sink, hipStream_t stream) {
  dv_status s = check_logits(logits, true);
  if (s != DV_OK) return s;
  if (tuning && tuning->shared_noise == 1) return fail(DV_ERR_ARG, "the probe reads no noise table");
  const dv_noise greedy{};
  Geometry g;
  if ((s = choose_geometry(logits, &greedy, tuning, g)) != DV_OK) return s;
  static_assert(kMaxSplit <= dv::kMaxProbeSplit, "the sink holds a word per slice");
  if (logits->rows == 0) return ok();
  if (!sink) return fail(DV_ERR_NULL, "sink is NULL");
  dv::VerifyLaunch p{};
  p.va = logits->verifier;
  p.vb = logits->drafter;
  p.rows = logits->rows;
  p.vocab = logits->vocab;
  p.ld = logits->ld;
  p.bf16 = logits->dtype == DV_BF16;
  p.split = g.split;
  p.slice_chunks = g.slice_chunks;
  p.rows_per_block = g.rows_per_block;
  return hip_status(dv::launch_read_probe(p, sink, stream), "dv_debug_read_probe launch");
}

const char *dv_status_str(dv_status s) {
  switch (s) {
    case DV_OK: return "DV_OK";
    case DV_ERR_NULL: return "DV_ERR_NULL";
    case DV_ERR_SHAPE: return "DV_ERR_SHAPE";
    case DV_ERR_DTYPE: return "DV_ERR_DTYPE";
    case DV_ERR_ALIGN: return "DV_ERR_ALIGN";
    case DV_ERR_ARG: return "DV_ERR_ARG";
    case DV_ERR_WORKSPACE: return "DV_ERR_WORKSPACE";
    case DV_ERR_UNSUPPORTED: return "DV_ERR_UNSUPPORTED";
    case DV_ERR_HIP: return "DV_ERR_HIP";
  }
  return "DV_UNKNOWN_STATUS";
}

const char *dv_last_error(void) { return g_err; }

int dv_version(void) { return DV_VERSION; }

}  // extern "C"
