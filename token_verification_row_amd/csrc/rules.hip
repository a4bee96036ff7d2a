// Per-position decisions, COVER seed score and per-sequence top-k selection
// (gfx950). All are light next to the verification pass:
// they touch tens of bytes per row.
#include <climits>
#include <cmath>

#include "dv_internal.h"

namespace dv {
namespace {

// ---------------------------------------------------------------- decide ----
// The uniform of a row's remask draw: the noise hash of (seed, position) at
// index 2^32 - 1, mapped like the Gumbel uniforms (exact in float32).
__device__ __forceinline__ float remask_uniform(const DecideLaunch &p, int64_t r) {
  const int64_t ps = p.pos ? p.pos[r] : (p.pos_period > 0 ? r % p.pos_period : r);
  const uint32_t key = mix32(p.seed_b ^ mix32(static_cast<uint32_t>(ps) ^ kPosSalt));
  const uint32_t h = mix32(key ^ (0xFFFFFFFFu * kIndexStep));
  return static_cast<float>(2u * (h >> 9) + 1u) * 0x1p-24f;
}

// Rule for one row in isolation ([DualDiffusion] §2 "Verification algorithms"
// items 1-3, item 2 also with its probabilistic clause, item 3 also read as the
// confidence in the drafted token; [COVER] §3 "Adaptive revision outcomes").
__device__ __forceinline__ uint8_t rule_of_row(const DecideLaunch &p, int64_t r, int32_t cur) {
  switch (p.rule) {
    case DV_RULE_TRUST:
      return DV_KEEP;
    case DV_RULE_KL:
      return p.kl[r] > p.tau_kl ? DV_REMASK : DV_KEEP;
    case DV_RULE_CONF:
      return p.conf[r] < p.conf_thr ? DV_REMASK : DV_KEEP;
    case DV_RULE_KL_OR_CONF:
      return (p.kl[r] > p.tau_kl || p.conf[r] < p.conf_thr) ? DV_REMASK : DV_KEEP;
    case DV_RULE_COVER:
      if (p.tok_v[r] == cur) return DV_KEEP;
      return p.conf[r] >= p.conf_thr ? DV_REPLACE : DV_REMASK;
    case DV_RULE_CONF_DRAFT:
      return p.p_tok[r] < p.conf_thr ? DV_REMASK : DV_KEEP;
    case DV_RULE_KL_STOCHASTIC:
      return __fmul_rn(remask_uniform(p, r), p.tau_kl) < p.kl[r] ? DV_REMASK : DV_KEEP;
    default:
      return DV_NONE;
  }
}

// rule_of_row with the rule fixed at compile time (a loop over rows then holds one rule's code only).
template <int RULE>
__device__ __forceinline__ uint8_t rule_of_row_t(const DecideLaunch &p, int64_t r, int32_t cur) {
  if constexpr (RULE == DV_RULE_TRUST) return DV_KEEP;
  if constexpr (RULE == DV_RULE_KL) return p.kl[r] > p.tau_kl ? DV_REMASK : DV_KEEP;
  if constexpr (RULE == DV_RULE_CONF) return p.conf[r] < p.conf_thr ? DV_REMASK : DV_KEEP;
  if constexpr (RULE == DV_RULE_KL_OR_CONF) return (p.kl[r] > p.tau_kl || p.conf[r] < p.conf_thr) ? DV_REMASK : DV_KEEP;
  if constexpr (RULE == DV_RULE_COVER) {
    if (p.tok_v[r] == cur) return DV_KEEP;
    return p.conf[r] >= p.conf_thr ? DV_REPLACE : DV_REMASK;
  }
  if constexpr (RULE == DV_RULE_CONF_DRAFT) return p.p_tok[r] < p.conf_thr ? DV_REMASK : DV_KEEP;
  if constexpr (RULE == DV_RULE_KL_STOCHASTIC)
    return __fmul_rn(remask_uniform(p, r), p.tau_kl) < p.kl[r] ? DV_REMASK : DV_KEEP;
  return DV_NONE;
}

__device__ __forceinline__ int32_t current_token(const DecideLaunch &p, int64_t r) {
  return p.cur_tok ? p.cur_tok[r] : p.tok_d[r];
}

__device__ __forceinline__ bool is_subject(const DecideLaunch &p, int64_t r) {
  return p.subject == nullptr || p.subject[r] != 0;
}

__device__ __forceinline__ void emit(const DecideLaunch &p, int64_t r, uint8_t d, int32_t cur) {
  if (p.decision) p.decision[r] = d;
  if (p.out_tok) {
    int32_t t = cur;
    if (d == DV_REPLACE) t = p.tok_v[r];
    if (d == DV_REMASK) t = p.mask_token;
    p.out_tok[r] = t;
  }
}

// One wave per group of group_len consecutive rows (a candidate). Pass 1 finds
// the first decided row that breaks the group (coupled acceptance: tokens
// disagree; other rules: decision is not KEEP); pass 2 writes the decisions.
// With group_len == 0 the rows are cut into 64-row tiles and no prefix exists.
__device__ __forceinline__ void decide_group(const DecideLaunch &p, int64_t g, int lane) {
  const int64_t G = p.group_len > 0 ? p.group_len : 64;
  const int64_t ngroups = (p.rows + G - 1) / G;
  if (g >= ngroups) return;
  const int64_t r0 = g * G;
  const int64_t r1 = min(r0 + G, p.rows);
  const bool coupled = p.rule == DV_RULE_COUPLED_ACCEPT;

  int64_t first = G;  // offset of the first breaking row
  if (coupled || p.prefix_len) {
    for (int64_t base = r0; base < r1 && first == G; base += 64) {
      const int64_t r = base + lane;
      bool brk = false;
      if (r < r1 && is_subject(p, r)) {
        const int32_t cur = current_token(p, r);
        brk = coupled ? (p.tok_v[r] != cur) : (rule_of_row(p, r, cur) != DV_KEEP);
      }
      const unsigned long long m = __ballot(brk);
      if (m) first = (base - r0) + __ffsll(m) - 1;
    }
  }
  for (int64_t base = r0; base < r1; base += 64) {
    const int64_t r = base + lane;
    if (r >= r1) continue;
    const int32_t cur = current_token(p, r);
    uint8_t d = DV_NONE;
    if (is_subject(p, r)) {
      if (coupled) {
        const int64_t j = r - r0;
        d = j < first ? DV_KEEP : (j == first ? DV_REPLACE : DV_REMASK);
      } else {
        d = rule_of_row(p, r, cur);
      }
    }
    emit(p, r, d, cur);
  }
  if (p.prefix_len && lane == 0) p.prefix_len[g] = static_cast<int32_t>(first);
}

__global__ __launch_bounds__(256) void decide_kernel(DecideLaunch p) {
  decide_group(p, static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// Longest accepted prefix over all groups, lowest group index on ties.
__global__ __launch_bounds__(1024) void best_group_kernel(const int32_t *prefix, int64_t ngroups, int32_t *best) {
  __shared__ long long s_key[1024];
  long long key = LLONG_MIN;
  for (int64_t g = threadIdx.x; g < ngroups; g += blockDim.x) {
    // larger prefix first; among equal prefixes the smaller index gives the larger key
    const long long k = (static_cast<long long>(prefix[g]) << 32) | static_cast<long long>(0xFFFFFFFFu - static_cast<uint32_t>(g));
    key = k > key ? k : key;
  }
  s_key[threadIdx.x] = key;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const long long other = s_key[threadIdx.x + o];
      if (other > s_key[threadIdx.x]) s_key[threadIdx.x] = other;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    best[0] = ngroups > 0 ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(s_key[0] & 0xFFFFFFFFll)) : -1;
  }
}

// Small batches in one launch: one workgroup finds the first breaking row of
// every group (LDS atomicMin over the rows), writes the decisions, the prefixes
// and the best group. The same results as decide_kernel + best_group_kernel.
constexpr int64_t kSmallDecideRows = 16384;
constexpr int64_t kSmallDecideGroups = 1024;

// Largest key of a workgroup of kThreads threads: xor shuffles inside each wave,
// then one LDS round over the waves' results. Every thread gets the answer.
template <int kThreads>
__device__ __forceinline__ long long block_max_key(long long key, long long *s_wave) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const long long other = __shfl_xor(key, o);
    key = other > key ? other : key;
  }
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = key;
  __syncthreads();
  long long m = s_wave[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = s_wave[w] > m ? s_wave[w] : m;
  return m;
}

// q = r / G and m = r - q G for 0 <= r < 2^24 and G >= 1: the quotient through the
// float reciprocal is off by at most one, which the remainder's range corrects
// (integer division is a long instruction sequence on this GPU).
__device__ __forceinline__ void divmod_small(int32_t r, int32_t G, float rcp_G, int32_t &q, int32_t &m) {
  q = static_cast<int32_t>(static_cast<float>(r) * rcp_G);
  m = r - q * G;
  if (m < 0) {
    --q;
    m += G;
  }
  if (m >= G) {
    ++q;
    m -= G;
  }
}

// The single-workgroup decision over all rows, for a workgroup of kThreads
// threads (group_len > 0 dividing rows, rows <= kSmallDecideRows, at most
// kSmallDecideGroups groups), with the rule fixed at compile time.
template <int kThreads, int RULE>
__device__ __forceinline__ void decide_small_rule(const DecideLaunch &p, int32_t *s_first, long long *s_wave) {
  constexpr bool coupled = RULE == DV_RULE_COUPLED_ACCEPT;
  const int32_t tid = static_cast<int32_t>(threadIdx.x);
  const int32_t rows = static_cast<int32_t>(p.rows), G = static_cast<int32_t>(p.group_len);
  const int32_t ngroups = rows / G;
  const float rcp_G = 1.0f / static_cast<float>(G);
  for (int32_t g = tid; g < ngroups; g += kThreads) s_first[g] = G;
  __syncthreads();
  // Rows go in batches of kBatch per thread, every load of a batch issued before the first
  // is used (at clamped, always valid rows, the optional arrays chosen outside the batch):
  // one memory round trip per batch, not one per row.
  constexpr int kBatch = 8;
  const int32_t *ctok = p.cur_tok ? p.cur_tok : p.tok_d;
  const auto load_batch = [&](int32_t base, bool (&subj)[kBatch], int32_t (&cur)[kBatch], int32_t (&tv)[kBatch]) {
    int32_t rc[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) rc[i] = min(base + i * kThreads, rows - 1);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) cur[i] = ctok[rc[i]];
    if constexpr (coupled) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) tv[i] = p.tok_v[rc[i]];
    }
    uint8_t sb[kBatch];
    if (p.subject) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) sb[i] = p.subject[rc[i]];
    } else {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) sb[i] = 1;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) subj[i] = base + i * kThreads < rows && sb[i] != 0;
  };
  for (int32_t base = tid; base < rows; base += kThreads * kBatch) {
    bool subj[kBatch], brk[kBatch];
    int32_t cur[kBatch], tv[kBatch];
    load_batch(base, subj, cur, tv);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if constexpr (coupled)
        brk[i] = subj[i] && tv[i] != cur[i];
      else
        brk[i] = subj[i] && rule_of_row_t<RULE>(p, min(base + i * kThreads, rows - 1), cur[i]) != DV_KEEP;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (brk[i]) {
        int32_t g, j;
        divmod_small(base + i * kThreads, G, rcp_G, g, j);
        atomicMin(&s_first[g], j);
      }
    }
  }
  __syncthreads();
  for (int32_t base = tid; base < rows; base += kThreads * kBatch) {
    bool subj[kBatch];
    int32_t cur[kBatch], tv[kBatch];
    uint8_t d[kBatch];
    load_batch(base, subj, cur, tv);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int32_t r = base + i * kThreads;
      d[i] = DV_NONE;
      if (subj[i]) {
        if constexpr (coupled) {
          int32_t g, j;
          divmod_small(r, G, rcp_G, g, j);
          const int32_t first = s_first[g];
          d[i] = j < first ? DV_KEEP : (j == first ? DV_REPLACE : DV_REMASK);
        } else {
          d[i] = rule_of_row_t<RULE>(p, r, cur[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int32_t r = base + i * kThreads;
      if (r < rows) {
        if (p.decision) p.decision[r] = d[i];
        if (p.out_tok) {
          int32_t t = cur[i];
          if (d[i] == DV_REPLACE) {
            if constexpr (coupled)
              t = tv[i];
            else
              t = p.tok_v[r];
          }
          if (d[i] == DV_REMASK) t = p.mask_token;
          p.out_tok[r] = t;
        }
      }
    }
  }
  long long key = LLONG_MIN;
  for (int32_t g = tid; g < ngroups; g += kThreads) {
    const int32_t f = s_first[g];
    if (p.prefix_len) p.prefix_len[g] = f;
    // larger prefix first; among equal prefixes the smaller index gives the larger key
    const long long k = (static_cast<long long>(f) << 32) | static_cast<long long>(0xFFFFFFFFu - static_cast<uint32_t>(g));
    key = k > key ? k : key;
  }
  if (p.best_group == nullptr) return;  // uniform: no barrier follows for anyone
  const long long best = block_max_key<kThreads>(key, s_wave);
  if (tid == 0)
    p.best_group[0] = ngroups > 0 ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFll)) : -1;
}

template <int kThreads>
__device__ __forceinline__ void decide_small_block(const DecideLaunch &p) {
  __shared__ int32_t s_first[kSmallDecideGroups];
  __shared__ long long s_wave[kThreads / 64];
  switch (p.rule) {
    case DV_RULE_COUPLED_ACCEPT: decide_small_rule<kThreads, DV_RULE_COUPLED_ACCEPT>(p, s_first, s_wave); break;
    case DV_RULE_TRUST: decide_small_rule<kThreads, DV_RULE_TRUST>(p, s_first, s_wave); break;
    case DV_RULE_KL: decide_small_rule<kThreads, DV_RULE_KL>(p, s_first, s_wave); break;
    case DV_RULE_CONF: decide_small_rule<kThreads, DV_RULE_CONF>(p, s_first, s_wave); break;
    case DV_RULE_KL_OR_CONF: decide_small_rule<kThreads, DV_RULE_KL_OR_CONF>(p, s_first, s_wave); break;
    case DV_RULE_COVER: decide_small_rule<kThreads, DV_RULE_COVER>(p, s_first, s_wave); break;
    case DV_RULE_CONF_DRAFT: decide_small_rule<kThreads, DV_RULE_CONF_DRAFT>(p, s_first, s_wave); break;
    case DV_RULE_KL_STOCHASTIC: decide_small_rule<kThreads, DV_RULE_KL_STOCHASTIC>(p, s_first, s_wave); break;
    default: break;
  }
}

__global__ __launch_bounds__(1024) void decide_small_kernel(DecideLaunch p) { decide_small_block<1024>(p); }

// ------------------------------------------------------------ seed score ----
// [COVER] §2, the Score equation: u (1 + d_in) / (1 + d_out).
__global__ __launch_bounds__(256) void seed_score_kernel(int64_t rows, const float *u, const float *d_in,
                                                        const float *d_out, const uint8_t *eligible, float *score) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float s = -INFINITY;
  if (eligible == nullptr || eligible[r] != 0) s = u[r] * (1.0f + d_in[r]) / (1.0f + d_out[r]);
  score[r] = s;
}

// A row's inputs to the row rules, loaded together: every pointer the rule may read is
// replaced, when the call left it NULL, by the current-token array (always given), so that
// no load sits behind a branch and none waits for another. The rule then reads only the
// fields the call checked it gives.
struct RowVals {
  float kl, conf, p_tok;
  int32_t tok_v, cur;
};
__device__ __forceinline__ RowVals load_row_vals(const DecideLaunch &p, int64_t r) {
  const int32_t *ctok = p.cur_tok ? p.cur_tok : p.tok_d;
  const float *any = reinterpret_cast<const float *>(ctok);
  RowVals v;
  v.cur = ctok[r];
  v.kl = (p.kl ? p.kl : any)[r];
  v.conf = (p.conf ? p.conf : any)[r];
  v.p_tok = (p.p_tok ? p.p_tok : any)[r];
  v.tok_v = (p.tok_v ? p.tok_v : ctok)[r];
  return v;
}

// rule_of_row on loaded values.
__device__ __forceinline__ uint8_t rule_of_vals(const DecideLaunch &p, int64_t r, const RowVals &v) {
  switch (p.rule) {
    case DV_RULE_TRUST:
      return DV_KEEP;
    case DV_RULE_KL:
      return v.kl > p.tau_kl ? DV_REMASK : DV_KEEP;
    case DV_RULE_CONF:
      return v.conf < p.conf_thr ? DV_REMASK : DV_KEEP;
    case DV_RULE_KL_OR_CONF:
      return (v.kl > p.tau_kl || v.conf < p.conf_thr) ? DV_REMASK : DV_KEEP;
    case DV_RULE_COVER:
      if (v.tok_v == v.cur) return DV_KEEP;
      return v.conf >= p.conf_thr ? DV_REPLACE : DV_REMASK;
    case DV_RULE_CONF_DRAFT:
      return v.p_tok < p.conf_thr ? DV_REMASK : DV_KEEP;
    case DV_RULE_KL_STOCHASTIC:
      return __fmul_rn(remask_uniform(p, r), p.tau_kl) < v.kl ? DV_REMASK : DV_KEEP;
    default:
      return DV_NONE;
  }
}

// --------------------------------------------------------------- top-k ----
// Keys sort descending: the upper word orders the scores (largest or smallest
// first), the lower word is ~index so that equal scores go to the lower index.
// Ineligible positions get key 0, below every real key.
__device__ __forceinline__ unsigned long long select_key(float s, uint32_t i, int32_t largest) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;  // -0 ranks as +0
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // increasing in s
  if (!largest) ord = ~ord;
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<unsigned long long>(0xFFFFFFFFu - i);
}

// Sequences of up to kRankMaxLen positions: the sorted position of each kept entry is its
// rank, the number of keys above its own (keys are distinct: the index is part of them).
// One 4-wave workgroup per (sequence, 64 positions): the workgroup builds all the
// sequence's keys in LDS (every load issued before the first is used) and counts the
// entries the threshold keeps; each wave then ranks the 64 positions against a quarter of
// the keys, and the quarters' counts are added in LDS. The workgroups of a sequence write
// disjoint outputs, so none waits for another. Scores are not NaN, so the kept entries (key
// above the threshold's key) are a prefix of the order and their number is
// min(k, number of kept entries). Same keys, same order as the sort. Given the seed score's
// inputs (p.u set) instead of scores, it computes the scores with seed_score_kernel's
// arithmetic, and each workgroup writes those of its own 64 positions.
constexpr int32_t kRankMaxLen = 2048;
constexpr int kRankThreads = 256;
// The workgroup of sequence seq and positions [64 by, 64 by + 64) (kRankThreads threads).
// DECIDE: then the decisions d over the same rows with the selection as their subject:
// wave 0 evaluates d's row rule at each selected position of its 64 (the row's inputs are
// loaded at the start, beside the selection's) and DV_NONE elsewhere.
template <bool DECIDE>
__device__ __forceinline__ void select_rank_block(const SelectLaunch &p, int64_t seq, int32_t by,
                                                  const DecideLaunch &d) {
  constexpr int kPer = kRankMaxLen / kRankThreads;  // keys built per thread, at most
  __shared__ unsigned long long keys[kRankMaxLen];
  __shared__ float vals[kRankMaxLen];
  __shared__ int32_t part[4][64];
  __shared__ int32_t wave_kept[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t L = static_cast<int32_t>(p.seq_len);
  const float *sc = p.score + seq * p.seq_len;
  const uint8_t *el = p.eligible ? p.eligible + seq * p.seq_len : nullptr;
  // the threshold's key without its index word: a score is kept iff its key's upper word is above it
  const uint32_t thr_ord = static_cast<uint32_t>(select_key(p.thr, 0u, p.largest) >> 32);
  // loads at clamped (always valid) positions, all issued before the first is used
  const int32_t i = by * 64 + lane;
  RowVals rv{};
  if (DECIDE && wave == 0) rv = load_row_vals(d, seq * p.seq_len + min(i, L - 1));
  float v[kPer];
  uint32_t e[kPer];
  if (el) {
#pragma unroll
    for (int t = 0; t < kPer; ++t) e[t] = el[min(t * kRankThreads + tid, L - 1)];
  } else {
#pragma unroll
    for (int t = 0; t < kPer; ++t) e[t] = 1u;
  }
  if (p.u) {
    // the seed scores, with seed_score_kernel's arithmetic
    const int64_t base = seq * p.seq_len;
    float uu[kPer], di[kPer], dd[kPer];
    uint32_t se[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int64_t j = base + min(t * kRankThreads + tid, L - 1);
      uu[t] = p.u[j];
      di[t] = p.d_in[j];
      dd[t] = p.d_out[j];
    }
    // the optional array chosen once, outside the loads (a choice per load would wait for each)
    if (p.seed_eligible) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) se[t] = p.seed_eligible[base + min(t * kRankThreads + tid, L - 1)];
    } else {
#pragma unroll
      for (int t = 0; t < kPer; ++t) se[t] = 1u;
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      float s = -INFINITY;
      if (se[t] != 0) s = uu[t] * (1.0f + di[t]) / (1.0f + dd[t]);
      v[t] = s;
      const int32_t j = t * kRankThreads + tid;
      if (p.score_out && j < L && (j >> 6) == by) p.score_out[base + j] = s;
    }
  } else {
#pragma unroll
    for (int t = 0; t < kPer; ++t) v[t] = sc[min(t * kRankThreads + tid, L - 1)];
  }
  int32_t kept = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int32_t j = t * kRankThreads + tid;
    const bool ok = j < L && e[t] != 0;
    const unsigned long long k = ok ? select_key(v[t], static_cast<uint32_t>(j), p.largest) : 0ull;
    if (j < L) {
      keys[j] = k;
      vals[j] = v[t];
    }
    const bool keep = k != 0 && (!p.use_thr || static_cast<uint32_t>(k >> 32) > thr_ord);
    kept += __popcll(__ballot(keep));
  }
  if (lane == 0) wave_kept[wave] = kept;
  __syncthreads();
  const int32_t count = min(p.k, wave_kept[0] + wave_kept[1] + wave_kept[2] + wave_kept[3]);
  const unsigned long long ki = i < L ? keys[i] : 0ull;
  const int32_t q = (L + 3) / 4, j0 = wave * q, j1 = min(L, j0 + q);
  int32_t r = 0;
#pragma unroll 16
  for (int32_t j = j0; j < j1; ++j) r += keys[j] > ki ? 1 : 0;
  part[wave][lane] = r;
  __syncthreads();
  if (wave != 0) return;
  const int32_t rank = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
  const bool sel = ki != 0 && rank < count;
  if (sel) {
    if (p.out_idx) p.out_idx[seq * p.k + rank] = i;
    if (p.out_val) p.out_val[seq * p.k + rank] = vals[i];
  }
  if (p.out_mask && i < L) p.out_mask[seq * p.seq_len + i] = sel ? 1 : 0;
  if (by == 0) {
    for (int32_t j = count + lane; j < p.k; j += 64) {
      if (p.out_idx) p.out_idx[seq * p.k + j] = -1;
      if (p.out_val) p.out_val[seq * p.k + j] = __builtin_nanf("");
    }
    if (lane == 0 && p.out_count) p.out_count[seq] = count;
  }
  if constexpr (DECIDE) {
    if (i < L) {
      const int64_t r = seq * p.seq_len + i;
      const uint8_t dr = sel ? rule_of_vals(d, r, rv) : DV_NONE;
      if (d.decision) d.decision[r] = dr;
      if (d.out_tok) d.out_tok[r] = dr == DV_REPLACE ? rv.tok_v : (dr == DV_REMASK ? d.mask_token : rv.cur);
    }
  }
}

__global__ __launch_bounds__(kRankThreads) void select_rank_kernel(SelectLaunch p) {
  select_rank_block<false>(p, blockIdx.x, static_cast<int32_t>(blockIdx.y), DecideLaunch{});
}

// dv_seed_select_decide: the selection, then the decisions over its seeds, in one launch.
__global__ __launch_bounds__(kRankThreads) void select_decide_kernel(SelectLaunch p, DecideLaunch d) {
  select_rank_block<true>(p, blockIdx.x, static_cast<int32_t>(blockIdx.y), d);
}

// Longer sequences: one workgroup per sequence, bitonic sort of pow2 keys in LDS.
__global__ __launch_bounds__(1024) void select_topk_kernel(SelectLaunch p, int32_t pow2) {
  extern __shared__ unsigned long long keys[];
  uint8_t *flags = reinterpret_cast<uint8_t *>(keys + pow2);
  __shared__ int s_count;
  const int64_t seq = blockIdx.x;
  const int32_t L = static_cast<int32_t>(p.seq_len);
  const float *sc = p.score + seq * p.seq_len;
  const uint8_t *el = p.eligible ? p.eligible + seq * p.seq_len : nullptr;
  for (int32_t i = threadIdx.x; i < pow2; i += blockDim.x) {
    unsigned long long k = 0;
    if (i < L && (el == nullptr || el[i] != 0)) k = select_key(sc[i], static_cast<uint32_t>(i), p.largest);
    keys[i] = k;
  }
  if (threadIdx.x == 0) s_count = p.k;
  for (int32_t size = 2; size <= pow2; size <<= 1) {
    for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int32_t t = threadIdx.x; t < (pow2 >> 1); t += blockDim.x) {
        const int32_t i = 2 * t - (t & (stride - 1));
        const int32_t j = i + stride;
        const bool desc = (i & size) == 0;
        const unsigned long long a = keys[i], b = keys[j];
        if ((a < b) == desc && a != b) {
          keys[i] = b;
          keys[j] = a;
        }
      }
    }
  }
  __syncthreads();
  // the kept entries are a prefix of the sorted list: find where it ends
  for (int32_t j = threadIdx.x; j < p.k; j += blockDim.x) {
    const unsigned long long k = keys[j];
    bool keep = k != 0;
    if (keep && p.use_thr) {
      const float v = sc[0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull)];
      keep = p.largest ? (v > p.thr) : (v < p.thr);
    }
    if (!keep) atomicMin(&s_count, j);
  }
  for (int32_t i = threadIdx.x; i < L; i += blockDim.x) flags[i] = 0;
  __syncthreads();
  const int32_t count = s_count;
  for (int32_t j = threadIdx.x; j < p.k; j += blockDim.x) {
    int32_t idx = -1;
    float val = __builtin_nanf("");
    if (j < count) {
      idx = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(keys[j] & 0xFFFFFFFFull));
      val = sc[idx];
      flags[idx] = 1;
    }
    if (p.out_idx) p.out_idx[seq * p.k + j] = idx;
    if (p.out_val) p.out_val[seq * p.k + j] = val;
  }
  if (threadIdx.x == 0 && p.out_count) p.out_count[seq] = count;
  __syncthreads();
  if (p.out_mask) {
    for (int32_t i = threadIdx.x; i < L; i += blockDim.x) p.out_mask[seq * p.seq_len + i] = flags[i];
  }
}

// ------------------------------------------------- decide + seed select ----
// dv_decide and dv_seed_select in one launch of kRankThreads-thread workgroups:
// the first nd workgroups decide (one workgroup for the whole batch on the
// small-batch path, else one group per wave as decide_kernel), the others
// select as select_rank_kernel, workgroup nd + seq * ny + y taking positions
// [64 y, 64 y + 64) of sequence seq. The two calls share no memory, so the
// order in which their workgroups run does not matter.
__global__ __launch_bounds__(kRankThreads) void decide_select_kernel(DecideLaunch d, SelectLaunch s, uint32_t nd,
                                                                    int32_t small, uint32_t ny) {
  const uint32_t b = blockIdx.x;
  if (b < nd) {
    if (small)
      decide_small_block<kRankThreads>(d);
    else
      decide_group(d, static_cast<int64_t>(b) * (kRankThreads / 64) + (threadIdx.x >> 6), threadIdx.x & 63);
    return;
  }
  select_rank_block<false>(s, (b - nd) / ny, static_cast<int32_t>((b - nd) % ny), d);
}

// ------------------------------------------------------------- noise dump ----
}  // namespace

hipError_t launch_decide(const DecideLaunch &p, hipStream_t stream) {
  const int64_t G = p.group_len > 0 ? p.group_len : 64;
  const int64_t ngroups = (p.rows + G - 1) / G;
  if (p.group_len > 0 && p.rows <= kSmallDecideRows && ngroups <= kSmallDecideGroups) {
    hipLaunchKernelGGL(decide_small_kernel, dim3(1), dim3(1024), 0, stream, p);
    return hipGetLastError();
  }
  if (p.rows > 0) {
    const unsigned blocks = static_cast<unsigned>((ngroups + 3) / 4);
    hipLaunchKernelGGL(decide_kernel, dim3(blocks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.best_group == nullptr) return hipSuccess;
  hipLaunchKernelGGL(best_group_kernel, dim3(1), dim3(1024), 0, stream, p.prefix_len, ngroups, p.best_group);
  return hipGetLastError();
}

hipError_t launch_seed_score(int64_t rows, const float *u, const float *d_in, const float *d_out,
                             const uint8_t *eligible, float *score, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((rows + 255) / 256);
  hipLaunchKernelGGL(seed_score_kernel, dim3(blocks), dim3(256), 0, stream, rows, u, d_in, d_out, eligible, score);
  return hipGetLastError();
}

hipError_t launch_seed_select(const SelectLaunch &p, hipStream_t stream) {
  if (p.nseq == 0) return hipSuccess;
  if (p.seq_len <= kRankMaxLen) {
    const dim3 grid(static_cast<unsigned>(p.nseq), static_cast<unsigned>((p.seq_len + 63) / 64));
    hipLaunchKernelGGL(select_rank_kernel, grid, dim3(kRankThreads), 0, stream, p);
    return hipGetLastError();
  }
  // longer sequences: the scores, then the sort
  hipError_t e = launch_seed_score(p.nseq * p.seq_len, p.u, p.d_in, p.d_out, p.seed_eligible, p.score_out, stream);
  if (e != hipSuccess) return e;
  SelectLaunch q = p;
  q.score = p.score_out;
  q.u = q.d_in = q.d_out = nullptr;
  q.seed_eligible = nullptr;
  q.score_out = nullptr;
  return launch_select_topk(q, stream);
}

hipError_t launch_decide_seed_select(const DecideLaunch &d, bool decide, const SelectLaunch &s, hipStream_t stream) {
  const int64_t G = d.group_len > 0 ? d.group_len : 64;
  const int64_t ngroups = (d.rows + G - 1) / G;
  const bool small = d.group_len > 0 && d.rows <= kSmallDecideRows && ngroups <= kSmallDecideGroups;
  // one launch when the decision is one workgroup or one wave per group with no best-group pass,
  // and the selection is the rank path
  const bool fusable = decide && d.rows > 0 && (small || d.best_group == nullptr) && s.nseq > 0 &&
                       s.seq_len <= kRankMaxLen;
  const int64_t ny = (s.seq_len + 63) / 64;
  const int64_t nd = small ? 1 : (ngroups + kRankThreads / 64 - 1) / (kRankThreads / 64);
  if (fusable && nd + s.nseq * ny <= 0x7FFFFFFFll) {
    hipLaunchKernelGGL(decide_select_kernel, dim3(static_cast<unsigned>(nd + s.nseq * ny)), dim3(kRankThreads), 0,
                       stream, d, s, static_cast<uint32_t>(nd), small ? 1 : 0, static_cast<uint32_t>(ny));
    return hipGetLastError();
  }
  // otherwise each call's own launches, in call order
  if (decide) {
    const hipError_t e = launch_decide(d, stream);
    if (e != hipSuccess) return e;
  }
  return launch_seed_select(s, stream);
}

hipError_t launch_seed_select_decide(const SelectLaunch &s, const DecideLaunch &d, hipStream_t stream) {
  if (s.nseq == 0) return hipSuccess;
  if (s.seq_len <= kRankMaxLen) {
    const dim3 grid(static_cast<unsigned>(s.nseq), static_cast<unsigned>((s.seq_len + 63) / 64));
    hipLaunchKernelGGL(select_decide_kernel, grid, dim3(kRankThreads), 0, stream, s, d);
    return hipGetLastError();
  }
  // longer sequences: the selection's own launches, then the decisions with its mask as their subject
  const hipError_t e = launch_seed_select(s, stream);
  if (e != hipSuccess) return e;
  DecideLaunch q = d;
  q.subject = s.out_mask;
  return launch_decide(q, stream);
}

hipError_t launch_select_topk(const SelectLaunch &p, hipStream_t stream) {
  if (p.nseq == 0) return hipSuccess;
  if (p.seq_len <= kRankMaxLen) {
    const dim3 grid(static_cast<unsigned>(p.nseq), static_cast<unsigned>((p.seq_len + 63) / 64));
    hipLaunchKernelGGL(select_rank_kernel, grid, dim3(kRankThreads), 0, stream, p);
    return hipGetLastError();
  }
  int32_t pow2 = 2;
  while (pow2 < p.seq_len) pow2 <<= 1;
  const size_t lds = static_cast<size_t>(pow2) * sizeof(unsigned long long) + static_cast<size_t>(p.seq_len);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_topk_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int threads = pow2 >= 2048 ? 1024 : (pow2 / 2 < 64 ? 64 : pow2 / 2);
  hipLaunchKernelGGL(select_topk_kernel, dim3(static_cast<unsigned>(p.nseq)), dim3(threads), lds, stream, p, pow2);
  return hipGetLastError();
}

}  // namespace dv
