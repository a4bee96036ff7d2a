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
__global__ __launch_bounds__(256) void decide_kernel(DecideLaunch p) {
  const int lane = threadIdx.x & 63;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
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

__global__ __launch_bounds__(1024) void decide_small_kernel(DecideLaunch p) {
  __shared__ int32_t s_first[kSmallDecideGroups];
  __shared__ long long s_key[1024];
  const int tid = threadIdx.x;
  const int64_t G = p.group_len;  // > 0 and dividing rows
  const int64_t ngroups = p.rows / G;
  const bool coupled = p.rule == DV_RULE_COUPLED_ACCEPT;
  for (int64_t g = tid; g < ngroups; g += 1024) s_first[g] = static_cast<int32_t>(G);
  __syncthreads();
  for (int64_t r = tid; r < p.rows; r += 1024) {
    if (!is_subject(p, r)) continue;
    const int32_t cur = current_token(p, r);
    const bool brk = coupled ? (p.tok_v[r] != cur) : (rule_of_row(p, r, cur) != DV_KEEP);
    if (brk) atomicMin(&s_first[r / G], static_cast<int32_t>(r % G));
  }
  __syncthreads();
  for (int64_t r = tid; r < p.rows; r += 1024) {
    const int32_t cur = current_token(p, r);
    uint8_t d = DV_NONE;
    if (is_subject(p, r)) {
      if (coupled) {
        const int64_t j = r % G, first = s_first[r / G];
        d = j < first ? DV_KEEP : (j == first ? DV_REPLACE : DV_REMASK);
      } else {
        d = rule_of_row(p, r, cur);
      }
    }
    emit(p, r, d, cur);
  }
  long long key = LLONG_MIN;
  for (int64_t g = tid; g < ngroups; g += 1024) {
    const int32_t f = s_first[g];
    if (p.prefix_len) p.prefix_len[g] = f;
    const long long k = (static_cast<long long>(f) << 32) | static_cast<long long>(0xFFFFFFFFu - static_cast<uint32_t>(g));
    key = k > key ? k : key;
  }
  if (p.best_group == nullptr) return;  // uniform: no barrier follows for anyone
  s_key[tid] = key;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) {
      const long long other = s_key[tid + o];
      if (other > s_key[tid]) s_key[tid] = other;
    }
    __syncthreads();
  }
  if (tid == 0)
    p.best_group[0] = ngroups > 0 ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(s_key[0] & 0xFFFFFFFFll)) : -1;
}

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
__global__ __launch_bounds__(kRankThreads) void select_rank_kernel(SelectLaunch p) {
  constexpr int kPer = kRankMaxLen / kRankThreads;  // keys built per thread, at most
  __shared__ unsigned long long keys[kRankMaxLen];
  __shared__ float vals[kRankMaxLen];
  __shared__ int32_t part[4][64];
  __shared__ int32_t wave_kept[4];
  const int64_t seq = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t L = static_cast<int32_t>(p.seq_len);
  const float *sc = p.score + seq * p.seq_len;
  const uint8_t *el = p.eligible ? p.eligible + seq * p.seq_len : nullptr;
  // the threshold's key without its index word: a score is kept iff its key's upper word is above it
  const uint32_t thr_ord = static_cast<uint32_t>(select_key(p.thr, 0u, p.largest) >> 32);
  // loads at clamped (always valid) positions, all issued before the first is used
  float v[kPer];
  uint32_t e[kPer];
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
      se[t] = p.seed_eligible ? p.seed_eligible[j] : 1u;
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      float s = -INFINITY;
      if (se[t] != 0) s = uu[t] * (1.0f + di[t]) / (1.0f + dd[t]);
      v[t] = s;
      const int32_t j = t * kRankThreads + tid;
      if (p.score_out && j < L && (j >> 6) == static_cast<int32_t>(blockIdx.y)) p.score_out[base + j] = s;
    }
  } else {
#pragma unroll
    for (int t = 0; t < kPer; ++t) v[t] = sc[min(t * kRankThreads + tid, L - 1)];
  }
  if (el) {
#pragma unroll
    for (int t = 0; t < kPer; ++t) e[t] = el[min(t * kRankThreads + tid, L - 1)];
  } else {
#pragma unroll
    for (int t = 0; t < kPer; ++t) e[t] = 1u;
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
  const int32_t i = static_cast<int32_t>(blockIdx.y) * 64 + lane;
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
  if (blockIdx.y == 0) {
    for (int32_t j = count + lane; j < p.k; j += 64) {
      if (p.out_idx) p.out_idx[seq * p.k + j] = -1;
      if (p.out_val) p.out_val[seq * p.k + j] = __builtin_nanf("");
    }
    if (lane == 0 && p.out_count) p.out_count[seq] = count;
  }
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
