// Fused verification pass over verifier and drafter logits (gfx950).
//
// One pass over both [rows][vocab] logit matrices produces, per row, both
// log-sum-exps, KL(p_v || p_d), the verifier entropy and max-probability
// confidence, both argmaxes and the Gumbel-max tokens of both models under
// shared noise:
//   [DualDiffusion] §2 "Verification algorithms" items 2-3 (KL and
//   confidence remasking read these statistics);
//   [SPOT] §1 and §3 (coupled-noise verification: both models draw with the
//   same Gumbel noise);
//   [COVER] §2 (the seed score's uncertainty u is the entropy).
//
// Design (HBM-bound streaming reduction, no matrix cores):
//   * a wavefront owns a (row, vocabulary slice); each lane reads 16-byte
//     chunks (8 bf16 or 4 fp32) of both rows with non-temporal loads, lanes
//     of a wave covering 1 KiB of contiguous memory per load;
//   * sums of exponentials are taken against a per-lane reference rho that is
//     only moved when a logit exceeds it by more than 64 (log2 units), so the
//     usual per-element online rescale disappears: the running maximum is
//     tracked separately, per 16-byte chunk, for the argmax;
//   * KL and entropy come from the same pass: D = sum e_v (a - b) and
//     W = sum e_v t_v with t_v = a log2(e) - rho;
//   * argmax and Gumbel-max tokens are tracked per chunk (value, chunk index);
//     the exact lowest index inside the winning chunk is recovered at the end
//     by re-reading 16 bytes, so the hot loop carries no per-element index;
//   * the noise is computed in registers from a counter hash; when rows share
//     positions (the candidates of a tree level), a workgroup computes it once
//     per (position, slice) into LDS and every row at that position reuses it;
//   * lane states are combined across the wave with cross-lane shuffles, then
//     per row in double precision (split rows go through a workspace of 64-byte
//     partials and a merge kernel).
#include <climits>
#include <cmath>

#include "dv_internal.h"

namespace dv {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLn2 = 0.693147180559945309417232121458;
constexpr float kRebase = 64.0f;                          // log2 units
constexpr float kOneMinusHalfUlp = 0.999999940395355224609375f;  // 1 - 2^-24

enum { kGreedy = 0, kInline = 1, kShared = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Chunk {
  static constexpr int N = BF16 ? 8 : 4;  // elements per 16-byte chunk
};

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// Gumbel noise in log2 units: G = -log2(-log2 u), u = (2 (h >> 9) + 1) 2^-24.
// argmax_i (x_i/T + g_i) with g = -ln(-ln u) equals argmax_i (x_i log2(e)/T + G_i),
// since g log2(e) = G - log2(e) ln(ln 2) is an increasing map of G.
__device__ __forceinline__ float gumbel_log2(uint32_t h) {
  // 23 hash bits as the mantissa of a float in [1, 2); subtracting 1 - 2^-24 is exact
  const float u = __uint_as_float(0x3F800000u | (h >> 9)) - kOneMinusHalfUlp;
  const float l = __builtin_amdgcn_logf(u);  // v_log_f32: log2, 1 ulp (relative) on (0, 1)
  return -__builtin_amdgcn_logf(-l);
}

__device__ __forceinline__ uint32_t row_key(uint32_t seed_b, int32_t pos) {
  return mix32(seed_b ^ mix32(static_cast<uint32_t>(pos) ^ kPosSalt));
}

__device__ __forceinline__ float noise_at(uint32_t key, uint32_t i) {
  return gumbel_log2(mix32(key ^ (i * kIndexStep)));
}

__device__ __forceinline__ int32_t position_of(const VerifyLaunch &p, int64_t r) {
  if (p.pos) return p.pos[r];
  if (p.pos_period > 0) return static_cast<int32_t>(r % p.pos_period);
  return static_cast<int32_t>(r);
}

template <bool BF16>
__device__ __forceinline__ void widen(const u32x4 &w, float (&x)[Chunk<BF16>::N]) {
  if constexpr (BF16) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xFFFF0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xFFFF0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xFFFF0000u);
  } else {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
}

// Per-lane accumulator of one (row, slice).
struct Lane {
  float rho_v, S_v, W_v, D_v, thr_v;
  float rho_d, S_d, thr_d;
  float m_v, m_d, s_v, s_d;
  int32_t cm_v, cm_d, cs_v, cs_d;

  __device__ __forceinline__ void init() {
    rho_v = rho_d = -INFINITY;
    thr_v = thr_d = -INFINITY;
    S_v = W_v = D_v = S_d = 0.0f;
    m_v = m_d = s_v = s_d = -INFINITY;
    cm_v = cm_d = cs_v = cs_d = INT_MAX;
  }
};

// Move the reference to x * log2(e) and rescale what was accumulated so far.
__device__ __forceinline__ void rebase_v(Lane &st, float x) {
  const float nr = x * kLog2e;
  if (st.S_v > 0.0f) {
    const float d = st.rho_v - nr;  // <= 0
    const float sc = __builtin_amdgcn_exp2f(d);
    st.W_v = sc * __builtin_fmaf(d, st.S_v, st.W_v);
    st.S_v *= sc;
    st.D_v *= sc;
  } else {
    st.S_v = st.W_v = st.D_v = 0.0f;
  }
  st.rho_v = nr;
  st.thr_v = (nr + kRebase) * (1.0f / kLog2e);
}

__device__ __forceinline__ void rebase_d(Lane &st, float x) {
  const float nr = x * kLog2e;
  if (st.S_d > 0.0f) {
    st.S_d *= __builtin_amdgcn_exp2f(st.rho_d - nr);
  } else {
    st.S_d = 0.0f;
  }
  st.rho_d = nr;
  st.thr_d = (nr + kRebase) * (1.0f / kLog2e);
}

template <int N>
__device__ __forceinline__ float max_of(const float (&x)[N]) {
  float m = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = fmaxf(m, x[j]);
  return m;
}

template <int N>
__device__ __forceinline__ float tree_sum(const float (&x)[N]) {
  if constexpr (N == 8) {
    return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
  } else {
    return (x[0] + x[1]) + (x[2] + x[3]);
  }
}

// Fold one chunk (N logits of each model, N noise values) into the lane state.
// MASKED: only the first nvalid elements are logits (last chunk of a row).
template <int N, bool NOISE, bool MASKED>
__device__ __forceinline__ void consume(Lane &st, float (&a)[N], float (&b)[N], const float (&g)[N],
                                        int32_t c, float cT, int nvalid) {
  float cma, cmb;
  if constexpr (MASKED) {
    cma = a[0];
    cmb = b[0];
#pragma unroll
    for (int j = 1; j < N; ++j) {
      if (j < nvalid) {
        cma = fmaxf(cma, a[j]);
        cmb = fmaxf(cmb, b[j]);
      }
    }
    // padding takes a finite stand-in value; its contributions are zeroed below
#pragma unroll
    for (int j = 1; j < N; ++j) {
      if (j >= nvalid) {
        a[j] = cma;
        b[j] = cmb;
      }
    }
  } else {
    cma = max_of(a);
    cmb = max_of(b);
  }
  if (cma > st.m_v) {
    st.m_v = cma;
    st.cm_v = c;
  }
  if (cmb > st.m_d) {
    st.m_d = cmb;
    st.cm_d = c;
  }
  if (cma > st.thr_v) rebase_v(st, cma);
  if (cmb > st.thr_d) rebase_d(st, cmb);

  float ev[N], ed[N];
  const float nrv = -st.rho_v, nrd = -st.rho_d;
  float W = st.W_v, D = st.D_v;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float tv = __builtin_fmaf(a[j], kLog2e, nrv);
    const float td = __builtin_fmaf(b[j], kLog2e, nrd);
    float e = __builtin_amdgcn_exp2f(tv);
    float f = __builtin_amdgcn_exp2f(td);
    if constexpr (MASKED) {
      if (j >= nvalid) {
        e = 0.0f;
        f = 0.0f;
      }
    }
    ev[j] = e;
    ed[j] = f;
    W = __builtin_fmaf(e, tv, W);
    D = __builtin_fmaf(e, a[j] - b[j], D);
  }
  st.W_v = W;
  st.D_v = D;
  st.S_v += tree_sum(ev);
  st.S_d += tree_sum(ed);

  if constexpr (NOISE) {
    float pa[N], pb[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      pa[j] = __builtin_fmaf(a[j], cT, g[j]);
      pb[j] = __builtin_fmaf(b[j], cT, g[j]);
      if constexpr (MASKED) {
        if (j >= nvalid) {
          pa[j] = -INFINITY;
          pb[j] = -INFINITY;
        }
      }
    }
    const float csa = max_of(pa), csb = max_of(pb);
    if (csa > st.s_v) {
      st.s_v = csa;
      st.cs_v = c;
    }
    if (csb > st.s_d) {
      st.s_d = csb;
      st.cs_d = c;
    }
  }
}

// Noise values of chunk c into g: computed from the hash (kInline) or read
// from the workgroup's LDS copy of the slice (kShared).
template <bool BF16, int MODE>
__device__ __forceinline__ void noise_chunk(float (&g)[Chunk<BF16>::N], int32_t c, int32_t c0, uint32_t key,
                                            const float *g_lds) {
  constexpr int N = Chunk<BF16>::N;
  if constexpr (MODE == kInline) {
    const uint32_t i0 = static_cast<uint32_t>(c) * N;
#pragma unroll
    for (int j = 0; j < N; ++j) g[j] = noise_at(key, i0 + j);
  } else if constexpr (MODE == kShared) {
    const f32x4 *q = reinterpret_cast<const f32x4 *>(g_lds + (c - c0) * N);
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      const f32x4 v = q[j];
      g[4 * j + 0] = v.x;
      g[4 * j + 1] = v.y;
      g[4 * j + 2] = v.z;
      g[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) g[j] = 0.0f;
  }
}

// Stream chunks [c0, c1) of one row pair through the lanes of a wave.
template <bool BF16, int MODE>
__device__ __forceinline__ void scan_slice(Lane &st, const u32x4 *ra, const u32x4 *rb, int32_t c0, int32_t c1,
                                           int32_t nfull, int nvalid_tail, float cT, uint32_t key,
                                           const float *g_lds, int lane) {
  constexpr int N = Chunk<BF16>::N;
  constexpr bool NOISE = MODE != kGreedy;
  const int32_t cend = c1 < nfull ? c1 : nfull;
  int32_t c = c0 + lane;
  for (; c + 64 < cend; c += 128) {
    const u32x4 wa0 = load_stream(ra + c), wb0 = load_stream(rb + c);
    const u32x4 wa1 = load_stream(ra + c + 64), wb1 = load_stream(rb + c + 64);
    float g0[N], g1[N];
    noise_chunk<BF16, MODE>(g0, c, c0, key, g_lds);
    noise_chunk<BF16, MODE>(g1, c + 64, c0, key, g_lds);
    float a0[N], b0[N], a1[N], b1[N];
    widen<BF16>(wa0, a0);
    widen<BF16>(wb0, b0);
    widen<BF16>(wa1, a1);
    widen<BF16>(wb1, b1);
    consume<N, NOISE, false>(st, a0, b0, g0, c, cT, N);
    consume<N, NOISE, false>(st, a1, b1, g1, c + 64, cT, N);
  }
  if (c < cend) {
    const u32x4 wa = load_stream(ra + c), wb = load_stream(rb + c);
    float g[N];
    noise_chunk<BF16, MODE>(g, c, c0, key, g_lds);
    float a[N], b[N];
    widen<BF16>(wa, a);
    widen<BF16>(wb, b);
    consume<N, NOISE, false>(st, a, b, g, c, cT, N);
  }
  // the last, partly filled chunk of the row (vocab not a multiple of N)
  if (nvalid_tail > 0 && nfull >= c0 && nfull < c1 && lane == ((nfull - c0) & 63)) {
    const u32x4 wa = ra[nfull], wb = rb[nfull];
    float g[N];
    noise_chunk<BF16, MODE>(g, nfull, c0, key, g_lds);
    float a[N], b[N];
    widen<BF16>(wa, a);
    widen<BF16>(wb, b);
    consume<N, NOISE, true>(st, a, b, g, nfull, cT, nvalid_tail);
  }
}

// ---- cross-lane combination ----
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int32_t wave_min_i(int32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
// (value, chunk): largest value, lowest chunk among equal values
__device__ __forceinline__ void wave_argmax(float &m, int32_t &c) {
  const float M = wave_max(m);
  c = wave_min_i(m == M ? c : INT_MAX);
  m = M;
}

// Reduce the lane states of a wave into one partial (valid in every lane).
__device__ __forceinline__ Partial wave_reduce(const Lane &st) {
  Partial t;
  {
    const float R = wave_max(st.rho_v);
    const bool has = st.S_v > 0.0f;
    const float d = has ? st.rho_v - R : 0.0f;
    const float sc = has ? __builtin_amdgcn_exp2f(d) : 0.0f;
    t.S_v = wave_sum(st.S_v * sc);
    t.W_v = wave_sum(sc * __builtin_fmaf(d, st.S_v, st.W_v));
    t.D_v = wave_sum(st.D_v * sc);
    t.rho_v = R;
  }
  {
    const float R = wave_max(st.rho_d);
    const bool has = st.S_d > 0.0f;
    const float sc = has ? __builtin_amdgcn_exp2f(st.rho_d - R) : 0.0f;
    t.S_d = wave_sum(st.S_d * sc);
    t.rho_d = R;
  }
  t.m_v = st.m_v;
  t.cm_v = st.cm_v;
  wave_argmax(t.m_v, t.cm_v);
  t.m_d = st.m_d;
  t.cm_d = st.cm_d;
  wave_argmax(t.m_d, t.cm_d);
  t.s_v = st.s_v;
  t.cs_v = st.cs_v;
  wave_argmax(t.s_v, t.cs_v);
  t.s_d = st.s_d;
  t.cs_d = st.cs_d;
  wave_argmax(t.s_d, t.cs_d);
  t.pad0 = t.pad1 = 0;
  return t;
}

// ---- per-row epilogue (double precision) ----
struct Totals {
  double rho_v, S_v, W_v, D_v, rho_d, S_d;
  float m_v, m_d, s_v, s_d;
  int32_t cm_v, cm_d, cs_v, cs_d;
};

__device__ __forceinline__ Totals totals_of(const Partial &t) {
  Totals o;
  o.rho_v = t.rho_v;
  o.S_v = t.S_v;
  o.W_v = t.W_v;
  o.D_v = t.D_v;
  o.rho_d = t.rho_d;
  o.S_d = t.S_d;
  o.m_v = t.m_v;
  o.m_d = t.m_d;
  o.s_v = t.s_v;
  o.s_d = t.s_d;
  o.cm_v = t.cm_v;
  o.cm_d = t.cm_d;
  o.cs_v = t.cs_v;
  o.cs_d = t.cs_d;
  return o;
}

// lowest index inside chunk c whose logit equals m. A chunk index outside the
// row (only possible when the logits hold NaN, which is not supported) gives
// -1 without touching memory.
template <bool BF16>
__device__ int32_t refine_max(const u32x4 *row, int32_t c, float m, int64_t vocab) {
  constexpr int N = Chunk<BF16>::N;
  if (c < 0 || static_cast<int64_t>(c) * N >= vocab) return -1;
  float x[N];
  widen<BF16>(row[c], x);
  for (int j = 0; j < N; ++j) {
    const int64_t i = static_cast<int64_t>(c) * N + j;
    if (i < vocab && x[j] == m) return static_cast<int32_t>(i);
  }
  return static_cast<int32_t>(static_cast<int64_t>(c) * N);
}

// lowest index inside chunk c whose perturbed score equals best (recomputed
// with exactly the arithmetic of the streaming pass)
template <bool BF16>
__device__ int32_t refine_score(const u32x4 *row, int32_t c, float best, int64_t vocab, float cT, uint32_t key) {
  constexpr int N = Chunk<BF16>::N;
  if (c < 0 || static_cast<int64_t>(c) * N >= vocab) return -1;
  float x[N];
  widen<BF16>(row[c], x);
  for (int j = 0; j < N; ++j) {
    const int64_t i = static_cast<int64_t>(c) * N + j;
    if (i < vocab && __builtin_fmaf(x[j], cT, noise_at(key, static_cast<uint32_t>(i))) == best)
      return static_cast<int32_t>(i);
  }
  return static_cast<int32_t>(static_cast<int64_t>(c) * N);
}

template <bool BF16>
__device__ void finalize_row(const VerifyLaunch &p, int64_t r, const Totals &t) {
  const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) +
                                                    r * p.ld * (BF16 ? 2 : 4));
  const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) +
                                                    r * p.ld * (BF16 ? 2 : 4));
  const double l2v = log2(t.S_v), l2d = log2(t.S_d);
  const double lse_v = kLn2 * (t.rho_v + l2v);
  const double lse_d = kLn2 * (t.rho_d + l2d);
  double kl = t.D_v / t.S_v - kLn2 * ((t.rho_v - t.rho_d) + (l2v - l2d));
  double ent = kLn2 * (l2v - t.W_v / t.S_v);
  double conf = exp2(static_cast<double>(t.m_v) * static_cast<double>(kLog2e) - t.rho_v) / t.S_v;
  kl = kl < 0.0 ? 0.0 : kl;
  ent = ent < 0.0 ? 0.0 : ent;
  conf = conf > 1.0 ? 1.0 : conf;
  const dv_row_stats &o = p.out;
  if (o.lse_v) o.lse_v[r] = static_cast<float>(lse_v);
  if (o.lse_d) o.lse_d[r] = static_cast<float>(lse_d);
  if (o.kl) o.kl[r] = static_cast<float>(kl);
  if (o.entropy) o.entropy[r] = static_cast<float>(ent);
  if (o.conf) o.conf[r] = static_cast<float>(conf);
  const bool want_am = o.argmax_v || o.argmax_d || (p.greedy && (o.tok_v || o.tok_d));
  int32_t am_v = 0, am_d = 0;
  if (want_am) {
    am_v = refine_max<BF16>(ra, t.cm_v, t.m_v, p.vocab);
    am_d = refine_max<BF16>(rb, t.cm_d, t.m_d, p.vocab);
  }
  if (o.argmax_v) o.argmax_v[r] = am_v;
  if (o.argmax_d) o.argmax_d[r] = am_d;
  if (o.tok_v || o.tok_d) {
    if (p.greedy) {
      if (o.tok_v) o.tok_v[r] = am_v;
      if (o.tok_d) o.tok_d[r] = am_d;
    } else {
      const uint32_t key = row_key(p.seed_b, position_of(p, r));
      if (o.tok_v) o.tok_v[r] = refine_score<BF16>(ra, t.cs_v, t.s_v, p.vocab, p.cT, key);
      if (o.tok_d) o.tok_d[r] = refine_score<BF16>(rb, t.cs_d, t.s_d, p.vocab, p.cT, key);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void row_geometry(const VerifyLaunch &p, int32_t &nfull, int &nvalid_tail, int32_t &nch) {
  constexpr int N = Chunk<BF16>::N;
  nfull = static_cast<int32_t>(p.vocab / N);
  nvalid_tail = static_cast<int>(p.vocab % N);
  nch = nfull + (nvalid_tail ? 1 : 0);
}

// One wave per (row, slice); noise per row in registers, or none when greedy.
template <bool BF16, int MODE>
__global__ __launch_bounds__(256) void verify_rows_kernel(VerifyLaunch p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + wave;
  if (task >= p.rows * p.split) return;
  const int64_t r = task / p.split;
  const int32_t s = static_cast<int32_t>(task % p.split);
  int32_t nfull, nch;
  int nvalid_tail;
  row_geometry<BF16>(p, nfull, nvalid_tail, nch);
  const int32_t c0 = s * p.slice_chunks;
  const int32_t c1 = min(c0 + p.slice_chunks, nch);
  const size_t row_bytes = static_cast<size_t>(p.ld) * (BF16 ? 2 : 4);
  const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) + r * row_bytes);
  const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) + r * row_bytes);
  const uint32_t key = MODE == kInline ? row_key(p.seed_b, position_of(p, r)) : 0u;
  Lane st;
  st.init();
  scan_slice<BF16, MODE>(st, ra, rb, c0, c1, nfull, nvalid_tail, p.cT, key, nullptr, lane);
  const Partial t = wave_reduce(st);
  if (lane == 0) {
    if (p.split == 1) {
      finalize_row<BF16>(p, r, totals_of(t));
    } else {
      p.ws[r * p.split + s] = t;
    }
  }
}

// One workgroup per (position group, slice): the noise of the slice is
// computed once into LDS, then the waves stream every row at that position.
// Rows of group q are q, q + P, q + 2P, ... (P = pos_period).
template <bool BF16>
__global__ __launch_bounds__(512) void verify_shared_kernel(VerifyLaunch p) {
  extern __shared__ float g_lds[];
  constexpr int N = Chunk<BF16>::N;
  const int64_t P = p.pos_period;
  const int64_t grp = blockIdx.x / p.split;
  const int32_t s = static_cast<int32_t>(blockIdx.x % p.split);
  int32_t nfull, nch;
  int nvalid_tail;
  row_geometry<BF16>(p, nfull, nvalid_tail, nch);
  const int32_t c0 = s * p.slice_chunks;
  const int32_t c1 = min(c0 + p.slice_chunks, nch);
  const uint32_t key = row_key(p.seed_b, static_cast<int32_t>(grp));
  const int n = (c1 > c0 ? c1 - c0 : 0) * N;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int64_t i = static_cast<int64_t>(c0) * N + idx;
    g_lds[idx] = i < p.vocab ? noise_at(key, static_cast<uint32_t>(i)) : 0.0f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int64_t nq = (p.rows - grp + P - 1) / P;
  const size_t row_bytes = static_cast<size_t>(p.ld) * (BF16 ? 2 : 4);
  for (int64_t q = wave; q < nq; q += nw) {
    const int64_t r = grp + q * P;
    const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) + r * row_bytes);
    const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) + r * row_bytes);
    Lane st;
    st.init();
    scan_slice<BF16, kShared>(st, ra, rb, c0, c1, nfull, nvalid_tail, p.cT, key, g_lds, lane);
    const Partial t = wave_reduce(st);
    if (lane == 0) {
      if (p.split == 1) {
        finalize_row<BF16>(p, r, totals_of(t));
      } else {
        p.ws[r * p.split + s] = t;
      }
    }
  }
}

// Combine the split partials of each row (double precision) and finish it.
template <bool BF16>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyLaunch p) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= p.rows) return;
  const Partial *w = p.ws + r * p.split;
  double Rv = -INFINITY, Rd = -INFINITY;
  for (int s = 0; s < p.split; ++s) {
    if (w[s].S_v > 0.0f) Rv = fmax(Rv, static_cast<double>(w[s].rho_v));
    if (w[s].S_d > 0.0f) Rd = fmax(Rd, static_cast<double>(w[s].rho_d));
  }
  Totals t;
  t.rho_v = Rv;
  t.rho_d = Rd;
  t.S_v = t.W_v = t.D_v = t.S_d = 0.0;
  t.m_v = t.m_d = t.s_v = t.s_d = -INFINITY;
  t.cm_v = t.cm_d = t.cs_v = t.cs_d = INT_MAX;
  for (int s = 0; s < p.split; ++s) {
    const Partial &x = w[s];
    if (x.S_v > 0.0f) {
      const double d = static_cast<double>(x.rho_v) - Rv;
      const double sc = exp2(d);
      t.S_v += sc * x.S_v;
      t.W_v += sc * (static_cast<double>(x.W_v) + d * x.S_v);
      t.D_v += sc * x.D_v;
    }
    if (x.S_d > 0.0f) t.S_d += exp2(static_cast<double>(x.rho_d) - Rd) * x.S_d;
    // slices are in increasing chunk order, so the first strict improvement
    // keeps the lowest chunk among equal values
    if (x.m_v > t.m_v) { t.m_v = x.m_v; t.cm_v = x.cm_v; }
    if (x.m_d > t.m_d) { t.m_d = x.m_d; t.cm_d = x.cm_d; }
    if (x.s_v > t.s_v) { t.s_v = x.s_v; t.cs_v = x.cs_v; }
    if (x.s_d > t.s_d) { t.s_d = x.s_d; t.cs_d = x.cs_d; }
  }
  finalize_row<BF16>(p, r, t);
}

template <bool BF16>
hipError_t launch_typed(const VerifyLaunch &p, hipStream_t stream) {
  constexpr int N = Chunk<BF16>::N;
  if (p.shared) {
    const int64_t groups = p.pos_period < p.rows ? p.pos_period : p.rows;
    const size_t lds = static_cast<size_t>(p.slice_chunks) * N * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&verify_shared_kernel<BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(verify_shared_kernel<BF16>, dim3(static_cast<unsigned>(groups * p.split)),
                       dim3(p.block), lds, stream, p);
  } else {
    const int64_t waves = p.rows * p.split;
    const int wpb = 256 / 64;
    const unsigned blocks = static_cast<unsigned>((waves + wpb - 1) / wpb);
    if (p.greedy) {
      hipLaunchKernelGGL((verify_rows_kernel<BF16, kGreedy>), dim3(blocks), dim3(256), 0, stream, p);
    } else {
      hipLaunchKernelGGL((verify_rows_kernel<BF16, kInline>), dim3(blocks), dim3(256), 0, stream, p);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split == 1) return e;
  const unsigned mblocks = static_cast<unsigned>((p.rows + 255) / 256);
  hipLaunchKernelGGL(verify_merge_kernel<BF16>, dim3(mblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyLaunch &p, hipStream_t stream) {
  return p.bf16 ? launch_typed<true>(p, stream) : launch_typed<false>(p, stream);
}

}  // namespace dv
