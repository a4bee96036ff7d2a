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
// Design (a streaming reduction with no matrix-core work; at T > 0 its VALU
// load is as large as its HBM traffic, so both are budgeted):
//   * a wavefront owns a (row, vocabulary slice); each lane reads 16-byte
//     chunks (8 bf16 or 4 fp32) of both rows with non-temporal loads, the
//     lanes of a wave covering 1 KiB of contiguous memory per load, and keeps
//     the next chunks' loads in flight in a second register set;
//   * sums of exponentials are taken against a per-lane reference rho that is
//     only moved when a logit exceeds it by more than 64 (log2 units), so the
//     usual per-element online rescale disappears; the running maximum is
//     tracked separately, per chunk, for the argmax;
//   * KL and entropy come from the same pass: D = sum e_v (a - b) and
//     W = sum e_v t_v with t_v = a log2(e) - rho;
//   * argmax and Gumbel-max tokens are tracked per chunk (value, chunk index);
//     the lowest index inside the winning chunk is recovered at the end by
//     re-reading 16 bytes, so the hot loop carries no per-element index;
//   * noise comes from a counter hash. A chunk's Gumbel scores are only
//     computed when max(x)/T + max(noise) reaches the best score the wave has
//     seen; the largest noise value of a chunk comes from the largest of its
//     hash words (two logarithms per chunk instead of two per element) or,
//     when rows share positions (the candidates of a tree level), from a table
//     built once per (position, chunk). Chunks that pass are queued in LDS
//     with their logits and scored 64 at a time, one per lane;
//   * lane states are combined across the wave with DPP; the vocabulary
//     slices of a row are waves of one workgroup, combined through LDS.
#include <climits>
#include <cmath>

#include "dv_internal.h"

namespace dv {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
static_assert(__builtin_bit_cast(uint32_t, kLog2e) == 0x3fb8aa3bu, "fma_log2e encodes log2(e) as this literal");
constexpr double kLn2 = 0.693147180559945309417232121458;
constexpr float kRebase = 64.0f;                                   // log2 units
constexpr float kOneMinusHalfUlp = 0.999999940395355224609375f;  // 1 - 2^-24

// Noise modes of the streaming kernel. With noise, a chunk is scored only when
// a bound on its best perturbed score reaches the best score seen so far; the
// bound's noise term is the largest noise value of the chunk, taken
//   kHashBound:  from the chunk's hash words, in registers (rows with their
//                own noise);
//   kTableBound: from a table built once per position (rows sharing noise).
enum { kGreedy = 0,      // T = 0: tokens are the argmaxes, no noise
       kHashBound = 1,
       kTableBound = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Chunk {
  static constexpr int N = BF16 ? 8 : 4;  // elements per 16-byte chunk
};

// A slice of a row as a buffer resource: loads address it with a 32-bit byte
// offset from a base held in scalar registers (one VALU operation per load
// instead of a 64-bit address), and a load at or past `bytes` returns zeros
// without touching memory. The third word is the gfx9 buffer format (raw
// 32-bit data).
constexpr int kBufferFormat = 0x00020000;
constexpr int kLoadNontemporal = 2;  // the nt bit of a buffer load's cache policy
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kBufferFormat);
}
__device__ __forceinline__ u32x4 load_stream_at(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNontemporal);
}

// Logits that may hold -inf (masked vocabulary entries): every value at or
// below -2^100, -inf included, is raised to -2^100 on the raw bits, before any
// arithmetic. Such an entry keeps probability 0 (its exponential underflows)
// while products like 0 * (x - rho) stay finite, and because -2^100 times
// log2(e) is exact in float, a reference taken at that value reproduces it
// exactly in the fused multiply-adds. Negative values order by their unsigned
// bit patterns in reverse, so an unsigned minimum does it: per 16-bit half
// for bf16 (0xF180), per word for fp32 (0xF1800000).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ u32x4 clamp_neg(u32x4 w) {
  // the words are copied out of the vector first: a bit cast takes whole
  // objects, not vector elements
  uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      const u16x2 lim = {0xF180u, 0xF180u};
      const u16x2 h = __builtin_bit_cast(u16x2, e[i]);
      e[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(h, lim));
    } else {
      e[i] = min(e[i], 0xF1800000u);
    }
  }
  return u32x4{e[0], e[1], e[2], e[3]};
}

// A plain read of a chunk (the tail chunk, the argmax refinement); with EXT
// the -inf clamp is applied, as to the streaming reads, so every later
// comparison sees the same values.
template <bool BF16, bool EXT>
__device__ __forceinline__ u32x4 read_chunk(const u32x4 *p) {
  const u32x4 w = *p;
  return EXT ? clamp_neg<BF16>(w) : w;
}

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

// The noise of a row is drawn in groups of kNoiseGroup = 8 consecutive vocabulary indices,
// largest first: a full group's maximum, G_max = -log2(-log2(u_max) / 8) (the law of the
// largest of 8 independent Gumbels), sits at place w & 7 of its group word w; every other
// index takes the Gumbel truncated below that maximum at its own uniform u,
// G = -log2(-(log2 u + log2(u_max) / 8)). Together these are 8 independent Gumbels. A partial
// last group draws each index on its own. The key pair of a row: kw for the index words, kg
// for the group words.
struct NoiseKey {
  uint32_t kw, kg;
};

__device__ __forceinline__ NoiseKey noise_key(uint32_t kw) { return NoiseKey{kw, mix32(kw ^ kGroupSalt)}; }

// uniform of a hash word: 23 bits as the mantissa of a float in [1, 2), minus 1 - 2^-24 (exact)
__device__ __forceinline__ float uniform_of(uint32_t h) {
  return __uint_as_float(0x3F800000u | (h >> 9)) - kOneMinusHalfUlp;
}

// log2(u_max) / 8 of a group word (exact scaling of the hardware log2)
__device__ __forceinline__ float group_lm8(uint32_t w) { return __builtin_amdgcn_logf(uniform_of(w)) * 0.125f; }
__device__ __forceinline__ float group_max_g(float lm8) { return -__builtin_amdgcn_logf(-lm8); }
__device__ __forceinline__ float truncated_g(uint32_t h, float lm8) {
  return -__builtin_amdgcn_logf(-(__builtin_amdgcn_logf(uniform_of(h)) + lm8));
}
__device__ __forceinline__ bool full_group(uint32_t grp, int64_t vocab) {
  return (static_cast<int64_t>(grp) + 1) * kNoiseGroup <= vocab;
}

// The noise of vocabulary index i, computed exactly as noise_chunk computes it.
__device__ __forceinline__ float noise_at(const NoiseKey &k, uint32_t i, int64_t vocab) {
  const uint32_t grp = i / kNoiseGroup;
  if (!full_group(grp, vocab)) return gumbel_log2(mix32(k.kw ^ (i * kIndexStep)));
  const uint32_t w = mix32(k.kg ^ (grp * kIndexStep));
  const float lm8 = group_lm8(w);
  if ((i & (kNoiseGroup - 1)) == (w & (kNoiseGroup - 1))) return group_max_g(lm8);
  return truncated_g(mix32(k.kw ^ (i * kIndexStep)), lm8);
}

__device__ __forceinline__ int32_t position_of(const VerifyLaunch &p, int64_t r) {
  if (p.pos) return p.pos[r];
  if (p.pos_period > 0) return static_cast<int32_t>(r % p.pos_period);
  return static_cast<int32_t>(r);
}

// x * log2(e) + c with one rounding, as v_fmamk_f32: on gfx950 the VOP2 form
// with a literal and VGPR operands issues in half the cycles of v_fma_f32,
// which the compiler picks once it has moved the constant into an SGPR.
__device__ __forceinline__ float fma_log2e(float x, float c) {
  float r;
  asm("v_fmamk_f32 %0, %1, 0x3fb8aa3b, %2" : "=v"(r) : "v"(x), "v"(c));
  return r;
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

// The noise of the N elements of chunk c (one group word per chunk: a chunk never spans two
// groups, since N divides the group size).
template <bool BF16>
__device__ __forceinline__ void noise_chunk(float (&g)[Chunk<BF16>::N], int32_t c, const NoiseKey &k, int64_t vocab) {
  constexpr int N = Chunk<BF16>::N;
  static_assert(kNoiseGroup % N == 0, "a chunk lies inside one noise group");
  const uint32_t i0 = static_cast<uint32_t>(c) * N;
  const uint32_t grp = i0 / kNoiseGroup;
  if (full_group(grp, vocab)) {
    const uint32_t w = mix32(k.kg ^ (grp * kIndexStep));
    const float lm8 = group_lm8(w);
    const float gmax = group_max_g(lm8);
    const uint32_t js = w & (kNoiseGroup - 1);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t i = i0 + j;
      g[j] = (i & (kNoiseGroup - 1)) == js ? gmax : truncated_g(mix32(k.kw ^ (i * kIndexStep)), lm8);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) g[j] = gumbel_log2(mix32(k.kw ^ ((i0 + j) * kIndexStep)));
  }
}

// Upper bound of the noise of chunk c: u, and with it G, grows with the hash
// word, so the largest word of the chunk gives its largest noise value. The
// slack covers a hardware log2 that is not exactly monotone (1 ulp), so the
// bound is never below a noise value the scoring recomputes.
__device__ __forceinline__ float noise_bound_of_word(uint32_t hmax) {
  const float g = gumbel_log2(hmax);
  return g + __builtin_fabsf(g) * 0x1p-20f + 0x1p-20f;
}

// The row key as a per-lane value: VOP2 operations that read an SGPR issue at
// the VOP3 rate on gfx950, so the hash's xor with the key is cheaper from a VGPR.
__device__ __forceinline__ uint32_t key_in_vgpr(uint32_t key) {
  asm volatile("" : "+v"(key));
  return key;
}

// Upper bound of the noise of chunk c (every element valid). In a full group it is the
// group's maximum itself, from one hash word, plus the slack that covers a hardware log2
// that is not exactly monotone. In a partial group the bound needs only an upper bound of
// the chunk's largest index word: the last step of the hash keeps a word's top 16 bits, so
// the largest word before that step, with its low 16 bits set, is one.
__device__ __forceinline__ float with_slack(float g) { return g + __builtin_fabsf(g) * 0x1p-20f + 0x1p-20f; }

template <int N>
__device__ __forceinline__ float chunk_noise_bound(int32_t c, const NoiseKey &k, int64_t vocab) {
  const uint32_t i0 = static_cast<uint32_t>(c) * N;
  const uint32_t grp = i0 / kNoiseGroup;
  if (full_group(grp, vocab)) return with_slack(group_max_g(group_lm8(mix32(k.kg ^ (grp * kIndexStep)))));
  uint32_t hm = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) hm = max(hm, mix32_head(k.kw ^ ((i0 + j) * kIndexStep)));
  return noise_bound_of_word(hm | 0xFFFFu);
}

// Per-lane accumulator of one (row, slice).
struct Lane {
  float rho_v, S_v, S_v2, W_v, D_v, thr_v;  // S_v + S_v2: even / odd elements (independent add chains)
  float rho_d, S_d, S_d2, thr_d, D_d;  // D_d = sum e_d (a - b): the reverse divergence (extended pass only)
  float m_v, m_d, s_v, s_d;
  int32_t cm_v, cm_d, cs_v, cs_d;
  float wb_v, wb_d;  // wave-wide lower bounds of the best perturbed scores (equal in all lanes)

  __device__ __forceinline__ void init() {
    wb_v = wb_d = -INFINITY;
    rho_v = rho_d = -INFINITY;
    thr_v = thr_d = -INFINITY;
    S_v = S_v2 = W_v = D_v = S_d = S_d2 = D_d = 0.0f;
    m_v = m_d = s_v = s_d = -INFINITY;
    cm_v = cm_d = cs_v = cs_d = INT_MAX;
  }
};

// ---- cross-lane combination ----
// Wave64 reductions with DPP moves (VALU, no LDS round trips): an inclusive
// scan inside each row of 16 lanes (row_shr 1, 2, 4, 8), then row_bcast:15
// and row_bcast:31 carry the row totals up, so lane 63 ends with the result,
// which readlane broadcasts to the whole wave.
enum : int { kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118, kRowBcast15 = 0x142,
             kRowBcast31 = 0x143 };

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float identity, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x), CTRL, ROW_MASK,
                                                    0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_i(int32_t identity, int32_t x) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kRowShr1, 0xF>(0.0f, x);
  x += dpp_f<kRowShr2, 0xF>(0.0f, x);
  x += dpp_f<kRowShr4, 0xF>(0.0f, x);
  x += dpp_f<kRowShr8, 0xF>(0.0f, x);
  x += dpp_f<kRowBcast15, 0xA>(0.0f, x);
  x += dpp_f<kRowBcast31, 0xC>(0.0f, x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kRowShr1, 0xF>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kRowShr2, 0xF>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kRowShr4, 0xF>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kRowShr8, 0xF>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kRowBcast15, 0xA>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kRowBcast31, 0xC>(-INFINITY, x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ int32_t wave_min_i(int32_t x) {
  x = min(x, dpp_i<kRowShr1, 0xF>(INT_MAX, x));
  x = min(x, dpp_i<kRowShr2, 0xF>(INT_MAX, x));
  x = min(x, dpp_i<kRowShr4, 0xF>(INT_MAX, x));
  x = min(x, dpp_i<kRowShr8, 0xF>(INT_MAX, x));
  x = min(x, dpp_i<kRowBcast15, 0xA>(INT_MAX, x));
  x = min(x, dpp_i<kRowBcast31, 0xC>(INT_MAX, x));
  return __builtin_amdgcn_readlane(x, 63);
}
// (value, chunk): largest value, lowest chunk among equal values
__device__ __forceinline__ void wave_argmax(float &m, int32_t &c) {
  const float M = wave_max(m);
  c = wave_min_i(m == M ? c : INT_MAX);
  m = M;
}

// Move the reference to x * log2(e) and rescale what was accumulated so far.
__device__ __forceinline__ void rebase_v(Lane &st, float x) {
  const float nr = x * kLog2e;
  const float S = st.S_v + st.S_v2;
  if (S > 0.0f) {
    const float d = st.rho_v - nr;  // <= 0
    const float sc = __builtin_amdgcn_exp2f(d);
    st.W_v = sc * __builtin_fmaf(d, S, st.W_v);
    st.S_v *= sc;
    st.S_v2 *= sc;
    st.D_v *= sc;
  } else {
    st.S_v = st.S_v2 = st.W_v = st.D_v = 0.0f;
  }
  st.rho_v = nr;
  st.thr_v = (nr + kRebase) * (1.0f / kLog2e);
}

__device__ __forceinline__ void rebase_d(Lane &st, float x) {
  const float nr = x * kLog2e;
  if (st.S_d + st.S_d2 > 0.0f) {
    const float sc = __builtin_amdgcn_exp2f(st.rho_d - nr);
    st.S_d *= sc;
    st.S_d2 *= sc;
    st.D_d *= sc;
  } else {
    st.S_d = st.S_d2 = st.D_d = 0.0f;
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

// Gumbel-max bookkeeping of one chunk: best perturbed score of each model.
// ANY_ORDER: chunks may arrive out of index order (queued scoring), so equal
// scores must compare chunk indices explicitly.
template <int N, bool MASKED, bool ANY_ORDER>
__device__ __forceinline__ void fold_tokens(Lane &st, const float (&a)[N], const float (&b)[N], const float (&g)[N],
                                            int32_t c, float cT, int nvalid) {
  float csa = -INFINITY, csb = -INFINITY;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float pa = __builtin_fmaf(a[j], cT, g[j]);
    float pb = __builtin_fmaf(b[j], cT, g[j]);
    if constexpr (MASKED) {
      if (j >= nvalid) {
        pa = -INFINITY;
        pb = -INFINITY;
      }
    }
    csa = fmaxf(csa, pa);
    csb = fmaxf(csb, pb);
  }
  if (csa > st.s_v || (ANY_ORDER && csa == st.s_v && c < st.cs_v)) {
    st.s_v = csa;
    st.cs_v = c;
  }
  if (csb > st.s_d || (ANY_ORDER && csb == st.s_d && c < st.cs_d)) {
    st.s_d = csb;
    st.cs_d = c;
  }
}

// Fold the statistics of one chunk (N logits of each model) into the lane
// state and return the chunk maxima of both rows in cma / cmb. MASKED: only
// the first nvalid elements are logits (last chunk of a row). One pass over
// the elements with running accumulators keeps few temporaries live.
template <int N, bool MASKED, bool EXT>
__device__ __forceinline__ void fold_stats(Lane &st, float (&a)[N], float (&b)[N], int32_t c, int nvalid, float &cma,
                                           float &cmb) {
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

  const float nrv = -st.rho_v, nrd = -st.rho_d;
  float W = st.W_v, D = st.D_v, Dd = st.D_d;
  float sv0 = st.S_v, sv1 = st.S_v2, sd0 = st.S_d, sd1 = st.S_d2;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float tv = fma_log2e(a[j], nrv);
    const float td = fma_log2e(b[j], nrd);
    float e = __builtin_amdgcn_exp2f(tv);
    float f = __builtin_amdgcn_exp2f(td);
    if constexpr (MASKED) {
      if (j >= nvalid) {
        e = 0.0f;
        f = 0.0f;
      }
    }
    if (j & 1) {
      sv1 += e;
      sd1 += f;
    } else {
      sv0 += e;
      sd0 += f;
    }
    W = __builtin_fmaf(e, tv, W);
    const float dab = a[j] - b[j];
    D = __builtin_fmaf(e, dab, D);
    if constexpr (EXT) Dd = __builtin_fmaf(f, dab, Dd);
  }
  st.W_v = W;
  st.D_v = D;
  if constexpr (EXT) st.D_d = Dd;
  st.S_v = sv0;
  st.S_v2 = sv1;
  st.S_d = sd0;
  st.S_d2 = sd1;
}

// One chunk, statistics and (unless greedy) tokens with noise from the hash.
// Chunks reach the token bookkeeping out of index order (queued scoring), so
// ties compare chunk indices.
template <bool BF16, int MODE, bool MASKED, bool EXT>
__device__ __forceinline__ void fold_chunk(Lane &st, const u32x4 &wa, const u32x4 &wb, int32_t c, const NoiseKey &key,
                                           int64_t vocab, float cT, int nvalid) {
  constexpr int N = Chunk<BF16>::N;
  float x[N], y[N], cma, cmb;
  widen<BF16>(wa, x);
  widen<BF16>(wb, y);
  fold_stats<N, MASKED, EXT>(st, x, y, c, nvalid, cma, cmb);
  if constexpr (MODE != kGreedy) {
    float g[N];
    noise_chunk<BF16>(g, c, key, vocab);
    fold_tokens<N, MASKED, true>(st, x, y, g, c, cT, nvalid);
  }
}

// Chunks whose bound did not rule them out, waiting to be scored: their
// index and raw logits. One queue per wave, in LDS.
struct ScoreQueue {
  int32_t c[64];
  u32x4 a[64], b[64];
};

// Score the queued chunks, one per lane, and raise the wave's bounds.
template <bool BF16>
__device__ __forceinline__ void flush_queue(Lane &st, ScoreQueue &q, int n, const NoiseKey &key, int64_t vocab, float cT,
                                            int lane) {
  constexpr int N = Chunk<BF16>::N;
  __builtin_amdgcn_wave_barrier();  // lanes read entries other lanes of the wave wrote
  if (lane < n) {
    const int32_t c = q.c[lane];
    float x[N], y[N], g[N];
    widen<BF16>(q.a[lane], x);
    widen<BF16>(q.b[lane], y);
    noise_chunk<BF16>(g, c, key, vocab);
    fold_tokens<N, false, true>(st, x, y, g, c, cT, N);
  }
  st.wb_v = wave_max(st.s_v);
  st.wb_d = wave_max(st.s_d);
  __builtin_amdgcn_wave_barrier();  // the entries are rewritten only after every lane read its own
}

#ifndef DV_STEP_CHUNKS
#define DV_STEP_CHUNKS 2
#endif
constexpr int kStep = DV_STEP_CHUNKS;  // chunks per lane per step of the streaming loop

// Raw registers of K chunks (c, c + 64, ..., c + 64 (K-1)) of both matrices
// and, with a noise table, the largest noise value of each chunk.
template <bool BF16, bool PRUNE, int K, bool EXT>
struct StepRegs {
  u32x4 a[K], b[K];
  float gm[K];

  // The chunks at offsets o, o + 64, ... (in chunks, from the start of the slice) of both rows
  // and of the noise table; past the end of the slice the buffers return zeros (not used).
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rg,
                                       int32_t o) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t off = static_cast<uint32_t>(o + 64 * k) * 16u;
      a[k] = load_stream_at(ra, off);
      b[k] = load_stream_at(rb, off);
      if constexpr (EXT) {
        a[k] = clamp_neg<BF16>(a[k]);
        b[k] = clamp_neg<BF16>(b[k]);
      }
      if constexpr (PRUNE) gm[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off / 4u, 0, 0));
    }
  }

  // Fold the K chunks in; chunk k exists only when c + 64 k < cend (lanes past
  // the end of the slice ran the step with the others but fold nothing). The
  // loaded registers are first read on every path (an empty asm that takes
  // them as inputs): were they read only inside the per-lane branch, the
  // compiler could not rule out a path on which a load is still in flight at
  // the loop's back edge, and would drain every load in flight there. The
  // queue operations are wave-wide, so every lane must reach them.
  template <int MODE>
  __device__ __forceinline__ void fold(Lane &st, int32_t c, int32_t cend, const NoiseKey &key, int64_t vocab, float cT,
                                       ScoreQueue *q, int &nq, int lane) const {
    constexpr int N = Chunk<BF16>::N;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      asm volatile("" ::"v"(a[k]), "v"(b[k]));
      if constexpr (PRUNE) asm volatile("" ::"v"(gm[k]));
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t ck = c + 64 * k;
      const bool valid = ck < cend;
      if constexpr (MODE != kGreedy) {
        // A chunk can hold a model's Gumbel-max token only if the bound
        // max(x)/T + max(noise) reaches the best score the wave has already
        // seen (fma is monotone, so the bound holds for the rounded scores;
        // >= keeps chunks that could tie). Those are queued.
        bool need = false;
        if (valid) {
          float x[N], y[N], cma, cmb;
          widen<BF16>(a[k], x);
          widen<BF16>(b[k], y);
          fold_stats<N, false, EXT>(st, x, y, ck, N, cma, cmb);
          const float g = MODE == kTableBound ? gm[k] : chunk_noise_bound<N>(ck, key, vocab);
          need = __builtin_fmaf(cma, cT, g) >= st.wb_v || __builtin_fmaf(cmb, cT, g) >= st.wb_d;
        }
        const unsigned long long mask = __ballot(need);
        if (mask) {
          const int cnt = __popcll(mask);
          if (nq + cnt > 64) {
            flush_queue<BF16>(st, *q, nq, key, vocab, cT, lane);
            nq = 0;
          }
          if (need) {
            const int slot = nq + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
            q->c[slot] = ck;
            q->a[slot] = a[k];
            q->b[slot] = b[k];
          }
          nq += cnt;
        }
      } else {
        if (valid) fold_chunk<BF16, kGreedy, false, EXT>(st, a[k], b[k], ck, key, vocab, cT, N);
      }
    }
  }
};

// Stream chunks [c0, c1) of one row pair through the lanes of a wave. Lane l
// takes chunks c0 + l, c0 + l + 64, ...; the loop runs the same number of
// steps in every lane (lanes past the end of the slice load a valid chunk and
// fold nothing), so wave-wide operations inside it see all lanes. Two register
// sets, X and Y, work in ping-pong: while one step of chunks is folded in, the
// loads of the next step land in the other set. The next loads are issued on
// every path (past the end of the slice the buffer returns zeros without a
// memory access), so the wait counts never have to cover a path without them
// and no register copy forces a wait at the back edge. The scheduling barrier
// after each step's loads keeps them ahead of the arithmetic on the other set:
// without it the compiler starts unpacking the set that is due before the next
// loads are issued, and the wave waits for its data with one step of loads in
// flight instead of two.
template <bool BF16, int MODE, bool EXT>
__device__ __forceinline__ void scan_slice(Lane &st, const u32x4 *ra, const u32x4 *rb, int32_t c0, int32_t c1,
                                           int32_t nfull, int nvalid_tail, float cT, const NoiseKey &key, int64_t vocab,
                                           const float *g_cmax, ScoreQueue *q, int lane) {
  constexpr int32_t kSpan = 64 * kStep;
  const int32_t cend = c1 < nfull ? c1 : nfull;  // whole chunks of the slice
  const int32_t nsteps = cend > c0 ? (cend - c0 + kSpan - 1) / kSpan : 0;
  int nq = 0;
  if (nsteps > 0) {
    // the slice's whole chunks as buffers: chunks past the end read as zeros and are not folded
    const uint32_t nbytes = static_cast<uint32_t>(cend - c0) * 16u;
    const __amdgpu_buffer_rsrc_t ba = slice_rsrc(ra + c0, nbytes), bb = slice_rsrc(rb + c0, nbytes);
    const __amdgpu_buffer_rsrc_t bg = slice_rsrc(MODE == kTableBound ? g_cmax + c0 : nullptr,
                                                 MODE == kTableBound ? nbytes / 4u : 0u);
    StepRegs<BF16, MODE == kTableBound, kStep, EXT> X, Y;
    int32_t c = c0 + lane;
    X.load(ba, bb, bg, c - c0);
    for (int32_t t = 0;;) {
      Y.load(ba, bb, bg, c + kSpan - c0);
      __builtin_amdgcn_sched_barrier(0);
      X.template fold<MODE>(st, c, cend, key, vocab, cT, q, nq, lane);
      if (++t == nsteps) break;
      c += kSpan;
      X.load(ba, bb, bg, c + kSpan - c0);
      __builtin_amdgcn_sched_barrier(0);
      Y.template fold<MODE>(st, c, cend, key, vocab, cT, q, nq, lane);
      if (++t == nsteps) break;
      c += kSpan;
    }
  }
  if constexpr (MODE != kGreedy) {
    if (nq > 0) flush_queue<BF16>(st, *q, nq, key, vocab, cT, lane);
  }
  // the last, partly filled chunk of the row (vocab not a multiple of N)
  if (nvalid_tail > 0 && nfull >= c0 && nfull < c1 && lane == ((nfull - c0) & 63))
    fold_chunk<BF16, MODE, true, EXT>(st, read_chunk<BF16, EXT>(ra + nfull), read_chunk<BF16, EXT>(rb + nfull), nfull, key,
                                      vocab, cT, nvalid_tail);
}

// Reduce the lane states of a wave into one partial (valid in every lane).
__device__ __forceinline__ Partial wave_reduce(const Lane &st) {
  Partial t;
  {
    const float R = wave_max(st.rho_v);
    const float S = st.S_v + st.S_v2;
    const bool has = S > 0.0f;
    const float d = has ? st.rho_v - R : 0.0f;
    const float sc = has ? __builtin_amdgcn_exp2f(d) : 0.0f;
    t.S_v = wave_sum(S * sc);
    t.W_v = wave_sum(sc * __builtin_fmaf(d, S, st.W_v));
    t.D_v = wave_sum(st.D_v * sc);
    t.rho_v = R;
  }
  {
    const float R = wave_max(st.rho_d);
    const float Sd = st.S_d + st.S_d2;
    const bool has = Sd > 0.0f;
    const float sc = has ? __builtin_amdgcn_exp2f(st.rho_d - R) : 0.0f;
    t.S_d = wave_sum(Sd * sc);
    t.D_d = wave_sum(st.D_d * sc);
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
  t.pad1 = 0;
  return t;
}

// ---- per-row epilogue (double precision) ----

// Lowest index inside chunk c of a row whose value equals target, found by the
// whole wave from the chunk's 16 bytes w (the same for every lane): lane j < N
// looks at element c*N + j. For scores the perturbed score is recomputed with
// exactly the arithmetic of the streaming pass. A chunk index outside the row
// (only possible when the logits hold NaN, which is not supported) gives -1.
template <bool BF16, bool SCORE>
__device__ __forceinline__ int32_t refine_in_chunk(const u32x4 &w, int32_t c, float target, int64_t vocab, float cT,
                                                   const NoiseKey &key, int lane) {
  constexpr int N = Chunk<BF16>::N;
  if (c < 0 || static_cast<int64_t>(c) * N >= vocab) return -1;
  float x[N];
  widen<BF16>(w, x);
  float v = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) v = (lane == j) ? x[j] : v;
  const int64_t i = static_cast<int64_t>(c) * N + lane;
  bool hit = false;
  if (lane < N && i < vocab) {
    if constexpr (SCORE) v = __builtin_fmaf(v, cT, noise_at(key, static_cast<uint32_t>(i), vocab));
    hit = v == target;
  }
  const unsigned long long m = __ballot(hit);
  return m ? static_cast<int32_t>(static_cast<int64_t>(c) * N + __ffsll(m) - 1) : -1;
}

// The 16 bytes of chunk c of a row (chunk 0 for an index outside the row, whose
// refinement gives -1 anyway), so that every chunk the epilogue needs can be
// requested before the first one is used.
template <bool BF16, bool EXT>
__device__ __forceinline__ u32x4 fetch_chunk(const u32x4 *row, int32_t c, int64_t vocab) {
  constexpr int N = Chunk<BF16>::N;
  const bool inside = c >= 0 && static_cast<int64_t>(c) * N < vocab;
  return read_chunk<BF16, EXT>(row + (inside ? c : 0));
}

// Row results from the reduced state of a whole row; every lane of the wave
// calls it (the refinements use the lanes), lane 0 writes.
template <bool BF16, bool EXT>
__device__ void finalize_row(const VerifyLaunch &p, int64_t r, const Partial &t, int lane) {
  constexpr int N = Chunk<BF16>::N;
  const size_t row_bytes = static_cast<size_t>(p.ld) * (BF16 ? 2 : 4);
  const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) + r * row_bytes);
  const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) + r * row_bytes);
  const dv_row_stats &o = p.out;
  const bool want_tok_d = o.tok_d || o.p_tok_d;
  const bool want_am = o.argmax_v || o.argmax_d || (p.greedy && (o.tok_v || want_tok_d));
  const bool want_tok = !p.greedy && (o.tok_v || want_tok_d);
  // every chunk the refinements read is requested before the first is used: one memory round trip, not four
  u32x4 wm_v{}, wm_d{}, ws_v{}, ws_d{};
  if (want_am) {
    wm_v = fetch_chunk<BF16, EXT>(ra, t.cm_v, p.vocab);
    wm_d = fetch_chunk<BF16, EXT>(rb, t.cm_d, p.vocab);
  }
  if (want_tok) {
    ws_v = fetch_chunk<BF16, EXT>(ra, t.cs_v, p.vocab);
    ws_d = fetch_chunk<BF16, EXT>(rb, t.cs_d, p.vocab);
  }
  int32_t am_v = 0, am_d = 0, tk_v = 0, tk_d = 0;
  if (want_am) {
    am_v = refine_in_chunk<BF16, false>(wm_v, t.cm_v, t.m_v, p.vocab, 0.0f, NoiseKey{0u, 0u}, lane);
    am_d = refine_in_chunk<BF16, false>(wm_d, t.cm_d, t.m_d, p.vocab, 0.0f, NoiseKey{0u, 0u}, lane);
  }
  if (o.tok_v || want_tok_d) {
    if (p.greedy) {
      tk_v = am_v;
      tk_d = am_d;
    } else {
      const NoiseKey key = noise_key(row_key(p.seed_b, position_of(p, r)));
      if (o.tok_v) tk_v = refine_in_chunk<BF16, true>(ws_v, t.cs_v, t.s_v, p.vocab, p.cT, key, lane);
      if (want_tok_d) tk_d = refine_in_chunk<BF16, true>(ws_d, t.cs_d, t.s_d, p.vocab, p.cT, key, lane);
    }
  }
  // the verifier's logit at the drafter's token
  float x_tok = 0.0f;
  if (o.p_tok_d && tk_d >= 0) {
    float x[N];
    widen<BF16>(read_chunk<BF16, EXT>(ra + tk_d / N), x);
    x_tok = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) x_tok = (tk_d % N == j) ? x[j] : x_tok;
  }
  if (lane != 0) return;
  const double S_v = t.S_v, S_d = t.S_d;
  const double l2v = log2(S_v), l2d = log2(S_d);
  const double rho_v = t.rho_v, rho_d = t.rho_d;
  const double lse_v = kLn2 * (rho_v + l2v);
  const double lse_d = kLn2 * (rho_d + l2d);
  double kl = static_cast<double>(t.D_v) / S_v - kLn2 * ((rho_v - rho_d) + (l2v - l2d));
  double ent = kLn2 * (l2v - static_cast<double>(t.W_v) / S_v);
  // the maximum's own term, computed as the streaming pass computed it for a
  // lane whose reference equals rho_v, so that a row with one dominant logit
  // gives conf == 1 exactly
  const float e_max = __builtin_amdgcn_exp2f(__builtin_fmaf(t.m_v, kLog2e, -t.rho_v));
  double conf = static_cast<double>(e_max) / S_v;
  kl = kl < 0.0 ? 0.0 : kl;
  ent = ent < 0.0 ? 0.0 : ent;
  conf = conf > 1.0 ? 1.0 : conf;
  if (p.neg_inf) {
    // a divergence this large only comes from mass where the other model
    // has a -inf logit (raised to -2^100): it is +inf
    if (kl >= 0x1p64) kl = INFINITY;
  }
  if (o.lse_v) o.lse_v[r] = static_cast<float>(lse_v);
  if (o.lse_d) o.lse_d[r] = static_cast<float>(lse_d);
  if (o.kl) o.kl[r] = static_cast<float>(kl);
  if (o.entropy) o.entropy[r] = static_cast<float>(ent);
  if (o.conf) o.conf[r] = static_cast<float>(conf);
  if (o.argmax_v) o.argmax_v[r] = am_v;
  if (o.argmax_d) o.argmax_d[r] = am_d;
  if (o.tok_v) o.tok_v[r] = tk_v;
  if (o.tok_d) o.tok_d[r] = tk_d;
  if constexpr (EXT) {
    if (o.kl_rev) {
      // KL(p_d || p_v) = sum p_d (b - a) - (lse_d - lse_v)
      double klr = -static_cast<double>(t.D_d) / S_d - kLn2 * ((rho_d - rho_v) + (l2d - l2v));
      klr = klr < 0.0 ? 0.0 : klr;
      if (p.neg_inf && klr >= 0x1p64) klr = INFINITY;
      o.kl_rev[r] = static_cast<float>(klr);
    }
  }
  if (o.p_tok_d) o.p_tok_d[r] = tk_d >= 0 ? static_cast<float>(exp(static_cast<double>(x_tok) - lse_v)) : 0.0f;
}

template <bool BF16>
__device__ __forceinline__ void row_geometry(const VerifyLaunch &p, int32_t &nfull, int &nvalid_tail, int32_t &nch) {
  constexpr int N = Chunk<BF16>::N;
  nfull = static_cast<int32_t>(p.vocab / N);
  nvalid_tail = static_cast<int>(p.vocab % N);
  nch = nfull + (nvalid_tail ? 1 : 0);
}

// Per-wave LDS of the streaming kernel: the score queue (with noise) and the
// reduced state handed to the first wave of the row (split rows).
struct WaveLds {
  ScoreQueue q;
  Partial part;
};

// One wave per (row, slice); the split slices of a row are consecutive waves
// of one workgroup and are combined through LDS by the row's first wave.
template <bool BF16, int MODE, bool EXT>
__global__ __launch_bounds__(1024) void verify_rows_kernel(VerifyLaunch p) {
  extern __shared__ WaveLds lds[];
  // the wave index is uniform across the wave: keep it (and all row
  // addressing derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int split = p.split;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * p.rows_per_block + wave / split;
  const int32_t s = wave % split;
  const bool live = r < p.rows;
  Lane st;
  st.init();
  if (live) {
    int32_t nfull, nch;
    int nvalid_tail;
    row_geometry<BF16>(p, nfull, nvalid_tail, nch);
    const int32_t c0 = s * p.slice_chunks;
    const int32_t c1 = min(c0 + p.slice_chunks, nch);
    const size_t row_bytes = static_cast<size_t>(p.ld) * (BF16 ? 2 : 4);
    const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) + r * row_bytes);
    const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) + r * row_bytes);
    const int32_t pos = MODE == kGreedy ? 0 : position_of(p, r);
    NoiseKey key = MODE == kGreedy ? NoiseKey{0u, 0u} : noise_key(row_key(p.seed_b, pos));
    if constexpr (MODE == kHashBound) key = NoiseKey{key_in_vgpr(key.kw), key_in_vgpr(key.kg)};
    const float *gcm = MODE == kTableBound ? p.noise_cmax + static_cast<int64_t>(pos) * p.cmax_ld : nullptr;
    scan_slice<BF16, MODE, EXT>(st, ra, rb, c0, c1, nfull, nvalid_tail, p.cT, key, p.vocab, gcm,
                           MODE == kGreedy ? nullptr : &lds[wave].q, lane);
  }
  const Partial t = wave_reduce(st);
  if (split == 1) {
    if (live) finalize_row<BF16, EXT>(p, r, t, lane);
    return;
  }
  if (lane == 0) lds[wave].part = t;
  __syncthreads();
  if (!live || s != 0) return;
  // lane l takes slice l of the row
  Lane m;
  m.init();
  if (lane < split) {
    const Partial x = lds[wave + lane].part;
    m.rho_v = x.rho_v;
    m.S_v = x.S_v;
    m.W_v = x.W_v;
    m.D_v = x.D_v;
    m.D_d = x.D_d;
    m.rho_d = x.rho_d;
    m.S_d = x.S_d;
    m.m_v = x.m_v;
    m.m_d = x.m_d;
    m.s_v = x.s_v;
    m.s_d = x.s_d;
    m.cm_v = x.cm_v;
    m.cm_d = x.cm_d;
    m.cs_v = x.cs_v;
    m.cs_d = x.cs_d;
  }
  finalize_row<BF16, EXT>(p, r, wave_reduce(m), lane);
}

// Chunk-max noise table: entry (q, c) bounds the noise of position q over the
// valid elements of chunk c, as chunk_noise_bound does in registers: a full
// group's maximum from its group word, or for the partial last group the largest
// index word without the hash's last step. Each thread fills kCmaxPerThread
// entries of one position, 256 apart, so that a launch has few workgroups.
// Entries number below 2^28 (the table is at most 1 GiB).
// Grid: x covers the chunks of a position, y the positions (strided past 65535), so
// the position's keys are uniform across the workgroup (scalar unit) and no thread divides.
constexpr uint32_t kCmaxPerThread = 4;

template <int N>
__global__ __launch_bounds__(256) void noise_cmax_kernel(uint32_t seed_b, uint32_t rows, uint32_t ld, int64_t vocab,
                                                        float *cmax) {
  for (uint32_t q = blockIdx.y; q < rows; q += gridDim.y) {
    const NoiseKey key = noise_key(row_key(seed_b, static_cast<int32_t>(q)));
#pragma unroll
    for (uint32_t k = 0; k < kCmaxPerThread; ++k) {
      const uint32_t c = (blockIdx.x * kCmaxPerThread + k) * 256u + threadIdx.x;
      if (c >= ld) break;
      const uint32_t grp = c * N / kNoiseGroup;  // vocab < 2^31
      float bound;
      if (full_group(grp, vocab)) {
        bound = with_slack(group_max_g(group_lm8(mix32(key.kg ^ (grp * kIndexStep)))));
      } else {
        uint32_t hm = 0;
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const uint32_t i = c * N + j;
          if (i < vocab) hm = max(hm, mix32_head(key.kw ^ (i * kIndexStep)));
        }
        bound = noise_bound_of_word(hm | 0xFFFFu);
      }
      cmax[static_cast<size_t>(q) * ld + c] = bound;
    }
  }
}

// Read-only streaming probe: the streaming kernel's access pattern (a wave per
// (row, slice) in the same launch shape, 16-byte non-temporal loads of both
// rows, kStep chunks per lane per step in two register sets) with no
// arithmetic but an xor fold. It measures the read rate this pattern can
// reach on the device, the ceiling of the verify pass. Each wave writes one
// word (the xor of everything it read) to sink[row * kMaxSplit + slice].
__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
  int32_t v = static_cast<int32_t>(x);
  v ^= dpp_i<kRowShr1, 0xF>(0, v);
  v ^= dpp_i<kRowShr2, 0xF>(0, v);
  v ^= dpp_i<kRowShr4, 0xF>(0, v);
  v ^= dpp_i<kRowShr8, 0xF>(0, v);
  v ^= dpp_i<kRowBcast15, 0xA>(0, v);
  v ^= dpp_i<kRowBcast31, 0xC>(0, v);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 63));
}

__global__ __launch_bounds__(1024) void read_probe_kernel(VerifyLaunch p, uint32_t *sink) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int split = p.split;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * p.rows_per_block + wave / split;
  const int32_t s = wave % split;
  if (r >= p.rows) return;
  const int32_t per = p.bf16 ? 8 : 4;
  const int32_t nch = static_cast<int32_t>((p.vocab + per - 1) / per);
  const int32_t c0 = s * p.slice_chunks;
  const int32_t c1 = min(c0 + p.slice_chunks, nch);
  const size_t row_bytes = static_cast<size_t>(p.ld) * (p.bf16 ? 2 : 4);
  const u32x4 *ra = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.va) + r * row_bytes);
  const u32x4 *rb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.vb) + r * row_bytes);
  constexpr int32_t kSpan = 64 * kStep;
  const int32_t nsteps = c1 > c0 ? (c1 - c0 + kSpan - 1) / kSpan : 0;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (nsteps > 0) {
    const uint32_t nbytes = static_cast<uint32_t>(c1 - c0) * 16u;
    const __amdgpu_buffer_rsrc_t ba = slice_rsrc(ra + c0, nbytes), bb = slice_rsrc(rb + c0, nbytes);
    u32x4 xa[kStep], xb[kStep], ya[kStep], yb[kStep];
    int32_t o = lane;
#pragma unroll
    for (int k = 0; k < kStep; ++k) {
      xa[k] = load_stream_at(ba, static_cast<uint32_t>(o + 64 * k) * 16u);
      xb[k] = load_stream_at(bb, static_cast<uint32_t>(o + 64 * k) * 16u);
    }
    for (int32_t t = 0;;) {
#pragma unroll
      for (int k = 0; k < kStep; ++k) {
        ya[k] = load_stream_at(ba, static_cast<uint32_t>(o + kSpan + 64 * k) * 16u);
        yb[k] = load_stream_at(bb, static_cast<uint32_t>(o + kSpan + 64 * k) * 16u);
      }
#pragma unroll
      for (int k = 0; k < kStep; ++k) acc ^= xa[k] ^ xb[k];
      if (++t == nsteps) break;
      o += kSpan;
#pragma unroll
      for (int k = 0; k < kStep; ++k) {
        xa[k] = load_stream_at(ba, static_cast<uint32_t>(o + kSpan + 64 * k) * 16u);
        xb[k] = load_stream_at(bb, static_cast<uint32_t>(o + kSpan + 64 * k) * 16u);
      }
#pragma unroll
      for (int k = 0; k < kStep; ++k) acc ^= ya[k] ^ yb[k];
      if (++t == nsteps) break;
      o += kSpan;
    }
  }
  const uint32_t x = wave_xor(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (lane == 0) sink[r * kMaxProbeSplit + s] = x;
}

// Test-only dump of the noise exactly as the kernels above derive it, so that
// it can be checked word for word: the index words, the group words, the
// Gumbel values in log2 units (noise_at), and the two per-chunk bounds the
// pruning uses (in registers, and the table). One thread per output entry of
// a row; rows on the grid's y dimension (strided past 65535).
template <int N>
__global__ __launch_bounds__(256) void debug_noise_kernel(uint32_t seed_b, const int32_t *pos, int64_t pos_period,
                                                         int64_t rows, int64_t vocab, int64_t width, int32_t what,
                                                         void *out) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int32_t ps = pos ? pos[r] : (pos_period > 0 ? static_cast<int32_t>(r % pos_period) : static_cast<int32_t>(r));
    const NoiseKey key = noise_key(row_key(seed_b, ps));
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < width;
         j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
      const int64_t o = r * width + j;
      const uint32_t i = static_cast<uint32_t>(j);
      switch (what) {
        case DV_DEBUG_INDEX_WORDS:
          static_cast<uint32_t *>(out)[o] = mix32(key.kw ^ (i * kIndexStep));
          break;
        case DV_DEBUG_GROUP_WORDS:
          static_cast<uint32_t *>(out)[o] = mix32(key.kg ^ (i * kIndexStep));
          break;
        case DV_DEBUG_NOISE_LOG2:
          static_cast<float *>(out)[o] = noise_at(key, i, vocab);
          break;
        case DV_DEBUG_CHUNK_BOUND: {
          // the tail chunk is scored whole, never bounded: its entry is +inf
          const bool whole = (static_cast<int64_t>(j) + 1) * N <= vocab;
          static_cast<float *>(out)[o] = whole ? chunk_noise_bound<N>(static_cast<int32_t>(j), key, vocab) : INFINITY;
          break;
        }
        default:
          break;
      }
    }
  }
}

template <bool BF16, int MODE, bool EXT>
hipError_t launch_rows(const VerifyLaunch &p, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((p.rows + p.rows_per_block - 1) / p.rows_per_block);
  const int waves = p.rows_per_block * p.split;
  const size_t lds = MODE == kGreedy ? (p.split > 1 ? waves * sizeof(WaveLds) : 0) : waves * sizeof(WaveLds);
  hipLaunchKernelGGL((verify_rows_kernel<BF16, MODE, EXT>), dim3(blocks), dim3(64 * waves), lds, stream, p);
  return hipGetLastError();
}

template <bool BF16, bool EXT>
hipError_t launch_noise(const VerifyLaunch &p, hipStream_t stream) {
  if (p.noise_cmax) return launch_rows<BF16, kTableBound, EXT>(p, stream);
  return p.greedy ? launch_rows<BF16, kGreedy, EXT>(p, stream) : launch_rows<BF16, kHashBound, EXT>(p, stream);
}

template <bool BF16>
hipError_t launch_typed(const VerifyLaunch &p, hipStream_t stream) {
  constexpr int N = Chunk<BF16>::N;
  if (p.noise_cmax) {
    const dim3 grid(static_cast<unsigned>((p.cmax_ld + 256 * kCmaxPerThread - 1) / (256 * kCmaxPerThread)),
                    static_cast<unsigned>(p.cmax_rows < 65535 ? p.cmax_rows : 65535));
    hipLaunchKernelGGL(noise_cmax_kernel<N>, grid, dim3(256), 0, stream, p.seed_b,
                       static_cast<uint32_t>(p.cmax_rows), static_cast<uint32_t>(p.cmax_ld), p.vocab, p.noise_cmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the extended pass: -inf logits and the reverse divergence
  return (p.neg_inf || p.out.kl_rev) ? launch_noise<BF16, true>(p, stream) : launch_noise<BF16, false>(p, stream);
}

}  // namespace

hipError_t launch_debug_noise(uint32_t seed_b, const int32_t *pos, int64_t pos_period, int64_t rows, int64_t vocab,
                              int32_t what, int32_t chunk_elems, void *out, hipStream_t stream) {
  const int64_t nch = (vocab + chunk_elems - 1) / chunk_elems;
  int64_t width = vocab;
  if (what == DV_DEBUG_GROUP_WORDS) width = vocab / kNoiseGroup;
  if (what == DV_DEBUG_CHUNK_BOUND || what == DV_DEBUG_TABLE_BOUND) width = nch;
  if (rows == 0 || width == 0) return hipSuccess;
  if (what == DV_DEBUG_TABLE_BOUND) {
    // the table as dv_verify_rows builds it, over positions 0 .. rows-1
    const dim3 grid(static_cast<unsigned>((nch + 256 * kCmaxPerThread - 1) / (256 * kCmaxPerThread)),
                    static_cast<unsigned>(rows < 65535 ? rows : 65535));
    if (chunk_elems == 8)
      hipLaunchKernelGGL(noise_cmax_kernel<8>, grid, dim3(256), 0, stream, seed_b, static_cast<uint32_t>(rows),
                         static_cast<uint32_t>(nch), vocab, static_cast<float *>(out));
    else
      hipLaunchKernelGGL(noise_cmax_kernel<4>, grid, dim3(256), 0, stream, seed_b, static_cast<uint32_t>(rows),
                         static_cast<uint32_t>(nch), vocab, static_cast<float *>(out));
    return hipGetLastError();
  }
  int64_t bx = (width + 255) / 256;
  if (bx > 4096) bx = 4096;
  const dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(rows < 65535 ? rows : 65535));
  if (chunk_elems == 8)
    hipLaunchKernelGGL(debug_noise_kernel<8>, grid, dim3(256), 0, stream, seed_b, pos, pos_period, rows, vocab, width,
                       what, out);
  else
    hipLaunchKernelGGL(debug_noise_kernel<4>, grid, dim3(256), 0, stream, seed_b, pos, pos_period, rows, vocab, width,
                       what, out);
  return hipGetLastError();
}

hipError_t launch_read_probe(const VerifyLaunch &p, uint32_t *sink, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((p.rows + p.rows_per_block - 1) / p.rows_per_block);
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(64 * p.rows_per_block * p.split), 0, stream, p, sink);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyLaunch &p, hipStream_t stream) {
  return p.bf16 ? launch_typed<true>(p, stream) : launch_typed<false>(p, stream);
}

}  // namespace dv
