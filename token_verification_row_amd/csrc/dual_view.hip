// COVER's dual-view attention with KV-cache override and diagonal correction
// ([COVER] "Method: COVER", part 1, Dual-View Feed Forward: seed columns read
// the K/V cached at the previous step, except a seed query's own diagonal,
// which reads the K/V of the masked input, with the weights renormalized).
// gfx950, MFMA.
//
//   k_eff(i, j) = K_prev[j] if seed[j] and j != i, else K_cur[j] (likewise v)
//   o_i = sum_j softmax_j(scale <q_i, k_eff(i, j)>) v_eff(i, j)
//
// Flash-attention style, bidirectional: one 4-wave workgroup per (sequence,
// head, 128 queries), one wave per 32 queries, key tiles of 32:
//   * S^T = K_eff Q^T with v_mfma_f32_32x32x16_bf16: a lane holds the scores
//     of one query (16 keys; the other 16 in lane ^ 32), so the online softmax
//     of a query is lane-local plus one exchange across the two halves. The A
//     operand is 16 bytes of one key row (K_prev or K_cur by the key's seed
//     flag); the B operand, the query's own 8 dimensions per step, stays in
//     registers for the whole kernel.
//   * O^T += V_eff^T P^T: V_eff goes to LDS transposed ([d][key]) so that an A
//     operand is one 16-byte LDS read; the B operand is assembled from the
//     probabilities in registers with one exchange across the halves.
//   * on the diagonal tile, a seed query's own score is recomputed from
//     K_cur, and its output gets p_ii (V_cur[i] - V_prev[i]) added in fp32 (the
//     tile's V_eff holds V_prev there).
// Inputs bf16, accumulation fp32, probabilities rounded to bf16 for the second
// product; output fp32.
#include <cmath>

#include "dv_internal.h"

namespace dv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ float bf16_to_float(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// round-to-nearest-even float -> bf16 bits (finite inputs)
__device__ __forceinline__ uint16_t float_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int D>
__global__ __launch_bounds__(256) void dual_view_kernel(DualViewLaunch p) {
  constexpr int KS = D / 16;  // k-steps of the score product
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  __shared__ uint16_t vT[D][32 + 8];  // V_eff tile, transposed; padded rows
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.z, h = blockIdx.y;
  const int64_t g = h / (p.heads / p.kv_heads);
  const int32_t L = static_cast<int32_t>(p.len);
  const int32_t qb = blockIdx.x * 128 + wave * 32;  // this wave's first query
  const bool live = qb < L;
  const uint16_t *Q = p.q + ((b * p.heads + h) * L) * D;
  const int64_t kvo = ((b * p.kv_heads + g) * L) * D;
  const uint16_t *Kc = p.k_cur + kvo, *Vc = p.v_cur + kvo, *Kp = p.k_prev + kvo, *Vp = p.v_prev + kvo;
  const uint8_t *seed = p.seed + b * L;

  // B operand of S^T: this lane's query, dims 16 s + 8 half + 0..7
  bf16x8 qf[KS];
  const int32_t qi = live ? qb + n : 0;
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_bf16x8(*reinterpret_cast<const u32x4 *>(Q + static_cast<int64_t>(qi) * D + 16 * s + 8 * half));
  const bool q_seed = live && seed[qi] != 0;

  f32x16 o[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;
  const float cs = p.scale * kLog2e;

  for (int32_t kb = 0; kb < L; kb += 32) {
    // V_eff tile -> LDS, transposed; 256 threads, D/8 segments of 8 dims per key
    __syncthreads();
    for (int e = tid; e < 32 * (D / 8); e += 256) {
      const int key = e / (D / 8), seg = e % (D / 8);
      const int32_t j = kb + key;
      const uint16_t *src = (seed[j] ? Vp : Vc) + static_cast<int64_t>(j) * D + 8 * seg;
      const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        vT[8 * seg + 2 * t][key] = static_cast<uint16_t>(ww[t] & 0xFFFFu);
        vT[8 * seg + 2 * t + 1][key] = static_cast<uint16_t>(ww[t] >> 16);
      }
    }
    __syncthreads();
    if (!live) continue;

    // scores of 32 keys for this wave's 32 queries: S^T[key][query]
    const int32_t kj = kb + n;  // the key row this lane feeds to the A operand
    const uint16_t *krow = (seed[kj] ? Kp : Kc) + static_cast<int64_t>(kj) * D + 8 * half;
    u32x4 ka[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) ka[s] = *reinterpret_cast<const u32x4 *>(krow + 16 * s);
    f32x16 sc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), qf[s], sc, 0, 0, 0);

    // register i holds key 8 (i / 4) + 4 half + i % 4 of this lane's query
    const bool diag = kb == qb;
    int di = -1;  // register of the diagonal key in this lane, if any
    if (diag && q_seed) {
      // a seed query's own score reads the current key
      float part = 0.0f;
      const uint16_t *kc = Kc + static_cast<int64_t>(qi) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(kc + 16 * s);
        const bf16x8 kk = as_bf16x8(w);
#pragma unroll
        for (int t = 0; t < 8; ++t) part = __builtin_fmaf(static_cast<float>(qf[s][t]), static_cast<float>(kk[t]), part);
      }
      const float own = part + __shfl_xor(part, 32);
      if (((n >> 2) & 1) == half) {
        di = 4 * (n >> 3) + (n & 3);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i == di) sc[i] = own;
      }
    }

    // online softmax of this lane's query (log2 domain)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] *= cs;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const float corr = __builtin_amdgcn_exp2f(m - mn);
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = __builtin_amdgcn_exp2f(sc[i] - mn);
      ps += sc[i];
    }
    lsum = lsum * corr + ps + __shfl_xor(ps, 32);
    m = mn;
#pragma unroll
    for (int c = 0; c < DB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[c][i] *= corr;

    // P^T as the B operand: for k-step u this lane needs keys 16 u + 8 half + 0..7
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint16_t own[4], give[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        own[t] = float_to_bf16(sc[8 * u + 4 * half + t]);
        give[t] = float_to_bf16(sc[8 * u + 4 * (1 - half) + t]);
      }
      const uint32_t g01 = give[0] | (static_cast<uint32_t>(give[1]) << 16);
      const uint32_t g23 = give[2] | (static_cast<uint32_t>(give[3]) << 16);
      const uint32_t r01 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(g01), 32));
      const uint32_t r23 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(g23), 32));
      const uint32_t o01 = own[0] | (static_cast<uint32_t>(own[1]) << 16);
      const uint32_t o23 = own[2] | (static_cast<uint32_t>(own[3]) << 16);
      const u32x4 pb = half == 0 ? u32x4{o01, o23, r01, r23} : u32x4{r01, r23, o01, o23};
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        const u32x4 va = *reinterpret_cast<const u32x4 *>(&vT[32 * c + n][16 * u + 8 * half]);
        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o[c], 0, 0, 0);
      }
    }

    if (diag && q_seed) {
      // the diagonal's value: the tile used V_prev, the seed query reads V_cur
      float pd = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i == di) pd = sc[i];
      pd += __shfl_xor(pd, 32);  // exactly one of the two lanes holds it
      const uint16_t *vc = Vc + static_cast<int64_t>(qi) * D;
      const uint16_t *vp = Vp + static_cast<int64_t>(qi) * D;
#pragma unroll
      for (int c = 0; c < DB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * c + 8 * (i / 4) + 4 * half + (i % 4);
          o[c][i] = __builtin_fmaf(pd, bf16_to_float(vc[d]) - bf16_to_float(vp[d]), o[c][i]);
        }
    }
  }
  if (!live) return;
  // O^T register i of block c: dim 32 c + 8 (i / 4) + 4 half + i % 4 of this lane's query
  const float inv = 1.0f / lsum;
  float *orow = p.out + ((b * p.heads + h) * L + qi) * D;
#pragma unroll
  for (int c = 0; c < DB; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(o[c][4 * q4] * inv, o[c][4 * q4 + 1] * inv, o[c][4 * q4 + 2] * inv, o[c][4 * q4 + 3] * inv);
      *reinterpret_cast<float4 *>(orow + 32 * c + 8 * q4 + 4 * half) = v;
    }
}

}  // namespace

hipError_t launch_dual_view(const DualViewLaunch &p, hipStream_t stream) {
  if (p.nseq == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.len + 127) / 128), static_cast<unsigned>(p.heads),
                  static_cast<unsigned>(p.nseq));
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(dual_view_kernel<128>, grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(dual_view_kernel<64>, grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dv
