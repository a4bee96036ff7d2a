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
// head, 128 queries), one wave per 32 queries, key tiles of 64 staged in LDS
// (K_eff and V_eff rows picked by each key's seed flag; the next tile is
// fetched into registers while the current one is computed):
//   * S^T = K_eff Q^T with v_mfma_f32_32x32x16_bf16: a lane holds the scores
//     of one query (32 of the 64 keys; the others in lane ^ 32), so the online
//     softmax of a query is lane-local plus one exchange across the two
//     halves. The A operand is 16 bytes of one key row in LDS; the B operand,
//     the query's own 8 dimensions per step, stays in registers.
//   * O^T += V_eff^T P^T: V_eff is stored transposed ([d][key]) so that an A
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (hardware round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// v_permlane32_swap: lanes 32..63 of a trade places with lanes 0..31 of b. With a == b
// on entry, each lane then holds its own value and its partner's (lane ^ 32), one in each.
__device__ __forceinline__ void swap_halves(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ float max_halves(float x) {
  uint32_t a = __float_as_uint(x), b = a;
  swap_halves(a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
// the same sum in both lanes of a pair: addition commutes bit for bit
__device__ __forceinline__ float sum_halves(float x) {
  uint32_t a = __float_as_uint(x), b = a;
  swap_halves(a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}

constexpr int kKeys = 64;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dual_view_kernel(DualViewLaunch p) {
  constexpr int KS = D / 16;                  // k-steps of the score product
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int SEG = D / 8;                  // 16-byte segments of a row
  constexpr int PER = kKeys * SEG / 256;      // segments of a tile per thread (K and V each)
  __shared__ uint16_t Ks[kKeys][D + 8];       // K_eff tile, row-major, padded rows
  __shared__ uint16_t Vt[D][kKeys + 8];       // V_eff tile, transposed, padded rows
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

  // the next tile staged in registers, rows picked by each key's seed flag: K row-major
  // (16-byte segments, SEG lanes per key), V one key per lane (segment wave + 4 r) so
  // that the transposed store below pairs neighbouring keys into 32-bit words
  u32x4 kst[PER], vst[PER];
  auto fetch = [&](int32_t kb) {
    const int32_t jl = min(kb + lane, L - 1);  // a tail of 32 keys repeats a valid row, weighted 0
    const uint64_t sm = __ballot(seed[jl] != 0);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r, key = e / SEG, seg = e % SEG;
      const int64_t off = static_cast<int64_t>(min(kb + key, L - 1)) * D + 8 * seg;
      kst[r] = *reinterpret_cast<const u32x4 *>((((sm >> key) & 1) ? Kp : Kc) + off);
    }
    const uint16_t *vrow = (((sm >> lane) & 1) ? Vp : Vc) + static_cast<int64_t>(jl) * D;
#pragma unroll
    for (int r = 0; r < PER; ++r) vst[r] = *reinterpret_cast<const u32x4 *>(vrow + 8 * (wave + 4 * r));
  };
  auto store = [&]() {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r, key = e / SEG, seg = e % SEG;
      *reinterpret_cast<u32x4 *>(&Ks[key][8 * seg]) = kst[r];
    }
    // lanes 2m and 2m + 1 hold keys 2m and 2m + 1: the even lane writes the words of
    // the even dimensions (both keys' values), the odd lane those of the odd ones
    const bool odd = lane & 1;
    const uint32_t pick = odd ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const uint32_t w[4] = {vst[r].x, vst[r].y, vst[r].z, vst[r].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t part = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(w[t]), 0xB1, 0xF, 0xF, false));  // lane ^ 1
        const uint32_t lo_key = odd ? part : w[t], hi_key = odd ? w[t] : part;
        *reinterpret_cast<uint32_t *>(&Vt[8 * (wave + 4 * r) + 2 * t + odd][lane & ~1]) =
            __builtin_amdgcn_perm(hi_key, lo_key, pick);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;
  const float cs = p.scale * kLog2e;

  fetch(0);
  store();
  __syncthreads();
  for (int32_t kb = 0; kb < L; kb += kKeys) {
    const bool more = kb + kKeys < L;
    if (more) fetch(kb + kKeys);  // lands while this tile is computed
    if (live) {
      // scores of 64 keys (two blocks of 32) for this wave's 32 queries: S^T[key][query];
      // register i of block kk holds key 32 kk + 8 (i / 4) + 4 half + i % 4 of this lane's query
      f32x16 sc[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        sc[kk] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 ka = *reinterpret_cast<const u32x4 *>(&Ks[32 * kk + n][16 * s + 8 * half]);
          sc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[s], sc[kk], 0, 0, 0);
        }
      }
      // the diagonal: a seed query's own score reads the current key. Key n of block dk
      // (this lane's query) sits in register 4 (n / 8) + n % 4 of the lanes with
      // half == (n / 4) % 2.
      const bool diag = qb >= kb && qb < kb + kKeys && q_seed;
      float own = 0.0f;
      if (diag) {
        float part = 0.0f;
        const uint16_t *kc = Kc + static_cast<int64_t>(qi) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kk = as_bf16x8(*reinterpret_cast<const u32x4 *>(kc + 16 * s));
#pragma unroll
          for (int t = 0; t < 8; ++t) part = __builtin_fmaf(static_cast<float>(qf[s][t]), static_cast<float>(kk[t]), part);
        }
        own = sum_halves(part);
        const int sel = ((n >> 2) & 1) == half ? 16 * ((qb - kb) >> 5) + 4 * (n >> 3) + (n & 3) : -1;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[kk][i] = sel == 16 * kk + i ? own : sc[kk][i];
      }
      // online softmax of this lane's query (log2 domain); len is a multiple of 32, so
      // the last tile may hold a single block of keys
      const bool blk1 = kb + 32 < L;
      float tmax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sc[kk][i] = (kk == 0 || blk1) ? sc[kk][i] * cs : -INFINITY;
          tmax = fmaxf(tmax, sc[kk][i]);
        }
      tmax = max_halves(tmax);
      const float mn = fmaxf(m, tmax);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      float ps = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sc[kk][i] = __builtin_amdgcn_exp2f(sc[kk][i] - mn);
          ps += sc[kk][i];
        }
      lsum = lsum * corr + sum_halves(ps);
      m = mn;
#pragma unroll
      for (int c = 0; c < DB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[c][i] *= corr;

      // P^T as the B operand: k-step u covers keys 16 u + 8 half + 0..7 (block u / 2),
      // four of them held by this lane and four by its partner: the lower half keeps its
      // registers 8 (u % 2) + 0..3 and takes the partner's, the upper half keeps
      // 8 (u % 2) + 4..7 and takes the partner's; one swap of halves does both
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = u >> 1, r0 = 8 * (u & 1);
        uint32_t l01 = pack_bf16(sc[kk][r0], sc[kk][r0 + 1]), l23 = pack_bf16(sc[kk][r0 + 2], sc[kk][r0 + 3]);
        uint32_t h01 = pack_bf16(sc[kk][r0 + 4], sc[kk][r0 + 5]), h23 = pack_bf16(sc[kk][r0 + 6], sc[kk][r0 + 7]);
        swap_halves(l01, h01);
        swap_halves(l23, h23);
        const u32x4 pb = u32x4{l01, l23, h01, h23};
#pragma unroll
        for (int c = 0; c < DB; ++c) {
          const u32x4 va = *reinterpret_cast<const u32x4 *>(&Vt[32 * c + n][16 * u + 8 * half]);
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o[c], 0, 0, 0);
        }
      }
      if (diag) {
        // the diagonal's value: the tile held V_prev, the seed query reads V_cur
        const float pd = __builtin_amdgcn_exp2f(own * cs - mn);  // its weight, as in the tile
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
    __syncthreads();  // every wave is done with this tile
    if (more) {
      store();
      __syncthreads();
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
