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
// head, 128 queries), one wave per 32 queries, key tiles of 64 in LDS (K_eff and
// V_eff rows picked by each key's seed flag), double-buffered: the next tile is
// fetched into registers while the current one is computed, then stored to the
// other buffer, one barrier per tile. Workgroups are renumbered so that the
// ones sharing a K/V head run on the same XCD (L2).
//   * S^T = K_eff Q^T with v_mfma_f32_32x32x16_bf16: a lane holds the scores
//     of one query (32 of the 64 keys; the others in lane ^ 32), so the online
//     softmax of a query is lane-local plus one swap of wave halves. The A
//     operand is 16 bytes of one key row in LDS; the B operand, the query's own
//     8 dimensions per step, stays in registers.
//   * O^T += V_eff^T P^T: V_eff is stored transposed ([d][key]) so that an A
//     operand is one 16-byte LDS read; the B operand is assembled from the
//     probabilities in registers with one swap of wave halves.
//   * the softmax reference is raised lazily (only when a score passes it by
//     2^8), so the accumulators are rarely rescaled.
//   * the diagonal: a seed query's own score against K_cur is computed once
//     up front and put in place of the tile's score on its diagonal tile; the
//     tile's V_eff holds V_prev there, so p_ii (V_cur[i] - V_prev[i]) is added
//     to the output at the end, in fp32.
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

constexpr int kKeys = 64;     // keys per tile
constexpr float kLazy = 8.0f;  // headroom of the softmax reference, log2 units

// one tile of K_eff (row-major) and V_eff (transposed) in LDS, rows padded by 16 bytes
template <int D>
struct Tile {
  uint16_t k[kKeys][D + 8];
  uint16_t vt[D][kKeys + 8];
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dual_view_kernel(DualViewLaunch p) {
  constexpr int KS = D / 16;                  // k-steps of the score product
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int SEG = D / 8;                  // 16-byte segments of a row
  constexpr int PER = kKeys * SEG / 256;      // segments of a tile per thread (K and V each)
  extern __shared__ uint4 lds_raw[];          // two tiles: one computed while the next is stored
  Tile<D> *const tiles = reinterpret_cast<Tile<D> *>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroups are dealt to the 8 XCDs in turn; renumber them so that each XCD takes a
  // contiguous range of (sequence, kv head, head, query block), whose K/V its L2 shares
  const int32_t L = static_cast<int32_t>(p.len);
  const uint32_t nqb = static_cast<uint32_t>(L + 127) / 128, total = gridDim.x, lin = blockIdx.x;
  const uint32_t even = total / 8 * 8;
  const uint32_t id = lin < even ? (lin % 8) * (even / 8) + lin / 8 : lin;
  const uint32_t qblk = id % nqb, hb = id / nqb;
  const int64_t h = hb % static_cast<uint32_t>(p.heads), b = hb / static_cast<uint32_t>(p.heads);
  const int64_t g = h / (p.heads / p.kv_heads);
  const int32_t qb = static_cast<int32_t>(qblk) * 128 + wave * 32;  // this wave's first query
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
  // a seed query's own score, against the key of the masked input (the diagonal)
  float own = 0.0f;
  if (q_seed) {  // both lanes of a query pair agree
    float part = 0.0f;
    const uint16_t *kc = Kc + static_cast<int64_t>(qi) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kk = as_bf16x8(*reinterpret_cast<const u32x4 *>(kc + 16 * s));
#pragma unroll
      for (int t = 0; t < 8; ++t) part = __builtin_fmaf(static_cast<float>(qf[s][t]), static_cast<float>(kk[t]), part);
    }
    own = sum_halves(part);
  }

  // the next tile staged in registers, rows picked by each key's seed flag: K row-major
  // (16-byte segments, SEG lanes per key), V one key per lane (segment wave + 4 r) so
  // that the transposed store below pairs neighbouring keys into 32-bit words
  u32x4 kst[PER], vst[PER];
  // sm: the tile's seed flags, one bit per key
  constexpr int KSTEP = 256 / SEG;            // keys between a thread's K rows
  const int kkey = tid / SEG, kseg = tid % SEG;
  auto fetch = [&](int32_t kb, uint64_t sm) {
    // a tail of 32 keys (len is a multiple of 32) repeats a valid row, weighted 0
    const bool tail = kb + kKeys > L;
    const int32_t jl = tail ? min(kb + lane, L - 1) : kb + lane;
    const uint64_t kbits = sm >> kkey;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int32_t row = tail ? min(kb + kkey + KSTEP * r, L - 1) : kb + kkey + KSTEP * r;
      const uint32_t off = static_cast<uint32_t>(row * D + 8 * kseg);
      kst[r] = *reinterpret_cast<const u32x4 *>((((kbits >> (KSTEP * r)) & 1) ? Kp : Kc) + off);
    }
    const uint16_t *vrow = (((sm >> lane) & 1) ? Vp : Vc) + static_cast<uint32_t>(jl * D);
#pragma unroll
    for (int r = 0; r < PER; ++r) vst[r] = *reinterpret_cast<const u32x4 *>(vrow + 8 * (wave + 4 * r));
  };
  auto store = [&](Tile<D> &tl) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r, key = e / SEG, seg = e % SEG;
      *reinterpret_cast<u32x4 *>(&tl.k[key][8 * seg]) = kst[r];
    }
    // lanes 2m and 2m + 1 hold keys 2m and 2m + 1: the even lane writes the words of
    // the even dimensions (both keys' values), the odd lane those of the odd ones
    const bool odd = lane & 1;
    // bytes 0..3 are this lane's word, 4..7 the partner's: the even lane takes its own
    // low half then the partner's, the odd lane the partner's high half then its own
    const uint32_t pick = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const uint32_t w[4] = {vst[r].x, vst[r].y, vst[r].z, vst[r].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t part = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(w[t]), 0xB1, 0xF, 0xF, false));  // lane ^ 1
        *reinterpret_cast<uint32_t *>(&tl.vt[8 * (wave + 4 * r) + 2 * t + odd][lane & ~1]) =
            __builtin_amdgcn_perm(part, w[t], pick);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;
  const float cs = p.scale * kLog2e;

  // seed flags are read a tile ahead of the rows they pick, so that no fetch waits on them
  uint32_t sv = seed[min(lane, L - 1)];
  fetch(0, __ballot(sv != 0));
  if (kKeys < L) sv = seed[min(kKeys + lane, L - 1)];
  store(tiles[0]);
  __syncthreads();
  for (int32_t kb = 0, cur = 0; kb < L; kb += kKeys, cur ^= 1) {
    const bool more = kb + kKeys < L;
    const Tile<D> &tl = tiles[cur];
    if (more) {
      fetch(kb + kKeys, __ballot(sv != 0));  // lands while this tile is computed
      if (kb + 2 * kKeys < L) sv = seed[min(kb + 2 * kKeys + lane, L - 1)];
    }
    if (live) {
      // scores of 64 keys (two blocks of 32) for this wave's 32 queries: S^T[key][query];
      // register i of block kk holds key 32 kk + 8 (i / 4) + 4 half + i % 4 of this lane's query
      // LDS operands are read a whole key block ahead of the products that use them, so
      // the matrix cores do not wait on LDS latency
      f32x16 sc[2] = {f32x16{}, f32x16{}};
      u32x4 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[s] = *reinterpret_cast<const u32x4 *>(&tl.k[n][16 * s + 8 * half]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead (the scheduler would sink them)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), qf[s], sc[0], 0, 0, 0);
        ka[s] = *reinterpret_cast<const u32x4 *>(&tl.k[32 + n][16 * s + 8 * half]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), qf[s], sc[1], 0, 0, 0);
      // the V operands of the first two k-steps of the second product
      u32x4 va[2][DB];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < DB; ++c)
          va[u][c] = *reinterpret_cast<const u32x4 *>(&tl.vt[32 * c + n][16 * u + 8 * half]);
      __builtin_amdgcn_sched_barrier(0);
      // the diagonal: a seed query's own score reads the current key. Key n of block
      // (qb - kb) / 32 (this lane's query) sits in register 4 (n / 8) + n % 4 of the
      // lane with half == (n / 4) % 2
      if (qb >= kb && qb < kb + kKeys && q_seed) {
        const int sel = ((n >> 2) & 1) == half ? 16 * ((qb - kb) >> 5) + 4 * (n >> 3) + (n & 3) : -1;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[kk][i] = sel == 16 * kk + i ? own : sc[kk][i];
      }
      // online softmax of this lane's query in the log2 domain, against a reference m
      // that is raised lazily: the weights exp2(s - m) stay at most 2^kLazy, and the
      // accumulators are rescaled only when some query's maximum passes m + kLazy (the
      // normalized result does not depend on m)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kk][i] *= cs;
      if (kb + 32 >= L) {  // len is a multiple of 32: the last tile may hold one block of keys
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[1][i] = -INFINITY;
      }
      float red[16];  // pairwise trees keep the dependency chains short
#pragma unroll
      for (int i = 0; i < 16; ++i) red[i] = fmaxf(sc[0][i], sc[1][i]);
#pragma unroll
      for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) red[i] = fmaxf(red[i], red[i + w]);
      const float tmax = max_halves(red[0]);
      const bool raise = tmax > m + kLazy;  // true on the first tile (m = -inf)
      if (__ballot(raise) != 0) {
        const float mn = raise ? tmax : m;
        const float corr = __builtin_amdgcn_exp2f(m - mn);
        lsum *= corr;
        m = mn;
#pragma unroll
        for (int c = 0; c < DB; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[c][i] *= corr;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kk][i] = __builtin_amdgcn_exp2f(sc[kk][i] - m);
#pragma unroll
      for (int i = 0; i < 16; ++i) red[i] = sc[0][i] + sc[1][i];
#pragma unroll
      for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) red[i] += red[i + w];
      lsum += sum_halves(red[0]);

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
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[u & 1][c]), as_bf16x8(pb), o[c], 0, 0, 0);
          if (u < 2) va[u & 1][c] = *reinterpret_cast<const u32x4 *>(&tl.vt[32 * c + n][16 * (u + 2) + 8 * half]);
        }
      }
    }
    // the other buffer was last read in the previous tile, which every wave has left
    if (more) store(tiles[cur ^ 1]);
    __syncthreads();
  }
  if (!live) return;
  if (q_seed) {
    // the diagonal's value: the tiles held V_prev there, a seed query reads V_cur; its
    // weight against the final reference m is the tile's weight times every later rescale
    const float pd = __builtin_amdgcn_exp2f(own * cs - m);
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

// two D = 128 tiles (70 KB) exceed the default 64 KB of dynamic LDS; gfx950 has 160 KB per CU
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

}  // namespace

hipError_t launch_dual_view(const DualViewLaunch &p, hipStream_t stream) {
  if (p.nseq == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.len + 127) / 128 * p.heads * p.nseq));
  if (p.head_dim == 128) {
    const hipError_t attr = allow_lds(dual_view_kernel<128>, 2 * sizeof(Tile<128>));  // on the current device
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(dual_view_kernel<128>, grid, dim3(256), 2 * sizeof(Tile<128>), stream, p);
  } else {
    hipLaunchKernelGGL(dual_view_kernel<64>, grid, dim3(256), 2 * sizeof(Tile<64>), stream, p);
  }
  return hipGetLastError();
}

}  // namespace dv
