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
// head, 128 queries), one wave per 32 queries. Key tiles (32 keys at head_dim
// 128, 64 at head_dim 64) go from global memory straight into LDS with
// global_load_lds, each row picked by the key's seed flag; K and V are both
// double-buffered, so the next tile loads while the current one is computed,
// one barrier per tile, and no register holds a tile in transit. Each buffer is
// an LDS variable of its own and the loop is unrolled by two tiles, so the
// compiler sees that the reads of one buffer cannot alias the loads landing in
// the other and does not make them wait for those loads (with one array
// indexed by a loop-carried buffer number, every tile's first read waited for
// the next tile's loads). Rows are
// stored row-major with their 16-byte segments XOR-swizzled so that the operand
// reads hit distinct banks. Workgroups are renumbered so that the ones sharing
// a K/V head run on the same XCD (L2). The kernel fits three waves per SIMD.
//   * S^T = K_eff Q^T with v_mfma_f32_32x32x16_bf16, per block of 32 keys: a
//     lane holds the scores of one query (16 keys; the others in lane ^ 32), so
//     the online softmax of a query is lane-local plus one swap of wave halves.
//     The A operand is 16 bytes of one key row in LDS; the B operand, the
//     query's own 8 dimensions per step, stays in registers.
//   * O^T += V_eff^T P^T: the A operand (8 keys of one dimension) comes from
//     two transposing LDS reads (ds_read_b64_tr_b16) of the row-major V tile;
//     the B operand is assembled from the probabilities in registers with one
//     swap of wave halves.
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

constexpr float kLazy = 8.0f;  // headroom of the softmax reference, log2 units

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define DV_LDS __attribute__((address_space(3)))

// K_eff and V_eff tiles live in LDS row-major, keys x D, unpadded; a row's 16-byte
// segment c sits at segment c ^ f(row), so that the operand reads below hit distinct
// banks of the 64-bank (256-byte) LDS. K, b128 reads of 16 consecutive rows at one
// segment: f spreads those rows over the 16 four-bank groups (a 256-byte row at D = 128,
// a 128-byte one at D = 64, where row parity already picks the half). V, transposed
// reads of rows r..r+3 (and r+8..r+11), 64 bytes each: f moves each row's bytes to its
// own quarter of the banks (bits 2-3 of the segment; at D = 64 row parity picks the half).
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// NW waves per workgroup (32 queries each) share every tile of KT keys.
template <int D, int NW, int KT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void dual_view_kernel(DualViewLaunch p) {
  constexpr int KS = D / 16;                  // k-steps of the score product
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int SEG = D / 8;                  // 16-byte segments of a row
  constexpr int RPI = 1024 / (2 * D);         // rows one wave-wide 16-byte-per-lane load fills
  constexpr int LPT = KT / RPI;               // such loads per tile (K and V each)
  constexpr int PER = (LPT + NW - 1) / NW;    // per wave, at most
  // double-buffered tiles, one LDS variable per buffer: every access below names its buffer
  // statically, so the compiler can tell the reads of one buffer from the loads in flight
  // into the other and does not make the reads wait for those loads
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT * D], K1[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[KT * D], V1[KT * D];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroups are dealt to the 8 XCDs in turn; renumber them so that each XCD takes a
  // contiguous range of (sequence, kv head, head, query block), whose K/V its L2 shares
  const int32_t L = static_cast<int32_t>(p.len);
  const uint32_t nqb = static_cast<uint32_t>(L + 32 * NW - 1) / (32 * NW), total = gridDim.x, lin = blockIdx.x;
  const uint32_t even = total / 8 * 8;
  const uint32_t id = lin < even ? (lin % 8) * (even / 8) + lin / 8 : lin;
  const uint32_t qblk = id % nqb, hb = id / nqb;
  const int64_t h = hb % static_cast<uint32_t>(p.heads), b = hb / static_cast<uint32_t>(p.heads);
  const int64_t g = h / (p.heads / p.kv_heads);
  const int32_t qb = static_cast<int32_t>(qblk) * 32 * NW + wave * 32;  // this wave's first query
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

  // A tile goes from global memory straight to LDS: wave-wide load r of wave w fills rows
  // RPI (w + 4 r) .. + RPI - 1, lane l writing row RPI (w + 4 r) + l / SEG at segment
  // l % SEG; it reads the row picked by the key's seed flag (sm, one bit per key), at the
  // segment the swizzle puts there. A tail of 32 keys (len is a multiple of 32) repeats a
  // valid row, weighted 0.
  auto load_tile = [&](uint16_t *dst, const uint16_t *cur, const uint16_t *prev, bool is_k, int32_t kb,
                       uint64_t sm) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int blk = wave + NW * r;
      if (LPT % NW != 0 && blk >= LPT) break;  // wave-uniform
      const int row = RPI * blk + lane / SEG;
      const int c = (lane % SEG) ^ (is_k ? swz_k<D>(row) : swz_v<D>(row));
      const int32_t key = kb + row < L ? kb + row : L - 1;
      const uint32_t boff = static_cast<uint32_t>(2 * (key * D + 8 * c));  // bytes, below 2^24
      // one load per source under complementary lane masks: each addresses a uniform base
      // plus a 32-bit offset, so no 64-bit per-lane pointer is kept
      if ((sm >> row) & 1) {
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(prev) + boff,
                                         (DV_LDS void *)(dst + blk * RPI * D), 16, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(cur) + boff,
                                         (DV_LDS void *)(dst + blk * RPI * D), 16, 0, 0);
      }
    }
  };
  // per-lane LDS element offsets of the operand reads; what varies per read (key block,
  // k-step) is a constant that goes into the instruction's offset field. K: row n (+ 32 kk),
  // segment (2 s + half) ^ f(row). V, transposed reads: within each 16-lane group, lane j
  // addresses 4 dims (from 32 c + 16 (group % 2) + 4 (j % 4)) of key row 8 (group / 2) + j / 4
  // (+ 16 u + 4 hh); the swizzle of those rows depends on the lane only
  int koff[KS], voff[DB];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = n * D + 8 * ((2 * s + half) ^ swz_k<D>(n));
  {
    const int grp = lane >> 4, gl = lane & 15, rowl = 8 * (grp >> 1) + (gl >> 2);
#pragma unroll
    for (int c = 0; c < DB; ++c) {
      const int dcol = 32 * c + 16 * (grp & 1) + 4 * (gl & 3);
      voff[c] = rowl * D + 8 * ((dcol >> 3) ^ swz_v<D>(rowl)) + (dcol & 7);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int c = 0; c < DB; ++c) o[c] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;
  const float cs = p.scale * kLog2e;

  // One tile of 32 keys: S^T for this wave's 32 queries, the diagonal, the online softmax
  // and the weights as B operands. Register i of the scores holds key 8 (i / 4) + 4 half
  // + i % 4 of the tile for this lane's query. The softmax is in the log2 domain against a
  // reference m that is raised lazily: the weights exp2(s - m) stay at most 2^kLazy, and
  // the accumulators are rescaled only when some query's maximum passes m + kLazy (the
  // normalized result does not depend on m).
  auto scores = [&](const uint16_t *kt, int32_t kb, u32x4 (&pb)[2]) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4 *>(&kt[koff[s]]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[s], sc, 0, 0, 0);
      if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // four reads in flight at most
    }
    // the diagonal: a seed query's own score reads the current key; key n of the block
    // holding this wave's queries sits in register 4 (n / 8) + n % 4 of the lane with
    // half == (n / 4) % 2
    if (qb == kb && q_seed) {
      const int sel = ((n >> 2) & 1) == half ? 4 * (n >> 3) + (n & 3) : -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = sel == i ? own : sc[i];
    }
    float red[8];  // pairwise trees keep the dependency chains short
#pragma unroll
    for (int i = 0; i < 8; ++i) red[i] = fmaxf(sc[i], sc[i + 8]);
#pragma unroll
    for (int w = 4; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) red[i] = fmaxf(red[i], red[i + w]);
    const float tmax = max_halves(red[0]) * cs;  // cs > 0: the maximum of the scaled scores
    const bool raise = tmax > m + kLazy;  // true on the first block (m = -inf)
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
    for (int i = 0; i < 16; ++i) sc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cs, -m));
#pragma unroll
    for (int i = 0; i < 8; ++i) red[i] = sc[i] + sc[i + 8];
#pragma unroll
    for (int w = 4; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) red[i] += red[i + w];
    lsum += sum_halves(red[0]);
    // P^T as the B operand: k-step u of the tile covers keys 16 u + 8 half + 0..7, four
    // held by this lane and four by its partner: the lower half keeps its registers
    // 8 u + 0..3 and takes the partner's, the upper half keeps 8 u + 4..7 and takes the
    // partner's; one swap of halves does both
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 8 * u;
      uint32_t l01 = pack_bf16(sc[r0], sc[r0 + 1]), l23 = pack_bf16(sc[r0 + 2], sc[r0 + 3]);
      uint32_t h01 = pack_bf16(sc[r0 + 4], sc[r0 + 5]), h23 = pack_bf16(sc[r0 + 6], sc[r0 + 7]);
      swap_halves(l01, h01);
      swap_halves(l23, h23);
      pb[u] = u32x4{l01, l23, h01, h23};
    }
  };
  // O^T += V^T P^T over one tile of 32 keys. The A operand (row d = 32 c + lane % 32,
  // keys 16 u + 8 (lane / 32) + 0..7) comes from two transposed reads (keys + 0..3,
  // + 4..7): the read hands lane j of a 16-lane group element j % 4 of group lane
  // 4 i + j / 4's word as its key i
  auto values = [&](const uint16_t *vt, const u32x4 (&pb)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int c = 0; c < DB; ++c) {
        i16x4 t2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          t2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DV_LDS i16x4 *)(&vt[voff[c] + (16 * u + 4 * hh) * D]));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t2[0], t2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(pb[u]), o[c], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // bounds the reads in flight (registers)
    }
  };

  // Tiles are double-buffered: the loads of tile t + 1 are issued right after the barrier
  // that opens tile t (it frees their buffer, last read in tile t - 1) and land while tile t
  // is computed; the barrier that opens tile t + 1 waits for them. Seed flags are read a
  // tile ahead of the rows they pick. Waves past the end of the sequence compute on a
  // valid query and store nothing.
  uint64_t sm = __ballot(seed[min(lane % KT, L - 1)] != 0);
  load_tile(K0, Kc, Kp, true, 0, sm);
  load_tile(V0, Vc, Vp, false, 0, sm);
  uint32_t sv = seed[min(KT + lane % KT, L - 1)];
  // one tile: kt/vt hold it, kn/vn receive the next one
  auto tile = [&](int32_t kb, const uint16_t *kt, const uint16_t *vt, uint16_t *kn, uint16_t *vn) {
    // vmcnt(0): this wave's loads of this tile have written LDS (a load to LDS counts until
    // its data is in); the barrier then makes the whole tile visible, and every wave is done
    // with the previous tile, whose buffers the next loads overwrite
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (kb + KT < L) {
      sm = __ballot(sv != 0);
      if (kb + 2 * KT < L) sv = seed[min(kb + 2 * KT + lane % KT, L - 1)];
      load_tile(kn, Kc, Kp, true, kb + KT, sm);
      load_tile(vn, Vc, Vp, false, kb + KT, sm);
    }
    // blocks of 32 keys; len is a multiple of 32, so the last tile may hold fewer blocks
    if (live) {
#pragma unroll
      for (int bk = 0; bk < KT / 32; ++bk) {
        if (bk > 0 && kb + 32 * bk >= L) break;
        u32x4 pb[2];
        scores(kt + 32 * bk * D, kb + 32 * bk, pb);
        values(vt + 32 * bk * D, pb);
      }
    }
  };
  for (int32_t kb = 0; kb < L; kb += 2 * KT) {
    tile(kb, K0, V0, K1, V1);
    if (kb + KT < L) tile(kb + KT, K1, V1, K0, V0);
  }
  if (!live) return;
  if (q_seed) {
    // the diagonal's value: the tiles held V_prev there, a seed query reads V_cur; its
    // weight against the final reference m is the tile's weight times every later rescale
    const float pd = __builtin_amdgcn_exp2f(__builtin_fmaf(own, cs, -m));
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

}  // namespace

hipError_t launch_dual_view(const DualViewLaunch &p, hipStream_t stream) {
  if (p.nseq == 0) return hipSuccess;
  // 4 waves (128 queries) per workgroup; both K and V tiles double-buffered in 32 KB:
  // 32-key tiles at head_dim 128, 64-key tiles at 64. (Six waves sharing 64-key tiles at
  // head_dim 128 measured 25% slower.)
  if (p.head_dim == 128) {
    constexpr int NW = 4;
    const dim3 grid(static_cast<unsigned>((p.len + 32 * NW - 1) / (32 * NW) * p.heads * p.nseq));
    hipLaunchKernelGGL((dual_view_kernel<128, NW, 32>), grid, dim3(64 * NW), 0, stream, p);
  } else {
    constexpr int NW = 4;
    const dim3 grid(static_cast<unsigned>((p.len + 32 * NW - 1) / (32 * NW) * p.heads * p.nseq));
    hipLaunchKernelGGL((dual_view_kernel<64, NW, 64>), grid, dim3(64 * NW), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dv
