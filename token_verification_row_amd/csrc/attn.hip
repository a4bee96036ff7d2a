// COVER's influence d_in and drift sensitivity d_out from attention
// probabilities ([COVER] "Method: COVER", part 2, Stability-Aware Seed
// Selection: the seed score weighs how much masked positions rely on a token
// (d_in) against how strongly the token attends to newly written positions
// (d_out)). gfx950.
//
//   d_in[b][j]  = (1/H) sum_h sum_{i masked} A[b][h][i][j]
//   d_out[b][i] = (1/H) sum_h sum_{k new}    A[b][h][i][k]
//
// Pass 1 reads every attention row once (HBM-bound): one workgroup per
// (sequence, head, tile of rows), lanes over 16-byte chunks of a row, a few rows
// in flight per wave. Each row's mass on new columns is a wave sum, kept by the
// lane of that row and collected in LDS; the rows of masked queries are summed
// into per-lane column accumulators, combined across the waves in LDS in a fixed
// order. The workgroup writes, for every group of 8 positions, its 8 column sums
// and its 8 row sums as one 64-byte partial, laid out so that the partials of a
// group from all heads and tiles are contiguous. Pass 2 sums each group's
// partials in double precision, in a fixed order, so results do not depend on
// scheduling.
#include "dv_internal.h"

namespace dv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum : int { kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118, kRowBcast15 = 0x142,
             kRowBcast31 = 0x143 };

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kRowShr1, 0xF>(x);
  x += dpp_f<kRowShr2, 0xF>(x);
  x += dpp_f<kRowShr4, 0xF>(x);
  x += dpp_f<kRowShr8, 0xF>(x);
  x += dpp_f<kRowBcast15, 0xA>(x);
  x += dpp_f<kRowBcast31, 0xC>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

template <bool BF16>
__device__ __forceinline__ void widen(const u32x4 &w, float (&x)[BF16 ? 8 : 4]) {
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

// M: 16-byte chunks of a row per lane (lane l holds chunks l, l + 64, ...); NW waves per
// workgroup; LOADS: 16-byte loads per lane in flight per wave (whole rows).
template <bool BF16, int M, int NW, int LOADS>
__global__ __launch_bounds__(64 * NW) void influence_rows_kernel(InfluenceLaunch p) {
  constexpr int N = BF16 ? 8 : 4;
  constexpr int U = M >= LOADS ? 1 : LOADS / M;  // rows in flight per wave
  constexpr int CAP = 64 * M * N;                 // positions of a row this instantiation covers
  __shared__ float col[CAP];
  __shared__ float rsum[CAP];  // the tile's row sums, by row - r0 (a tile has at most len rows)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.z, h = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const int32_t L = static_cast<int32_t>(p.len);
  const int32_t nch = (L + N - 1) / N;
  const int32_t r0 = tile * p.tile_rows;
  const int32_t r1 = min(L, r0 + p.tile_rows);
  const int64_t bh = b * p.heads + h;
  const size_t pitch = static_cast<size_t>(p.ld) * (BF16 ? 2 : 4);
  const char *head = static_cast<const char *>(p.probs) + static_cast<size_t>(bh) * L * pitch;
  const uint8_t *qmask = p.query_masked + b * L;
  const uint8_t *newc = p.new_cols + b * L;

  // per element of my chunks: 1.0 where the column is newly written, else 0.0
  // (in registers, or for long rows in LDS, shared by the workgroup); and, per
  // 32-bit word, the bits that belong to the row (the partly filled last
  // chunk of a row carries padding, which is cleared before use)
  constexpr bool kNewInLds = M >= 8;
  __shared__ float s_new[kNewInLds ? CAP : 1];
  float newf[kNewInLds ? 1 : M][N];
  u32x4 keep[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int32_t c = lane + 64 * m;
    uint32_t kw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int32_t j = c * N + e;
      const bool valid = c < nch && j < L;
      if constexpr (!kNewInLds) newf[m][e] = valid && newc[j] ? 1.0f : 0.0f;
      if (valid) kw[BF16 ? e / 2 : e] |= BF16 ? (0xFFFFu << (16 * (e & 1))) : 0xFFFFFFFFu;
    }
    keep[m] = u32x4{kw[0], kw[1], kw[2], kw[3]};
  }
  if constexpr (kNewInLds) {
    for (int32_t j = threadIdx.x; j < nch * N; j += 64 * NW) s_new[j] = (j < L && newc[j]) ? 1.0f : 0.0f;
    __syncthreads();
  }
  float acc[M][N];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[m][e] = 0.0f;

  auto load_row = [&](int32_t i, u32x4 (&w)[M]) {
    const u32x4 *row = reinterpret_cast<const u32x4 *>(head + static_cast<size_t>(i) * pitch);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int32_t c = lane + 64 * m;
      w[m] = c < nch ? __builtin_nontemporal_load(row + c) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // folds one row; returns its mass on new columns (uniform across the wave)
  auto fold_row = [&](bool masked_query, const u32x4 (&w)[M]) {
    float rs = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float x[N];
      widen<BF16>(w[m] & keep[m], x);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        float f;
        if constexpr (kNewInLds) {
          const int32_t c = lane + 64 * m;
          f = c < nch ? s_new[c * N + e] : 0.0f;
        } else {
          f = newf[m][e];
        }
        rs = __builtin_fmaf(x[e], f, rs);
      }
      if (masked_query) {
#pragma unroll
        for (int e = 0; e < N; ++e) acc[m][e] += x[e];
      }
    }
    return wave_sum(rs);
  };

  // this wave's rows: r0 + wave + NW k, k < K; taken 64 at a time so that lane
  // k holds the query mask and, at the end, the row sum of row k of the group
  const int32_t K = r1 > r0 + wave ? (r1 - r0 - wave + NW - 1) / NW : 0;
  for (int32_t g = 0; g < K; g += 64) {
    const int32_t kn = min(64, K - g);
    const int32_t my_row = r0 + wave + NW * (g + lane);
    const unsigned long long qbits = __ballot(lane < kn && qmask[my_row] != 0);
    float my_sum = 0.0f;
    int32_t k = 0;
    for (; k + U <= kn; k += U) {  // U rows of this wave in flight
      u32x4 w[U][M];
#pragma unroll
      for (int u = 0; u < U; ++u) load_row(r0 + wave + NW * (g + k + u), w[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float su = fold_row((qbits >> (k + u)) & 1ull, w[u]);
        my_sum = lane == k + u ? su : my_sum;
      }
    }
    for (; k < kn; ++k) {
      u32x4 w0[M];
      load_row(r0 + wave + NW * (g + k), w0);
      const float s0 = fold_row((qbits >> k) & 1ull, w0);
      my_sum = lane == k ? s0 : my_sum;
    }
    if (lane < kn) rsum[my_row - r0] = my_sum;
  }

  // column sums of the tile: wave 0 writes, the others add, in wave order
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int32_t c = lane + 64 * m;
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const int32_t j = c * N + e;
          if (c < nch && j < L) col[j] = (w == 0 ? 0.0f : col[j]) + acc[m][e];
        }
      }
    }
    __syncthreads();
  }
  // the partials: 64 bytes per group of 8 positions, four 16-byte stores (columns 0-3,
  // 4-7, rows 0-3, 4-7 of the group)
  const int32_t G = (L + 7) / 8;
  const int64_t mtot = p.heads * p.tiles, mine = h * p.tiles + tile;
  float4 *out = reinterpret_cast<float4 *>(p.part);
  for (int32_t x = threadIdx.x; x < 4 * G; x += 64 * NW) {
    const int32_t grp = x >> 2, q = x & 3;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t i = 8 * grp + 4 * (q & 1) + e;
      if (q < 2) v[e] = i < L ? col[i] : 0.0f;
      else v[e] = (i >= r0 && i < r1) ? rsum[i - r0] : 0.0f;
    }
    out[((b * G + grp) * mtot + mine) * 4 + q] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// d_in and d_out of every (sequence, group of 8 positions): the group's partials
// from all heads and tiles, contiguous, summed in double precision. Thread (s, q)
// sums float4 q of partials s, s + 256, ... in order, then a fixed binary tree over
// s adds the 256 sums, so the result does not depend on scheduling.
constexpr int kRedSplit = 256;
__global__ __launch_bounds__(4 * kRedSplit) void influence_reduce_kernel(InfluenceLaunch p) {
  __shared__ double red[kRedSplit][17];  // 16 sums per split, padded against bank conflicts
  const int q = threadIdx.x & 3, sp = threadIdx.x >> 2;
  const int64_t b = blockIdx.y, grp = blockIdx.x;
  const int64_t G = (p.len + 7) / 8, mtot = p.heads * p.tiles;
  const float4 *src = reinterpret_cast<const float4 *>(p.part) + (b * G + grp) * mtot * 4 + q;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll 4
  for (int64_t m = sp; m < mtot; m += kRedSplit) {
    const float4 v = src[m * 4];
    s0 += v.x;
    s1 += v.y;
    s2 += v.z;
    s3 += v.w;
  }
  red[sp][4 * q] = s0;
  red[sp][4 * q + 1] = s1;
  red[sp][4 * q + 2] = s2;
  red[sp][4 * q + 3] = s3;
  __syncthreads();
  for (int stride = kRedSplit / 2; stride > 0; stride >>= 1) {
    if (sp < stride) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[sp][4 * q + e] += red[sp + stride][4 * q + e];
    }
    __syncthreads();
  }
  if (sp == 0) {
    const double inv = 1.0 / static_cast<double>(p.heads);
    float *dst = q < 2 ? p.d_in : p.d_out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = 8 * grp + 4 * (q & 1) + e;
      if (dst && i < p.len) dst[b * p.len + i] = static_cast<float>(red[0][4 * q + e] * inv);
    }
  }
}

// Rows of one 16-byte chunk per lane (up to 512 bf16 positions) stream best from two waves with
// eight rows each in flight; longer rows from four waves with four 16-byte loads per lane.
template <bool BF16, int M>
hipError_t launch_rows(const InfluenceLaunch &p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(p.heads), static_cast<unsigned>(p.nseq));
  if constexpr (M == 1)
    hipLaunchKernelGGL((influence_rows_kernel<BF16, M, 2, 8>), grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL((influence_rows_kernel<BF16, M, 4, 4>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_typed(const InfluenceLaunch &p, hipStream_t stream) {
  constexpr int N = BF16 ? 8 : 4;
  const int64_t per_lane = ((p.len + N - 1) / N + 63) / 64;
  if (per_lane <= 1) return launch_rows<BF16, 1>(p, stream);
  if (per_lane <= 2) return launch_rows<BF16, 2>(p, stream);
  if (per_lane <= 4) return launch_rows<BF16, 4>(p, stream);
  if (per_lane <= 8) return launch_rows<BF16, 8>(p, stream);
  if constexpr (!BF16) {
    if (per_lane <= 16) return launch_rows<BF16, 16>(p, stream);
  }
  return hipErrorInvalidValue;  // excluded by the host checks (len <= kMaxInfluenceLen)
}

}  // namespace

hipError_t launch_influence(const InfluenceLaunch &p, hipStream_t stream) {
  if (p.nseq == 0 || p.heads == 0) return hipSuccess;
  hipError_t e = p.bf16 ? launch_typed<true>(p, stream) : launch_typed<false>(p, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((p.len + 7) / 8), static_cast<unsigned>(p.nseq));
  hipLaunchKernelGGL(influence_reduce_kernel, grid, dim3(4 * kRedSplit), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dv
