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
// (sequence, head, tile of rows), lanes over 16-byte chunks of a row, two rows
// in flight per wave. Each row's mass on new columns is a wave sum written to
// a per-(sequence, head) row partial; the rows of masked queries are summed
// into per-lane column accumulators, combined across the four waves in LDS in
// a fixed order and written as a per-tile column partial. Pass 2 sums the
// partials of each position over heads and tiles in double precision, in a
// fixed order, so results do not depend on scheduling.
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

// M: 16-byte chunks of a row per lane (lane l holds chunks l, l + 64, ...).
template <bool BF16, int M>
__global__ __launch_bounds__(256) void influence_rows_kernel(InfluenceLaunch p) {
  constexpr int N = BF16 ? 8 : 4;
  __shared__ float col[kMaxInfluenceLen];
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

  // which of my elements are newly written columns, and which lie inside the row
  uint32_t newbits[M], validbits[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    newbits[m] = validbits[m] = 0;
    const int32_t c = lane + 64 * m;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int32_t j = c * N + e;
      if (c < nch && j < L) {
        validbits[m] |= 1u << e;
        if (newc[j]) newbits[m] |= 1u << e;
      }
    }
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
  auto fold_row = [&](int32_t i, const u32x4 (&w)[M]) {
    const bool masked_query = qmask[i] != 0;  // uniform across the wave
    float rs = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float x[N];
      widen<BF16>(w[m], x);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float v = ((validbits[m] >> e) & 1u) ? x[e] : 0.0f;  // the padding after the row is not read as data
        rs += ((newbits[m] >> e) & 1u) ? v : 0.0f;
        if (masked_query) acc[m][e] += v;
      }
    }
    rs = wave_sum(rs);
    if (lane == 0) p.row_part[bh * L + i] = rs;
  };

  int32_t i = r0 + wave;
  for (; i + 4 < r1; i += 8) {  // two rows of this wave in flight
    u32x4 w0[M], w1[M];
    load_row(i, w0);
    load_row(i + 4, w1);
    fold_row(i, w0);
    fold_row(i + 4, w1);
  }
  if (i < r1) {
    u32x4 w0[M];
    load_row(i, w0);
    fold_row(i, w0);
  }

  // column sums of the tile: wave 0 writes, waves 1..3 add, in that order
  for (int w = 0; w < 4; ++w) {
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
  float *out = p.col_part + (bh * p.tiles + tile) * L;
  for (int32_t j = threadIdx.x; j < L; j += 256) out[j] = col[j];
}

// d_in and d_out of every (sequence, position): the partials summed over heads
// (and tiles) in double precision, heads in order.
__global__ __launch_bounds__(256) void influence_reduce_kernel(InfluenceLaunch p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= p.nseq * p.len) return;
  const int64_t b = idx / p.len, j = idx - b * p.len;
  double si = 0.0, so = 0.0;
  for (int64_t h = 0; h < p.heads; ++h) {
    const int64_t bh = b * p.heads + h;
    for (int32_t t = 0; t < p.tiles; ++t) si += p.col_part[(bh * p.tiles + t) * p.len + j];
    so += p.row_part[bh * p.len + j];
  }
  if (p.d_in) p.d_in[idx] = static_cast<float>(si / static_cast<double>(p.heads));
  if (p.d_out) p.d_out[idx] = static_cast<float>(so / static_cast<double>(p.heads));
}

template <bool BF16, int M>
hipError_t launch_rows(const InfluenceLaunch &p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(p.heads), static_cast<unsigned>(p.nseq));
  hipLaunchKernelGGL((influence_rows_kernel<BF16, M>), grid, dim3(256), 0, stream, p);
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
  const int64_t n = p.nseq * p.len;
  hipLaunchKernelGGL(influence_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dv
