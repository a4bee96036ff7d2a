// Internal declarations shared by the host API (api.cpp) and the HIP kernels.
// Not part of the public interface (include/dlmverify.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dlmverify.h"

namespace dv {

// ---- noise hash: 32-bit finalizer of MurmurHash3 (Appleby, public domain) ----
// The noise word for (seed, position, vocabulary index) is built from it as
// follows (the generator behind [SPOT]'s shared Gumbel noise; the review does
// not say how the noise is drawn, so this keying is this library's choice):
//   A = mix32(seed_hi ^ kSeedSalt), B = mix32(A ^ seed_lo)
//   key(pos) = mix32(B ^ mix32(pos ^ kPosSalt))
//   word(pos, i) = mix32(key(pos) ^ (i * kIndexStep))
// and each full group of kNoiseGroup consecutive indices is drawn largest first
// from a group word (verify.hip has the construction):
//   gkey(pos) = mix32(key(pos) ^ kGroupSalt)
//   gword(pos, c) = mix32(gkey(pos) ^ (c * kIndexStep))
constexpr uint32_t kSeedSalt = 0x243F6A88u;
constexpr uint32_t kPosSalt = 0x85A308D3u;
constexpr uint32_t kIndexStep = 0x9E3779B9u;
constexpr uint32_t kGroupSalt = 0x6A09E667u;
constexpr int kNoiseGroup = 8;

// mix32 without its last step (x ^= x >> 16), which leaves the top 16 bits as they are:
// mix32(x) >> 16 == mix32_head(x) >> 16
__host__ __device__ __forceinline__ uint32_t mix32_head(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  return x;
}

__host__ __device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x = mix32_head(x);
  x ^= x >> 16;
  return x;
}

inline uint32_t seed_word(uint64_t seed) {
  uint32_t a = mix32(static_cast<uint32_t>(seed >> 32) ^ kSeedSalt);
  return mix32(a ^ static_cast<uint32_t>(seed));
}

// ---- per-(row, slice) partial state handed between the waves of a row: 64 bytes ----
// rho: reference (log2 units) the exponentials were taken against, i.e.
//      e_i = 2^(x_i * log2e - rho); S = sum e_i; W = sum e_i * (x_i*log2e - rho);
//      D = sum e_v,i * (a_i - b_i) (nats).
// m: running maximum logit, cm: 16-byte chunk holding its first occurrence.
// s: best perturbed score (log2 units), cs: its chunk.
struct alignas(16) Partial {
  float rho_v, S_v, W_v, D_v;
  float rho_d, S_d, m_v, m_d;
  float s_v, s_d;
  int32_t cm_v, cm_d;
  int32_t cs_v, cs_d;
  float D_d;  // sum e_d (a - b) against rho_d (extended pass; 0 otherwise)
  int32_t pad1;
};
static_assert(sizeof(Partial) == 64, "partial state must be 64 bytes");

struct VerifyLaunch {
  const void *va;
  const void *vb;
  int64_t rows;
  int64_t vocab;
  int64_t ld;          // elements
  int32_t bf16;
  int32_t greedy;      // temperature == 0
  int32_t neg_inf;     // logits may hold -inf (DV_LOGITS_NEG_INF)
  float cT;            // log2(e) / temperature (0 when greedy)
  uint32_t seed_b;     // seed word B
  const int32_t *pos;  // device or NULL
  int64_t pos_period;
  int32_t split;           // vocabulary slices per row: consecutive waves of one workgroup
  int32_t slice_chunks;    // 16-byte chunks per slice
  int32_t rows_per_block;  // rows of one workgroup (rows_per_block * split <= 16 waves)
  float *noise_cmax;       // [cmax_rows][cmax_ld] chunk-max noise table (workspace), or NULL
  int64_t cmax_rows;     // positions 0 .. cmax_rows-1
  int64_t cmax_ld;       // chunks per row
  dv_row_stats out;
};

hipError_t launch_verify(const VerifyLaunch &p, hipStream_t stream);

// Device address of the library's fixed scratch on the device of `stream` (noalloc.hip): resolved once per
// device, DV_NOALLOC_SCRATCH_BYTES long, shared by every call on that device.
hipError_t noalloc_scratch(hipStream_t stream, void **ptr);

// the read-only streaming probe (dv_debug_read_probe): sink holds kMaxProbeSplit words per row
constexpr int kMaxProbeSplit = 16;
hipError_t launch_read_probe(const VerifyLaunch &p, uint32_t *sink, hipStream_t stream);

struct DecideLaunch {
  int32_t rule;
  float tau_kl, conf_thr;
  int32_t mask_token;
  int64_t rows, group_len;
  const float *kl, *conf, *p_tok;
  const int32_t *tok_v, *tok_d;
  const uint8_t *subject;
  const int32_t *cur_tok;
  uint8_t *decision;
  int32_t *out_tok, *prefix_len, *best_group;
  uint32_t seed_b;  // KL_STOCHASTIC: the seed word B of the noise hash
  const int32_t *pos;
  int64_t pos_period;
};
hipError_t launch_decide(const DecideLaunch &p, hipStream_t stream);

hipError_t launch_seed_score(int64_t rows, const float *u, const float *d_in, const float *d_out,
                             const uint8_t *eligible, float *score, hipStream_t stream);

struct SelectLaunch {
  int64_t nseq, seq_len;
  const float *score;
  const uint8_t *eligible;
  int32_t k, largest, use_thr;
  float thr;
  int32_t *out_idx;
  float *out_val;
  int32_t *out_count;
  uint8_t *out_mask;
  // seed scores computed in the selection (u set): u (1 + d_in) / (1 + d_out) where
  // seed_eligible (or everywhere), -inf elsewhere, written to score_out; score is then unused
  const float *u, *d_in, *d_out;
  const uint8_t *seed_eligible;
  float *score_out;
};
constexpr int64_t kMaxSelectLen = 16384;
hipError_t launch_select_topk(const SelectLaunch &p, hipStream_t stream);
hipError_t launch_seed_select(const SelectLaunch &p, hipStream_t stream);
// dv_decide (when decide is set) and dv_seed_select, fused into one launch where both fit it
hipError_t launch_decide_seed_select(const DecideLaunch &d, bool decide, const SelectLaunch &s, hipStream_t stream);
// dv_seed_select, then dv_decide with the selection's mask (s.out_mask, required) as the subject
hipError_t launch_seed_select_decide(const SelectLaunch &s, const DecideLaunch &d, hipStream_t stream);

constexpr int kMaxTreeNodes = 1024;
constexpr int kMaxTreeBlockLen = 1024;
struct TreeLaunch {
  int64_t ntrees, nodes, block_len;
  const int32_t *parent, *node_pos, *node_tok;
  const uint8_t *root_masked;
  const float *conf;
  const int32_t *tok_v;
  uint8_t *accepted;
  int32_t *depth, *best_node, *commit_pos, *commit_tok, *commit_len, *block_tokens;
  uint8_t *out_masked;
};
hipError_t launch_tree_accept(const TreeLaunch &p, hipStream_t stream);

constexpr int kMaxInfluenceLen = 4096;
struct InfluenceLaunch {
  const void *probs;  // [nseq][heads][len][ld]
  int32_t bf16;
  int32_t tiles, tile_rows;  // row tiles per head
  int64_t nseq, heads, len, ld;
  const uint8_t *query_masked, *new_cols;  // [nseq][len]
  float *d_in, *d_out;                     // [nseq][len]
  // workspace [nseq][ceil(len / 8)][heads * tiles][16]: for each group of 8 positions and each
  // (head, tile), the tile's 8 column sums (d_in) then its 8 row sums (d_out; 0 for rows
  // outside the tile), so that the reduction reads each group's partials contiguously
  float *part;
};
hipError_t launch_influence(const InfluenceLaunch &p, hipStream_t stream);

struct DualViewLaunch {
  const uint16_t *q, *k_cur, *v_cur, *k_prev, *v_prev;  // bf16 bits
  const uint8_t *seed;
  float *out;
  float scale;
  int32_t head_dim;  // 64 or 128
  int64_t nseq, heads, kv_heads, len;
};
hipError_t launch_dual_view(const DualViewLaunch &p, hipStream_t stream);

// what: a dv_debug_noise mode; chunk_elems: 8 (bf16 chunks) or 4 (fp32 chunks)
hipError_t launch_debug_noise(uint32_t seed_b, const int32_t *pos, int64_t pos_period, int64_t rows, int64_t vocab,
                              int32_t what, int32_t chunk_elems, void *out, hipStream_t stream);

}  // namespace dv
