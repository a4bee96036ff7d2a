// Acceptance over trees of candidate block states and the commit it yields
// ([SPOT] §1 "Key Terms & Definitions", §3 "Method & Key Results": the
// drafter proposes a multi-level tree of block states, the target verifies all
// of them in one batched pass, and under coupled noise a proposed child is
// right exactly when it equals the target's own transition). gfx950.
//
// One workgroup per tree:
//   1. the node arrays go to LDS;
//   2. the target's transition from each node's state: the masked positions
//      are the root's minus those committed on the path (pointer jumping in LDS), the
//      transition is the masked position with the highest confidence, lowest
//      position on ties, with the verifier's token (one thread per (node,
//      position) for blocks of up to 64 positions, else one wave per node);
//   3. one thread per node accepts it when every node on its path matches its
//      parent's transition, and counts its depth (pointer jumping);
//   4. the deepest accepted node (lowest index on ties), its path and the
//      target's transition there form the commit list, which can be applied
//      to the block's tokens and mask.
// An accepted path commits distinct masked positions, so a node deeper than
// block_len cannot be accepted: a path of more than block_len edges gets no
// transition and its node is not accepted.
// Device data that breaks the layout (a parent not below its node, a position
// outside the block) makes that node unacceptable, never an access outside
// the arrays.
#include <climits>

#include "dv_internal.h"

namespace dv {
namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
static_assert(kMaxTreeNodes <= kTreeThreads, "one node per thread in the pointer jumping");
constexpr int kPosPerLane = kMaxTreeBlockLen / 64;
constexpr int kPre = 4;  // (node, position) entries per thread read ahead in small trees

// A small tree's confidences, tokens and root mask flags, read by each thread at the start for the
// entries tid + kTreeThreads k it handles later, so that every global read of the kernel is in
// flight at once (one round trip to memory instead of one per phase).
struct Prefetch {
  bool on;
  float conf[kPre];
  int32_t tok[kPre];
  uint32_t masked[kPre];
};

struct TreeLds {
  int32_t parent[kMaxTreeNodes];
  int32_t pos[kMaxTreeNodes];
  int32_t tok[kMaxTreeNodes];
  int32_t ttok[kMaxTreeNodes];         // transition token of each node's state
  int16_t tpos[kMaxTreeNodes];         // transition position (-1: none, or not needed)
  int16_t depth[kMaxTreeNodes];        // accepted depth, -1 when not accepted (edges so far while jumping)
  int16_t anc[kMaxTreeNodes];          // pointer jumping: the ancestor a node's summary reaches (-1: the root)
  unsigned long long pmask[kMaxTreeNodes];  // blocks of <= 64 positions: positions committed on the path
  unsigned long long tkey[kMaxTreeNodes];   // blocks of <= 64 positions: best (confidence, position) key
  int32_t commit_pos[kMaxTreeBlockLen + 1];
  int32_t commit_tok[kMaxTreeBlockLen + 1];
  unsigned long long best_key[kTreeWaves];
  int32_t ncommit;
};

// Parent of node i, or -1 when the layout is broken (parent not in [0, i)).
__device__ __forceinline__ int32_t parent_of(const TreeLds &s, int32_t i) {
  const int32_t q = s.parent[i];
  return (q >= 0 && q < i) ? q : -1;
}

// Pointer jumping to the root, one node per thread: a node's summary is (anc, bits, steps): the
// ancestor it reaches, the OR of the positions committed on the way (path masks only) and the number
// of edges, -1 once a link on the way is broken. Each round adds the ancestor's summary to the node's
// and jumps to the ancestor's ancestor, so after ceil(log2 n) rounds every summary reaches the root:
// log2 n dependent LDS reads instead of one per level. The caller has published every node's first
// summary (s.depth, s.anc, and s.pmask with bits) and synchronised.
template <bool BITS>
__device__ __forceinline__ void jump_to_root(TreeLds &s, int32_t n, int32_t &anc, int32_t &steps,
                                             unsigned long long &bits) {
  const int tid = threadIdx.x;
  for (int32_t span = 1; span < n; span <<= 1) {
    const bool act = tid < n && anc >= 0;
    unsigned long long b2 = 0;
    int32_t s2 = 0, a2 = -1;
    if (act) {
      if (BITS) b2 = s.pmask[anc];
      s2 = s.depth[anc];
      a2 = s.anc[anc];
    }
    __syncthreads();
    if (act) {
      bits |= b2;
      steps = (steps < 0 || s2 < 0) ? -1 : steps + s2;
      anc = steps < 0 ? -1 : a2;
      if (BITS) s.pmask[tid] = bits;
      s.depth[tid] = static_cast<int16_t>(steps);
      s.anc[tid] = static_cast<int16_t>(anc);
    }
    __syncthreads();
  }
}

// Order-preserving unsigned image of a float (larger float, larger image).
__device__ __forceinline__ uint32_t float_order(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Blocks of up to 64 positions. Each node's path (at most block_len edges: a
// longer path cannot be accepted and gets no transition) gives a 64-bit mask of
// committed positions, by pointer jumping; then one thread per (node, position)
// offers its masked position to the node's transition with an LDS atomic max on
// (confidence, lowest position), and the winner records its token. Every load of
// confidence and token is independent of the others.
__device__ void transitions_small(TreeLds &s, const TreeLaunch &p, int64_t nb, const uint8_t *root_masked,
                                  int32_t n, int32_t L, const Prefetch &pf) {
  const int tid = threadIdx.x;  // node tid (n <= kTreeThreads)
  int32_t anc = -1, steps = 0;
  unsigned long long bits = 0;
  if (tid < n) {
    if (tid > 0) {
      const int32_t up = parent_of(s, tid);
      if (up < 0) {
        steps = -1;
      } else {
        anc = up;
        steps = 1;
        const int32_t q = s.pos[tid];
        if (q >= 0 && q < L) bits = 1ull << q;
      }
    }
    s.pmask[tid] = bits;
    s.depth[tid] = static_cast<int16_t>(steps);
    s.anc[tid] = static_cast<int16_t>(anc);
  }
  __syncthreads();
  jump_to_root<true>(s, n, anc, steps, bits);
  if (tid < n) {
    s.pmask[tid] = (steps >= 0 && steps <= L) ? bits : ~0ull;  // all positions taken: no transition
    s.tkey[tid] = 0;
  }
  __syncthreads();
  const int64_t total = static_cast<int64_t>(n) * L;
  auto offer = [&](int64_t e, bool masked, float c) {
    const int32_t i = static_cast<int32_t>(e / L), q = static_cast<int32_t>(e - static_cast<int64_t>(i) * L);
    if (!masked || ((s.pmask[i] >> q) & 1ull)) return;
    const unsigned long long key = (static_cast<unsigned long long>(float_order(c)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(q));
    atomicMax(&s.tkey[i], key);
  };
  auto claim = [&](int64_t e, int32_t tok) {
    const int32_t i = static_cast<int32_t>(e / L), q = static_cast<int32_t>(e - static_cast<int64_t>(i) * L);
    const unsigned long long k = s.tkey[i];
    if (k != 0 && static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull)) == q) {
      s.tpos[i] = static_cast<int16_t>(q);
      s.ttok[i] = tok;
    }
  };
  if (pf.on) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int64_t e = tid + static_cast<int64_t>(k) * kTreeThreads;
      if (e < total) offer(e, pf.masked[k] != 0, pf.conf[k]);
    }
  } else {
    for (int64_t e = tid; e < total; e += kTreeThreads) {
      const int32_t q = static_cast<int32_t>(e % L);
      if (root_masked[q]) offer(e, true, p.conf[nb * L + e]);
    }
  }
  __syncthreads();
  if (pf.on) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int64_t e = tid + static_cast<int64_t>(k) * kTreeThreads;
      if (e < total) claim(e, pf.tok[k]);
    }
  } else {
    for (int64_t e = tid; e < total; e += kTreeThreads) {
      const int32_t i = static_cast<int32_t>(e / L);
      const unsigned long long k = s.tkey[i];
      // only the winner reads its token
      if (k != 0 && static_cast<int64_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull)) == e - static_cast<int64_t>(i) * L)
        claim(e, p.tok_v[nb * L + e]);
    }
  }
}

// Longer blocks: one wave per node; lane l holds positions l, l + 64, ...
__device__ void transitions_wide(TreeLds &s, const TreeLaunch &p, int64_t nb, const uint8_t *root_masked,
                                 int32_t n, int32_t L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t root_bits = 0;
#pragma unroll
  for (int k = 0; k < kPosPerLane; ++k) {
    const int32_t q = lane + 64 * k;
    if (q < L && root_masked[q]) root_bits |= 1u << k;
  }
  for (int32_t i = wave; i < n; i += kTreeWaves) {
    uint32_t bits = root_bits;
    int32_t j = i, steps = 0;
    bool broken = false;
    while (j > 0) {  // uniform across the wave
      const int32_t up = parent_of(s, j);
      if (++steps > L || up < 0) {
        broken = true;
        break;
      }
      const int32_t q = s.pos[j];
      if (q >= 0 && q < L && (q & 63) == lane) bits &= ~(1u << (q >> 6));
      j = up;
    }
    if (broken) continue;
    const float *crow = p.conf + (nb + i) * p.block_len;
    const int32_t *trow = p.tok_v + (nb + i) * p.block_len;
    float best_c = -INFINITY;
    int32_t best_q = INT_MAX, best_t = -1;
#pragma unroll
    for (int k = 0; k < kPosPerLane; ++k) {
      const int32_t q = lane + 64 * k;
      if ((bits >> k) & 1u) {
        const float c = crow[q];
        if (best_q == INT_MAX || c > best_c) {  // positions rise with k: keep the first of equal values
          best_c = c;
          best_q = q;
          best_t = trow[q];
        }
      }
    }
    // wave argmax: largest confidence, then lowest position
    for (int o = 32; o > 0; o >>= 1) {
      const float oc = __shfl_xor(best_c, o);
      const int32_t oq = __shfl_xor(best_q, o);
      const int32_t ot = __shfl_xor(best_t, o);
      if (oq != INT_MAX && (best_q == INT_MAX || oc > best_c || (oc == best_c && oq < best_q))) {
        best_c = oc;
        best_q = oq;
        best_t = ot;
      }
    }
    if (lane == 0 && best_q != INT_MAX) {
      s.tpos[i] = static_cast<int16_t>(best_q);
      s.ttok[i] = best_t;
    }
  }
}

__global__ __launch_bounds__(kTreeThreads) void tree_accept_kernel(TreeLaunch p) {
  __shared__ TreeLds s;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n = static_cast<int32_t>(p.nodes), L = static_cast<int32_t>(p.block_len);
  const int64_t nb = t * p.nodes;  // node base of this tree
  const uint8_t *root_masked = p.root_masked + t * p.block_len;
  const int64_t total = static_cast<int64_t>(n) * L;
  Prefetch pf;
  pf.on = L <= 64 && total <= static_cast<int64_t>(kPre) * kTreeThreads;
  if (pf.on) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      // entries past the tree read its last entry (always inside the arrays) and are not used
      const int64_t e = min(tid + static_cast<int64_t>(k) * kTreeThreads, total - 1);
      pf.conf[k] = p.conf[nb * L + e];
      pf.tok[k] = p.tok_v[nb * L + e];
      pf.masked[k] = root_masked[e % L];
    }
  }
  // the root mask flag of position tid, for the updated mask at the end (block_len <= kTreeThreads)
  const uint32_t own_masked = tid < L ? root_masked[tid] : 0u;
  for (int32_t i = tid; i < n; i += kTreeThreads) {
    s.parent[i] = i == 0 ? -1 : p.parent[nb + i];
    s.pos[i] = p.node_pos[nb + i];
    s.tok[i] = p.node_tok[nb + i];
    s.tpos[i] = -1;
    s.ttok[i] = -1;
  }
  __syncthreads();

  // 2. the target's transition from every node's state that could be accepted
  if (L <= 64) {
    transitions_small(s, p, nb, root_masked, n, L, pf);
  } else {
    transitions_wide(s, p, nb, root_masked, n, L);
  }
  __syncthreads();

  // 3. acceptance and depth, one thread per node: a node is accepted when every node on its path
  // matches its parent's transition and the path has at most block_len edges (pointer jumping)
  {
    int32_t anc = -1, steps = 0;
    unsigned long long none = 0;
    if (tid < n) {
      if (tid > 0) {
        const int32_t up = parent_of(s, tid);
        const bool ok = up >= 0 && s.tpos[up] >= 0 && s.pos[tid] == s.tpos[up] && s.tok[tid] == s.ttok[up];
        anc = ok ? up : -1;
        steps = ok ? 1 : -1;
      }
      s.depth[tid] = static_cast<int16_t>(steps);
      s.anc[tid] = static_cast<int16_t>(anc);
    }
    __syncthreads();
    jump_to_root<false>(s, n, anc, steps, none);
    if (tid < n) s.depth[tid] = static_cast<int16_t>(steps >= 0 && steps <= L ? steps : -1);
  }
  __syncthreads();

  // 4. best node: deepest, lowest index (key = (depth + 1) << 32 | ~index)
  unsigned long long key = 0;
  for (int32_t i = tid; i < n; i += kTreeThreads) {
    const int32_t d = s.depth[i];
    if (d >= 0) {
      const unsigned long long k = (static_cast<unsigned long long>(d + 1) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
      key = k > key ? k : key;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(key, o);
    key = other > key ? other : key;
  }
  if (lane == 0) s.best_key[wave] = key;
  __syncthreads();
  if (tid == 0) {
    unsigned long long k = s.best_key[0];
    for (int w = 1; w < kTreeWaves; ++w) k = s.best_key[w] > k ? s.best_key[w] : k;
    const int32_t best = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));  // the root at least
    const int32_t d = s.depth[best];
    int32_t j = best;
    for (int32_t m = d - 1; m >= 0; --m) {  // the path, written from its end
      s.commit_pos[m] = s.pos[j];
      s.commit_tok[m] = s.tok[j];
      j = s.parent[j];
    }
    int32_t c = d;
    if (s.tpos[best] >= 0) {
      s.commit_pos[c] = s.tpos[best];
      s.commit_tok[c] = s.ttok[best];
      ++c;
    }
    s.ncommit = c;
    if (p.best_node) p.best_node[t] = best;
    if (p.commit_len) p.commit_len[t] = c;
  }
  __syncthreads();
  for (int32_t i = tid; i < n; i += kTreeThreads) {
    if (p.accepted) p.accepted[nb + i] = s.depth[i] >= 0 ? 1 : 0;
    if (p.depth) p.depth[nb + i] = s.depth[i];
  }
  const int32_t nc = s.ncommit;
  for (int32_t m = tid; m < L; m += kTreeThreads) {
    if (p.commit_pos) p.commit_pos[t * p.block_len + m] = m < nc ? s.commit_pos[m] : -1;
    if (p.commit_tok) p.commit_tok[t * p.block_len + m] = m < nc ? s.commit_tok[m] : -1;
  }
  // apply the commits (committed positions are distinct); out_masked may alias
  // root_masked: every read of it happened before the barriers above
  for (int32_t m = tid; m < nc; m += kTreeThreads) {
    const int32_t q = s.commit_pos[m];
    if (p.block_tokens) p.block_tokens[t * p.block_len + q] = s.commit_tok[m];
  }
  if (p.out_masked && tid < L) {
    const int32_t q = tid;
    bool m = own_masked != 0;
    for (int32_t c = 0; c < nc && m; ++c) m = s.commit_pos[c] != q;
    p.out_masked[t * p.block_len + q] = m ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_tree_accept(const TreeLaunch &p, hipStream_t stream) {
  if (p.ntrees == 0) return hipSuccess;
  hipLaunchKernelGGL(tree_accept_kernel, dim3(static_cast<unsigned>(p.ntrees)), dim3(kTreeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dv
