// tree_build.hip -- best-first draft-tree construction on the GPU.
//
// Computes the tree the pages' GPU builder replaces the per-request CPU heap
// queue with ("The Architecture of a Thousand-Parameter Decision ...", "What to
// Build New", item 3; "The Architecture of Closure ...", "The Table as a
// Decision Artifact", tree_build row): best-first top-k expansion over the
// drafter's per-depth top-K log-probs, emitted as parent indices, visibility
// bitsets and first-child / next-sibling links.
//
// One 64-lane wavefront per request.  The frontier (never more than Q <= 128
// live candidates) lives in registers, two slots per lane, each as a 64-bit key
// whose unsigned order is the pop order: the fp32 score mapped to an
// order-preserving integer in the high word, then 0xFFFF - parent and
// 0xFFFF - rank in the low word, so a wave-wide max is "highest score, then
// lowest parent index, then lowest rank".  Every pop is one 64-bit max
// reduction plus one ballot to find the owning slot; the popped slot is reused
// for the child and a fresh slot takes the sibling.
#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kMaxQ = 128;
constexpr int kMaxDK = 4096;

// Order-preserving map from fp32 to u32 (larger value -> larger key).  Only
// non-NaN values reach it.
__device__ __forceinline__ uint32_t order_bits(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Every live key is > 0 (the score part of any value above -inf is > 0x007FFFFF).
__device__ __forceinline__ uint64_t frontier_key(float s, int parent, int rank) {
  return ((uint64_t)order_bits(s) << 32) |
         ((uint64_t)(uint32_t)(0xFFFF - parent) << 16) | (uint64_t)(uint32_t)(0xFFFF - rank);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(kWave) void tree_build_kernel(
    const float* __restrict__ topk_logp, const int32_t* __restrict__ topk_ids,
    const int32_t* __restrict__ root_token, const int32_t* __restrict__ prefix_len,
    int D, int K, int Q, int32_t* __restrict__ node_token, int32_t* __restrict__ parent,
    int32_t* __restrict__ depth, int32_t* __restrict__ position,
    int32_t* __restrict__ first_child, int32_t* __restrict__ next_sibling,
    float* __restrict__ score, uint64_t* __restrict__ vis, int32_t* __restrict__ n_nodes) {
  __shared__ float s_logp[kMaxDK];
  __shared__ int32_t s_ids[kMaxDK];
  __shared__ int32_t s_par[kMaxQ];
  __shared__ int32_t s_dep[kMaxQ];
  __shared__ int32_t s_tok[kMaxQ];
  __shared__ float s_sc[kMaxQ];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int DK = D * K;
  const size_t in0 = (size_t)b * DK;
  for (int t = lane; t < DK; t += kWave) {
    s_logp[t] = topk_logp[in0 + t];
    s_ids[t] = topk_ids[in0 + t];
  }
  if (lane == 0) {
    s_par[0] = -1;
    s_dep[0] = 0;
    s_tok[0] = root_token[b];
    s_sc[0] = 0.0f;
  }
  __syncthreads();

  // Frontier slot s lives in lane (s & 63), register (s >> 6); key 0 = empty.
  uint64_t key0 = 0, key1 = 0;
  int dep0 = 0, dep1 = 0;  // depth of the candidate held in the slot
  int used = 0;            // slots handed out so far (never exceeds n <= Q)
  if (D >= 1 && K >= 1) {
    const float s = __fadd_rn(0.0f, s_logp[0]);
    if (s > -INFINITY) {
      if (lane == 0) {
        key0 = frontier_key(s, 0, 0);
        dep0 = 1;
      }
      used = 1;
    }
  }

  int n = 1;
  while (n < Q) {
    const uint64_t best = wave_max_u64(key0 > key1 ? key0 : key1);
    if (best == 0) break;  // nothing left on offer: underfull tree
    const uint64_t m0 = __ballot(key0 == best);
    const uint64_t m1 = __ballot(key1 == best);
    const int slot = m0 ? (__ffsll((unsigned long long)m0) - 1)
                        : (64 + __ffsll((unsigned long long)m1) - 1);
    const int d0 = __shfl(dep0, slot & 63);
    const int d1 = __shfl(dep1, slot & 63);
    const int cdep = slot < 64 ? d0 : d1;
    const float csc = unorder_bits((uint32_t)(best >> 32));
    const int cpar = 0xFFFF - (int)((best >> 16) & 0xFFFFu);
    const int crank = 0xFFFF - (int)(best & 0xFFFFu);
    const int i = n++;

    // Offer the new node's rank-0 child and its next-ranked sibling.
    uint64_t kc = 0, ks = 0;
    if (cdep < D) {
      const float s = __fadd_rn(csc, s_logp[cdep * K]);
      if (s > -INFINITY) kc = frontier_key(s, i, 0);
    }
    if (crank + 1 < K) {
      const float s = __fadd_rn(s_sc[cpar], s_logp[(cdep - 1) * K + crank + 1]);
      if (s > -INFINITY) ks = frontier_key(s, cpar, crank + 1);
    }
    if (lane == 0) {
      s_par[i] = cpar;
      s_dep[i] = cdep;
      s_tok[i] = s_ids[(cdep - 1) * K + crank];
      s_sc[i] = csc;
    }
    __syncthreads();

    int slot_a = slot, slot_b = -1, dep_a = 0, dep_b = cdep;
    uint64_t key_a = 0, key_b = 0;
    if (kc) {
      key_a = kc;
      dep_a = cdep + 1;
      if (ks) {
        slot_b = used++;
        key_b = ks;
      }
    } else if (ks) {
      key_a = ks;
      dep_a = cdep;
    }
    if (lane == (slot_a & 63)) {
      if (slot_a < 64) { key0 = key_a; dep0 = dep_a; } else { key1 = key_a; dep1 = dep_a; }
    }
    if (slot_b >= 0 && lane == (slot_b & 63)) {
      if (slot_b < 64) { key0 = key_b; dep0 = dep_b; } else { key1 = key_b; dep1 = dep_b; }
    }
  }
  __syncthreads();

  // Derived arrays, one node per lane (two passes for Q > 64).
  const int W = (Q + 63) >> 6;
  const int32_t L = prefix_len[b];
  for (int i = lane; i < Q; i += kWave) {
    const size_t o = (size_t)b * Q + i;
    if (i < n) {
      const int p = s_par[i], d = s_dep[i];
      int fc = -1, ns = -1;
      for (int c = i + 1; c < n; ++c)
        if (s_par[c] == i) { fc = c; break; }
      if (i > 0)
        for (int c = i + 1; c < n; ++c)
          if (s_par[c] == p) { ns = c; break; }
      uint64_t v0 = 0, v1 = 0;
      for (int a = i; a >= 0; a = s_par[a]) {
        if (a < 64) v0 |= 1ull << a; else v1 |= 1ull << (a - 64);
      }
      node_token[o] = s_tok[i];
      parent[o] = p;
      depth[o] = d;
      position[o] = (int32_t)((uint32_t)L + (uint32_t)d);
      first_child[o] = fc;
      next_sibling[o] = ns;
      score[o] = s_sc[i];
      vis[o * W] = v0;
      if (W > 1) vis[o * W + 1] = v1;
    } else {
      node_token[o] = parent[o] = depth[o] = position[o] = -1;
      first_child[o] = next_sibling[o] = -1;
      score[o] = -INFINITY;
      vis[o * W] = 0;
      if (W > 1) vis[o * W + 1] = 0;
    }
  }
  if (lane == 0) n_nodes[b] = n;
}

}  // namespace

hipError_t launch_tree_build(const float* topk_logp, const int32_t* topk_ids,
                             const int32_t* root_token, const int32_t* prefix_len,
                             int B, int D, int K, int Q, int32_t* node_token,
                             int32_t* parent, int32_t* depth, int32_t* position,
                             int32_t* first_child, int32_t* next_sibling,
                             float* score, uint64_t* vis, int32_t* n_nodes,
                             hipStream_t stream) {
  hipLaunchKernelGGL(tree_build_kernel, dim3(B), dim3(kWave), 0, stream, topk_logp,
                     topk_ids, root_token, prefix_len, D, K, Q, node_token, parent,
                     depth, position, first_child, next_sibling, score, vis, n_nodes);
  return hipGetLastError();
}

}  // namespace ddt
