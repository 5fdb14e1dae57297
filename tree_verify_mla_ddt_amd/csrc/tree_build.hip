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
// 0xFFFF - rank in the low word, so the largest key is "highest score, then
// lowest parent index, then lowest rank".  Every pop is a 32-bit DPP max
// reduction of the high words (a second one over the low words only when
// scores tie) plus a ballot to find the owning slot; the popped slot is reused for the
// child and a fresh slot takes the sibling.  Node i's fields live in lane i%64
// (register i/64) and are read back with readlane; its visibility row is its
// parent's row plus its own bit, set when it is popped.
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

// One DPP step of a 32-bit max: combine with the lane selected by CTRL (rows
// outside ROW_MASK contribute 0, the identity of an unsigned max).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}

// Wave-wide unsigned max: pair swaps, quad swaps, half-row and row mirrors give
// every lane its row's max; two row broadcasts carry it to lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = max_dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = max_dpp<0x141, 0xF>(v);  // row_half_mirror
  v = max_dpp<0x140, 0xF>(v);  // row_mirror
  v = max_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = max_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ int read_i(int v0, int v1, int idx) {
  const int a = __builtin_amdgcn_readlane(v0, idx & 63);
  const int b = __builtin_amdgcn_readlane(v1, idx & 63);
  return idx < 64 ? a : b;
}
__device__ __forceinline__ float read_f(float v0, float v1, int idx) {
  return __int_as_float(read_i(__float_as_int(v0), __float_as_int(v1), idx));
}
__device__ __forceinline__ uint64_t read_u64(uint64_t v0, uint64_t v1, int idx) {
  const uint32_t lo = (uint32_t)read_i((int)(uint32_t)v0, (int)(uint32_t)v1, idx);
  const uint32_t hi = (uint32_t)read_i((int)(uint32_t)(v0 >> 32), (int)(uint32_t)(v1 >> 32), idx);
  return ((uint64_t)hi << 32) | lo;
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
  __shared__ unsigned long long s_kids[kMaxQ][2];  // children of each node, as bitsets

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int DK = D * K;
  const size_t in0 = (size_t)b * DK;
  // Loaded first so that its latency overlaps the build (positions use it).
  const int32_t L = prefix_len[b];
  for (int t = lane; t < DK; t += kWave) {
    s_logp[t] = topk_logp[in0 + t];
    s_ids[t] = topk_ids[in0 + t];
  }
  s_kids[lane][0] = s_kids[lane][1] = 0;
  s_kids[lane + kWave][0] = s_kids[lane + kWave][1] = 0;
  __syncthreads();

  // Node fields: node `lane` in the *0 registers, node `lane + 64` in the *1.
  int par0 = -1, par1 = -1, dep0 = -1, dep1 = -1, tok0 = -1, tok1 = -1;
  float sc0 = -INFINITY, sc1 = -INFINITY;
  uint64_t va0 = 0, vb0 = 0, va1 = 0, vb1 = 0;  // visibility words 0 and 1
  if (lane == 0) {
    par0 = -1;
    dep0 = 0;
    tok0 = root_token[b];
    sc0 = 0.0f;
    va0 = 1;
  }

  // Frontier slot s lives in lane (s & 63), register (s >> 6); key 0 = empty.
  uint64_t key0 = 0, key1 = 0;
  int fd0 = 0, fd1 = 0;  // depth of the candidate held in the slot
  int used = 0;          // slots handed out so far (never exceeds n <= Q)
  if (D >= 1 && K >= 1) {
    const float s = __fadd_rn(0.0f, s_logp[0]);
    if (s > -INFINITY) {
      if (lane == 0) {
        key0 = frontier_key(s, 0, 0);
        fd0 = 1;
      }
      used = 1;
    }
  }

  // One pop.  With std::true_type (fewer than 64 nodes exist) every node,
  // parent and frontier slot index is below 64, so only the first register of
  // each pair is read or written (slots are handed out one per node at most);
  // std::false_type is the general pop.
  int n = 1;
  auto pop = [&](auto low_tag) __attribute__((always_inline)) -> bool {
    constexpr bool kLow = decltype(low_tag)::value;
    // The best key: the largest score word (one 32-bit DPP max), then, only
    // when several slots share it, the largest low word among them.  Live
    // candidates have distinct (parent, rank), so one slot remains.
    const uint32_t h0 = (uint32_t)(key0 >> 32), h1 = kLow ? 0u : (uint32_t)(key1 >> 32);
    const uint32_t hbest = wave_max_u32(kLow ? h0 : max(h0, h1));
    if (hbest == 0) return false;  // nothing left on offer: underfull tree
    uint64_t m0 = __ballot(h0 == hbest);
    uint64_t m1 = kLow ? 0ull : __ballot(h1 == hbest);
    if (__popcll(m0) + __popcll(m1) > 1) {
      const uint32_t l0 = h0 == hbest ? (uint32_t)key0 : 0u;
      const uint32_t l1 = (!kLow && h1 == hbest) ? (uint32_t)key1 : 0u;
      const uint32_t lbest = wave_max_u32(kLow ? l0 : max(l0, l1));
      m0 = __ballot(h0 == hbest && (uint32_t)key0 == lbest);
      m1 = kLow ? 0ull : __ballot(h1 == hbest && (uint32_t)key1 == lbest);
    }
    const int slot = m0 ? (__ffsll((unsigned long long)m0) - 1)
                        : (64 + __ffsll((unsigned long long)m1) - 1);
    const uint32_t low =
        kLow ? (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key0, slot)
             : (uint32_t)read_i((int)(uint32_t)key0, (int)(uint32_t)key1, slot);
    const int cdep = kLow ? __builtin_amdgcn_readlane(fd0, slot) : read_i(fd0, fd1, slot);
    const float csc = unorder_bits(hbest);
    const int cpar = 0xFFFF - (int)(low >> 16);
    const int crank = 0xFFFF - (int)(low & 0xFFFFu);
    const int i = n++;

    // Table reads of this pop, issued together: the node's token, its rank-0
    // child's log-prob and its next sibling's (indices clamped in range; the
    // values are used only where the candidate exists).
    const int row = (cdep - 1) * K;
    const int ctok = s_ids[row + crank];
    const float lp_child = s_logp[(cdep < D ? cdep : cdep - 1) * K];
    const float lp_sib = s_logp[row + (crank + 1 < K ? crank + 1 : crank)];
    const float psc = kLow ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc0), cpar))
                           : read_f(sc0, sc1, cpar);

    // The new node: fields into its owner lane, visibility = parent's + self.
    if (kLow) {
      const uint64_t pva = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)va0, cpar) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(va0 >> 32), cpar) << 32);
      const uint64_t pvb = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)vb0, cpar) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(vb0 >> 32), cpar) << 32);
      if (lane == i) { par0 = cpar; dep0 = cdep; tok0 = ctok; sc0 = csc; va0 = pva | (1ull << i); vb0 = pvb; }
    } else {
      const uint64_t pva = read_u64(va0, va1, cpar);
      const uint64_t pvb = read_u64(vb0, vb1, cpar);
      if (lane == (i & 63)) {
        const uint64_t nva = pva | (i < 64 ? (1ull << i) : 0ull);
        const uint64_t nvb = pvb | (i >= 64 ? (1ull << (i - 64)) : 0ull);
        if (i < 64) { par0 = cpar; dep0 = cdep; tok0 = ctok; sc0 = csc; va0 = nva; vb0 = nvb; }
        else        { par1 = cpar; dep1 = cdep; tok1 = ctok; sc1 = csc; va1 = nva; vb1 = nvb; }
      }
    }

    // Offer the new node's rank-0 child and its next-ranked sibling.
    uint64_t kc = 0, ks = 0;
    const float s_child = __fadd_rn(csc, lp_child);
    if (cdep < D && s_child > -INFINITY) kc = frontier_key(s_child, i, 0);
    const float s_sib = __fadd_rn(psc, lp_sib);
    if (crank + 1 < K && s_sib > -INFINITY) ks = frontier_key(s_sib, cpar, crank + 1);
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
    if (kLow) {
      if (lane == slot_a) { key0 = key_a; fd0 = dep_a; }
      if (lane == slot_b) { key0 = key_b; fd0 = dep_b; }
    } else {
      if (lane == (slot_a & 63)) {
        if (slot_a < 64) { key0 = key_a; fd0 = dep_a; } else { key1 = key_a; fd1 = dep_a; }
      }
      if (slot_b >= 0 && lane == (slot_b & 63)) {
        if (slot_b < 64) { key0 = key_b; fd0 = dep_b; } else { key1 = key_b; fd1 = dep_b; }
      }
    }
    return true;
  };
  // The first 64 nodes, then the rest; a frontier that runs empty ends the
  // build in either phase (the second starts only once 64 nodes exist).
  const int q_low = Q < kWave ? Q : kWave;
  while (n < q_low && pop(std::true_type{})) {
  }
  while (n >= kWave && n < Q && pop(std::false_type{})) {
  }

  // Children bitsets, then the links: first child = lowest child index; next
  // sibling = lowest child of the same parent above this node.
  if (lane > 0 && lane < n) atomicOr(&s_kids[par0][lane >> 6], 1ull << (lane & 63));
  if (lane + kWave < n) atomicOr(&s_kids[par1][1], 1ull << lane);
  __syncthreads();

  const int W = (Q + 63) >> 6;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + k * kWave;
    if (i >= Q) break;
    const size_t o = (size_t)b * Q + i;
    if (i < n) {
      const int p = k ? par1 : par0, d = k ? dep1 : dep0;
      const unsigned long long c0 = s_kids[i][0], c1 = s_kids[i][1];
      int fc = c0 ? __ffsll(c0) - 1 : (c1 ? 64 + __ffsll(c1) - 1 : -1);
      int ns = -1;
      if (i > 0) {
        unsigned long long s0 = s_kids[p][0], s1 = s_kids[p][1];
        // keep siblings with index > i
        if (i < 63) s0 &= ~0ull << (i + 1); else s0 = 0;
        if (i >= 64) s1 &= (i - 64 < 63) ? (~0ull << (i - 63)) : 0ull;
        ns = s0 ? __ffsll(s0) - 1 : (s1 ? 64 + __ffsll(s1) - 1 : -1);
      }
      node_token[o] = k ? tok1 : tok0;
      parent[o] = p;
      depth[o] = d;
      position[o] = (int32_t)((uint32_t)L + (uint32_t)d);
      first_child[o] = fc;
      next_sibling[o] = ns;
      score[o] = k ? sc1 : sc0;
      vis[o * W] = k ? va1 : va0;
      if (W > 1) vis[o * W + 1] = k ? vb1 : vb0;
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
