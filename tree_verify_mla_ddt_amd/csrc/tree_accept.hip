// tree_accept.hip -- greedy follow-the-verified-tree acceptance on the GPU.
//
// Implements the tree_accept stage of "The Architecture of Closure ...", "The
// Table as a Decision Artifact": starting at the root, follow the child whose
// draft token equals the target model's greedy token at the current node, and
// commit the accepted draft tokens plus the target's token at the last one.
//
// One 64-lane wavefront per request; lane l holds nodes l and l+64.  Each step
// is one ballot over "my node is a child of cur and carries the wanted token";
// the lowest set bit is the next node, so duplicate sibling tokens resolve to
// the lowest index.  Node indices strictly increase along the walk, so it ends
// after at most Q steps whatever the input.
#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kMaxQ = 128;

__global__ __launch_bounds__(kWave) void tree_accept_kernel(
    const int32_t* __restrict__ node_token, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ target,
    int Q, int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ next_root) {
  __shared__ int32_t s_path[kMaxQ];
  __shared__ int32_t s_tok[kMaxQ];  // s_tok[k]: token of path node k+1 (= the target's token at node k)
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const size_t base = (size_t)b * Q;
  int nb = n_nodes[b];
  nb = nb < 1 ? 1 : (nb > Q ? Q : nb);

  int tok0 = 0, par0 = -2, tgt0 = 0, tok1 = 0, par1 = -2, tgt1 = 0;
  if (lane < Q) {
    tok0 = node_token[base + lane];
    par0 = parent[base + lane];
    tgt0 = target[base + lane];
  }
  if (lane + kWave < Q) {
    tok1 = node_token[base + lane + kWave];
    par1 = parent[base + lane + kWave];
    tgt1 = target[base + lane + kWave];
  }
  if (lane == 0) s_path[0] = 0;

  int cur = 0, len = 1, want = 0;
  for (;;) {
    // cur is the same in every lane: read the target token straight from its lane.
    want = __builtin_amdgcn_readlane(cur < kWave ? tgt0 : tgt1, cur & 63);
    const bool hit0 = lane < nb && lane > cur && par0 == cur && tok0 == want;
    const bool hit1 = lane + kWave < nb && lane + kWave > cur && par1 == cur && tok1 == want;
    const uint64_t b0 = __ballot(hit0);
    const uint64_t b1 = __ballot(hit1);
    if (b0 == 0 && b1 == 0) break;
    const int nxt = b0 ? (__ffsll((unsigned long long)b0) - 1)
                       : (kWave + __ffsll((unsigned long long)b1) - 1);
    if (lane == 0) {
      s_path[len] = nxt;
      s_tok[len - 1] = want;  // the matched child carries the wanted token
    }
    ++len;
    cur = nxt;
  }
  __syncthreads();

  for (int i = lane; i < Q; i += kWave) {
    accept_nodes[base + i] = i < len ? s_path[i] : -1;
    int t = -1;
    if (i + 1 < len) t = s_tok[i];
    else if (i + 1 == len) t = want;  // bonus token
    out_tokens[base + i] = t;
  }
  if (lane == 0) {
    accept_len[b] = len;
    next_root[b] = want;
  }
}

}  // namespace

hipError_t launch_tree_accept(const int32_t* node_token, const int32_t* parent,
                              const int32_t* n_nodes, const int32_t* target_argmax,
                              int B, int Q, int32_t* accept_len,
                              int32_t* accept_nodes, int32_t* out_tokens,
                              int32_t* next_root, hipStream_t stream) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(B), dim3(kWave), 0, stream, node_token,
                     parent, n_nodes, target_argmax, Q, accept_len, accept_nodes,
                     out_tokens, next_root);
  return hipGetLastError();
}

}  // namespace ddt
