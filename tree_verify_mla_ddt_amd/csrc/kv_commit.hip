// kv_commit.hip -- append the accepted path to the committed prefix.
//
// The append step after greedy acceptance ("The Architecture of a
// Thousand-Parameter Decision ...", "What to Build New", item 5: paged
// MLA-latent KV cache, draft -> build -> verify -> accept -> append).  With one
// token per page the latent KV of every tree node already sits in its own pool
// slot, written during verification at position L + depth; committing the
// accepted root path is therefore a rewrite of the request's slot table: path
// node j (depth j) becomes prefix entry L + j, the other tree nodes' slots are
// handed back to the caller.
//
// One 64-lane wavefront per request; lane l handles tree entries / path
// positions l and l + 64.  Every value is read (slot table into LDS) before any
// entry is written, so the in-place rewrite never reads an entry it changed.
#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kMaxQ = 128;

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

__global__ __launch_bounds__(kWave) void kv_commit_kernel(
    int32_t* __restrict__ req_to_slot, int max_kv, int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accept_nodes, int Q, int32_t* __restrict__ freed_slots,
    int32_t* __restrict__ n_freed) {
  __shared__ int32_t s_old[kMaxQ];      // slot of tree node k before the rewrite
  __shared__ unsigned char s_acc[kMaxQ];  // tree node k is on the committed path
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* row = req_to_slot + (size_t)b * max_kv;
  const int L = clampi(prefix_len[b], 0, max_kv);
  const int cap = Q < max_kv - L ? Q : max_kv - L;
  const int n = clampi(n_nodes[b], 0, cap);
  const int a_in = clampi(accept_len[b], 0, n);

  // The path, cut before its first entry outside [0, n) or not above the one
  // before it.
  const size_t pb = (size_t)b * Q;
  const int j0 = lane, j1 = lane + kWave;
  const int p0 = j0 < a_in ? accept_nodes[pb + j0] : -1;
  const int p1 = j1 < a_in ? accept_nodes[pb + j1] : -1;
  const int prev0 = __shfl_up(p0, 1);
  const int last0 = __shfl(p0, kWave - 1);
  const int prev1 = lane == 0 ? last0 : __shfl_up(p1, 1);
  const bool ok0 = p0 >= 0 && p0 < n && (j0 == 0 || p0 > prev0);
  const bool ok1 = p1 >= 0 && p1 < n && p1 > prev1;
  const uint64_t bad0 = __ballot(j0 < a_in && !ok0);
  const uint64_t bad1 = __ballot(j1 < a_in && !ok1);
  int a = a_in;
  if (bad0) a = __ffsll((unsigned long long)bad0) - 1;
  else if (bad1) a = kWave + __ffsll((unsigned long long)bad1) - 1;

  // Old slots of the tree entries, and the committed-path marks.
  for (int k = lane; k < kMaxQ; k += kWave) {
    s_old[k] = k < n ? row[L + k] : -1;
    s_acc[k] = 0;
  }
  __syncthreads();
  if (j0 < a) s_acc[p0] = 1;
  if (j1 < a) s_acc[p1] = 1;
  __syncthreads();

  // Rewrite [L, L + n): the path's slots, then -1 for the entries past it.
  if (j0 < n) row[L + j0] = j0 < a ? s_old[p0] : -1;
  if (j1 < n) row[L + j1] = j1 < a ? s_old[p1] : -1;
  // Released slots in increasing node index, compacted through LDS.
  const bool f0 = j0 < n && !s_acc[j0];
  const bool f1 = j1 < n && !s_acc[j1];
  const uint64_t m0 = __ballot(f0), m1 = __ballot(f1);
  const unsigned below0 = __builtin_amdgcn_mbcnt_hi((unsigned)(m0 >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)m0, 0u));
  const unsigned below1 = __builtin_amdgcn_mbcnt_hi((unsigned)(m1 >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)m1, 0u));
  const int nf0 = __popcll(m0);
  __shared__ int32_t s_fr[kMaxQ];
  if (f0) s_fr[below0] = s_old[j0];
  if (f1) s_fr[nf0 + below1] = s_old[j1];
  __syncthreads();
  const int nfree = n - a;
  for (int k = lane; k < Q; k += kWave) freed_slots[pb + k] = k < nfree ? s_fr[k] : -1;
  if (lane == 0) {
    n_freed[b] = n - a;
    prefix_len[b] = L + a;
  }
}

}  // namespace

hipError_t launch_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                            const int32_t* n_nodes, const int32_t* accept_len,
                            const int32_t* accept_nodes, int B, int Q, int32_t* freed_slots,
                            int32_t* n_freed, hipStream_t stream) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3(B), dim3(kWave), 0, stream, req_to_slot, max_kv,
                     prefix_len, n_nodes, accept_len, accept_nodes, Q, freed_slots, n_freed);
  return hipGetLastError();
}

}  // namespace ddt
