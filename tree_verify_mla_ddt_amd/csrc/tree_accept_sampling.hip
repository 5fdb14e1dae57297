// tree_accept_sampling.hip -- sampling acceptance of a verified draft tree.
//
// The sampling-probability path of tree verification ("The Architecture of a
// Thousand-Parameter Decision ...", "What to Build New", item 2: normalized
// target probabilities at the tree nodes; "What to Reuse", item 3: target-only
// tree speculative sampling from the verified distribution; item 5: the
// temperature commit path).  Per request, with p = softmax(logits[node] / T):
// from the root, the children of the current node are tried in index order and
// a child with token t is accepted when coin[child] < p(t) / (1 - R), R the
// mass of the tokens rejected so far at that node; the walk moves to the
// accepted child.  When none is accepted the bonus token is the first entry of
// the residual (p without the rejected tokens) whose running sum exceeds
// coin_final times the residual mass.  A temperature that is not a finite
// value > 0, and a node whose largest logit is not finite, make the node greedy
// (a point mass on the lowest-index argmax).
//
// Two kernels on one stream:
//  * sampling_stats_kernel, one 256-thread workgroup per (node row, chunk)
//    (rows along the grid's x, so any batch fits): 16-byte loads of the chunk
//    kept in registers; one pass gives each thread's max and sum of
//    exp((x - max) / T), combined into the chunk's, and the threads holding
//    the chunk max find its lowest index.  This pass reads every live node's
//    logits once and bounds the path by HBM bandwidth.
//  * sampling_accept_kernel, one workgroup per request: combines the chunk
//    statistics of every node (staged in LDS), reads the one logit each
//    child's acceptance needs, walks the tree on one wavefront (a DPP prefix
//    sum over the siblings gives each one's rejected mass, a ballot the first
//    accepted), then draws the bonus token: the chunk holding the draw comes
//    from the chunks' residual masses, its residual weights are staged in LDS,
//    and a block-wide scan over runs of entries finds the token.
#include <float.h>

#include "logit_rows.h"

namespace ddt {
namespace {

constexpr int kMaxQ = 128;
constexpr int kStatBatch = 1024;  // chunk records staged in LDS at a time
constexpr int kSerialChunks = 16;  // up to this many chunks a thread combines a node alone
static_assert(kRowChunksMax <= kStatBatch, "a batch holds at least one node");
constexpr float kLog2e = 1.4426950408889634f;

struct ChunkStat {
  float m;   // chunk max (NaN counted as -inf)
  float s;   // sum of exp((x - m) / T) over the chunk (0 for greedy requests)
  int amax;  // lowest row index holding m
  int pad;
};

// exp((x - ref) / T) with k2 = log2(e) / T: exactly 1 at x == ref (also when
// k2 overflowed), 0 for x = -inf.  x is never NaN here.
__device__ __forceinline__ float weight(float x, float ref, float k2) {
  const float d = x - ref;
  return d == 0.0f ? 1.0f : exp2f(d * k2);
}

__device__ __forceinline__ float no_nan(float x) { return x != x ? -INFINITY : x; }

__device__ __forceinline__ int clamp_nodes(int n, int Q) { return n < 1 ? 1 : (n > Q ? Q : n); }

__device__ __forceinline__ bool sampled_temperature(float T) { return T > 0.0f && T <= FLT_MAX; }

// v from the lane CTRL selects, 0 where that lane is outside the row or the row
// is masked off (DPP with bound_ctrl off and a zero old value).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive sum over lanes 0..lane with DPP row shifts and row broadcasts.
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp0<0x111, 0xF>(v);  // row_shr:1
  v += dpp0<0x112, 0xF>(v);  // row_shr:2
  v += dpp0<0x114, 0xF>(v);  // row_shr:4
  v += dpp0<0x118, 0xF>(v);  // row_shr:8
  v += dpp0<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp0<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <typename E>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 8 : 5)))
void sampling_stats_kernel(
    const E* __restrict__ logits, int V, int Q, const float* __restrict__ temperature,
    const int32_t* __restrict__ n_nodes, int S, int C, ChunkStat* __restrict__ ws) {
  constexpr int kN = Vec16<E>::kN;
  constexpr int kVPT = kRowChunkMax / kN / kRowThreads;
  constexpr int kW = kVPT * 4;
  __shared__ float s_m[kRowThreads / kWave];
  __shared__ int s_a[kRowThreads / kWave];
  __shared__ float s_s[kRowThreads / kWave];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int c = blockIdx.y;
  const int b = row / Q, node = row - b * Q;
  if (node >= clamp_nodes(n_nodes[b], Q)) return;  // a pad slot: never read
  const float T = temperature[b];
  const bool sampled = sampled_temperature(T);
  // log2(e) / T, kept finite so that (x - ref) * k2 is 0 at x == ref for any T.
  const float k2 = sampled ? fminf(kLog2e / T, FLT_MAX) : 0.0f;
  const int v0 = c * C;
  const int n = V - v0 < C ? V - v0 : C;  // > 0: the host sizes chunks so none is empty
  const E* src = logits + (long long)row * V + v0;

  // The chunk in registers as loaded (entry j of group u of a thread is chunk
  // entry (tid + 256*u)*kN + j, -inf where the chunk has none).
  uint32_t w[kW];
  load_chunk_words<E, kVPT>(src, n, tid, w);
  auto val = [&](int u, int j) -> float { return word_entry<E>(w[4 * u + j / (kN / 4)], j); };

  // The thread's max tm and, for a sampled request, its sum ts of
  // exp((x - tm) / T), in one pass (the sum is rescaled when a group raises the
  // max).  A NaN never wins a comparison, so it counts as -inf for the max; in
  // the sum it turns ts into NaN, and only then does the thread sum again,
  // skipping NaN entries.
  float tm = -INFINITY, ts = 0.0f;
#pragma unroll
  for (int u = 0; u < kVPT; ++u) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const float x = val(u, j);
      lm = x > lm ? x : lm;
    }
    if (sampled) {
      if (lm > tm) {
        ts *= __builtin_amdgcn_exp2f((tm - lm) * k2);  // 0 while tm is -inf
        tm = lm;
      }
      if (tm > -INFINITY && tm < INFINITY) {
#pragma unroll
        for (int j = 0; j < kN; ++j) ts += __builtin_amdgcn_exp2f((val(u, j) - tm) * k2);
      }
    } else {
      tm = lm > tm ? lm : tm;
    }
  }
  mark_rewritten<kW>(w);
  if (ts != ts && tm < INFINITY) {
    ts = 0.0f;
#pragma unroll
    for (int u = 0; u < kVPT; ++u)
#pragma unroll
      for (int j = 0; j < kN; ++j) {
        const float x = val(u, j);
        if (x == x) ts += __builtin_amdgcn_exp2f((x - tm) * k2);
      }
  }
  float m = wave_max(tm);
  if (lane == 0) s_m[wave] = m;
  __syncthreads();
  m = s_m[0];
#pragma unroll
  for (int q = 1; q < kRowThreads / kWave; ++q) m = fmaxf(m, s_m[q]);

  // The lowest index holding the max: only threads whose max equals it look,
  // in index order.  If the max is -inf every entry counts as -inf (NaN
  // included), so it is the chunk's first entry.
  int a = 0x7FFFFFFF;
  if (m == -INFINITY) {
    a = 0;
  } else if (tm == m) {
    mark_rewritten<kW>(w);
#pragma unroll
    for (int u = kVPT - 1; u >= 0; --u)
#pragma unroll
      for (int j = kN - 1; j >= 0; --j)
        if (val(u, j) == m) a = (tid + kRowThreads * u) * kN + j;
  }
  a = wave_min(a);
  // The thread's share of the chunk's sum of exp((x - m) / T) (m >= tm).
  float part = 0.0f;
  if (sampled && m > -INFINITY && m < INFINITY && tm > -INFINITY)
    part = ts * __builtin_amdgcn_exp2f((tm - m) * k2);
  part = wave_sum(part);
  if (lane == 0) {
    s_a[wave] = a;
    s_s[wave] = part;
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f;
    int am = s_a[0];
#pragma unroll
    for (int q = 0; q < kRowThreads / kWave; ++q) {
      t += s_s[q];
      am = min(am, s_a[q]);
    }
    ChunkStat st;
    st.m = m;
    st.s = t;
    st.amax = v0 + am;
    st.pad = 0;
    ws[(long long)row * S + c] = st;
  }
}

template <typename E>
__global__ __launch_bounds__(kRowThreads) void sampling_accept_kernel(
    const E* __restrict__ logits, int V, int Q, const float* __restrict__ temperature,
    const int32_t* __restrict__ node_token, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ n_nodes, const float* __restrict__ coins,
    const float* __restrict__ coin_final, int S, int C, const ChunkStat* __restrict__ ws,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ next_root) {
  __shared__ float s_M[kMaxQ], s_Z[kMaxQ], s_e[kMaxQ], s_coin[kMaxQ];
  __shared__ int s_amax[kMaxQ], s_tok[kMaxQ], s_par[kMaxQ], s_greedy[kMaxQ];
  __shared__ int s_path[kMaxQ];
  __shared__ int s_rtok[kMaxQ];  // tokens rejected at the last node, with their masses
  __shared__ float s_re[kMaxQ];
  __shared__ float s_w[kRowChunksMax];
  __shared__ float s_r[kRowChunkMax];  // residual weights of the chunk holding the bonus draw
  __shared__ ChunkStat s_cs[kStatBatch];  // chunk records of a batch of nodes
  __shared__ int s_len, s_nrej, s_chunk, s_first, s_lastpos, s_bonus;
  __shared__ float s_tgt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int n = clamp_nodes(n_nodes[b], Q);
  const float T = temperature[b];
  const bool sampled = sampled_temperature(T);
  const float k2 = sampled ? kLog2e / T : 0.0f;
  const E* rows = logits + (long long)b * Q * V;

  // Target statistics of every node: the chunks' maxima and sums combined.  The
  // chunk records of a batch of nodes are first staged in LDS by all threads
  // (one round trip to memory per batch, not one per node); then each thread
  // combines one node's chunks in chunk order when there are few chunks, else
  // each wavefront one node at a time with the lanes over the chunks.
  if (tid < n) {  // requested first: the statistics below do not depend on them
    s_tok[tid] = node_token[b * Q + tid];
    s_par[tid] = parent[b * Q + tid];
    s_coin[tid] = coins[b * Q + tid];
  }
  // Nodes per batch (S <= kRowChunksMax <= kStatBatch), one per thread.
  const int npb = min(kStatBatch / S, kRowThreads);
  for (int nb0 = 0; nb0 < n; nb0 += npb) {
    const int nn = min(npb, n - nb0);
    const ChunkStat* src = ws + ((long long)b * Q + nb0) * S;
#pragma unroll 4
    for (int i = tid; i < nn * S; i += kRowThreads) s_cs[i] = src[i];
    __syncthreads();
    if (S <= kSerialChunks) {
      if (tid < nn) {  // one node per thread, its chunks in order
        const ChunkStat* st = s_cs + tid * S;
        const ChunkStat f = st[0];
        float M = f.m, Z = f.s;
        int am = f.amax;
        for (int c = 1; c < S; ++c) {
          const ChunkStat g = st[c];
          if (g.m > M) {
            Z = (M > -INFINITY ? Z * weight(M, g.m, k2) : 0.0f) + g.s;
            M = g.m;
            am = g.amax;
          } else if (g.m > -INFINITY) {
            Z += g.s * weight(g.m, M, k2);
          }
        }
        const int node = nb0 + tid;
        const bool greedy = !sampled || !(M > -INFINITY && M < INFINITY);
        s_M[node] = M;
        s_Z[node] = greedy ? 1.0f : Z;
        s_amax[node] = am;
        s_greedy[node] = greedy ? 1 : 0;
      }
    } else {
      // One node per wavefront at a time, lanes over its chunks.
      for (int k = wave; k < nn; k += kRowThreads / kWave) {
        const ChunkStat* st = s_cs + k * S;
        float M = -INFINITY, Z = 0.0f;
        int am = 0x7FFFFFFF;
        for (int c = lane; c < S; c += kWave) {
          const ChunkStat g = st[c];
          if (g.m > M) {
            Z = (M > -INFINITY ? Z * weight(M, g.m, k2) : 0.0f) + g.s;
            M = g.m;
            am = g.amax;
          } else if (g.m == M) {
            Z += g.s;
            am = min(am, g.amax);
          } else if (g.m > -INFINITY) {
            Z += g.s * weight(g.m, M, k2);
          }
        }
        // Every lane's (M, Z) against the wave's max; the lowest index among
        // the lanes holding the max (the lowest chunk's when all are -inf).
        const float Mw = wave_max(M);
        const float z = M > -INFINITY ? Z * weight(M, Mw, k2) : 0.0f;
        const float Zw = wave_sum(z);
        int a = M == Mw ? am : 0x7FFFFFFF;
        a = wave_min(a);
        if (lane == 0) {
          const int node = nb0 + k;
          const bool greedy = !sampled || !(Mw > -INFINITY && Mw < INFINITY);
          s_M[node] = Mw;
          s_Z[node] = greedy ? 1.0f : Zw;
          s_amax[node] = a;
          s_greedy[node] = greedy ? 1 : 0;
        }
      }
    }
    __syncthreads();
  }
  // Unnormalized target mass of each child's token at its parent.
  if (tid < n) {
    const int p = s_par[tid], t = s_tok[tid];
    float e = 0.0f;
    if (tid >= 1 && p >= 0 && p < tid && t >= 0 && t < V) {
      if (s_greedy[p])
        e = t == s_amax[p] ? 1.0f : 0.0f;
      else
        e = weight(no_nan(to_f32(rows[(long long)p * V + t])), s_M[p], k2);
    }
    s_e[tid] = e;
  }
  __syncthreads();

  // The walk, on wavefront 0: lane l looks after nodes l and l + 64.
  if (wave == 0) {
    // Per-node values of nodes lane and lane + 64, read once.
    const bool in_a = lane < n, in_b = lane + kWave < n;
    const int tok_a = in_a ? s_tok[lane] : -1, tok_b = in_b ? s_tok[lane + kWave] : -1;
    const int par_a = in_a ? s_par[lane] : -1, par_b = in_b ? s_par[lane + kWave] : -1;
    const float e_a = in_a ? s_e[lane] : 0.0f, e_b = in_b ? s_e[lane + kWave] : 0.0f;
    const float coin_a = in_a ? s_coin[lane] : 0.0f, coin_b = in_b ? s_coin[lane + kWave] : 0.0f;
    const uint64_t below = (1ull << lane) - 1;
    int cur = 0, len = 1;
    if (lane == 0) s_path[0] = 0;
    for (;;) {
      const int c0 = lane, c1 = lane + kWave;
      const bool ch0 = in_a && c0 > cur && par_a == cur;
      const bool ch1 = in_b && c1 > cur && par_b == cur;
      const uint64_t m0 = __ballot(ch0), m1 = __ballot(ch1);
      float e0 = ch0 ? e_a : 0.0f, e1 = ch1 ? e_b : 0.0f;
      // A token already tried at this node (an earlier sibling with the same
      // token) has no mass left.  The siblings are visited in index order by a
      // wave-uniform loop; their tokens come from registers.
      bool dup0 = false, dup1 = false;
      for (uint64_t mm = m0; mm; mm &= mm - 1) {
        const int sl = __ffsll((unsigned long long)mm) - 1;
        const int ts = __builtin_amdgcn_readlane(tok_a, sl);
        dup0 |= lane > sl && tok_a == ts;
        dup1 |= tok_b == ts;  // every sibling below 64 precedes c1
      }
      for (uint64_t mm = m1; mm; mm &= mm - 1) {
        const int sl = __ffsll((unsigned long long)mm) - 1;
        const int ts = __builtin_amdgcn_readlane(tok_b, sl);
        dup1 |= lane > sl && tok_b == ts;
      }
      if (dup0) e0 = 0.0f;
      if (dup1) e1 = 0.0f;
      // Mass of the earlier siblings, in index order.
      const float i0 = wave_incl_scan(e0);
      const float tot0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(i0), kWave - 1));
      const float i1 = wave_incl_scan(e1);
      const float r0 = i0 - e0;
      const float r1 = tot0 + (i1 - e1);
      bool a0, a1;
      if (s_greedy[cur]) {
        a0 = e0 > 0.0f;
        a1 = e1 > 0.0f;
      } else {
        // coin < e / (Z - r), written without the division.
        const float Z = s_Z[cur];
        a0 = e0 > 0.0f && coin_a * (Z - r0) < e0;
        a1 = e1 > 0.0f && coin_b * (Z - r1) < e1;
      }
      const uint64_t acc0 = __ballot(a0), acc1 = __ballot(a1);
      int next = -1;
      if (acc0)
        next = __ffsll((unsigned long long)acc0) - 1;
      else if (acc1)
        next = kWave + __ffsll((unsigned long long)acc1) - 1;
      if (next < 0) {
        // Every child with mass was tried and rejected: list them for the bonus draw.
        const uint64_t rj0 = __ballot(e0 > 0.0f), rj1 = __ballot(e1 > 0.0f);
        const int base1 = __popcll(rj0);
        if (e0 > 0.0f) {
          const int k = __popcll(rj0 & below);
          s_rtok[k] = tok_a;
          s_re[k] = e0;
        }
        if (e1 > 0.0f) {
          const int k = base1 + __popcll(rj1 & below);
          s_rtok[k] = tok_b;
          s_re[k] = e1;
        }
        if (lane == 0) {
          s_nrej = base1 + __popcll(rj1);
          s_len = len;
        }
        break;
      }
      if (lane == 0) s_path[len] = next;
      ++len;
      cur = next;  // strictly increasing, so the walk ends within n steps
    }
  }
  if (tid == 0) {
    s_first = 0x7FFFFFFF;
    s_lastpos = -1;
  }
  __syncthreads();

  const int len = s_len, cur = s_path[len - 1];
  if (s_greedy[cur]) {
    if (tid == 0) s_bonus = s_amax[cur];
  } else {
    // The bonus token from the residual distribution at `cur`.
    const int nrej = s_nrej;
    const float M = s_M[cur];
    const ChunkStat* st = ws + ((long long)b * Q + cur) * S;
    for (int c = tid; c < S; c += kRowThreads) {
      const ChunkStat g = st[c];
      const float mass = g.m > -INFINITY ? g.s * weight(g.m, M, k2) : 0.0f;
      float w = mass;
      for (int j = 0; j < nrej; ++j) {
        const int t = s_rtok[j];
        if (t >= c * C && t < c * C + C) w -= s_re[j];
      }
      // What is left below the rounding of the chunk's own sum is nothing.
      s_w[c] = w > 1e-6f * mass ? w : 0.0f;
    }
    __syncthreads();
    if (tid == 0) {
      float Zr = 0.0f;
      for (int c = 0; c < S; ++c) Zr += s_w[c];
      const float target = coin_final[b] * Zr;
      float cum = 0.0f;
      int ch = -1, last = -1;
      for (int c = 0; c < S; ++c) {
        if (!(s_w[c] > 0.0f)) continue;
        last = c;
        if (cum + s_w[c] > target) {
          ch = c;
          break;
        }
        cum += s_w[c];
      }
      // No crossing (a draw >= 1, NaN, or rounding): the last entry left.
      s_chunk = ch >= 0 ? ch : last;
      s_tgt = ch >= 0 ? target - cum : INFINITY;
    }
    __syncthreads();
    const int ch = s_chunk;
    if (ch < 0) {
      if (tid == 0) s_bonus = s_amax[cur];  // no residual mass at all
    } else {
      // The chunk's residual weights, staged in LDS with coalesced loads: each
      // entry's weight against the node's max, 0 for the rejected tokens.
      const int v0 = ch * C;
      const int nc = V - v0 < C ? V - v0 : C;
      const E* src = rows + (long long)cur * V + v0;
      {
        // All of a thread's loads are issued before any is used (entry j of
        // group u is chunk entry (tid + 256*u)*kN + j, -inf past the chunk).
        constexpr int kN = Vec16<E>::kN;
        constexpr int kVPT = kRowChunkMax / kN / kRowThreads;
        uint32_t w[kVPT * 4];
        load_chunk_words<E, kVPT>(src, nc, tid, w);
#pragma unroll
        for (int u = 0; u < kVPT; ++u) {
          const int e0 = (tid + kRowThreads * u) * kN;
          if (e0 < nc) {
#pragma unroll
            for (int j = 0; j < kN; ++j)
              s_r[e0 + j] = weight(no_nan(word_entry<E>(w[4 * u + j / (kN / 4)], j)), M, k2);
          }
        }
      }
      __syncthreads();
      if (tid < nrej) {
        const int t = s_rtok[tid] - v0;
        if (t >= 0 && t < nc) s_r[t] = 0.0f;
      }
      __syncthreads();
      // Thread t scans a run of consecutive entries of the chunk.
      const int run = (nc + kRowThreads - 1) / kRowThreads;
      const int lo = min(nc, tid * run), hi = min(nc, lo + run);
      float sum = 0.0f;
      int lastpos = -1;
      for (int i = lo; i < hi; ++i) {
        const float r = s_r[i];
        if (r > 0.0f) {
          sum += r;
          lastpos = v0 + i;
        }
      }
      // Exclusive scan of the runs' sums over the block.
      float inc = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
      }
      if (lane == kWave - 1) s_w[wave] = inc;  // the chunk masses are no longer needed
      __syncthreads();
      float excl = __shfl_up(inc, 1);
      if (lane == 0) excl = 0.0f;
      for (int w = 0; w < wave; ++w) excl += s_w[w];
      const float tgt = s_tgt;
      // The first run whose end passes the target holds the draw; its own
      // running sum ends at exactly the value tested here.
      if (excl + sum > tgt) atomicMin(&s_first, tid);
      if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
      __syncthreads();
      if (tid == s_first) {
        float part = 0.0f;
        for (int i = lo; i < hi; ++i) {
          const float r = s_r[i];
          if (r > 0.0f) {
            part += r;
            if (excl + part > tgt) {
              s_bonus = v0 + i;
              break;
            }
          }
        }
      } else if (tid == 0 && s_first == 0x7FFFFFFF) {
        s_bonus = s_lastpos >= 0 ? s_lastpos : s_amax[cur];
      }
    }
  }
  __syncthreads();

  const int bonus = s_bonus;
  if (tid < Q) {
    accept_nodes[b * Q + tid] = tid < len ? s_path[tid] : -1;
    int o = -1;
    if (tid < len - 1)
      o = s_tok[s_path[tid + 1]];
    else if (tid == len - 1)
      o = bonus;
    out_tokens[b * Q + tid] = o;
  }
  if (tid == 0) {
    accept_len[b] = len;
    next_root[b] = bonus;
  }
}

}  // namespace

SamplingPlan plan_tree_accept_sampling(int B, int Q, int V, int num_cu) {
  const RowChunks rc = plan_row_chunks((long long)B * Q, V, num_cu, 2);
  SamplingPlan p;
  p.chunks = rc.chunks;
  p.chunk = rc.chunk;
  p.ws_bytes = (size_t)B * Q * rc.chunks * sizeof(ChunkStat);
  return p;
}

size_t tree_accept_sampling_ws_bound(int B, int Q) {
  return (size_t)B * Q * kRowChunksMax * sizeof(ChunkStat);
}

hipError_t launch_tree_accept_sampling(int dtype, const void* logits, int V,
                                       const float* temperature, const int32_t* node_token,
                                       const int32_t* parent, const int32_t* n_nodes,
                                       const float* coins, const float* coin_final, int B, int Q,
                                       int32_t* accept_len, int32_t* accept_nodes,
                                       int32_t* out_tokens, int32_t* next_root, void* workspace,
                                       const SamplingPlan& plan, hipStream_t stream) {
  ChunkStat* ws = static_cast<ChunkStat*>(workspace);
  const dim3 grid1(B * Q, plan.chunks);
  if (dtype == 1)
    hipLaunchKernelGGL(sampling_stats_kernel<uint16_t>, grid1, dim3(kRowThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, Q, temperature, n_nodes,
                       plan.chunks, plan.chunk, ws);
  else
    hipLaunchKernelGGL(sampling_stats_kernel<float>, grid1, dim3(kRowThreads), 0, stream,
                       static_cast<const float*>(logits), V, Q, temperature, n_nodes,
                       plan.chunks, plan.chunk, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1)
    hipLaunchKernelGGL(sampling_accept_kernel<uint16_t>, dim3(B), dim3(kRowThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, Q, temperature, node_token,
                       parent, n_nodes, coins, coin_final, plan.chunks, plan.chunk, ws,
                       accept_len, accept_nodes, out_tokens, next_root);
  else
    hipLaunchKernelGGL(sampling_accept_kernel<float>, dim3(B), dim3(kRowThreads), 0, stream,
                       static_cast<const float*>(logits), V, Q, temperature, node_token, parent,
                       n_nodes, coins, coin_final, plan.chunks, plan.chunk, ws, accept_len,
                       accept_nodes, out_tokens, next_root);
  return hipGetLastError();
}

}  // namespace ddt
