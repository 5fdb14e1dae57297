// draft_topk.hip -- per-depth top-K extraction from drafter logits.
//
// The "per-depth top-k logit extraction" of the fused draft helpers ("The
// Architecture of a Thousand-Parameter Decision ...", "What to Build New",
// item 4), producing the tree builder's input: for every (request, depth) row
// of logits over the vocabulary, log-softmax and the K largest logits (largest
// first, lower index first among equal logits).
//
// It is one streaming read of the logits, so HBM bandwidth bounds it.  Rows
// are cut into chunks of at most 12288 entries so that the grid fills the chip
// even for a handful of rows:
//  * draft_topk_partial_kernel (one 256-thread workgroup per chunk): 16-byte
//    loads kept in registers as loaded words; one pass gives each thread's max
//    and its sum of exp(x - max), combined into the chunk's.  Each wave's K-th
//    largest thread max has K entries at or above it, so the largest of the
//    four bounds the chunk's K-th entry from below; the entries at or above it
//    -- a few times K on ordinary rows -- are gathered into LDS as
//    order-preserving (key, index) pairs and ranked (each candidate counts the
//    larger ones).  When the bound is -inf or wide ties make the candidates too
//    many, a radix selection (four 8-bit digits, LDS histograms) finds the K-th
//    key exactly and the lowest-index ties are taken in index order;
//  * draft_topk_merge_kernel (one workgroup per row): the chunks' log-sum-exps
//    combined, their candidates ranked (or bitonic-sorted in LDS when there are
//    more than 1024) and the first K written as log-probs and ids.
#include "logit_rows.h"

namespace ddt {
namespace {

constexpr int kTopkThreads = kRowThreads;
constexpr int kMaxChunk = kRowChunkMax;  // entries of one chunk (keys held in registers)
constexpr int kMaxChunks = kRowChunksMax;
constexpr int kMaxK = 64;
constexpr int kCandCap = 1024;    // candidates of the threshold pass held in LDS

// Order-preserving key of a logit (larger logit -> larger key).  NaN counts as
// -inf and -0 as +0, so equal logits get equal keys.  Every key is > 0.
__device__ __forceinline__ uint32_t logit_key(float x) {
  if (x != x) x = -INFINITY;
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Candidate: key in the high word, ~index in the low word (larger = better).
__device__ __forceinline__ uint64_t cand(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// Descending bitonic sort of P (a power of two) entries in LDS by all threads.
template <typename U>
__device__ __forceinline__ void bitonic_desc(U* a, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += kTopkThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const U x = a[lo], y = a[hi];
        if ((x < y) == desc) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Writes the kk best of the nc distinct candidates in a[0..nc) to out[0..kk),
// best first: each candidate's rank is the number of larger ones (reads of one
// LDS word by a whole wave are broadcasts).  For up to a few hundred entries
// this beats a bitonic sort's barrier per step.
__device__ __forceinline__ void rank_select(const uint64_t* a, int nc, int kk, uint64_t* out) {
  for (int i = threadIdx.x; i < nc; i += kTopkThreads) {
    const uint64_t x = a[i];
    int r = 0;
    for (int j = 0; j < nc; ++j) r += a[j] > x ? 1 : 0;
    if (r < kk) out[r] = x;
  }
}

template <typename T>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 8 : 5))) void draft_topk_partial_kernel(
    const T* __restrict__ logits, int V, int K, int S, int C, uint64_t* __restrict__ ws_cand,
    float2* __restrict__ ws_ms) {
  constexpr int kN = Vec16<T>::kN;
  constexpr int kVPT = kMaxChunk / kN / kTopkThreads;  // 16-byte loads per thread at most
  static_assert(kVPT * kN * kTopkThreads == kMaxChunk, "chunk tiling");
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ uint64_t s_cand[kCandCap];
  __shared__ uint32_t s_hist[256];
  __shared__ float s_max[kTopkThreads / kWave];
  __shared__ float s_sum[kTopkThreads / kWave];
  __shared__ uint32_t s_wtau[kTopkThreads / kWave];
  __shared__ int s_pick[2];  // digit, count above it
  __shared__ int s_cnt;
  __shared__ int s_wties[kTopkThreads / kWave];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const long long row = blockIdx.y;
  const int v0 = c * C;
  const int n = V - v0 < C ? V - v0 : C;  // > 0: the host sizes S so every chunk has entries
  const T* src = logits + row * (long long)V + v0;

  // The chunk stays in registers as loaded (entry j of group u of a thread is
  // chunk entry (tid + 256*u)*kN + j, -inf where the chunk has none).
  constexpr int kW = kVPT * 4;
  uint32_t w[kW];
  load_chunk_words<T, kVPT>(src, n, tid, w);
  auto val = [&](int u, int j) -> float { return word_entry<T>(w[4 * u + j / (kN / 4)], j); };
  auto entry = [&](int u, int j) -> int { return (tid + kTopkThreads * u) * kN + j; };
  auto refresh = [&]() { mark_rewritten<kW>(w); };

  // The thread's max tm and sum ts of exp(x - tm), in one pass over its loads
  // (the sum is rescaled when a load raises the max).  A NaN never wins a
  // comparison, so it counts as -inf for the max; in the sum it turns ts into
  // NaN, and only then does the thread sum again, skipping NaN entries.
  float tm = -INFINITY, ts = 0.0f;
#pragma unroll
  for (int u = 0; u < kVPT; ++u) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const float x = val(u, j);
      lm = x > lm ? x : lm;
    }
    if (lm > tm) {
      ts *= __builtin_amdgcn_exp2f((tm - lm) * kLog2e);  // 0 while tm is -inf
      tm = lm;
    }
    if (tm > -INFINITY) {
      const float mk = tm * kLog2e;
#pragma unroll
      for (int j = 0; j < kN; ++j) ts += __builtin_amdgcn_exp2f(__builtin_fmaf(val(u, j), kLog2e, -mk));
    }
  }
  refresh();
  if (ts != ts) {
    ts = 0.0f;
    const float mk = tm * kLog2e;
#pragma unroll
    for (int u = 0; u < kVPT; ++u)
#pragma unroll
      for (int j = 0; j < kN; ++j) {
        const float x = val(u, j);
        if (x == x) ts += __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mk));
      }
  }
  // Butterfly shuffles here rather than the DPP reductions: two per workgroup,
  // and the DPP form's registers would push this kernel past 64 VGPRs.
  float wm = tm;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
  if (lane == 0) s_max[wave] = wm;

  // Threshold: each wave sorts its threads' maxima (lane-exchange bitonic
  // network, descending); the kk-th largest of a wave has at least kk entries
  // at or above it, so the largest of the four is a lower bound of the chunk's
  // kk-th largest entry, and the entries at or above it -- at most a few times
  // kk on ordinary rows -- hold the chunk's answer.
  const int kk = K < n ? K : n;
  uint32_t v = logit_key(tm);
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, stride);
      const bool desc = (lane & size) == 0 || size == kWave;
      const bool lower = (lane & stride) == 0;
      v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  if (lane == kk - 1) s_wtau[wave] = v;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  float M = s_max[0];
  uint32_t tau = s_wtau[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / kWave; ++w) {
    M = fmaxf(M, s_max[w]);
    tau = s_wtau[w] > tau ? s_wtau[w] : tau;
  }
  // The thread's share of the chunk's sum of exp(x - M) (M >= tm).
  float part = tm > -INFINITY ? ts * __builtin_amdgcn_exp2f((tm - M) * kLog2e) : 0.0f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) s_sum[wave] = part;

  // Fast path (threshold above -inf): threads whose max reaches it gather their
  // entries at or above it; NaN and missing entries never qualify.
  refresh();
  const bool fast = tau > logit_key(-INFINITY);
  const float tau_f = key_value(tau);
  if (fast && tm >= tau_f) {
#pragma unroll
    for (int u = 0; u < kVPT; ++u)
#pragma unroll
      for (int j = 0; j < kN; ++j) {
        const float x = val(u, j);
        if (x >= tau_f) {
          const int at = atomicAdd(&s_cnt, 1);
          if (at < kCandCap) s_cand[at] = cand(logit_key(x), v0 + entry(u, j));
        }
      }
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kTopkThreads / kWave; ++w) t += s_sum[w];
    ws_ms[row * S + c] = make_float2(M, t);
  }
  uint64_t* out = ws_cand + (row * S + c) * (long long)K;
  const int nc = fast ? s_cnt : kCandCap + 1;
  if (nc <= kCandCap) {
    rank_select(s_cand, nc, kk, out);
    for (int j = kk + tid; j < K; j += kTopkThreads) out[j] = 0;
    return;
  }

  // Slow path (the threshold is -inf, or many entries tie at it): radix
  // selection of the kk-th largest key over the registers, most significant
  // digit first; `need` counts how many keys equal to or above the selected
  // prefix are still wanted.  Key 0 marks a missing entry (every real key is > 0).
  refresh();
  auto key_at = [&](int u, int j) -> uint32_t {
    return entry(u, j) < n ? logit_key(val(u, j)) : 0u;
  };
  uint32_t prefix = 0, mask = 0;
  int need = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    refresh();  // keys are formed again in every pass, never kept
    s_hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kVPT; ++u)
#pragma unroll
      for (int j = 0; j < kN; ++j) {
        const uint32_t k = key_at(u, j);
        if (k != 0 && (k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
      }
    __syncthreads();
    if (wave == 0) {
      // Bins 255..0 as 4 per lane, lane 0 holding the top ones.
      int h[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = (int)s_hist[255 - (lane * 4 + j)];
        tot += h[j];
      }
      // Inclusive scan of the per-lane totals (counts from the top).
      int inc = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
      }
      const int exc = inc - tot;
      const uint64_t hit = __ballot(exc < need && inc >= need);
      const int wl = __ffsll((unsigned long long)hit) - 1;
      if (lane == wl) {
        int above = exc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above + h[j] >= need) {
            s_pick[0] = 255 - (lane * 4 + j);
            s_pick[1] = above;
            break;
          }
          above += h[j];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_pick[0] << shift;
    mask |= 255u << shift;
    need -= s_pick[1];
    __syncthreads();
  }
  // prefix is now the kk-th largest key; `need` of the keys equal to it are
  // taken (the lowest indices), with every key above it.
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  refresh();
#pragma unroll
  for (int u = 0; u < kVPT; ++u)
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const uint32_t k = key_at(u, j);
      if (k > prefix) out[atomicAdd(&s_cnt, 1)] = cand(k, v0 + entry(u, j));
    }
  // Ties in index order: the chunk is read again (from the caches) 256
  // consecutive entries at a time.
  int taken = 0;
  const int base_gt = kk - need;
  for (int b0 = 0; b0 < n && taken < need; b0 += kTopkThreads) {
    const int i = b0 + tid;
    const bool tie = i < n && logit_key(to_f32(src[i])) == prefix;
    const uint64_t bal = __ballot(tie);
    if (lane == 0) s_wties[wave] = __popcll(bal);
    __syncthreads();
    int before = taken;
    for (int w = 0; w < wave; ++w) before += s_wties[w];
    const int rank = before + (int)__builtin_amdgcn_mbcnt_hi(
                                  (unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
    if (tie && rank < need) out[base_gt + rank] = cand(prefix, v0 + i);
    int tot = 0;
    for (int w = 0; w < kTopkThreads / kWave; ++w) tot += s_wties[w];
    taken += tot;
    __syncthreads();
  }
  // Chunks shorter than K pad with 0 (below every real candidate).
  for (int j = kk + tid; j < K; j += kTopkThreads) out[j] = 0;
}

__global__ __launch_bounds__(kTopkThreads) void draft_topk_merge_kernel(
    int K, int S, const uint64_t* __restrict__ ws_cand, const float2* __restrict__ ws_ms,
    float* __restrict__ topk_logp, int32_t* __restrict__ topk_ids) {
  __shared__ uint64_t s_c[kMaxChunks * kMaxK];  // 64 KiB
  __shared__ float s_lse;
  const int tid = threadIdx.x;
  const long long row = blockIdx.x;
  const int n = S * K;
  int P = 1;
  while (P < n) P <<= 1;
  const uint64_t* src = ws_cand + row * (long long)S * K;
  for (int i = tid; i < P; i += kTopkThreads) s_c[i] = i < n ? src[i] : 0ull;
  // Combined log-sum-exp of the chunks (each chunk: max, sum of exp(x - max)),
  // one chunk per thread.
  static_assert(kMaxChunks <= kTopkThreads, "one chunk per thread");
  __shared__ float s_rm[kTopkThreads / kWave];
  __shared__ float s_rs[kTopkThreads / kWave];
  const int lane = tid & 63, wave = tid >> 6;
  float cm = -INFINITY, cs = 0.0f;
  if (tid < S) {
    const float2 ms = ws_ms[row * S + tid];
    cm = ms.x;
    cs = ms.y;
  }
  float M = wave_max(cm);
  if (lane == 0) s_rm[wave] = M;
  __syncthreads();
  M = s_rm[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / kWave; ++w) M = fmaxf(M, s_rm[w]);
  float part = cm > -INFINITY ? cs * __expf(cm - M) : 0.0f;
  part = wave_sum(part);
  if (lane == 0) s_rs[wave] = part;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kTopkThreads / kWave; ++w) tot += s_rs[w];
    s_lse = M > -INFINITY ? M + __logf(tot) : -INFINITY;
  }
  __syncthreads();
  __shared__ uint64_t s_top[kMaxK];
  const uint64_t* best = s_c;
  if (n <= 1024) {
    rank_select(s_c, n, K, s_top);
    __syncthreads();
    best = s_top;
  } else {
    bitonic_desc(s_c, P);
  }
  const float lse = s_lse;
  for (int k = tid; k < K; k += kTopkThreads) {
    const uint64_t e = best[k];
    const float x = key_value((uint32_t)(e >> 32));
    topk_ids[row * K + k] = (int32_t)(0xFFFFFFFFu - (uint32_t)e);
    topk_logp[row * K + k] = (x == -INFINITY || lse == -INFINITY) ? -INFINITY : x - lse;
  }
}

}  // namespace

TopkPlan plan_draft_topk(int B, int D, int V, int K, int num_cu) {
  const long long rows = (long long)B * D;
  // One workgroup per compute unit: with few rows, more chunks would mostly add
  // candidates for the merge to rank (S * K of them per row).
  const RowChunks rc = plan_row_chunks(rows, V, num_cu, 1);
  TopkPlan p;
  p.chunks = rc.chunks;
  p.chunk = rc.chunk;
  p.ws_bytes = (size_t)rows * p.chunks * ((size_t)K * sizeof(uint64_t) + sizeof(float2));
  return p;
}

size_t draft_topk_ws_bound(int B, int D, int K) {
  return (size_t)B * D * kMaxChunks * ((size_t)K * sizeof(uint64_t) + sizeof(float2));
}

hipError_t launch_draft_topk(int dtype, const void* logits, int B, int D, int V, int K,
                             float* topk_logp, int32_t* topk_ids, void* workspace,
                             const TopkPlan& plan, hipStream_t stream) {
  const int rows = B * D;
  uint64_t* ws_cand = static_cast<uint64_t*>(workspace);
  float2* ws_ms = reinterpret_cast<float2*>(ws_cand + (size_t)rows * plan.chunks * K);
  const dim3 grid1(plan.chunks, rows);
  if (dtype == 1)
    hipLaunchKernelGGL(draft_topk_partial_kernel<uint16_t>, grid1, dim3(kTopkThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, K, plan.chunks, plan.chunk,
                       ws_cand, ws_ms);
  else
    hipLaunchKernelGGL(draft_topk_partial_kernel<float>, grid1, dim3(kTopkThreads), 0, stream,
                       static_cast<const float*>(logits), V, K, plan.chunks, plan.chunk, ws_cand,
                       ws_ms);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(draft_topk_merge_kernel, dim3(rows), dim3(kTopkThreads), 0, stream, K,
                     plan.chunks, ws_cand, ws_ms, topk_logp, topk_ids);
  return hipGetLastError();
}

}  // namespace ddt
