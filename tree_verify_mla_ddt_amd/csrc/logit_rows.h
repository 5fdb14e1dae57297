// logit_rows.h -- helpers of the kernels that stream rows of logits over a
// vocabulary (per-depth top-K extraction, sampling acceptance).
//
// A row is cut into chunks of at most kRowChunkMax entries, one 256-thread
// workgroup per (row, chunk), so that even a handful of rows fills the chip;
// each thread holds up to kRowChunkMax / 256 entries in registers.
#pragma once

#include "ddt_internal.h"

namespace ddt {

constexpr int kRowThreads = 256;
constexpr int kRowChunkMax = 12288;  // entries of one chunk
constexpr int kRowChunksMax = 128;   // chunks of one row

struct RowChunks {
  int chunks;  // chunks per row, 1..kRowChunksMax
  int chunk;   // entries per chunk: a multiple of 8, <= kRowChunkMax; no chunk is empty
};

// About `per_cu` workgroups per compute unit, at most 64 chunks per row unless
// the chunk size forces more.
inline RowChunks plan_row_chunks(long long rows, int V, int num_cu, int per_cu) {
  const int s_min = (V + kRowChunkMax - 1) / kRowChunkMax;
  const long long want = (long long)per_cu * (num_cu > 0 ? num_cu : 256);
  long long s = (want + rows - 1) / rows;
  if (s > 64) s = 64;
  if (s < s_min) s = s_min;
  if (s > kRowChunksMax) s = kRowChunksMax;
  const long long s_cap = (V + 7) / 8;  // at most one chunk per 8 entries
  if (s > s_cap) s = s_cap;
  if (s < 1) s = 1;
  int C = (int)((V + s - 1) / s);
  C = (C + 7) / 8 * 8;
  RowChunks p;
  p.chunks = (V + C - 1) / C;
  p.chunk = C;
  return p;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T> struct Vec16;  // 16 bytes of logits
template <> struct Vec16<float> { static constexpr int kN = 4; };
template <> struct Vec16<uint16_t> { static constexpr int kN = 8; };

// The 32-bit word holding entries i0 .. i0 + 4/sizeof(T) - 1 of a chunk of n
// entries (-inf for entries past n).
__device__ __forceinline__ uint32_t load_word(const float* src, int i0, int n) {
  return i0 < n ? __float_as_uint(src[i0]) : 0xFF800000u;
}
__device__ __forceinline__ uint32_t load_word(const uint16_t* src, int i0, int n) {
  const uint32_t lo = i0 < n ? src[i0] : 0xFF80u;
  const uint32_t hi = i0 + 1 < n ? src[i0 + 1] : 0xFF80u;
  return lo | (hi << 16);
}

// A thread's share of a chunk of n entries, kept in registers as loaded, in
// 32-bit words: entry j of 16-byte group u is chunk entry (tid + 256*u)*kN + j
// (kN entries per group), or -inf where the chunk has none.  16-byte loads when
// the chunk is aligned and a whole number of groups, else word by word.
template <typename T, int kVPT>
__device__ __forceinline__ void load_chunk_words(const T* src, int n, int tid,
                                                 uint32_t (&w)[kVPT * 4]) {
  constexpr int kN = Vec16<T>::kN;
  constexpr uint32_t kFill = kN == 8 ? 0xFF80FF80u : 0xFF800000u;
  if (((reinterpret_cast<uintptr_t>(src) & 15) == 0) && n % kN == 0) {
    const int nv = n / kN;
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int i = tid + u * kRowThreads;
      uint4 r = make_uint4(kFill, kFill, kFill, kFill);
      if (i < nv) r = *reinterpret_cast<const uint4*>(src + (long long)i * kN);
      w[4 * u] = r.x;
      w[4 * u + 1] = r.y;
      w[4 * u + 2] = r.z;
      w[4 * u + 3] = r.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kVPT * 4; ++q) {
      const int u = q >> 2;
      w[q] = load_word(src, (tid + u * kRowThreads) * kN + (q & 3) * (kN / 4), n);
    }
  }
}

// Entry j of a 16-byte group, from the word that holds it.
template <typename T> __device__ __forceinline__ float word_entry(uint32_t word, int j);
template <> __device__ __forceinline__ float word_entry<float>(uint32_t word, int) {
  return __uint_as_float(word);
}
template <> __device__ __forceinline__ float word_entry<uint16_t>(uint32_t word, int j) {
  return __uint_as_float((j & 1) ? (word & 0xFFFF0000u) : (word << 16));
}

// Marks the words as rewritten (an empty asm statement), so that a later pass
// converts them again instead of the compiler keeping every entry as a float.
template <int kW>
__device__ __forceinline__ void mark_rewritten(uint32_t (&w)[kW]) {
#pragma unroll
  for (int q = 0; q < kW; ++q) asm volatile("" : "+v"(w[q]));
}

// Wave-wide reductions with DPP row operations: quad swaps, half-row and row
// mirrors give every lane its row's result, two row broadcasts carry it to lane
// 63, whose value every lane then reads (the result is wave-uniform).  Rows a
// broadcast leaves out take the identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t identity, Op op) {
  const int id = (int)identity;
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), __float_as_uint(-INFINITY),
                                     [](uint32_t a, uint32_t b) {
                                       return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                                     }));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ int wave_min(int v) {
  return (int)wave_reduce((uint32_t)v, 0x7FFFFFFFu, [](uint32_t a, uint32_t b) {
    return (uint32_t)min((int)a, (int)b);
  });
}

}  // namespace ddt
