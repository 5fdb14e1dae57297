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

// About two workgroups per compute unit, at most 64 chunks per row unless the
// chunk size forces more.
inline RowChunks plan_row_chunks(long long rows, int V, int num_cu) {
  const int s_min = (V + kRowChunkMax - 1) / kRowChunkMax;
  const long long want = 2LL * (num_cu > 0 ? num_cu : 256);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace ddt
