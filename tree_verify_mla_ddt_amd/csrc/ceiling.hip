// ceiling.hip -- measured ceilings of the attention tile on gfx950 (a
// measurement aid, built into its own library; not part of libddt.so).
//
// One workgroup of four waves per CU (one wave per SIMD, like the attention
// kernels), every wave issuing v_mfma_f32_32x32x16_bf16 on operands whose
// values are random bf16 (the matrix cores draw more power on random data,
// which lowers the clock the chip sustains):
//   mode 0  MFMA only: 16 independent accumulators, operands in registers;
//   mode 1  the tile's operand traffic: per 32-key tile, 36 score MFMAs fed by
//           16-byte LDS reads of swizzled 1 KiB key rows, then 32 value MFMAs
//           fed by transposing LDS reads, one barrier per tile;
//   mode 2  mode 1 plus the next tile's 36 KiB global->LDS loads (nine
//           16-byte-per-lane loads per wave) issued at the top of each tile,
//           waited for before the barrier.
// ddt_ceiling_run reports TFLOP/s (32768 flops per MFMA) over the wall time of
// the launch and the shader-clock cycles per MFMA of a wave.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4_lds_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
#define CL_LDS __attribute__((address_space(3)))

constexpr int kStage = 36864;          // one 32-key tile: 32 x 1 KiB latent rows + 4 KiB rope
constexpr int kRows = 8192;            // 1 KiB rows of the global source
constexpr int kGrid = 256;             // one workgroup per CU

__device__ __forceinline__ int swz(int r) {
  return ((0xEA40 >> (4 * (r & 3))) & 15) ^ ((r >> 2) & 3);
}

// Transposing reads of the value operand from swizzled 1 KiB key rows, in the
// attention kernels' bank-conflict-free pattern: keys 4g + j/4 (+8) of the
// lane's column chunk.
struct VtRead {
  uint32_t p0, p1;
  __device__ __forceinline__ VtRead(uint32_t tile, int lane) {
    const int j = lane & 15, q = lane >> 4, g = lane >> 5;
    const int x = 2 * (q & 1) + ((j & 3) >> 1);
    const int f0 = ((0xEA40 >> (4 * ((j >> 2) & 3))) & 15) ^ g, f1 = f0 ^ 2;
    const uint32_t rb = tile + (4 * g + (j >> 2)) * 1024 + 8 * (j & 1);
    p0 = rb + 16 * ((x ^ f0) & 3) + 64 * (f0 >> 2);
    p1 = rb + 16 * ((x ^ f1) & 3) + 64 * (f1 >> 2);
  }
  __device__ __forceinline__ bf16x8_t read(int cb, int k1) const {
    const uint32_t c = 64 * (cb & 3), h = 256 * (cb >> 2) + 16384 * k1;
    const bf16x4_lds_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CL_LDS bf16x4_lds_t*)(uintptr_t)((p0 ^ c) + h));
    const bf16x4_lds_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (CL_LDS bf16x4_lds_t*)(uintptr_t)((p1 ^ c) + h + 8192));
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8_t, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
  }
};

// Score-chain step with the accumulator in VGPRs (the 16 value accumulators
// take the AGPRs), as in the attention kernels.
__device__ __forceinline__ void mfma_chain(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  __asm__ __volatile__("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  __asm__ __volatile__("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :
                       : "v"(src), "s"(lds)
                       : "memory", "m0");
}
#pragma clang diagnostic pop

template <int MODE>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ceiling_kernel(const bf16x8_t* __restrict__ in, const uint16_t* __restrict__ rows,
                    float* __restrict__ out, unsigned long long* __restrict__ cycles, int iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[3 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  bf16x8_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = in[(threadIdx.x * 32 + i) & 1023];
  for (int i = threadIdx.x; i < 3 * kStage / 16; i += 256)
    reinterpret_cast<uint4*>(lds)[i] = reinterpret_cast<const uint4*>(rows)[i];
  __syncthreads();
  f32x16_t o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16_t{};
  f32x16_t s = {};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(CL_LDS void*)lds;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
#pragma unroll
      for (int k = 0; k < 32; ++k)
        o[k & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[k], q[(k + 3) & 31], o[k & 15], 0, 0, 0);
    } else {
      const uint32_t st = lds0 + (it % 3) * kStage;
      if constexpr (MODE == 2) {
        const uint32_t dst = lds0 + ((it + 1) % 3) * kStage + wave * 8 * 1024;
#pragma unroll
        for (int j = 0; j < 9; ++j) {
          const int r = (it * 37 + j * 11 + wave * 1000) & (kRows - 1);
          dma16(rows + (size_t)r * 512 + lane * 8, __builtin_amdgcn_readfirstlane(dst + j * 1024));
        }
      }
      const int n = lane & 31, g = lane >> 5;
      const uint32_t kb = st + n * 1024 + 16 * (g ^ swz(n));
      auto kread = [&](int t) -> bf16x8_t {
        t &= 31;  // the four rope steps read latent rows as stand-ins
        return *(const CL_LDS bf16x8_t*)(uintptr_t)((kb ^ ((t & 7) << 5)) + 256 * (t >> 3));
      };
      bf16x8_t kop[36];
#pragma unroll
      for (int i = 0; i < 4; ++i) kop[i] = kread(i);
#pragma unroll
      for (int k = 0; k < 36; ++k) {
        if (k + 4 < 36) kop[k + 4] = kread(k + 4);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chain(s, kop[k], q[k & 31]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const VtRead va(st, lane);
      bf16x8_t vop[32];
#pragma unroll
      for (int i = 0; i < 6; ++i) vop[i] = va.read(i % 16, i / 16);
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k + 6 < 32) vop[k + 6] = va.read((k + 6) % 16, (k + 6) / 16);
        __builtin_amdgcn_sched_barrier(0);
        o[k & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k], q[k], o[k & 15], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += s[i] + o[i][i];
  out[blockIdx.x * 256 + threadIdx.x] = acc;
  if (threadIdx.x == 0) atomicAdd(cycles, t1 - t0);
}

template <int MODE>
hipError_t launch(int iters, const bf16x8_t* in, const uint16_t* rows, float* out,
                  unsigned long long* cyc) {
  hipLaunchKernelGGL(ceiling_kernel<MODE>, dim3(kGrid), dim3(256), 0, 0, in, rows, out, cyc,
                     iters);
  return hipGetLastError();
}

hipError_t launch_mode(int mode, int iters, const bf16x8_t* in, const uint16_t* rows, float* out,
                       unsigned long long* cyc) {
  if (mode == 0) return launch<0>(iters, in, rows, out, cyc);
  if (mode == 1) return launch<1>(iters, in, rows, out, cyc);
  return launch<2>(iters, in, rows, out, cyc);
}

}  // namespace

// mode 0..2 (see above), iters >= 1, random != 0 for random operand values
// (else all zero).  Writes TFLOP/s and cycles per MFMA of one wave; returns 0,
// or -1 for invalid arguments, -3 for a HIP failure.
extern "C" int ddt_ceiling_run(int mode, int iters, int random, double* tflops,
                               double* cycles_per_mfma) {
  if (mode < 0 || mode > 2 || iters < 1 || iters > 1000000 || !tflops || !cycles_per_mfma)
    return -1;
  const size_t row_bytes = (size_t)kRows * 1024;
  bf16x8_t* in = nullptr;
  uint16_t* rows = nullptr;
  float* out = nullptr;
  unsigned long long* cyc = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -3;
  uint16_t* host = static_cast<uint16_t*>(malloc(row_bytes));
  if (!host) return -3;
  // Values of magnitude in [0.5, 1) with random mantissa and sign (a linear
  // congruential generator), or zeros.
  uint32_t x = 12345u;
  for (size_t i = 0; i < row_bytes / 2; ++i) {
    x = x * 1664525u + 1013904223u;
    host[i] = random ? (uint16_t)(0x3f00u + ((x >> 16) & 0xffu) + ((x >> 30) << 15)) : 0;
  }
  float ms = 0.0f;
  unsigned long long c = 0;
  if (hipMalloc(&in, 1024 * 16) == hipSuccess && hipMalloc(&rows, row_bytes) == hipSuccess &&
      hipMalloc(&out, kGrid * 256 * sizeof(float)) == hipSuccess &&
      hipMalloc(&cyc, sizeof(unsigned long long)) == hipSuccess &&
      hipMemcpy(rows, host, row_bytes, hipMemcpyHostToDevice) == hipSuccess &&
      hipMemcpy(in, host, 1024 * 16, hipMemcpyHostToDevice) == hipSuccess &&
      hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess &&
      launch_mode(mode, 10, in, rows, out, cyc) == hipSuccess &&
      hipDeviceSynchronize() == hipSuccess &&
      hipMemset(cyc, 0, sizeof(unsigned long long)) == hipSuccess &&
      hipEventRecord(e0, 0) == hipSuccess &&
      launch_mode(mode, iters, in, rows, out, cyc) == hipSuccess &&
      hipEventRecord(e1, 0) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
      hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
      hipMemcpy(&c, cyc, sizeof(c), hipMemcpyDeviceToHost) == hipSuccess) {
    const double mfma_per_iter = mode == 0 ? 32.0 : 68.0;
    const double n = (double)iters * mfma_per_iter;   // MFMAs per wave
    *tflops = (double)kGrid * 4 * n * 32768.0 / (ms * 1e-3) / 1e12;
    *cycles_per_mfma = (double)c / kGrid / n;
    rc = 0;
  }
  free(host);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (in) (void)hipFree(in);
  if (rows) (void)hipFree(rows);
  if (out) (void)hipFree(out);
  if (cyc) (void)hipFree(cyc);
  return rc;
}
