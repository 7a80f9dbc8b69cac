// Measurement-only microbenchmarks (attainable bf16 MFMA rate, HBM streaming
// read rate) for gfx950.  Not part of the attention method.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cosa_calib.h"

namespace cosa_calib {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// 8 independent accumulator chains per wave, so consecutive MFMAs never wait on
// each other's results; the operands vary with the lane so nothing folds away.
__global__ __launch_bounds__(256) void mfma_bf16_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16_t acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[x][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[x], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[x][e];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// The same chains on operands with every bit pattern in play: bf16 values with random signs and
// mantissas and exponents spread over about 2^-8 .. 2^8, two operand sets taken in turn, so the
// datapath toggles as it does on real data (the constant operands above draw less power and let
// the clock stay higher).  The values come from a 32-bit integer hash of (seed, lane, element).
__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ bf16x8_t calib_operand(uint32_t seed, uint32_t lane, uint32_t set) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = calib_hash(seed ^ (lane * 64u + set * 8u + (uint32_t)e) * 0x9e3779b9u);
    const uint32_t sign = (h >> 31) << 15;
    const uint32_t expo = 119u + ((h >> 8) & 0xffu) % 17u;  // 2^-8 .. 2^8
    const uint32_t mant = h & 0x7fu;
    const uint16_t bits = (uint16_t)(sign | (expo << 7) | mant);
    r[e] = __builtin_bit_cast(__bf16, bits);
  }
  return r;
}

__global__ __launch_bounds__(256) void mfma_bf16_data_kernel(float* out, int pairs, uint32_t seed) {
  const uint32_t lane = threadIdx.x & 63;
  const bf16x8_t a0 = calib_operand(seed, lane, 0), b0 = calib_operand(seed, lane, 1);
  const bf16x8_t a1 = calib_operand(seed, lane, 2), b1 = calib_operand(seed, lane, 3);
  f32x16_t acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[x][e] = 0.f;
  for (int it = 0; it < pairs; ++it) {
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[x], 0, 0, 0);
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[x], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[x][e];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ src, size_t n16, uint32_t* out) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(&src[i]);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace cosa_calib

extern "C" int32_t cosa_calib_mfma_bf16(float* out, int32_t num_workgroups, int32_t iters, hipStream_t stream) {
  if (out == nullptr || num_workgroups < 1 || iters < 1) return COSA_CALIB_ERR_ARG;
  hipLaunchKernelGGL(cosa_calib::mfma_bf16_kernel, dim3((unsigned)num_workgroups), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? COSA_CALIB_OK : COSA_CALIB_ERR_LAUNCH;
}

extern "C" double cosa_calib_mfma_bf16_flop(int32_t num_workgroups, int32_t iters) {
  // per MFMA: 32 x 32 x 16 multiply-adds
  return 2.0 * 32 * 32 * 16 * 8.0 * (double)iters * 4.0 * (double)num_workgroups;
}

extern "C" int32_t cosa_calib_mfma_bf16_data(float* out, int32_t num_workgroups, int32_t iters, uint32_t seed,
                                             hipStream_t stream) {
  if (out == nullptr || num_workgroups < 1 || iters < 2 || iters % 2 != 0) return COSA_CALIB_ERR_ARG;
  hipLaunchKernelGGL(cosa_calib::mfma_bf16_data_kernel, dim3((unsigned)num_workgroups), dim3(256), 0, stream, out,
                     iters / 2, seed);
  return hipGetLastError() == hipSuccess ? COSA_CALIB_OK : COSA_CALIB_ERR_LAUNCH;
}

extern "C" int32_t cosa_calib_read(const void* src, size_t bytes, uint32_t* out, int32_t num_workgroups,
                                   hipStream_t stream) {
  if (src == nullptr || out == nullptr || num_workgroups < 1 || bytes % 16 != 0 ||
      ((uintptr_t)src & 15u) != 0)
    return COSA_CALIB_ERR_ARG;
  hipLaunchKernelGGL(cosa_calib::read_kernel, dim3((unsigned)num_workgroups), dim3(256), 0, stream,
                     static_cast<const cosa_calib::u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? COSA_CALIB_OK : COSA_CALIB_ERR_LAUNCH;
}
