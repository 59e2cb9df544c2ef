// Internal helpers shared by the HIP kernels of libspecverify (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2, v);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Lane permutation within a row of 16 lanes through DPP.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
// xor 1, xor 2 (quad permutes), then the half-row and row mirrors.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide reductions; every thread receives the result. `lds` holds one
// slot per wave. The summation order is fixed, so results are deterministic.
template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_sum_f64(v);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) t += lds[w];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ float block_max_f32(float v, float* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_max_f32(v);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) t = fmaxf(t, lds[w]);
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ int block_min_i32(int v, int* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) t = min(t, lds[w]);
  __syncthreads();
  return t;
}

}  // namespace specv
