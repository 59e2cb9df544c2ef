// Achievable ceilings beside the published peaks: a read-only stream over a
// large buffer (HBM read bandwidth) and a loop of independent MFMAs (dense
// bf16 matrix-core rate). The verify pass is priced against the published
// figures; these say how close to them a kernel on this part can get
// ("Speculative Decoding: Guess Several Tokens, Check Them in One Pass",
// Step 1: checking is cheap because the step is the weight read).

#include "common.h"
#include "internal.h"

#define SPECV_PROBE_GLOBAL __attribute__((address_space(1)))

namespace specv {

constexpr int kProbeThreads = 512;  // eight waves

// Every lane reads 16-byte units of the buffer, U at a time: unit
// (it * U + j) * G * T + bid * T + tid, so each wave instruction reads 1 KB
// contiguous and the grid sweeps the buffer front to back. The loaded words
// are folded into one value that is stored only if it equals `never` (a
// value the caller picks so that it never matches in practice), which keeps
// the loads from being removed.
template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(
    const u32x4* __restrict__ buf, size_t units, unsigned never, unsigned* sink) {
  const size_t T = blockDim.x, G = gridDim.x;
  const size_t stride = G * T;
  size_t i = (size_t)blockIdx.x * T + threadIdx.x;
  unsigned acc = 0;
  const SPECV_PROBE_GLOBAL u32x4* src = (const SPECV_PROBE_GLOBAL u32x4*)buf;
  for (; i + (U - 1) * stride < units; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < units; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[0] = acc;
}

// s_waitcnt vmcnt(N), the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void probe_wait_vmcnt() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// The same sweep with the loads going straight to LDS (global_load_lds, the
// path the tile kernels feed their operand rings with): each wave keeps a
// ring of U one-kilobyte slots and U loads in flight, waiting for the
// oldest before its slot is loaded again. Every wave runs the same number
// of iterations; lanes past the end reload the last unit.
template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read_lds_kernel(
    const u32x4* __restrict__ buf, size_t units, unsigned never, unsigned* sink) {
  __shared__ u32x4 ring[kProbeThreads / 64 * U * 64];
  const size_t T = blockDim.x, G = gridDim.x;
  const size_t stride = G * T;
  const size_t n_it = (units + stride - 1) / stride;
  const size_t i0 = (size_t)blockIdx.x * T + threadIdx.x;
  const int wave = threadIdx.x >> 6;
  const SPECV_PROBE_GLOBAL u32x4* src = (const SPECV_PROBE_GLOBAL u32x4*)buf;
  for (size_t it = 0; it < n_it; ++it) {
    if (it >= U) probe_wait_vmcnt<U - 1>();
    const size_t i = min(i0 + it * stride, units - 1);
    __attribute__((address_space(3))) void* dst =
        (__attribute__((address_space(3))) void*)(ring + (wave * U + (int)(it % U)) * 64);
    __builtin_amdgcn_global_load_lds((const SPECV_PROBE_GLOBAL void*)(src + i), dst, 16, 0, 0);
  }
  probe_wait_vmcnt<0>();
  __syncthreads();
  const u32x4 v = ring[threadIdx.x];
  const unsigned acc = v.x ^ v.y ^ v.z ^ v.w;
  if (acc == never) sink[0] = acc;
}

// NCH independent accumulator chains per wave, each `iters` MFMAs long, on
// register operands only (no memory traffic inside the loop). The
// accumulators are folded and stored only if they equal `never`.
template <int SHAPE>  // 16: v_mfma_f32_16x16x32_bf16; 32: v_mfma_f32_32x32x16_bf16
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, unsigned never,
                                                         unsigned* sink) {
  constexpr int NCH = SHAPE == 16 ? 8 : 4;  // 32 accumulator registers either way
  constexpr int NACC = SHAPE == 16 ? 4 : 16;
  typedef float facc __attribute__((ext_vector_type(NACC)));
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (lane + k));
    b[k] = (__bf16)(0.002f * (lane - k));
  }
  facc acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < NACC; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (SHAPE == 16)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < NACC; ++r) s += acc[c][r];
  if (__float_as_uint(s) == never) sink[0] = __float_as_uint(s);
}

hipError_t launch_probe_read(const void* buf, size_t bytes, int loads, unsigned* sink, int grid,
                             hipStream_t s) {
  const u32x4* b = static_cast<const u32x4*>(buf);
  switch (loads) {
    case 1: hipLaunchKernelGGL(probe_read_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, s, b,
                               bytes / 16, 0x9E3779B9u, sink); break;
    case 2: hipLaunchKernelGGL(probe_read_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, s, b,
                               bytes / 16, 0x9E3779B9u, sink); break;
    case 4: hipLaunchKernelGGL(probe_read_kernel<4>, dim3(grid), dim3(kProbeThreads), 0, s, b,
                               bytes / 16, 0x9E3779B9u, sink); break;
    default: hipLaunchKernelGGL(probe_read_kernel<8>, dim3(grid), dim3(kProbeThreads), 0, s, b,
                                bytes / 16, 0x9E3779B9u, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_read_lds(const void* buf, size_t bytes, int loads, unsigned* sink,
                                 int grid, hipStream_t s) {
  const u32x4* b = static_cast<const u32x4*>(buf);
  switch (loads) {
    case 1: hipLaunchKernelGGL(probe_read_lds_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, s,
                               b, bytes / 16, 0x9E3779B9u, sink); break;
    case 2: hipLaunchKernelGGL(probe_read_lds_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, s,
                               b, bytes / 16, 0x9E3779B9u, sink); break;
    case 4: hipLaunchKernelGGL(probe_read_lds_kernel<4>, dim3(grid), dim3(kProbeThreads), 0, s,
                               b, bytes / 16, 0x9E3779B9u, sink); break;
    default: hipLaunchKernelGGL(probe_read_lds_kernel<8>, dim3(grid), dim3(kProbeThreads), 0, s,
                                b, bytes / 16, 0x9E3779B9u, sink); break;
  }
  return hipGetLastError();
}

// FLOPs of one launch: grid * 4 waves * iters * 131072 (per wave and
// iteration 8 x 16x16x32 or 4 x 32x32x16, 2 * 8192 * 8 FLOPs either way).
hipError_t launch_probe_mfma(int shape, int iters, unsigned* sink, int grid, hipStream_t s) {
  if (shape == 16)
    hipLaunchKernelGGL(probe_mfma_kernel<16>, dim3(grid), dim3(256), 0, s, iters, 0x7FC00001u,
                       sink);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<32>, dim3(grid), dim3(256), 0, s, iters, 0x7FC00001u,
                       sink);
  return hipGetLastError();
}

}  // namespace specv
