// Verify-pass linears for many verify positions: y[M][N] = x[M][K] . w[N][K]^T
// with bf16 MFMA (v_mfma_f32_16x16x32_bf16) and fp32 accumulators.
//
// Once B*(K+1) positions make the product a real dense contraction (the
// batch crossover of "Speculative Decoding: Guess Several Tokens, Check Them
// in One Pass", What happens at larger batches), tiles of x and w are staged
// in LDS and multiplied on the matrix cores. Few positions use the
// weight-streaming kernel in gemm_stream.hip instead.

#include "common.h"
#include "internal.h"

namespace specv {

// ---------------------------------------------------------------------------
// Large-M MFMA GEMM
// ---------------------------------------------------------------------------

constexpr int kMfmaThreads = 256;
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row (+16 B pad)

// BM x BN output tile; WM x (4/WM) waves; each wave owns (BM/WM) x (BN*WM/4).
// v_mfma_f32_16x16x32_bf16 operands: lane l supplies row (l % 16) of its
// 16-row block and 8 consecutive reduction elements starting at 8 * (l / 16);
// the 4 accumulator values of lane l are rows 4 * (l / 16) + r, column l % 16.
template <int BM, int BN, int WM, bool OUT_BF16>
__global__ __launch_bounds__(kMfmaThreads) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y, int M,
    int N, int K) {
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int A_UNITS = BM * kBK / 8 / kMfmaThreads;  // 16-byte units per thread
  constexpr int B_UNITS = BN * kBK / 8 / kMfmaThreads;
  static_assert(A_UNITS >= 1 && B_UNITS >= 1, "tile too small");
  __shared__ u32x4 As[BM * kLdsStride / 8];
  __shared__ u32x4 Bs[BN * kLdsStride / 8];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_UNITS], rb[B_UNITS];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * kMfmaThreads;
      const int r = u / (kBK / 8), c = u % (kBK / 8);
      const int gm = m0 + r, gk = k0 + c * 8;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4*>(X + (size_t)gm * K + gk)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      const int u = tid + i * kMfmaThreads;
      const int r = u / (kBK / 8), c = u % (kBK / 8);
      const int gn = n0 + r, gk = k0 + c * 8;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4*>(W + (size_t)gn * K + gk)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * kMfmaThreads;
      const int r = u / (kBK / 8), c = u % (kBK / 8);
      As[(r * kLdsStride) / 8 + c] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      const int u = tid + i * kMfmaThreads;
      const int r = u / (kBK / 8), c = u % (kBK / 8);
      Bs[(r * kLdsStride) / 8 + c] = rb[i];
    }
  };

  const int n_k = (K + kBK - 1) / kBK;
  load_tiles(0);
  for (int kt = 0; kt < n_k; ++kt) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (kt + 1 < n_k) load_tiles((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 a[TM], b[TN];
      const int kunit = (kk + (lane >> 4) * 8) / 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / WM) + i * 16 + (lane & 15);
        a[i] = __builtin_bit_cast(bf16x8, As[(r * kLdsStride) / 8 + kunit]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / WN) + j * 16 + (lane & 15);
        b[j] = __builtin_bit_cast(bf16x8, Bs[(r * kLdsStride) / 8 + kunit]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
        if (row < M && col < N) {
          const float v = acc[i][j][r];
          if (OUT_BF16)
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * N + col] = f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(Y)[(size_t)row * N + col] = v;
        }
      }
    }
}

template <int BM, int BN, int WM>
static hipError_t launch_mfma_t(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                                int K, int N, hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, true>), grid, dim3(kMfmaThreads), 0, s, x, w,
                       y, M, N, K);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, false>), grid, dim3(kMfmaThreads), 0, s, x,
                       w, y, M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                            int K, int N, hipStream_t s) {
  if (M <= 32) return launch_mfma_t<32, 64, 1>(x, w, y, out_bf16, M, K, N, s);
  if (M <= 128) return launch_mfma_t<64, 64, 2>(x, w, y, out_bf16, M, K, N, s);
  return launch_mfma_t<128, 128, 2>(x, w, y, out_bf16, M, K, N, s);
}

}  // namespace specv
