// Verify-pass linear layers: y[M][N] = x[M][K] . w[N][K]^T, bf16 in, fp32
// accumulation, for the M = B*(K+1) positions of one verify step.
//
// One read of w serves every verify position: the pass costs what a
// one-token decode step costs as long as it stays bandwidth-bound
// ("What Actually Happens During Speculative Decoding in LLMs", the
// 5-candidate pass; "Speculative Decoding: Guess Several Tokens, Check Them
// in One Pass", Step 1: 5 FLOPs per weight byte at K = 4). Two kernels:
//
//  * gemm_stream: small M. Vector-ALU weight streaming. Each lane group of 16
//    lanes walks RPL rows of w with 16-byte loads (one 256-byte contiguous
//    piece per row per segment); the activation tile x[:, chunk] is staged
//    once per workgroup in LDS and read with 16-byte LDS loads; products use
//    v_dot2c_f32_bf16 (two bf16 products per lane-op, fp32 accumulate).
//    The four waves of a workgroup split the reduction dimension; partial
//    sums are reduced across 16 lanes with DPP and across waves through LDS
//    in a fixed order (deterministic).
//  * gemm_mfma: large M, where the product is a dense contraction. Tiles of
//    x and w staged in LDS, v_mfma_f32_16x16x32_bf16, fp32 accumulators.
//
// Names follow the pages: K in a template or loop here is the reduction
// length d_in; the draft length never appears in this file.

#include "common.h"
#include "internal.h"

namespace specv {

// ---------------------------------------------------------------------------
// Small-M weight streaming
// ---------------------------------------------------------------------------

constexpr int kStreamThreads = 256;
constexpr int kSeg = 128;  // reduction elements per lane group per segment

__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

// M: rows of x (verify positions). RPL: rows of w per lane group.
// U: segments per wave per pipeline stage. Rows per workgroup: 4 * RPL.
template <int M, int RPL, int U, bool OUT_BF16>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int K, int N, int KC) {
  extern __shared__ u32x4 lds[];
  constexpr int NR = 4 * RPL;
  constexpr int ELEMS_PER_IT = 4 * U * kSeg;  // all four waves, one stage
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, sub = lane & 15;
  const int row_base = blockIdx.x * NR + grp * RPL;
  const int kc_units = KC / 8;
  const int its_per_chunk = KC / ELEMS_PER_IT;
  const int n_it = (K + ELEMS_PER_IT - 1) / ELEMS_PER_IT;

  const u32x4* wrow[RPL];
  bool row_ok[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int row = row_base + r;
    row_ok[r] = row < N;
    wrow[r] = reinterpret_cast<const u32x4*>(W + (size_t)(row_ok[r] ? row : 0) * K);
  }

  float acc[RPL][M];
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  auto stage_x = [&](int chunk) {
    const int k0 = chunk * KC;
    const int kc = min(KC, K - k0);
    const int units = kc / 8;
    for (int u = tid; u < M * units; u += kStreamThreads) {
      const int m = u / units, c = u - m * units;
      lds[m * kc_units + c] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + k0 + c * 8);
    }
  };
  // element offset (in K) of this lane's 8 elements for segment u of stage it
  auto kofs = [&](int it, int u) { return ((it * U + u) * 4 + wave) * kSeg + sub * 8; };

  auto load_w = [&](u32x4 (&buf)[U][RPL], int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kofs(it, u);
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        buf[u][r] = (row_ok[r] && k < K) ? wrow[r][k >> 3] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto compute = [&](const u32x4 (&buf)[U][RPL], int it) {
    const int chunk_base = (it / its_per_chunk) * KC;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kofs(it, u);
      if (k < K) {
        const int lu = (k - chunk_base) >> 3;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 xv = lds[m * kc_units + lu];
#pragma unroll
          for (int r = 0; r < RPL; ++r) acc[r][m] = dot8_bf16(buf[u][r], xv, acc[r][m]);
        }
      }
    }
  };

  u32x4 wa[U][RPL], wb[U][RPL];
  load_w(wa, 0);
  stage_x(0);
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    if (it + 1 < n_it) load_w(wb, it + 1);
    compute(wa, it);
    if ((it + 1) % its_per_chunk == 0 && it + 1 < n_it) {
      __syncthreads();
      stage_x((it + 1) / its_per_chunk);
      __syncthreads();
    }
    if (it + 1 >= n_it) break;
    if (it + 2 < n_it) load_w(wa, it + 2);
    compute(wb, it + 1);
    if ((it + 2) % its_per_chunk == 0 && it + 2 < n_it) {
      __syncthreads();
      stage_x((it + 2) / its_per_chunk);
      __syncthreads();
    }
  }

  // reduce over the 16 lanes of each group, then over the 4 waves
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = row16_sum(acc[r][m]);
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [wave][NR][M]
  if (sub == 0) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) red[(wave * NR + grp * RPL + r) * M + m] = acc[r][m];
  }
  __syncthreads();
  for (int i = tid; i < NR * M; i += kStreamThreads) {
    const int m = i / NR, rr = i - m * NR;
    const int row = blockIdx.x * NR + rr;
    if (row < N) {
      const float v = ((red[(0 * NR + rr) * M + m] + red[(1 * NR + rr) * M + m]) +
                       red[(2 * NR + rr) * M + m]) + red[(3 * NR + rr) * M + m];
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(Y)[(size_t)m * N + row] = f32_to_bf16_bits(v);
      else
        reinterpret_cast<float*>(Y)[(size_t)m * N + row] = v;
    }
  }
}

template <int M, int RPL, int U>
static hipError_t launch_stream_m(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16,
                                  int K, int N, hipStream_t s) {
  constexpr int ELEMS_PER_IT = 4 * U * kSeg;
  // Activation chunk staged in LDS: at most ~48 KB, a multiple of one stage.
  const int max_kc = ((48 * 1024) / (2 * M)) / ELEMS_PER_IT * ELEMS_PER_IT;
  const int k_pad = (K + ELEMS_PER_IT - 1) / ELEMS_PER_IT * ELEMS_PER_IT;
  const int cap = max_kc > ELEMS_PER_IT ? max_kc : ELEMS_PER_IT;
  const int n_chunks = (k_pad + cap - 1) / cap;
  int kc = (k_pad / ELEMS_PER_IT + n_chunks - 1) / n_chunks * ELEMS_PER_IT;
  size_t lds = (size_t)M * kc * 2;
  const size_t red = (size_t)4 * 4 * RPL * M * 4;
  if (lds < red) lds = red;
  const int grid = (N + 4 * RPL - 1) / (4 * RPL);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_stream_kernel<M, RPL, U, true>), dim3(grid), dim3(kStreamThreads), lds,
                       s, x, w, y, K, N, kc);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<M, RPL, U, false>), dim3(grid), dim3(kStreamThreads),
                       lds, s, x, w, y, K, N, kc);
  return hipGetLastError();
}

hipError_t launch_gemm_stream(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                              int K, int N, hipStream_t s) {
  switch (M) {
#define SPECV_STREAM_CASE(MM, RPL, U) \
  case MM:                            \
    return launch_stream_m<MM, RPL, U>(x, w, y, out_bf16, K, N, s);
    SPECV_STREAM_CASE(1, 2, 4)
    SPECV_STREAM_CASE(2, 2, 4)
    SPECV_STREAM_CASE(3, 2, 4)
    SPECV_STREAM_CASE(4, 2, 4)
    SPECV_STREAM_CASE(5, 2, 4)
    SPECV_STREAM_CASE(6, 2, 4)
    SPECV_STREAM_CASE(7, 2, 4)
    SPECV_STREAM_CASE(8, 2, 4)
    SPECV_STREAM_CASE(9, 2, 2)
    SPECV_STREAM_CASE(10, 2, 2)
    SPECV_STREAM_CASE(11, 2, 2)
    SPECV_STREAM_CASE(12, 2, 2)
    SPECV_STREAM_CASE(13, 2, 2)
    SPECV_STREAM_CASE(14, 2, 2)
    SPECV_STREAM_CASE(15, 2, 2)
    SPECV_STREAM_CASE(16, 2, 2)
#undef SPECV_STREAM_CASE
    default:
      return hipErrorInvalidValue;
  }
}

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
