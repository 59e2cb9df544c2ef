// Verify-pass linears for 17..128 positions: y[M][N] = x[M][K] . w[N][K]^T
// on the matrix cores (v_mfma_f32_16x16x32_bf16), streaming w once.
//
// Between a handful of positions (the VALU streaming kernel) and a real
// dense contraction (the tiled MFMA kernel) the product is still bound by
// reading w: M FLOPs per weight byte stay below the chip's ridge of about
// 312 ("Speculative Decoding: Guess Several Tokens, Check Them in One Pass",
// What happens at larger batches). The kernel is built around keeping
// enough weight bytes in flight on every CU:
//
//  * A workgroup owns 16 * NT consecutive rows of w over the whole
//    reduction dimension; there are N / (16 * NT) workgroups, so the grid
//    fills the chip without splitting the reduction across workgroups.
//  * Its eight waves interleave 64-element segments of the reduction (128
//    contiguous bytes of each row per segment); a pipeline stage holds U
//    segments, which keeps 64 to 128 KB of weights in flight per workgroup. Each lane loads its 16-byte weight
//    fragments straight into MFMA operand registers; no weight byte passes
//    through LDS.
//  * No two waves of a workgroup need the same activation element, so the
//    activation fragments also go straight from global memory (L2) into
//    operand registers, once per workgroup.
//  * Two register stages are in flight ahead of the matrix instructions.
//  * Partial sums of the waves are added into one LDS buffer in wave
//    order: results are deterministic.
//
// MFMA operand layout (16x16x32): lane l supplies row (l % 16) of a 16-row
// operand block and the 8 reduction elements starting at 8 * (l / 16); lane
// l receives D[4 * (l / 16) + r][l % 16], r = 0..3. Here A = x (rows are
// positions), B = w (rows are outputs), so D[m][n] = sum_k x[m][k] w[n][k].

#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kSegK = 64;  // reduction elements per wave segment

#define SPECV_SK_GLOBAL __attribute__((address_space(1)))

// MT 16-row tiles of positions, NT 16-row tiles of weight rows per
// workgroup, KW waves splitting the reduction dimension, U segments per
// pipeline stage (two stages in flight).
template <int MT, int NT, int KW, int U, bool OUT_BF16>
__global__ __launch_bounds__(KW * kWave) void gemm_skinny_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y, int M,
    int N, int K) {
  constexpr int kOut = NT * MT * 4 * kWave;  // accumulator values per wave
  __shared__ float red[kOut];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);

  // Per-lane row pointers: positions (x rows) and outputs (w rows). Rows
  // past the end are clamped to a valid row: they only feed outputs that are
  // never stored.
  const SPECV_SK_GLOBAL u32x4* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xrow[t] = (const SPECV_SK_GLOBAL u32x4*)(X + (size_t)min(t * 16 + row16, M - 1) * K);
  const SPECV_SK_GLOBAL u32x4* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wrow[t] = (const SPECV_SK_GLOBAL u32x4*)(W + (size_t)min(n0 + t * 16 + row16, N - 1) * K);

  // Segments s = wave, wave + KW, ...; segment s covers k in [64 s, 64 s + 64).
  // In segment s, MFMA j (0, 1) takes k = 64 s + 32 j + 8 * grp + (0..7).
  // Stage i of a wave holds its segments i * U .. i * U + U - 1.
  const int n_seg = (K + kSegK - 1) / kSegK;
  const int my_seg = n_seg > wave ? (n_seg - wave + KW - 1) / KW : 0;
  const int n_st = (my_seg + U - 1) / U;
  const int K8 = K >> 3;  // 16-byte units per row

  f32x4 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loaded values are used only by the matrix instructions: no instruction
  // between a load and its MFMA reads them, so the loads of both register
  // stages stay in flight. Reduction elements past K (the ragged tail, and
  // the unused segments of a wave's last stage) load a clamped valid unit;
  // the weight fragment is zeroed at use.
  struct Frag {
    u32x4 x[U][2][MT];
    u32x4 w[U][2][NT];
    bool kok[U][2];
  };
  auto load = [&](Frag& f, int i) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = wave + KW * (i * U + u);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int unit = s * (kSegK / 8) + j * 4 + grp;  // 16-byte unit index along k
        f.kok[u][j] = unit < K8;
        const int uc = min(unit, K8 - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) f.w[u][j][t] = __builtin_nontemporal_load(wrow[t] + uc);
#pragma unroll
        for (int t = 0; t < MT; ++t) f.x[u][j][t] = xrow[t][uc];
      }
    }
  };
  auto mma = [&](const Frag& f, bool last) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          u32x4 wv = f.w[u][j][i];
          if (last) wv = f.kok[u][j] ? wv : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, f.x[u][j][t]), __builtin_bit_cast(bf16x8, wv),
                acc[i][t], 0, 0, 0);
        }
  };

  // The prologue and the steady-state loop issue their loads on every path
  // (a stage past the wave's last one reads clamped valid addresses and is
  // never used), so the compiler's vmcnt waits keep both stages in flight;
  // the last zero to three stages are finished after the loop. Only a
  // wave's last stage can reach past K.
  Frag fa, fb;
  load(fa, 0);
  load(fb, 1);
  int i = 0;
  for (; i + 4 <= n_st; i += 2) {
    mma(fa, false);
    load(fa, i + 2);
    mma(fb, false);
    load(fb, i + 3);
  }
  const int rem = n_st - i;  // 0..3 stages left, already loaded up to 2
  if (rem >= 1) mma(fa, rem == 1);
  if (rem >= 3) load(fa, i + 2);
  if (rem >= 2) mma(fb, rem == 2);
  if (rem >= 3) mma(fa, true);

  // The KW partial sums of each output are added into one LDS buffer in
  // wave order (deterministic), then stored.
#pragma unroll 1
  for (int w = 0; w < KW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float& d = red[((a * MT + t) * 4 + r) * kWave + lane];
            d = w == 0 ? acc[a][t][r] : d + acc[a][t][r];
          }
    }
    __syncthreads();
  }
  for (int e = tid; e < kOut; e += KW * kWave) {
    const int l = e % kWave, rr = (e / kWave) % 4, t = (e / (4 * kWave)) % MT, a = e / (4 * kWave * MT);
    const int m = t * 16 + (l >> 4) * 4 + rr;
    const int n = n0 + a * 16 + (l & 15);
    if (m < M && n < N) {
      const float v = red[e];
      const size_t o = (size_t)m * N + n;
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(Y)[o] = f32_to_bf16_bits(v);
      else
        reinterpret_cast<float*>(Y)[o] = v;
    }
  }
}

template <int MT, int NT, int U>
static hipError_t launch_skinny_t(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16,
                                  int M, int K, int N, hipStream_t s) {
  constexpr int KW = 8;
  const dim3 grid((N + 16 * NT - 1) / (16 * NT));
  if (out_bf16)
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KW, U, true>), grid, dim3(KW * kWave), 0, s, x,
                       w, y, M, N, K);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KW, U, false>), grid, dim3(KW * kWave), 0, s, x,
                       w, y, M, N, K);
  return hipGetLastError();
}

// Tile choice per count of position tiles, measured on the Llama-shaped
// linears. Narrow linears (N < 16384) use NT1 16-row weight tiles per
// workgroup (one keeps 256 workgroups at N = 4096), wide ones NT2 (more
// rows reuse each activation fragment for more weight bytes). U segments
// per pipeline stage; the register file (256 VGPRs per lane at two waves
// per SIMD) bounds NT, U and the position tiles together.
#define SPECV_SKINNY_TABLE(X) \
  X(2, 1, 1, 4, 1)            \
  X(3, 1, 2, 2, 2)            \
  X(4, 1, 2, 2, 1)            \
  X(5, 1, 1, 2, 1)            \
  X(6, 1, 1, 1, 1)            \
  X(7, 1, 1, 1, 1)            \
  X(8, 1, 1, 1, 1)
// (MT, NT1, U1, NT2, U2)

template <int MT, int NT1, int U1, int NT2, int U2>
static hipError_t launch_skinny_m(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16,
                                  int M, int K, int N, hipStream_t s) {
  if (N >= 16384) return launch_skinny_t<MT, NT2, U2>(x, w, y, out_bf16, M, K, N, s);
  return launch_skinny_t<MT, NT1, U1>(x, w, y, out_bf16, M, K, N, s);
}

hipError_t launch_gemm_skinny(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                              int K, int N, hipStream_t s) {
  switch (max((M + 15) / 16, 2)) {
#define SPECV_SKINNY_CASE(MT, NT1, U1, NT2, U2) \
  case MT:                                      \
    return launch_skinny_m<MT, NT1, U1, NT2, U2>(x, w, y, out_bf16, M, K, N, s);
    SPECV_SKINNY_TABLE(SPECV_SKINNY_CASE)
#undef SPECV_SKINNY_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace specv
