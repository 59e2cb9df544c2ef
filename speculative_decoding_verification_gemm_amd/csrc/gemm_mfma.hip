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

#define SPECV_TILE_GLOBAL __attribute__((address_space(1)))

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

// ---------------------------------------------------------------------------
// Pipelined tile kernel (K a multiple of 64): NW waves (eight for the large
// tiles), LDS ring filled by direct-to-LDS loads
// ---------------------------------------------------------------------------
//
// Both operands reach LDS as whole 128-byte lines: one load instruction of a
// wave moves 8 rows x 128 bytes (64 reduction elements) straight into LDS
// (global_load_lds, no registers). Inside a row the eight 16-byte units are
// stored XOR-swizzled by the row index mod 8, so the fragment reads of
// v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, unit l / 16) hit eight
// distinct bank groups in every eight lanes. S tile stages are in flight;
// each wave waits (vmcnt) for its own loads of the stage it computes on and
// a workgroup barrier makes every wave's loads visible. The barrier is a
// bare s_barrier: a memory fence there would make the compiler wait for all
// loads in flight. Tiles are numbered so that the workgroups of one XCD
// (bid mod 8) take consecutive tiles, which share weight tiles in that XCD's
// L2.

constexpr int kTileKAlign = 64;  // the kernel needs K to be a multiple of this

// BK reduction elements per stage: 64 (a whole 128-byte line of each row) or
// 32 (half a line; the other half follows in the next stage, from L2), which
// halves a stage so that more of them fit in LDS.
// KS > 1 splits the reduction inside the workgroup: the waves form KS
// groups of NW / KS, group g takes k-tiles g, g + KS, ... through a ring of
// its own, and the KS partial tiles are added through LDS in group order at
// the end (deterministic). A small tile then still has NW waves' loads in
// flight.
template <int BM, int BN, int WM, int S, int BK, int NW, int KS = 1>
struct TileCfg {
  static constexpr int NWG = NW / KS;            // waves per k-group
  static constexpr int WN = NWG / WM;            // a group's waves: WM along M, WN along N
  static constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  static constexpr int ROWS = BM + BN;           // LDS rows per stage (x rows, then w rows)
  static constexpr int UPR = BK / 8;             // 16-byte units per row
  static constexpr int RPI = 64 / UPR;           // rows per load instruction
  static constexpr int RPL = 128 / (2 * BK);     // rows per 128-byte bank line
  static constexpr int ROW_BYTES = 2 * BK;
  static constexpr int L = ROWS / (NWG * RPI);   // load instructions per wave per stage
  static constexpr int STAGE_BYTES = ROWS * ROW_BYTES;
  static constexpr int RING_BYTES = KS * S * STAGE_BYTES;
  static constexpr int RED_BYTES = KS > 1 ? KS * BM * BN * 4 : 0;  // partial tiles, over the drained ring
  static constexpr int LDS_BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(TM >= 1 && TN >= 1 && BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(NWG * KS == NW && WM * WN == NWG && ROWS % (NWG * RPI) == 0,
                "whole load instructions per wave");
  static_assert(S >= 2 && LDS_BYTES <= 160 * 1024 && NW * 64 <= 1024, "LDS ring, workgroup");
};
// Stored position of unit u of LDS row r, XOR-swizzled so that a fragment
// read (16 consecutive rows at one unit) is free of bank conflicts whether
// the banks serve 128 bytes (eight lanes) or 256 bytes (sixteen lanes) at a
// time: eight consecutive rows map to distinct 16-byte slots of a 128-byte
// bank line, and the second eight rows of the 16 to the opposite slots.
template <class C>
__device__ __forceinline__ int tile_unit_pos(int r, int u) {
  return u ^ ((r / C::RPL) % C::UPR) ^ ((r / (C::RPL * C::UPR)) & 1);
}

__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Address-space casts live in device helpers: the kernel body is also
// checked by the host pass, where they are not valid.
__device__ __forceinline__ void tile_load_lds(const uint16_t* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((const SPECV_TILE_GLOBAL void*)src,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
template <class T>
__device__ __forceinline__ void tile_store(void* y, size_t i, T v) {
  ((SPECV_TILE_GLOBAL T*)y)[i] = v;
}

template <int N>
__device__ __forceinline__ void tile_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int S, int BK, int NW, int KS, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void gemm_tile_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y, int M,
    int N, int K, int n_tiles, int per_xcd) {
  using C = TileCfg<BM, BN, WM, S, BK, NW, KS>;
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-grouped tile order: workgroup bid runs on XCD bid % 8
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= n_tiles) return;
  const int MT = (M + BM - 1) / BM;
  const int tm = t % MT, tn = t / MT;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kg = wave / C::NWG, wr = wave % C::NWG;  // k-group, wave inside it
  const int wm = wr / C::WN, wn = wr % C::WN;
  const int n_k = K / BK;
  const int n_j = (n_k + KS - 1) / KS;  // ring steps; group kg's step st is k-tile st * KS + kg

  // This lane's source row and unit for each of its L load instructions: the
  // instruction covers LDS rows RPI*g .. RPI*g + RPI-1 (g = wr + NWG*q); lane
  // l writes LDS row RPI*g + l/UPR at stored unit l%UPR, which holds the
  // row's global unit tile_unit_pos(row, l%UPR) (the swizzle is its own
  // inverse).
  const uint16_t* src[C::L];
#pragma unroll
  for (int q = 0; q < C::L; ++q) {
    const int r = C::RPI * (wr + C::NWG * q) + lane / C::UPR;
    const int u = tile_unit_pos<C>(r, lane % C::UPR);
    const uint16_t* p;
    if (r < BM)
      p = X + (size_t)min(m0 + r, M - 1) * K + u * 8;
    else
      p = W + (size_t)min(n0 + (r - BM), N - 1) * K + u * 8;
    src[q] = p;
  }
  auto issue = [&](int st) __attribute__((always_inline)) {
    // k-tiles past the end reload the last one into a slot nobody reads
    const int kc = min(st * KS + kg, n_k - 1);
    const int slot = kg * S + st % S;
#pragma unroll
    for (int q = 0; q < C::L; ++q) {
      tile_load_lds(src[q] + (size_t)kc * BK, reinterpret_cast<char*>(lds) + slot * C::STAGE_BYTES +
                                                  C::RPI * (wr + C::NWG * q) * C::ROW_BYTES);
    }
  };

  f32x4 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);

  for (int st = 0; st < n_j; ++st) {
    tile_wait_vmcnt<(S - 2) * C::L>();  // this wave's loads of step st have landed
    tile_barrier();                     // everyone's; and step st-1's slots are free
    issue(st + S - 1);
    if (KS > 1 && st * KS + kg >= n_k) continue;  // this group has no k-tile left
    const char* base = reinterpret_cast<const char*>(lds) + (kg * S + st % S) * C::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int unit = kk * 4 + (lane >> 4);
      bf16x8 a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int r = wm * (BM / WM) + i * 16 + (lane & 15);
        a[i] = *reinterpret_cast<const bf16x8*>(base + r * C::ROW_BYTES +
                                                 (tile_unit_pos<C>(r, unit) << 4));
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = BM + wn * (BN / C::WN) + j * 16 + (lane & 15);
        b[j] = *reinterpret_cast<const bf16x8*>(base + r * C::ROW_BYTES +
                                                 (tile_unit_pos<C>(r, unit) << 4));
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  tile_wait_vmcnt<0>();  // the reloads past the end land before the workgroup leaves

  if constexpr (KS > 1) {
    // partial tiles of the k-groups into LDS (over the ring, once every wave
    // is done with it), then each output is the sum over groups in order
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int jj = 0; jj < C::TN; ++jj) {
        const int col = wn * (BN / C::WN) + jj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
          red[(kg * BM + row) * BN + col] = acc[i][jj][r];
        }
      }
    __syncthreads();
    for (int e = tid; e < BM * BN; e += NW * 64) {
      const int row = m0 + e / BN, col = n0 + e % BN;
      float v = red[e];
#pragma unroll
      for (int g = 1; g < KS; ++g) v += red[g * BM * BN + e];
      if (row < M && col < N) {
        if (OUT_BF16)
          tile_store<uint16_t>(Y, (size_t)row * N + col, f32_to_bf16_bits(v));
        else
          tile_store<float>(Y, (size_t)row * N + col, v);
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int col = n0 + wn * (BN / C::WN) + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
        if (row < M && col < N) {
          const float v = acc[i][j][r];
          if (OUT_BF16)
            tile_store<uint16_t>(Y, (size_t)row * N + col, f32_to_bf16_bits(v));
          else
            tile_store<float>(Y, (size_t)row * N + col, v);
        }
      }
    }
}

template <int BM, int BN, int WM, int S, int BK, int NW = 8, int KS = 1>
static hipError_t launch_tile_t(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16,
                                int M, int K, int N, hipStream_t s) {
  using C = TileCfg<BM, BN, WM, S, BK, NW, KS>;
  const int n_tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int per_xcd = (n_tiles + 7) / 8;
  const dim3 grid(8 * per_xcd);
  static const hipError_t a1 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, true>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  static const hipError_t a2 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, false>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  if (out_bf16)
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, true>), grid, dim3(NW * 64),
                       C::LDS_BYTES, s, x, w, y, M, N, K, n_tiles, per_xcd);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, false>), grid, dim3(NW * 64),
                       C::LDS_BYTES, s, x, w, y, M, N, K, n_tiles, per_xcd);
  return hipGetLastError();
}

// Tile shapes (BM, BN), indexed as in the launch switch of
// launch_gemm_mfma; the first seven use eight waves, the last four (for
// linears with few positions) two or four, so that several of them share a
// CU.
static const int kTileShapes[][2] = {{256, 256}, {256, 128}, {128, 256}, {128, 128},
                                     {128, 64},  {64, 128},  {64, 64},   {64, 32},
                                     {32, 32},   {32, 16},   {32, 64}};

// Time model of one launch, per reduction element: a tile costs
// a * (BM + BN) (operand lines into LDS and out to the matrix cores) plus
// b * BM * BN (the products), and the tiles run in ceil(tiles / CUs) rounds.
// a and b were fitted to measured Llama-shaped linears at M = 320 and 1280
// on MI355X. At M = 20 to 128 the shapes it picks for the Llama-3.1-8B
// linears were checked against every small shape forced in turn: the pick
// was the fastest, or within about 10 % of it.
static int pick_tile(int M, int N, int cus) {
  const double a = 3.6e-5, b = 8.1e-8;
  const int n = sizeof(kTileShapes) / sizeof(kTileShapes[0]);
  int best = 0;
  double best_t = 0.0;
  for (int i = 0; i < n; ++i) {
    const int bm = kTileShapes[i][0], bn = kTileShapes[i][1];
    const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const long rounds = (tiles + cus - 1) / cus;
    const double t = rounds * (a * (bm + bn) + b * (double)bm * bn);
    if (i == 0 || t < best_t) {
      best_t = t;
      best = i;
    }
  }
  return best;
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
  if (K % kTileKAlign == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const int pick = pick_tile(M, N, cus);
    const long tiles = (long)((M + kTileShapes[pick][0] - 1) / kTileShapes[pick][0]) *
                       ((N + kTileShapes[pick][1] - 1) / kTileShapes[pick][1]);
    if (tiles <= cus) {
      // One round of small tiles: the same tile with the reduction split over
      // k-groups of eight waves in all, so that each CU has as many loads in
      // flight as a large tile's (measured on the Llama linears at M = 20 to
      // 128: O and down 15-30 % faster, QKV 5-20 %).
      switch (pick) {
        case 6: return launch_tile_t<64, 64, 2, 4, 64, 8, 2>(x, w, y, out_bf16, M, K, N, s);
        case 7: return launch_tile_t<64, 32, 2, 4, 64, 8, 2>(x, w, y, out_bf16, M, K, N, s);
        case 8: return launch_tile_t<32, 32, 2, 4, 64, 8, 2>(x, w, y, out_bf16, M, K, N, s);
        case 9: return launch_tile_t<32, 16, 2, 4, 64, 8, 4>(x, w, y, out_bf16, M, K, N, s);
        default: break;
      }
    }
    switch (pick) {
      case 0: return launch_tile_t<256, 256, 4, 2, 64>(x, w, y, out_bf16, M, K, N, s);
      case 1: return launch_tile_t<256, 128, 4, 3, 64>(x, w, y, out_bf16, M, K, N, s);
      case 2: return launch_tile_t<128, 256, 2, 3, 64>(x, w, y, out_bf16, M, K, N, s);
      case 3: return launch_tile_t<128, 128, 2, 4, 64>(x, w, y, out_bf16, M, K, N, s);
      case 4: return launch_tile_t<128, 64, 4, 4, 64>(x, w, y, out_bf16, M, K, N, s);
      case 5: return launch_tile_t<64, 128, 2, 4, 64>(x, w, y, out_bf16, M, K, N, s);
      case 6: return launch_tile_t<64, 64, 2, 4, 64>(x, w, y, out_bf16, M, K, N, s);
      case 7: return launch_tile_t<64, 32, 2, 4, 64, 4>(x, w, y, out_bf16, M, K, N, s);
      case 8: return launch_tile_t<32, 32, 2, 6, 64, 4>(x, w, y, out_bf16, M, K, N, s);
      case 9: return launch_tile_t<32, 16, 2, 6, 64, 2>(x, w, y, out_bf16, M, K, N, s);
      default: return launch_tile_t<32, 64, 1, 4, 64, 4>(x, w, y, out_bf16, M, K, N, s);
    }
  }
  if (M <= 32) return launch_mfma_t<32, 64, 1>(x, w, y, out_bf16, M, K, N, s);
  if (M <= 128) return launch_mfma_t<64, 64, 2>(x, w, y, out_bf16, M, K, N, s);
  return launch_mfma_t<128, 128, 2>(x, w, y, out_bf16, M, K, N, s);
}

}  // namespace specv
