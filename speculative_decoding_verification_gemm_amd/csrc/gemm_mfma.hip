// Verify-pass linears for many verify positions: y[M][N] = x[M][K] . w[N][K]^T
// with bf16 MFMA (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16) and
// fp32 accumulators; w bf16, or FP8 E4M3 codes with a scale per row.
//
// Once B*(K+1) positions make the product a real dense contraction (the
// batch crossover of "Speculative Decoding: Guess Several Tokens, Check Them
// in One Pass", What happens at larger batches), tiles of x and w are staged
// in LDS and multiplied on the matrix cores. Few positions use the
// weight-streaming kernel in gemm_stream.hip instead.

#include <stdlib.h>
#include <string.h>

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
// (global_load_lds, no registers). Inside a row the 16-byte units are
// stored XOR-swizzled (tile_unit_pos below), so that the MFMA fragment reads
// are free of LDS bank conflicts. S tile stages are in flight;
// each wave waits (vmcnt) for its own loads of the stage it computes on and
// a workgroup barrier makes every wave's loads visible. The barrier is a
// bare s_barrier: a memory fence there would make the compiler wait for all
// loads in flight. Tiles are numbered so that the workgroups of one XCD
// (bid mod 8) take consecutive tiles, which share weight tiles in that XCD's
// L2.

constexpr int kTileKAlign = 64;  // the kernel needs K to be a multiple of this

// BK reduction elements per stage: 64 (a whole 128-byte line of each row) or
// 32 (half a line; the other half follows in the next stage, from L2), which
// halves a stage so that more of them fit in LDS; with FP8 weights also 128
// (a whole 128-byte line of each weight row).
// KS > 1 splits the reduction inside the workgroup: the waves form KS
// groups of NW / KS, group g takes k-tiles g, g + KS, ... through a ring of
// its own, and the KS partial tiles are added through LDS in group order at
// the end (deterministic). A small tile then still has NW waves' loads in
// flight.
//
// MF is the MFMA block: 16 (v_mfma_f32_16x16x32_bf16, a k-step of 32) or 32
// (v_mfma_f32_32x32x16_bf16, a k-step of 16). Both read one 16-byte operand
// unit per lane per k-step, so a wave tile reads the same LDS bytes per
// reduction element either way; the 32x32 form issues half as many MFMAs
// for the same products, and measured on MI355X a stream of independent
// 32x32x16 MFMAs reaches about 1.9 PFLOP/s where 16x16x32 reaches about 1.2.
// W8: the weights are FP8 E4M3 codes (one byte each) with one fp32 scale
// per output row (weight-only 8-bit storage, "Speculative Decoding: The
// Algebra and the Proof", Where it breaks). A weight row then takes BK
// bytes of LDS per stage instead of 2 BK; fragment reads fetch 8 codes (8
// bytes) per lane and widen them exactly to bf16 before the same MFMA, and
// the row's scale multiplies the fp32 sum in the epilogue.
template <int BM, int BN, int WM, int S, int BK, int NW, int KS = 1, int MF = 16, bool W8 = false,
          bool WL = false>
struct TileCfg {
  static constexpr int NWG = NW / KS;            // waves per k-group
  static constexpr int WN = NWG / WM;            // a group's waves: WM along M, WN along N
  static constexpr int TM = BM / WM / MF, TN = BN / WN / MF;
  static constexpr int MFB = MF;
  static constexpr int KSTEP = MF == 16 ? 32 : 16;  // reduction elements per MFMA
  static constexpr int NACC = MF == 16 ? 4 : 16;    // accumulator floats per lane per block
  // A stage holds BM x rows (bf16), then BN w rows (bf16, or FP8 codes).
  static constexpr int ROW_A = 2 * BK;
  static constexpr int ROW_B = (W8 ? 1 : 2) * BK;
  static constexpr int UPR_A = ROW_A / 16, UPR_B = ROW_B / 16;  // 16-byte units per row
  static constexpr int RPI_A = 64 / UPR_A, RPI_B = 64 / UPR_B;  // rows per 1 KB load instruction
  static constexpr int IA = BM / RPI_A, IB = BN / RPI_B;        // load instructions per stage
  // load instructions per wave per stage; when the stage's IA + IB do not
  // divide among the NWG waves, the spare ones reload one line of x into a
  // dummy kilobyte that nothing reads, so every wave's vmcnt waits are equal
  static constexpr int L = (IA + IB + NWG - 1) / NWG;
  static constexpr int DUMMY_BYTES = L * NWG > IA + IB ? 1024 : 0;
  static constexpr int B_OFF = BM * ROW_A;       // w rows' offset in a stage
  static constexpr int STAGE_BYTES = B_OFF + BN * ROW_B;
  static constexpr int RING_BYTES = KS * S * STAGE_BYTES;
  static constexpr int RED_BYTES = KS > 1 ? KS * BM * BN * 4 : 0;  // partial tiles, over the drained ring
  // WL (FP8 weights): each stage's codes are widened once per workgroup
  // into a bf16 region of BN rows of 2 BK bytes after the ring
  static constexpr int ROW_W = 2 * BK, UPR_W = ROW_W / 16;
  static constexpr int WIDE_BYTES = WL ? BN * ROW_W : 0;
  static constexpr int LDS_BYTES =
      (RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES) + DUMMY_BYTES + WIDE_BYTES;
  static constexpr int DUMMY_OFF = LDS_BYTES - WIDE_BYTES - DUMMY_BYTES;
  static_assert(!WL || (W8 && KS == 1), "widening in LDS: FP8 weights, one k-group");
  static_assert(BK == 32 || BK == 64 || (W8 && BK == 128), "stage depth");
  static_assert(MF == 16 || MF == 32, "MFMA block");
  static_assert(TM >= 1 && TN >= 1 && BM % (MF * WM) == 0 && BN % (MF * WN) == 0, "wave tile");
  static_assert(NWG * KS == NW && WM * WN == NWG && BM % RPI_A == 0 && BN % RPI_B == 0,
                "whole load instructions");
  static_assert(S >= 2 && LDS_BYTES <= 160 * 1024 && NW * 64 <= 1024, "LDS ring, workgroup");
};
// Stored position of unit u of LDS row r in a region of UPR 16-byte units
// per row, XOR-swizzled so that fragment reads are free of bank conflicts.
// Measured on MI355X (SQ_LDS_BANK_CONFLICT of a probe kernel): a
// 16-byte-per-lane LDS read is served for lanes 0-7 together with lanes
// 32-39 (and 8-15 with 40-47, ...), over 256 bytes of banks, so those 16
// lanes must hit 16 distinct 16-byte slots of a 256-byte window.
//  * 32x32 fragments (lane l: row l % 32, unit l / 32 of the k-step): rows
//    r and r of the next unit meet, so the rows of one parity need distinct
//    positions that stay distinct after flipping the unit's low bit: the
//    row index itself, u ^ (r mod 8) ^ (bit 3 of r).
//  * 16x16 fragments (row l % 16, unit l / 16): rows r at units u and
//    u + 2 meet, so positions must stay distinct after flipping bit 1:
//    u ^ g(r) with g taking 0, 0, 1, 1, 4, 4, 5, 5 over r mod 8 (rows of one
//    parity take 0, 1, 4, 5), and bit 1 set for rows 8-15.
// The former (row index) swizzle costs four conflict cycles per 16x16
// fragment read; both forms here measure zero. 64-byte rows (BK = 32, or
// FP8 weight rows) keep the row-index form over two rows per 128 bytes.
template <int UPR, int MF>
__device__ __forceinline__ int tile_unit_pos(int r, int u) {
  // 256-byte rows (activations of 128-element FP8 stages): one row fills
  // the 256-byte window, so the 16 lanes that meet need distinct positions
  // among 16: g(r) keeps g and g ^ 2 apart for 16x16 (0, 1, 4, 5, 8, 9, 12,
  // 13 over r mod 8), g and g ^ 1 for 32x32 (0, 2, 4, ..., 14).
  if constexpr (UPR == 16) {
    if constexpr (MF == 16) return u ^ ((r & 1) | ((r & 6) << 1));
    return u ^ ((r & 7) << 1);
  }
  if constexpr (MF == 16 && UPR == 8)
    return u ^ ((((r >> 1) & 1) | (((r >> 2) & 1) << 2)) ^ (((r >> 3) & 1) << 1));
  constexpr int RPL = 8 / UPR;  // rows per 128-byte line
  return u ^ ((r / RPL) % UPR) ^ ((r / (RPL * UPR)) & 1);
}

__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Address-space casts live in device helpers: the kernel body is also
// checked by the host pass, where they are not valid.
__device__ __forceinline__ void tile_load_lds(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((const SPECV_TILE_GLOBAL void*)src,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
template <class T>
__device__ __forceinline__ void tile_store(void* y, size_t i, T v) {
  ((SPECV_TILE_GLOBAL T*)y)[i] = v;
}
__device__ __forceinline__ float tile_scale(const float* ws, int col) {
  return ((const SPECV_TILE_GLOBAL float*)ws)[col];
}
__device__ __forceinline__ void tile_store16(void* base, size_t byte_off, u32x4 v) {
  *(SPECV_TILE_GLOBAL u32x4*)(static_cast<char*>(base) + byte_off) = v;
}

// One staged block of the epilogue (R rows of WTN fp32 values, LDW floats
// apart in LDS) to rows row0.. and columns col0.. of an output of ld
// elements per row: each lane takes 16 bytes of a row per store (8 bf16 or
// 4 fp32 outputs), so a wave's store covers whole runs of a row instead of
// one 16- or 32-column piece per row. Element by element at the right edge
// and where the output is not 16-byte aligned.
template <int R, int WTN, int LDW, bool BF>
__device__ __forceinline__ void tile_emit_block(const float* stg, void* base, int ld, bool vec_ok,
                                                int row0, int col0, int M, int N, int lane) {
  constexpr int VEC = BF ? 8 : 4, CPR = WTN / VEC;
  static_assert(WTN % VEC == 0, "whole stores per row");
#pragma unroll
  for (int it = 0; it < (R * CPR + 63) / 64; ++it) {
    const int c = lane + 64 * it;
    if (R * CPR % 64 != 0 && c >= R * CPR) break;
    const int rr = c / CPR, cc = (c - rr * CPR) * VEC;
    const int row = row0 + rr, col = col0 + cc;
    if (row >= M) continue;
    const float* sp = stg + rr * LDW + cc;
    const size_t off = (size_t)row * ld + col;
    if (vec_ok && col + VEC <= N) {
      if constexpr (BF) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sp);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sp + 4);
        auto pk = [](uint32_t a, uint32_t b) {
          return (uint32_t)f32_to_bf16_bits(__builtin_bit_cast(float, a)) |
                 ((uint32_t)f32_to_bf16_bits(__builtin_bit_cast(float, b)) << 16);
        };
        tile_store16(base, off * 2,
                     u32x4{pk(lo.x, lo.y), pk(lo.z, lo.w), pk(hi.x, hi.y), pk(hi.z, hi.w)});
      } else {
        tile_store16(base, off * 4, *reinterpret_cast<const u32x4*>(sp));
      }
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        if (col + v < N) {
          if constexpr (BF)
            tile_store<uint16_t>(base, off + v, f32_to_bf16_bits(sp[v]));
          else
            tile_store<float>(base, off + v, sp[v]);
        }
    }
  }
}

template <int N>
__device__ __forceinline__ void tile_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// lgkmcnt(0): this wave's LDS accesses are complete. The builtin alone is
// not ordered against LDS accesses by the compiler; the empty asm with a
// memory clobber on both sides keeps them where they are written.
__device__ __forceinline__ void tile_wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt at their maxima, lgkmcnt 0
  asm volatile("" ::: "memory");
}

// Two FP8 E4M3 codes (the low or high 16 bits of v) widened to a bf16 pair;
// every E4M3 value is exact in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t tile_widen_fp8x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

// One MFMA on a pair of 16-byte operand fragments.
template <int MF, class Acc>
__device__ __forceinline__ Acc tile_mfma(bf16x8 a, bf16x8 b, Acc c) {
  if constexpr (MF == 16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int BM, int BN, int WM, int S, int BK, int NW, int KS, int MF, bool W8, bool WL,
          bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void gemm_tile_kernel(
    const uint16_t* __restrict__ X, const void* __restrict__ W, const float* __restrict__ WS,
    void* __restrict__ Y, int M, int N, int K, int n_tiles, int per_xcd, int sk, int ldy) {
  using C = TileCfg<BM, BN, WM, S, BK, NW, KS, MF, W8, WL>;
  typedef float facc __attribute__((ext_vector_type(C::NACC)));
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-grouped tile order: workgroup bid runs on XCD bid % 8
  // Work item (tile t, reduction split s): with sk > 1 the K stages of a
  // tile are split over sk workgroups, each storing an fp32 partial tile
  // (to Y, then a workspace of sk x M x N floats) that the split-sum kernel
  // adds up in split order.
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= n_tiles * sk) return;
  const int t = item / sk, split = item - t * sk;
  const int MT = (M + BM - 1) / BM;
  const int tm = t % MT, tn = t / MT;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kg = wave / C::NWG, wr = wave % C::NWG;  // k-group, wave inside it
  const int wm = wr / C::WN, wn = wr % C::WN;
  const int k_begin = split * (K / BK) / sk, k_end = (split + 1) * (K / BK) / sk;
  const int n_k = k_end - k_begin;      // this work item's k-tiles, from k_begin
  const int n_j = (n_k + KS - 1) / KS;  // ring steps; group kg's step st is k-tile st * KS + kg

  // This lane's source address for each of its L load instructions. Load
  // instruction g = wr + NWG q fills bytes [1 KB g, 1 KB (g + 1)) of a stage:
  // x rows RPI_A g .. while g < IA, then w rows RPI_B (g - IA) ... Lane l
  // writes row RPI g' + l / UPR of its region at stored unit l % UPR, which
  // holds the row's global unit tile_unit_pos(row, l % UPR) (the swizzle is
  // its own inverse). kstride: bytes of one k-tile along the row.
  const char* src[C::L];
  int kstride[C::L];
#pragma unroll
  for (int q = 0; q < C::L; ++q) {
    const int g = wr + C::NWG * q;
    if (C::DUMMY_BYTES > 0 && g >= C::IA + C::IB) {
      // a spare instruction: the same valid line at every stage
      src[q] = reinterpret_cast<const char*>(X);
      kstride[q] = 0;
    } else if (g < C::IA) {
      const int r = C::RPI_A * g + lane / C::UPR_A;
      const int u = tile_unit_pos<C::UPR_A, MF>(r, lane % C::UPR_A);
      src[q] = reinterpret_cast<const char*>(X + (size_t)min(m0 + r, M - 1) * K) + u * 16;
      kstride[q] = C::ROW_A;
    } else {
      const int r = C::RPI_B * (g - C::IA) + lane / C::UPR_B;
      const int u = tile_unit_pos<C::UPR_B, MF>(r, lane % C::UPR_B);
      src[q] = static_cast<const char*>(W) + (size_t)min(n0 + r, N - 1) * K * (W8 ? 1 : 2) + u * 16;
      kstride[q] = C::ROW_B;
    }
  }
  auto issue = [&](int st) __attribute__((always_inline)) {
    // k-tiles past the end reload the last one into a slot nobody reads
    const int kc = k_begin + min(st * KS + kg, n_k - 1);
    const int slot = kg * S + st % S;
#pragma unroll
    for (int q = 0; q < C::L; ++q) {
      const int g = wr + C::NWG * q;
      char* dst = reinterpret_cast<char*>(lds) + slot * C::STAGE_BYTES + g * 1024;
      if constexpr (C::DUMMY_BYTES > 0)
        if (g >= C::IA + C::IB) dst = reinterpret_cast<char*>(lds) + C::DUMMY_OFF;
      tile_load_lds(src[q] + (size_t)kc * kstride[q], dst);
    }
  };

  facc acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) acc[i][j][e] = 0.f;
  // Output position of accumulator float e of block (i, j) held by this
  // lane: 16x16 blocks hold rows 4 (lane / 16) + e of column lane % 16;
  // 32x32 blocks rows 8 (e / 4) + 4 (lane / 32) + e % 4 of column lane % 32.
  auto out_row = [&](int i, int e) __attribute__((always_inline)) {
    return MF == 16 ? wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + e
                    : wm * (BM / WM) + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
  };
  auto out_col = [&](int j) __attribute__((always_inline)) {
    return wn * (BN / C::WN) + j * MF + (lane & (MF - 1));
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);

  for (int st = 0; st < n_j; ++st) {
    tile_wait_vmcnt<(S - 2) * C::L>();  // this wave's loads of step st have landed
    tile_barrier();                     // everyone's; and step st-1's slots are free
    issue(st + S - 1);
    if (KS > 1 && st * KS + kg >= n_k) continue;  // this group has no k-tile left
    const char* base = reinterpret_cast<const char*>(lds) + (kg * S + st % S) * C::STAGE_BYTES;
    char* wide = reinterpret_cast<char*>(lds) + C::LDS_BYTES - C::WIDE_BYTES;
    if constexpr (WL) {
      // widen the stage's codes once for the workgroup: 16 codes (one
      // 16-byte unit) per thread and pass into two bf16 units of the wide
      // region (whose previous contents every wave finished with before the
      // barrier above); then make them visible to every wave
      constexpr int UPB = BK / 16;  // code units per weight row
      for (int c = tid; c < BN * UPB; c += NW * 64) {
        const int r = c / UPB, u = c - r * UPB;
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            base + C::B_OFF + r * C::ROW_B + (tile_unit_pos<C::UPR_B, MF>(r, u) << 4));
        const u32x4 lo{tile_widen_fp8x2<false>(v.x), tile_widen_fp8x2<true>(v.x),
                       tile_widen_fp8x2<false>(v.y), tile_widen_fp8x2<true>(v.y)};
        const u32x4 hi{tile_widen_fp8x2<false>(v.z), tile_widen_fp8x2<true>(v.z),
                       tile_widen_fp8x2<false>(v.w), tile_widen_fp8x2<true>(v.w)};
        *reinterpret_cast<u32x4*>(wide + r * C::ROW_W + (tile_unit_pos<C::UPR_W, MF>(r, 2 * u) << 4)) = lo;
        *reinterpret_cast<u32x4*>(wide + r * C::ROW_W +
                                  (tile_unit_pos<C::UPR_W, MF>(r, 2 * u + 1) << 4)) = hi;
      }
      tile_wait_lgkm0();  // this wave's LDS writes are done
      tile_barrier();
    }
#pragma unroll
    for (int kk = 0; kk < BK / C::KSTEP; ++kk) {
      // lane l supplies row l % MF of its block and the 8 reduction
      // elements starting at 8 (l / MF) of the k-step
      const int k8 = kk * C::KSTEP + 8 * (lane / MF);
      bf16x8 a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int r = wm * (BM / WM) + i * MF + (lane & (MF - 1));
        a[i] = *reinterpret_cast<const bf16x8*>(
            base + r * C::ROW_A + (tile_unit_pos<C::UPR_A, MF>(r, k8 >> 3) << 4));
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = wn * (BN / C::WN) + j * MF + (lane & (MF - 1));
        const char* row = base + C::B_OFF + r * C::ROW_B;
        if constexpr (WL) {
          b[j] = *reinterpret_cast<const bf16x8*>(
              wide + r * C::ROW_W + (tile_unit_pos<C::UPR_W, MF>(r, k8 >> 3) << 4));
        } else if constexpr (W8) {
          // 8 codes: half (k8 / 8) % 2 of unit k8 / 16, widened to 8 bf16
          const uint2 v = *reinterpret_cast<const uint2*>(
              row + (tile_unit_pos<C::UPR_B, MF>(r, k8 >> 4) << 4) + ((k8 >> 3) & 1) * 8);
          const u32x4 wv{tile_widen_fp8x2<false>(v.x), tile_widen_fp8x2<true>(v.x),
                         tile_widen_fp8x2<false>(v.y), tile_widen_fp8x2<true>(v.y)};
          b[j] = __builtin_bit_cast(bf16x8, wv);
        } else {
          b[j] = *reinterpret_cast<const bf16x8*>(
              row + (tile_unit_pos<C::UPR_B, MF>(r, k8 >> 3) << 4));
        }
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = tile_mfma<MF>(a[i], b[j], acc[i][j]);
    }
  }
  tile_wait_vmcnt<0>();  // the reloads past the end land before the workgroup leaves

  // Epilogue through LDS (one k-group, and 64 or more outputs per lane):
  // each wave writes one row of its blocks (MF rows of its wave tile) into a
  // padded staging block of its own over the drained ring, then stores it
  // along the rows, 16 bytes a lane (tile_emit_block). Stored directly, the
  // blocks' own layout (4 rows of 16 columns, or 2 of 32, per store) takes
  // one store instruction per output of a lane, each writing 32- to 128-byte
  // pieces of rows. Measured on the Llama-3.1-8B linears: 2-5 % faster with
  // 320x256, 256x256 and 320x128 tiles (up to 14 % with FP8 weights); 1-2 %
  // slower with 32 or fewer outputs per lane, which keep the direct stores.
  constexpr int WTN = BN / C::WN;           // wave tile columns
  constexpr int LDW = WTN + 4;              // staged row, floats (padded against bank conflicts)
  constexpr int STG_BYTES = MF * LDW * 4;   // one wave's staging block
  if constexpr (KS == 1 && C::TM * C::TN * C::NACC >= 64 && NW * STG_BYTES <= C::LDS_BYTES &&
                WTN % 8 == 0) {
    __syncthreads();  // every wave's loads have landed and its ring reads are done
    float* stg = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + wave * STG_BYTES);
    const int r0 = wm * (BM / WM), c0 = wn * WTN;  // wave tile origin in the tile
    const bool partial = sk > 1;
    // a partial tile goes to split `split` of the workspace (fp32, unscaled)
    void* dst = partial ? static_cast<void*>(static_cast<float*>(Y) + (size_t)split * M * N) : Y;
    const int ld = partial ? N : ldy;
    float sc[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int col = n0 + out_col(j);
      sc[j] = W8 && !partial && col < N ? tile_scale(WS, col) : 1.0f;
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int col = out_col(j) - c0;
#pragma unroll
        for (int e = 0; e < C::NACC; ++e)
          stg[(out_row(i, e) - r0 - i * MF) * LDW + col] =
              W8 ? acc[i][j][e] * sc[j] : acc[i][j][e];
      }
      tile_wait_lgkm0();  // the block is in LDS (one wave writes and reads it)
      if (!partial && OUT_BF16) {
        const bool vec_ok = (reinterpret_cast<uintptr_t>(dst) & 15) == 0 && ld % 8 == 0;
        tile_emit_block<MF, WTN, LDW, true>(stg, dst, ld, vec_ok, m0 + r0 + i * MF, n0 + c0, M, N,
                                            lane);
      } else {
        const bool vec_ok = (reinterpret_cast<uintptr_t>(dst) & 15) == 0 && ld % 4 == 0;
        tile_emit_block<MF, WTN, LDW, false>(stg, dst, ld, vec_ok, m0 + r0 + i * MF, n0 + c0, M,
                                             N, lane);
      }
      tile_wait_lgkm0();  // its reads are done before the next block overwrites it
    }
    return;
  }

  if (sk > 1) {
    // a partial tile: fp32, unscaled, to split `split` of the workspace
    float* part = static_cast<float*>(Y) + (size_t)split * M * N;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int col = n0 + out_col(j);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int e = 0; e < C::NACC; ++e) {
          const int row = m0 + out_row(i, e);
          if (row < M && col < N) tile_store<float>(part, (size_t)row * N + col, acc[i][j][e]);
        }
    }
    return;
  }
  auto store = [&](int row, int col, float v) __attribute__((always_inline)) {
    if (OUT_BF16)
      tile_store<uint16_t>(Y, (size_t)row * ldy + col, f32_to_bf16_bits(v));
    else
      tile_store<float>(Y, (size_t)row * ldy + col, v);
  };
  if constexpr (KS > 1) {
    // partial tiles of the k-groups into LDS (over the ring, once every wave
    // is done with it), then each output is the sum over groups in order
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int jj = 0; jj < C::TN; ++jj) {
        const int col = out_col(jj);
#pragma unroll
        for (int e = 0; e < C::NACC; ++e) red[(kg * BM + out_row(i, e)) * BN + col] = acc[i][jj][e];
      }
    __syncthreads();
    for (int e = tid; e < BM * BN; e += NW * 64) {
      const int row = m0 + e / BN, col = n0 + e % BN;
      float v = red[e];
#pragma unroll
      for (int g = 1; g < KS; ++g) v += red[g * BM * BN + e];
      if (row < M && col < N) store(row, col, W8 ? v * tile_scale(WS, col) : v);
    }
    return;
  }

#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int col = n0 + out_col(j);
    const float sc = W8 && col < N ? tile_scale(WS, col) : 1.0f;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) {
        const int row = m0 + out_row(i, e);
        if (row < M && col < N) store(row, col, W8 ? acc[i][j][e] * sc : acc[i][j][e]);
      }
  }
}

// The sk partial tiles of a split reduction added in split order (fixed, so
// the result is deterministic), scaled by the row scale for FP8 weights and
// stored as the output. Each thread takes four consecutive outputs with
// 16-byte loads when M * N is a multiple of four (every partial slice is
// then 16-byte aligned), else one at a time.
template <bool OUT_BF16, bool W8>
__global__ __launch_bounds__(256) void gemm_split_sum_kernel(const float* __restrict__ P,
                                                             const float* __restrict__ WS,
                                                             void* __restrict__ Y, int M, int N,
                                                             int sk) {
  const size_t mn = (size_t)M * N;
  const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= mn) return;
  float v[4];
  int cnt = 4;
  if ((mn & 3) == 0) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const SPECV_TILE_GLOBAL f32x4* p4 = (const SPECV_TILE_GLOBAL f32x4*)(P + i0);
    f32x4 a = p4[0];
    for (int p = 1; p < sk; ++p) a += p4[(size_t)p * (mn / 4)];
    v[0] = a.x;
    v[1] = a.y;
    v[2] = a.z;
    v[3] = a.w;
  } else {
    cnt = (int)min((size_t)4, mn - i0);
    for (int e = 0; e < cnt; ++e) {
      float a = P[i0 + e];
      for (int p = 1; p < sk; ++p) a += P[(size_t)p * mn + i0 + e];
      v[e] = a;
    }
  }
  for (int e = 0; e < cnt; ++e) {
    const size_t i = i0 + e;
    const float x = W8 ? v[e] * tile_scale(WS, (int)(i % N)) : v[e];
    if (OUT_BF16)
      tile_store<uint16_t>(Y, i, f32_to_bf16_bits(x));
    else
      tile_store<float>(Y, i, x);
  }
}

// sk > 1: the reduction is split over sk workgroups per tile (whole k-tiles,
// at least one each) whose fp32 partial tiles go to `partials` (sk x M x N
// floats), then added up by the split-sum kernel; one k-group per workgroup.
template <int BM, int BN, int WM, int S, int BK, int NW = 8, int KS = 1, int MF = 16,
          bool W8 = false, bool WL = false>
static hipError_t launch_tile_t(const uint16_t* x, const void* w, const float* ws, void* y,
                                bool out_bf16, int M, int K, int N, hipStream_t s,
                                float* partials = nullptr, int sk = 1, int ldy = 0) {
  using C = TileCfg<BM, BN, WM, S, BK, NW, KS, MF, W8, WL>;
  if (ldy == 0) ldy = N;  // output rows of N elements unless a wider stride is given
  if (K % BK != 0 || ldy < N) return hipErrorInvalidValue;  // whole stages only
  if (sk < 1 || (sk > 1 && (KS != 1 || partials == nullptr || K / BK < sk || ldy != N)))
    return hipErrorInvalidValue;
  const int n_tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int per_xcd = (n_tiles * sk + 7) / 8;
  const dim3 grid(8 * per_xcd);
  static const hipError_t a1 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, MF, W8, WL, true>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  static const hipError_t a2 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, MF, W8, WL, false>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  if (sk > 1) {
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, MF, W8, WL, false>), grid,
                       dim3(NW * 64), C::LDS_BYTES, s, x, w, ws, partials, M, N, K, n_tiles,
                       per_xcd, sk, N);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 sgrid((unsigned)(((size_t)M * N + 1023) / 1024));  // four outputs per thread
    if (out_bf16)
      hipLaunchKernelGGL((gemm_split_sum_kernel<true, W8>), sgrid, dim3(256), 0, s, partials, ws, y,
                         M, N, sk);
    else
      hipLaunchKernelGGL((gemm_split_sum_kernel<false, W8>), sgrid, dim3(256), 0, s, partials, ws,
                         y, M, N, sk);
    return hipGetLastError();
  }
  if (out_bf16)
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, MF, W8, WL, true>), grid,
                       dim3(NW * 64), C::LDS_BYTES, s, x, w, ws, y, M, N, K, n_tiles, per_xcd, 1,
                       ldy);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, S, BK, NW, KS, MF, W8, WL, false>), grid,
                       dim3(NW * 64), C::LDS_BYTES, s, x, w, ws, y, M, N, K, n_tiles, per_xcd, 1,
                       ldy);
  return hipGetLastError();
}

// Tile shapes (BM, BN), indexed as in the launch switch of
// launch_gemm_mfma: the first seven and the two 320-row tiles use eight
// waves; the four small ones (for linears with few positions) two or four,
// so that several of them share a CU, or eight in k-groups when their tiles
// fit one round. The last kExactFillShapes are candidates only where their
// tiles number exactly one per CU: 80x64 (ten waves in two k-groups),
// 160x128 (eight waves), 160x224 (fourteen waves), 160x192 (eight) and
// 64x48 (eight waves in two k-groups).
// Measured on the Llama-3.1-8B O projection (4096 -> 4096): at M = 320,
// 80x64 22.7 against 26.6 us (128x64); at M = 1280, 160x128 48.3 against
// 55.8 (320x128 tiles, two splits); on gate/up (4096 -> 28672) at M = 320,
// 160x224 85-86 against 92-93 us (320x128), and on the Llama-3.1-70B
// gate/up (8192 -> 57344) at M = 160, 195 against 242; 160x192 on QKV
// (4096 -> 6144) at M = 1280, 66 against 67-69 us (256x128); 64x48 on
// QKV at M = 80 (B = 16 step 4.33 against 4.37 ms with 64x64 tiles). A
// 32x112 exact fill for gate/up at M = 20 made the B = 4 step 6 % slower
// and is not in the table.
static const int kTileShapes[][2] = {{256, 256}, {256, 128}, {128, 256}, {128, 128},
                                     {128, 64},  {64, 128},  {64, 64},   {64, 32},
                                     {32, 32},   {32, 16},   {32, 64},   {320, 128},
                                     {320, 256}, {80, 64},   {160, 128}, {160, 224},
                                     {160, 192}, {64, 48}};
constexpr int kExactFillShapes = 5;

// Time model of one launch, per reduction element: a tile costs
// a * (BM + wb BN) (operand lines into LDS and out to the matrix cores; wb
// is the bytes of a weight element relative to bf16, 1/2 for FP8) plus
// b * BM * BN (the products), and the tiles run in ceil(tiles / CUs)
// rounds. a and b are a relative least-squares fit to the measured times of
// eight tile shapes (256x256, 256x128, 128x256, 128x128, 128x64, 64x128,
// 320x128, 320x256) on the five Llama-3.1-8B linears at M = 320 and 1280 on
// MI355X: the model then picks the fastest measured shape for nine of the
// ten linears and one within 2 % for the tenth. At M = 20 to 256 it picks
// what the earlier fit picked there, which was checked against every small
// shape forced in turn at M = 20 to 128 (the fastest, or within about 10 %).
static int pick_tile(int M, int N, int cus, const int (*shapes)[2], int n, double wb = 1.0,
                     int n_exact = 0) {
  const double a = 2.5e-5, b = 1.88e-7;
  int best = 0;
  double best_t = 0.0;
  for (int i = 0; i < n; ++i) {
    const int bm = shapes[i][0], bn = shapes[i][1];
    const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    if (i >= n - n_exact && tiles != cus) continue;  // exact-fill shapes: one tile per CU only
    const long rounds = (tiles + cus - 1) / cus;
    const double t = rounds * (a * (bm + wb * bn) + b * (double)bm * bn);
    if (i == 0 || t < best_t) {
      best_t = t;
      best = i;
    }
  }
  return best;
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return cus;
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

#if defined(SPECV_DIAGNOSTICS)
// Diagnostic builds: SPECV_TILE_FORCE=<id> replaces the picked tile by one
// of these (timing experiments only).
static hipError_t launch_tile_forced(int id, const uint16_t* x, const uint16_t* w, void* y,
                                     bool o, int M, int K, int N, hipStream_t s) {
  switch (id) {
    case 100: return launch_tile_t<256, 256, 4, 4, 32, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 101: return launch_tile_t<256, 256, 4, 5, 32, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 102: return launch_tile_t<128, 256, 2, 6, 32, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 103: return launch_tile_t<256, 128, 4, 6, 32, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 104: return launch_tile_t<128, 128, 2, 8, 32, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 105: return launch_tile_t<256, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 106: return launch_tile_t<192, 256, 2, 2, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 108: return launch_tile_t<320, 128, 2, 2, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 110: return launch_tile_t<256, 256, 4, 2, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 111: return launch_tile_t<128, 256, 2, 3, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 112: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 113: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 120: return launch_tile_t<128, 256, 2, 3, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 121: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 122: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 123: return launch_tile_t<128, 64, 4, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 124: return launch_tile_t<256, 128, 4, 3, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 125: return launch_tile_t<320, 128, 2, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 126: return launch_tile_t<320, 256, 2, 2, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 127: return launch_tile_t<128, 64, 4, 4, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 128: return launch_tile_t<256, 128, 4, 3, 64, 8, 1, 32>(x, w, nullptr, y, o, M, K, N, s);
    case 133: return launch_tile_t<320, 128, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 134: return launch_tile_t<320, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    case 135: return launch_tile_t<320, 192, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s);
    default: return hipErrorInvalidValue;
  }
}
#endif

hipError_t launch_gemm_mfma(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                            int K, int N, hipStream_t s) {
#if defined(SPECV_DIAGNOSTICS)
  if (const char* f = getenv("SPECV_TILE_FORCE"))
    if (K % kTileKAlign == 0) return launch_tile_forced(atoi(f), x, w, y, out_bf16, M, K, N, s);
#endif
  if (K % kTileKAlign == 0) {
    const int cus = device_cus();
    constexpr int n_shapes = sizeof(kTileShapes) / sizeof(kTileShapes[0]);
    int pick = pick_tile(M, N, cus, kTileShapes, n_shapes, 1.0, kExactFillShapes);
#if defined(SPECV_DIAGNOSTICS)
    if (const char* f = getenv("SPECV_TILE_PICK")) pick = max(0, min(atoi(f), n_shapes - 1));
#endif
    const long tiles = (long)((M + kTileShapes[pick][0] - 1) / kTileShapes[pick][0]) *
                       ((N + kTileShapes[pick][1] - 1) / kTileShapes[pick][1]);
    if (tiles <= cus) {
      // One round of small tiles: the same tile with the reduction split over
      // k-groups of eight waves in all, so that each CU has as many loads in
      // flight as a large tile's (measured on the Llama linears at M = 20 to
      // 128: O and down 15-30 % faster, QKV 5-20 %).
      switch (pick) {
        case 6: return launch_tile_t<64, 64, 2, 4, 64, 8, 2>(x, w, nullptr, y, out_bf16, M, K, N, s);
        case 7: return launch_tile_t<64, 32, 2, 4, 64, 8, 2>(x, w, nullptr, y, out_bf16, M, K, N, s);
        case 8: return launch_tile_t<32, 32, 2, 4, 64, 8, 2>(x, w, nullptr, y, out_bf16, M, K, N, s);
        case 9: return launch_tile_t<32, 16, 2, 4, 64, 8, 4>(x, w, nullptr, y, out_bf16, M, K, N, s);
        default: break;
      }
    }
    if (pick == 12) {
      // 320x256 tiles over two or more rounds with a partial last one (the
      // gate/up projection, 4096 -> 28672, at M = 1280 has 448 tiles for 256
      // CUs): the columns of the whole rounds keep 320x256 tiles, and the
      // rest run as a second launch of 320x192 tiles when those fit one
      // round, so the last round costs a 320x192 tile's time instead of a
      // 320x256 one's. Measured at M = 1280 on that linear, with the 2x2
      // 320-row forms of the time: 306 against 369 us (the whole linear on
      // 320x256 tiles) and 327 (on 256x256).
      const int mt = (M + 319) / 320;
      const long tiles = (long)mt * ((N + 255) / 256);
      const long rounds = (tiles + cus - 1) / cus;
      if (rounds >= 2 && tiles % cus != 0) {
        const int n1 = (int)((rounds - 1) * cus / mt) * 256;
        const int n2 = N - n1;
        if (n2 > 0 && (long)mt * ((n2 + 191) / 192) <= cus) {
          const hipError_t e = launch_tile_t<320, 256, 4, 2, 64, 8, 1, 16>(
              x, w, nullptr, y, out_bf16, M, K, n1, s, nullptr, 1, N);
          if (e != hipSuccess) return e;
          void* y2 = static_cast<char*>(y) + (size_t)n1 * (out_bf16 ? 2 : 4);
          return launch_tile_t<320, 192, 4, 2, 64, 8, 1, 16>(
              x, w + (size_t)n1 * K, nullptr, y2, out_bf16, M, K, n2, s, nullptr, 1, N);
        }
      }
    }
    switch (pick) {
      // 16x16x32 blocks: measured faster than 32x32x16 on every shape both
      // forms exist for (by 3-15 %, e.g. 256x128 at M = 1280: QKV 66 against
      // 71 us, down 197 against 220; 256x256 lm-head 1193 against 1275)
      case 0: return launch_tile_t<256, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 1: return launch_tile_t<256, 128, 4, 3, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 2: return launch_tile_t<128, 256, 2, 3, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 3: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 4: return launch_tile_t<128, 64, 4, 4, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 5: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 6: return launch_tile_t<64, 64, 2, 4, 64>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 7: return launch_tile_t<64, 32, 2, 4, 64, 4>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 8: return launch_tile_t<32, 32, 2, 6, 64, 4>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 9: return launch_tile_t<32, 16, 2, 6, 64, 2>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 10: return launch_tile_t<32, 64, 1, 4, 64, 4>(x, w, nullptr, y, out_bf16, M, K, N, s);
      // 320 rows: B = 64 and B = 256 sequences of K + 1 = 5 positions fill
      // one or four of them without padding (M = 320: gate/up 89 against
      // 144 us with 256x256 tiles; lm-head with 320x256, 334 against 419 us;
      // M = 1280 gate/up with 320x256, 282 against 316 us). 320x256 tiles
      // lay the eight waves out 4x2 (80x128 wave tiles of 16x16x32 blocks):
      // measured faster than 2x2 with 160x64 wave tiles of 32x32x16 blocks
      // (lm-head at M = 1280: 1174 against 1240 us; gate/up 267-284 against
      // 284-307), and so are the split forms below (down projection at
      // M = 1280 with sk = 4: 165-177 against 176-202 us).
      case 11: return launch_tile_t<320, 128, 2, 2, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 12: return launch_tile_t<320, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      // exact-fill shapes (one tile per CU)
      case 13: return launch_tile_t<80, 64, 5, 3, 64, 10, 2, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 14: return launch_tile_t<160, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 15: return launch_tile_t<160, 224, 2, 3, 64, 14, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 16: return launch_tile_t<160, 192, 2, 3, 64, 8, 1, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      case 17: return launch_tile_t<64, 48, 4, 4, 64, 8, 2, 16>(x, w, nullptr, y, out_bf16, M, K, N, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (M <= 32) return launch_mfma_t<32, 64, 1>(x, w, y, out_bf16, M, K, N, s);
  if (M <= 128) return launch_mfma_t<64, 64, 2>(x, w, y, out_bf16, M, K, N, s);
  return launch_mfma_t<128, 128, 2>(x, w, y, out_bf16, M, K, N, s);
}

// Reduction split over workgroups (spec_verify_gemm_ws). When few tiles of
// a large shape would leave CUs idle (the down projection at M = 320 has
// 192 tiles of 128x64 for 256 CUs and K = 14336), each tile's K stages are
// split over sk workgroups writing fp32 partial tiles to a caller
// workspace, and a second kernel adds them in split order.
static const int kSplitShapes[][2] = {{256, 256}, {256, 128}, {128, 256}, {128, 128},
                                      {64, 128},  {320, 128}, {320, 256}, {128, 64},
                                      {64, 64},   {32, 64}};
constexpr int kSplitShapeCount = sizeof(kSplitShapes) / sizeof(kSplitShapes[0]);
constexpr int kPlanCUs = 256;  // plans depend on the shape only, not the device

static hipError_t launch_split_shape(int shape, const uint16_t* x, const uint16_t* w, void* y,
                                     bool o, int M, int K, int N, float* part, int sk,
                                     hipStream_t s) {
  switch (shape) {
    case 0: return launch_tile_t<256, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 1: return launch_tile_t<256, 128, 4, 3, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 2: return launch_tile_t<128, 256, 2, 3, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 3: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 4: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 5: return launch_tile_t<320, 128, 2, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 6: return launch_tile_t<320, 256, 4, 2, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 7: return launch_tile_t<128, 64, 4, 4, 64, 8, 1, 16>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 8: return launch_tile_t<64, 64, 2, 4, 64>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    case 9: return launch_tile_t<32, 64, 1, 4, 64, 4>(x, w, nullptr, y, o, M, K, N, s, part, sk);
    default: return hipErrorInvalidValue;
  }
}

struct SplitPlan {
  int shape, sk;  // sk == 1: no split (the per-linear kernel's own pick)
};

// Time of one launch in microseconds: the tile model's term (scaled by a
// fit to measured launches) plus, for a split, a fixed cost and the fp32
// partial tiles written and read back by the split-sum kernel. The fit is to
// 250 launches on MI355X (the Llama-3.1-8B linears except the lm-head at
// M = 20, 80, 320, 1280, every split of the split shapes above from 2 to
// 16): rms error 12 %; on each of the 16 linears the plan it picks is the
// fastest measured or within 5.2 % of it. Checked on the Llama-3.1-8B and 70B
// linears at M = 5 to 1280: where it splits, the split runs 0.64 to 1.00 of
// the unsplit time.
static double tile_us(int M, int N, int K, int bm, int bn, int sk, int cus) {
  const double a = 2.5e-5, b = 1.88e-7;
  const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const long rounds = (tiles * sk + cus - 1) / cus;
  const double t = 0.962 * rounds * (a * (bm + bn) + b * (double)bm * bn) * K / sk + 4.15;
  if (sk == 1) return t;
  return t + 2.65 + 0.19e-6 * ((double)sk * M * N * 8 + (double)M * N * 2);
}

static SplitPlan split_plan(int M, int N, int K) {
  SplitPlan p{0, 1};
#if defined(SPECV_DIAGNOSTICS)
  if (const char* f = getenv("SPECV_SPLITK")) {  // "shape,sk"
    p.shape = max(0, min(atoi(f), kSplitShapeCount - 1));
    if (const char* c = strchr(f, ',')) p.sk = max(1, atoi(c + 1));
    return p;
  }
#endif
  constexpr int n_shapes = sizeof(kTileShapes) / sizeof(kTileShapes[0]);
  // The exact-fill shapes stand as the unsplit pick only up to 4096 columns:
  // at 8192 (the Llama-3.1-70B O projection at M = 160 and 640) they were
  // 2-5 % slower than the split plans the model put behind them.
  const int n_exact = N <= 4096 ? kExactFillShapes : 0;
  const int base = pick_tile(M, N, kPlanCUs, kTileShapes, n_shapes - kExactFillShapes + n_exact,
                             1.0, n_exact);
  const long base_tiles = (long)((M + kTileShapes[base][0] - 1) / kTileShapes[base][0]) *
                          ((N + kTileShapes[base][1] - 1) / kTileShapes[base][1]);
  // A split must beat the unsplit pick by 5 % of the model's time, or by
  // 20 % where that pick runs in k-groups (one round of the small 64x64 to
  // 32x16 tiles), which the model does not credit: measured, such picks
  // beat the splits the model put 10 to 18 % ahead of them (the 8192x8192
  // and 28672x8192 linears at M = 10 to 80).
  const bool k_groups = base_tiles <= kPlanCUs && base >= 6 && base <= 9;
  double best = (k_groups ? 0.80 : 0.95) *
                tile_us(M, N, K, kTileShapes[base][0], kTileShapes[base][1], 1, kPlanCUs);
  for (int i = 0; i < kSplitShapeCount; ++i) {
    const long tiles =
        (long)((M + kSplitShapes[i][0] - 1) / kSplitShapes[i][0]) *
        ((N + kSplitShapes[i][1] - 1) / kSplitShapes[i][1]);
    // at least two k-tiles per split, at most four rounds of work items
    for (int sk = 2; sk <= 16 && 2 * sk <= K / 64 && tiles * sk <= 4 * kPlanCUs; ++sk) {
      const double t = tile_us(M, N, K, kSplitShapes[i][0], kSplitShapes[i][1], sk, kPlanCUs);
      if (t < best) {
        best = t;
        p = SplitPlan{i, sk};
      }
    }
  }
  return p;
}

size_t gemm_split_workspace_bytes(int M, int K, int N) {
  if (K % kTileKAlign != 0) return 0;
  const SplitPlan p = split_plan(M, N, K);
  return p.sk > 1 ? (size_t)p.sk * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm_split(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                             int K, int N, void* workspace, size_t workspace_bytes, hipStream_t s) {
  const SplitPlan p = split_plan(M, N, K);
  if (K % kTileKAlign != 0 || p.sk <= 1) return launch_gemm_mfma(x, w, y, out_bf16, M, K, N, s);
  if (workspace == nullptr || workspace_bytes < (size_t)p.sk * M * N * sizeof(float) ||
      K / 64 < p.sk)
    return hipErrorInvalidValue;
  return launch_split_shape(p.shape, x, w, y, out_bf16, M, K, N, static_cast<float*>(workspace),
                            p.sk, s);
}

// FP8 E4M3 weights with per-row scales. The tile shapes are those whose
// load instructions divide evenly over the waves once a weight row takes
// 64 bytes per stage (8 x rows or 16 w rows per instruction); an FP8 stage
// is 3/4 the size of a bf16 one, so the largest tile keeps three stages.
static const int kTileShapesW8[][2] = {{256, 256}, {128, 256}, {128, 128}, {64, 128},
                                       {64, 64},   {32, 32},   {32, 16},   {32, 64},
                                       {64, 32},   {320, 128}, {320, 256}};

// Stages of 128 reduction elements (K a multiple of 128): a weight row is
// then one whole 128-byte line per stage instead of half of one. Measured
// on the Llama-3.1-8B linears at M = 20 to 1280 against the 64-element
// form of the same shape, these are faster wherever they appear below
// (e.g. 64x32 at M = 80 on the down projection 48 against 61 us, 32x16 at
// M = 20 24 against 31 us, 128x256 at M = 1280 on QKV 85 against 96 us).
// The others keep 64-element stages: 64x128, and 32x32 and 32x64 over
// several rounds, hold more workgroups per CU that way (the doubled stage
// would halve it) and measured slower with 128; 256x256 and the 320-row
// tiles would not fit their stages in LDS.
static bool w8_has_k128(int pick, bool one_round) {
  return pick == 1 || pick == 2 || pick == 4 || pick == 6 || pick == 8 ||
         ((pick == 5 || pick == 7) && one_round);
}

static hipError_t launch_w8_k128(int pick, const uint16_t* x, const uint8_t* w, const float* ws,
                                 void* y, bool o, int M, int K, int N, hipStream_t s) {
  switch (pick) {
    case 1: return launch_tile_t<128, 256, 2, 2, 128, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 2: return launch_tile_t<128, 128, 2, 3, 128, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 4: return launch_tile_t<64, 64, 2, 3, 128, 8, 2, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 5: return launch_tile_t<32, 32, 2, 3, 128, 8, 4, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 6: return launch_tile_t<32, 16, 1, 2, 128, 8, 8, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 7: return launch_tile_t<32, 64, 1, 4, 128, 8, 2, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 8: return launch_tile_t<64, 32, 2, 2, 128, 8, 4, 16, true>(x, w, ws, y, o, M, K, N, s);
    default: return hipErrorInvalidValue;
  }
}

// Each stage's codes widened once per workgroup into a bf16 LDS region
// (behind a second barrier per stage) instead of once per wave row at every
// fragment read: 1 / WM of the conversions. v_cvt_scalef32_pk_bf16_fp8
// costs about two plain VALU slots (measured), and the per-wave widening
// spends 4 / TM of them per MFMA, enough to compete with the matrix cores
// once the products dominate. Measured on the Llama-3.1-8B linears at
// M = 320: QKV 46.5 -> 41.3 us, O 47.2 -> 40.3, gate/up 130 -> 98.5, down
// 169 -> 123, lm-head 392 -> 359; at M = 1280 1-6 % on the 320-row tiles
// and 64x128 / 128x128 down. Tiles whose per-wave widening costs little
// (128x256 with 128-element stages, 256x256) measured slower with it, and
// so did 64x128 at M = 80 on gate/up: the 320-row tiles always take it,
// 64x128 and 128x128 from M = 256.
static bool w8_wide(int pick, int M) {
  return pick == 9 || pick == 10 || (M >= 256 && (pick == 2 || pick == 3));
}
static hipError_t launch_w8_wide(int pick, const uint16_t* x, const uint8_t* w, const float* ws,
                                 void* y, bool o, int M, int K, int N, hipStream_t s) {
  switch (pick) {
    case 2: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    case 3: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    case 9: return launch_tile_t<320, 128, 2, 3, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    case 10: return launch_tile_t<320, 256, 2, 2, 64, 8, 1, 32, true, true>(x, w, ws, y, o, M, K, N, s);
    default: return hipErrorInvalidValue;
  }
}

#if defined(SPECV_DIAGNOSTICS)
// Diagnostic builds: further 128-element FP8 forms (K a multiple of 128).
static hipError_t launch_w8_forced(int id, const uint16_t* x, const uint8_t* w, const float* ws,
                                   void* y, bool o, int M, int K, int N, hipStream_t s) {
  if (K % 128 != 0) return hipErrorInvalidValue;
  switch (id) {
    case 105: return launch_tile_t<64, 128, 2, 4, 128, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 108: return launch_tile_t<32, 64, 1, 4, 128, 4, 1, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 109: return launch_tile_t<32, 32, 2, 4, 128, 4, 2, 16, true>(x, w, ws, y, o, M, K, N, s);
    case 110: return launch_tile_t<320, 256, 4, 2, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    case 111: return launch_tile_t<320, 256, 2, 2, 64, 8, 1, 32, true, true>(x, w, ws, y, o, M, K, N, s);
    case 112: return launch_tile_t<320, 128, 4, 2, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    case 113: return launch_tile_t<320, 128, 2, 3, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s);
    default: return hipErrorInvalidValue;
  }
}
#endif

hipError_t launch_gemm_tile_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                               bool out_bf16, int M, int K, int N, hipStream_t s) {
  if (K % kTileKAlign != 0) return hipErrorInvalidValue;
  const int cus = device_cus();
  constexpr int n_shapes = sizeof(kTileShapesW8) / sizeof(kTileShapesW8[0]);
  int pick = pick_tile(M, N, cus, kTileShapesW8, n_shapes, 0.5);
  bool allow_k128 = true;
#if defined(SPECV_DIAGNOSTICS)
  if (const char* f = getenv("SPECV_TILE_FORCE_W8")) {
    const int id = atoi(f);
    if (id >= 100) return launch_w8_forced(id, x, w, w_scale, y, out_bf16, M, K, N, s);
    pick = max(0, min(id, n_shapes - 1));
  }
  if (getenv("SPECV_W8_NO_K128")) allow_k128 = false;
#endif
  const long tiles = (long)((M + kTileShapesW8[pick][0] - 1) / kTileShapesW8[pick][0]) *
                     ((N + kTileShapesW8[pick][1] - 1) / kTileShapesW8[pick][1]);
  const bool one_round = tiles <= cus;
  if (pick == 10 && w8_wide(pick, M)) {
    // as for bf16 weights: 320x256 tiles over two or more rounds with a
    // partial last one run the columns of the whole rounds on 320x256 and
    // the rest on 320x192 (both widened once per workgroup) when those fit
    // one round
    const int mt = (M + 319) / 320;
    const long tiles = (long)mt * ((N + 255) / 256);
    const long rounds = (tiles + cus - 1) / cus;
    if (rounds >= 2 && tiles % cus != 0) {
      const int n1 = (int)((rounds - 1) * cus / mt) * 256;
      const int n2 = N - n1;
      if (n2 > 0 && (long)mt * ((n2 + 191) / 192) <= cus) {
        const hipError_t e = launch_tile_t<320, 256, 2, 2, 64, 8, 1, 32, true, true>(
            x, w, w_scale, y, out_bf16, M, K, n1, s, nullptr, 1, N);
        if (e != hipSuccess) return e;
        void* y2 = static_cast<char*>(y) + (size_t)n1 * (out_bf16 ? 2 : 4);
        return launch_tile_t<320, 192, 2, 2, 64, 8, 1, 16, true, true>(
            x, w + (size_t)n1 * K, w_scale + n1, y2, out_bf16, M, K, n2, s, nullptr, 1, N);
      }
    }
  }
  if (w8_wide(pick, M)) return launch_w8_wide(pick, x, w, w_scale, y, out_bf16, M, K, N, s);
  if (allow_k128 && K % 128 == 0 && w8_has_k128(pick, one_round))
    return launch_w8_k128(pick, x, w, w_scale, y, out_bf16, M, K, N, s);
  if (one_round) {
    // one round of small tiles: eight waves per tile in k-groups, so that
    // each CU keeps eight waves' loads in flight (as for bf16 weights)
    switch (pick) {
      case 5: return launch_tile_t<32, 32, 2, 4, 64, 8, 4, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
      case 7: return launch_tile_t<32, 64, 1, 4, 64, 8, 2, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
      default: break;
    }
  }
  switch (pick) {
    case 0: return launch_tile_t<256, 256, 4, 3, 64, 8, 1, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 1: return launch_tile_t<128, 256, 2, 4, 64, 8, 1, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 2: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 3: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 4: return launch_tile_t<64, 64, 2, 4, 64, 8, 2, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    // 64x32 needs four k-groups of two waves for whole load instructions
    case 8: return launch_tile_t<64, 32, 2, 4, 64, 8, 4, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 5: return launch_tile_t<32, 32, 2, 4, 64, 4, 2, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    // (the model picks 32x16 only where its tiles fit one round)
    case 6: return launch_tile_t<32, 16, 1, 3, 64, 8, 8, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    case 7: return launch_tile_t<32, 64, 1, 4, 64, 4, 1, 16, true>(x, w, w_scale, y, out_bf16, M, K, N, s);
    default: return hipErrorInvalidValue;
  }
}

// FP8 weights with a split reduction: the KS = 1 forms of the FP8 tile
// table (the widen-once 64x128, 128x128 and 320-row tiles, 128-element
// stages for 128x256 where d_in allows).
static const int kSplitShapesW8[][2] = {{256, 256}, {128, 256}, {128, 128},
                                        {64, 128},  {320, 128}, {320, 256}};
constexpr int kSplitShapeCountW8 = sizeof(kSplitShapesW8) / sizeof(kSplitShapesW8[0]);

static hipError_t launch_split_shape_w8(int shape, const uint16_t* x, const uint8_t* w,
                                        const float* ws, void* y, bool o, int M, int K, int N,
                                        float* part, int sk, hipStream_t s) {
  const bool k128 = K % 128 == 0;
  switch (shape) {
    case 0: return launch_tile_t<256, 256, 4, 3, 64, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    case 1:
      if (k128) return launch_tile_t<128, 256, 2, 2, 128, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s, part, sk);
      return launch_tile_t<128, 256, 2, 4, 64, 8, 1, 16, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    case 2: return launch_tile_t<128, 128, 2, 4, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    case 3: return launch_tile_t<64, 128, 2, 4, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    case 4: return launch_tile_t<320, 128, 2, 3, 64, 8, 1, 16, true, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    case 5: return launch_tile_t<320, 256, 2, 2, 64, 8, 1, 32, true, true>(x, w, ws, y, o, M, K, N, s, part, sk);
    default: return hipErrorInvalidValue;
  }
}

// k-tiles of a split form: 128-element stages for the 128x256 form when
// d_in allows, 64 elsewhere
static int split_k_tiles_w8(int shape, int K) {
  return (shape == 1 && K % 128 == 0) ? K / 128 : K / 64;
}

// The FP8 tile model's term (weights at half the bytes of bf16) for `sk`
// splits of one tile shape.
static double tile_term_w8(int M, int N, int K, int bm, int bn, int sk, int cus) {
  const double a = 2.5e-5, b = 1.88e-7;
  const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const long rounds = (tiles * sk + cus - 1) / cus;
  return rounds * (a * (bm + 0.5 * bn) + b * (double)bm * bn) * K / sk;
}

// Two fits (microseconds) to 277 launches on MI355X (six Llama-3.1-8B and
// 70B linears at M = 20, 80, 320, 1280, unsplit and every split of the
// shapes above from 2 to 16): the unsplit kernels, whose several FP8 forms
// the tile model prices alike (rms error 15 %), and the split ones with the
// cost of their fp32 partials (rms 8 %). A split must beat the unsplit
// estimate by 5 %; on those 24 linears the plans sum to 1.01 of the fastest
// measured choice, and none is slower than the unsplit kernel.
static SplitPlan split_plan_w8(int M, int N, int K) {
  SplitPlan p{0, 1};
#if defined(SPECV_DIAGNOSTICS)
  if (const char* f = getenv("SPECV_SPLITK_W8")) {  // "shape,sk"
    p.shape = max(0, min(atoi(f), kSplitShapeCountW8 - 1));
    if (const char* c = strchr(f, ',')) p.sk = max(1, atoi(c + 1));
    return p;
  }
#endif
  constexpr int n_shapes = sizeof(kTileShapesW8) / sizeof(kTileShapesW8[0]);
  const int base = pick_tile(M, N, kPlanCUs, kTileShapesW8, n_shapes, 0.5);
  double best =
      0.95 * (1.595 * tile_term_w8(M, N, K, kTileShapesW8[base][0], kTileShapesW8[base][1], 1,
                                   kPlanCUs) + 2.59);
  for (int i = 0; i < kSplitShapeCountW8; ++i) {
    const int bm = kSplitShapesW8[i][0], bn = kSplitShapesW8[i][1];
    const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    for (int sk = 2; sk <= 16 && 2 * sk <= split_k_tiles_w8(i, K) && tiles * sk <= 4 * kPlanCUs;
         ++sk) {
      const double t = 1.365 * tile_term_w8(M, N, K, bm, bn, sk, kPlanCUs) +
                       0.182e-6 * ((double)sk * M * N * 8 + (double)M * N * 2) + 7.79;
      if (t < best) {
        best = t;
        p = SplitPlan{i, sk};
      }
    }
  }
  return p;
}

size_t gemm_split_workspace_bytes_w8(int M, int K, int N) {
  if (K % kTileKAlign != 0) return 0;
  const SplitPlan p = split_plan_w8(M, N, K);
  return p.sk > 1 ? (size_t)p.sk * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm_split_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                                bool out_bf16, int M, int K, int N, void* workspace,
                                size_t workspace_bytes, hipStream_t s) {
  const SplitPlan p = split_plan_w8(M, N, K);
  if (K % kTileKAlign != 0 || p.sk <= 1)
    return launch_gemm_tile_w8(x, w, w_scale, y, out_bf16, M, K, N, s);
  if (workspace == nullptr || workspace_bytes < (size_t)p.sk * M * N * sizeof(float) ||
      split_k_tiles_w8(p.shape, K) < p.sk)
    return hipErrorInvalidValue;
  return launch_split_shape_w8(p.shape, x, w, w_scale, y, out_bf16, M, K, N,
                               static_cast<float*>(workspace), p.sk, s);
}

}  // namespace specv
