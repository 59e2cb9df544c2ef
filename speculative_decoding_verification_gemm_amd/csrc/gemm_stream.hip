// Weight-streaming linears for few verify positions: y = x . w^T with M <= 16
// rows of x, bf16 in, fp32 accumulation.
//
// At M = B*(K+1) of 5 a linear does 5 FLOPs per weight byte, far below the
// chip's ridge, so the pass is bound by reading w once from HBM ("Speculative
// Decoding: Guess Several Tokens, Check Them in One Pass", Step 1; "What
// Actually Happens During Speculative Decoding in LLMs", the 5-candidate
// pass). The kernel is built around that read:
//
//  * One persistent workgroup of eight waves per CU walks row blocks of w
//    round-robin. (A second co-resident workgroup measurably received less
//    bandwidth than the first; with one, every CU streams alike.) Each lane
//    group of 16 lanes owns RPL rows of a row block; one 16-byte
//    non-temporal load per lane covers 256 contiguous bytes of a row per
//    segment, and the eight waves interleave segments along the reduction
//    dimension.
//  * The activation tile x[:, chunk] is staged in LDS and stays there across
//    row blocks; lanes read it back with 16-byte LDS loads. Chunks are as
//    large as LDS allows, so most linears stage their activations once.
//  * Products use v_dot2c_f32_bf16 (two bf16 products per lane-op).
//  * Weight-only 8-bit storage ("Speculative Decoding: The Algebra and the
//    Proof", Where it breaks): with FP8 E4M3 weights a 16-byte load holds
//    16 weights, which v_cvt_scalef32_pk_bf16_fp8 widens exactly to bf16
//    before the same dot products; the row's scale multiplies the reduced
//    sum. Half the bytes stream per weight.
//  * DEPTH register stages of weights are in flight ahead of the compute,
//    across row-block and linear boundaries, so the next linear's weights
//    stream while the current one finishes. Weight loads are issued on every
//    path (clamped addresses, no selects on loaded values), which keeps the
//    compiler's vmcnt waits exact.
//  * Partial sums are reduced across the 16 lanes of a group with DPP and
//    across the waves through LDS in a fixed order: outputs are
//    deterministic.

// Chain mode runs a list of linears in order in one launch. Linear l+1 reads
// its activations only after every workgroup has finished linear l (an
// arrival counter per linear), as the next layer of a forward pass would;
// its weight loads, which depend on nothing, are issued before that wait.
// The per-XCD L2 caches are kept out of the hand-off instead of being
// flushed: outputs are written and activations read with device-scope (sc1)
// accesses, and a workgroup bumps the counter only after its own output
// stores have completed (vmcnt), so no cache write-back or invalidate is
// issued per barrier. Counters are generation-based, so the workspace never
// needs clearing between launches; a bounded spin turns a stalled barrier
// into an error flag instead of a hang.
//
// Diagnostic builds (SPECV_DIAGNOSTICS defined) also record per-workgroup
// timestamps at every barrier and accept tile-parameter overrides; the
// library as built for use has neither.

#include <limits.h>
#include <math.h>

#include <type_traits>

#include "chain_sync.h"
#include "common.h"
#include "internal.h"

namespace specv {

#if !defined(SPECV_DIAGNOSTICS) || !defined(SPECV_STREAM_WAVES)
#undef SPECV_STREAM_WAVES
#define SPECV_STREAM_WAVES 8
#endif
constexpr int kStreamWaves = SPECV_STREAM_WAVES;  // one workgroup per CU
constexpr int kStreamThreads = kStreamWaves * kWave;
// Weight element format: elements per 16-byte load (kEpl), reduction
// elements per lane group per segment (16 lanes x 16 bytes), bytes per
// element.
template <bool W8>
struct WFmt {
  static constexpr int kEpl = W8 ? 16 : 8;
  static constexpr int kEplShift = W8 ? 4 : 3;
  static constexpr int kSeg = 16 * kEpl;
  static constexpr int kEsz = W8 ? 1 : 2;
};
constexpr int kCachePolicyDevice = 16;  // buffer-load aux bits: sc1 (device scope)
constexpr int kPollSleep = 4;  // s_sleep units (64 clocks each) between polls

// Pointers taken from a descriptor are generic; naming the global address
// space lets the compiler emit global (not flat) loads and stores, which
// count only on vmcnt.
#define SPECV_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const SPECV_GLOBAL T* gptr(const void* p) {
  return (const SPECV_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ SPECV_GLOBAL T* gptr_mut(void* p) {
  return (SPECV_GLOBAL T*)(p);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// A pointer every lane holds the same value of, made visibly uniform (a
// buffer resource built from it then lives in scalar registers).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
}

// Calls f(std::integral_constant<int, i>) for i = 0..N-1, unrolled.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

// Two FP8 E4M3 weights (the low or high 16 bits of v) as a bf16 pair; every
// E4M3 value is exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8).
template <bool HI>
__device__ __forceinline__ uint32_t widen_fp8x2_t(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}
#define widen_fp8x2(v, hi) widen_fp8x2_t<hi>(v)

// Per-workgroup schedule of one linear.
struct LinSched {
  const uint16_t* x;
  const void* w;
  const float* scale;  // FP8 weights: per-row scales
  void* y;
  int K, N;
  int n_it;    // pipeline stages per row block (ceil(K / elems per stage))
  int n_rb;    // row blocks of the linear
  int my_rb;   // row blocks this workgroup owns (bid, bid + G, ..., see sched)
  int q;       // whole rounds of G row blocks
  int extra;   // this workgroup's row block in the last, partial round, or -1
  int kc;      // activation chunk length (multiple of a stage)
  int ipc;     // stages per chunk
  int xs;      // LDS row stride of the activation chunk, elements (multiple of 512)
  int bf16;
  int ragged_k;
};

template <int M, int RPL, int U, int KCMAX, bool W8>
struct Stream {
  static constexpr int NR = 4 * RPL;              // rows per row block
  static constexpr int EPI = kStreamWaves * U * WFmt<W8>::kSeg;  // reduction elements per stage
  // Activation region rounded up to whole 1 KB blocks: staging writes one
  // 1 KB block (64 lanes x 16 bytes) per wave instruction.
  static constexpr size_t kXBytes = ((size_t)M * KCMAX * 2 + 1023) / 1024 * 1024;
  // two partial-sum buffers, used by alternate row blocks
  static constexpr size_t kRedFloats = (size_t)kStreamWaves * NR * M;
  static constexpr size_t kRedBytes = 2 * kRedFloats * 4;
  static constexpr size_t kLdsBytes = kXBytes + kRedBytes;
  static_assert(KCMAX % 512 == 0 && KCMAX >= EPI, "LDS rows are whole 64-lane blocks");
  static_assert(EPI % 512 == 0, "a chunk row must be whole 64-lane staging blocks");

  __device__ static LinSched sched(const StreamLinear& d) {
    LinSched s;
    s.x = d.x;
    s.w = d.w;
    s.scale = d.w_scale;
    s.y = d.y;
    s.K = d.K;
    s.N = d.N;
    s.bf16 = d.out_bf16;
    s.n_it = (d.K + EPI - 1) / EPI;
    s.n_rb = (d.N + NR - 1) / NR;
    const int bid = blockIdx.x, G = gridDim.x;
    // Whole rounds of G row blocks go round-robin (block bid + j G). The r
    // blocks of a last, partial round go to workgroups on even XCDs first
    // (bid mod 8 even): those stream 5-8 % faster than the odd ones, so the
    // extra block lands where it costs least.
    s.q = s.n_rb / G;
    const int r = s.n_rb - s.q * G;
    const int rank = G % 2 != 0 ? bid : (bid & 1) ? (G >> 1) + (bid >> 1) : (bid >> 1);
    s.extra = rank < r ? s.q * G + rank : -1;
    s.my_rb = s.q + (s.extra >= 0 ? 1 : 0);
    if (d.K <= KCMAX) {
      // the whole reduction dimension is staged once; LDS rows hold K
      // rounded up to a 512-element block, which may be less than the
      // stages span (the last stage's elements past K are never read)
      s.ipc = s.n_it;
      s.kc = s.n_it * EPI;
      s.xs = (d.K + 511) / 512 * 512;
    } else {
      const int ipc_max = KCMAX / EPI;
      const int n_chunks = (s.n_it + ipc_max - 1) / ipc_max;
      s.ipc = (s.n_it + n_chunks - 1) / n_chunks;
      s.kc = s.ipc * EPI;
      s.xs = s.kc;
    }
    s.ragged_k = (d.K % EPI) != 0;
    return s;
  }
};

// A position in a workgroup's stage sequence: linear l, its j-th row block,
// stage it.
struct Cursor {
  int l, j, it;
  bool valid;
};

template <int M, int RPL, int U, int KCMAX, int DEPTH, bool W8>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream_kernel(StreamLinear single,
                                                                     const StreamLinear* chain,
                                                                     int n_lin, ChainSync* sync,
                                                                     LogitStats st) {
  using S = Stream<M, RPL, U, KCMAX, W8>;
  using F = WFmt<W8>;
  constexpr int NR = S::NR, EPI = S::EPI;
  extern __shared__ u32x4 lds[];
  float* const red_base = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + S::kXBytes);
  int red_par = 0;  // partial-sum buffer of the next row block
  __shared__ unsigned s_gen;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, sub = lane & 15;
  const int bid = blockIdx.x, G = gridDim.x;
  const bool is_chain = chain != nullptr;
  // Fused softmax statistics of the outputs (single launch of a logits
  // linear): the thread of row 0 of each position's 16-row group keeps the
  // workgroup's running maximum, fp64 sum of exp((l - max) * inv) and first
  // index of the maximum.
  const bool want_stats = !is_chain && st.pmax != nullptr;
  float st_max = -INFINITY;
  double st_sum = 0.0;
  int st_arg = INT_MAX;
  unsigned* counts = is_chain ? reinterpret_cast<unsigned*>(sync + 1) : nullptr;
  if (is_chain && (sync->magic != (W8 ? kChainMagicW8 : kChainMagic) || sync->n != n_lin ||
                   sync->M != M || sync->grid != G)) {
    if (bid == 0 && tid == 0)
      __hip_atomic_fetch_or(&sync->error, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;  // every workgroup reads the same header and leaves
  }

  // Descriptors are read-only while the kernel runs: read them through the
  // constant address space (scalar loads, counted on lgkmcnt), so that
  // moving to the next linear never waits on the weight loads in flight.
  auto desc = [&](int l) __attribute__((always_inline)) -> StreamLinear {
    if (!is_chain) return single;
    const __attribute__((address_space(4))) StreamLinear* d =
        (const __attribute__((address_space(4))) StreamLinear*)(chain + l);
    return StreamLinear{d->x, d->w, d->w_scale, d->y, d->K, d->N, d->out_bf16, d->reserved};
  };

  // ---- barrier between linears (chain mode)
  // gen1: launches of this chain including this one; every counter target
  // of the launch derives from it (modulo 2^32, as the counters wrap).
  unsigned gen1 = 0, target = 0;
  int spin_limit = 0;
  if (is_chain) {
    if (tid == 0) s_gen = __hip_atomic_load(&sync->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    gen1 = s_gen + 1u;
    target = chain_target(gen1, G);
    spin_limit = sync->spin_limit;
  }
  // Arrival: every wave's device-scope output stores have completed (the
  // caller waited on vmcnt) before the barrier, so the count only rises once
  // the linear's outputs are visible at device scope.
  // Global (not flat) stores: a pending flat access would make the
  // compiler wait for every load in flight wherever it needs a vmcnt wait.
#if defined(SPECV_DIAGNOSTICS)
  SPECV_GLOBAL unsigned long long* const trace =
      is_chain ? gptr_mut<unsigned long long>(sync->trace) : nullptr;
#else
  SPECV_GLOBAL unsigned long long* const trace = nullptr;  // no timestamps
#endif
  // Arrivals are counted in two levels: each workgroup bumps the counter of
  // its group (bid mod kArriveGroups, one 64-byte line each), and the last of
  // a group bumps the linear's counter. When every workgroup finishes a
  // linear at nearly the same moment, no counter serializes more than a
  // group's worth of atomics. The last group to arrive publishes the target
  // to kReleaseLanes flags on separate lines, and waiters poll the flag of
  // their lane, so polls do not queue on the lines the arrivals update.
  unsigned* release = is_chain ? counts + chain_release_offset(n_lin) : nullptr;
  auto flag = [&](int l, int lane_id) __attribute__((always_inline)) {
    return release + ((size_t)l * kBarrierLines + lane_id) * 16;
  };
  const int n_groups = G < kArriveGroups ? G : kArriveGroups;
  auto arrive = [&](int l) __attribute__((always_inline)) {
    __syncthreads();
    if (tid == 0) {
      if (trace) trace[((size_t)l * G + bid) * 4] = wall_clock64();
      const int g = bid % kArriveGroups;
      const unsigned gsize = chain_group_size(G, g, kArriveGroups);
      unsigned* gc = release + ((size_t)l * kBarrierLines + kReleaseLanes + g) * 16;
      const unsigned gp = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (chain_group_complete(gp, gen1, gsize)) {
        const unsigned prev =
            __hip_atomic_fetch_add(&counts[l], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (chain_linear_complete(prev, gen1, n_groups)) {
          for (int x = 0; x < kReleaseLanes; ++x)
            __hip_atomic_store(flag(l, x), target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  auto wait = [&](int l) __attribute__((always_inline)) {
    if (tid == 0) {
      int spins = 0;
      const unsigned* f = flag(l, bid % kReleaseLanes);
      while (!chain_released(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                             target)) {
        if (++spins > spin_limit) {
          __hip_atomic_fetch_or(&sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(kPollSleep);
      }
      if (trace) trace[((size_t)(l + 1) * G + bid) * 4 + 1] = wall_clock64();
    }
    __syncthreads();
  };

  // ---- cursors: first stage of the first linear this workgroup works on
  LinSched cs, ps;
  Cursor c{0, 0, 0, false}, p;
  auto seek = [&](Cursor& cur, LinSched& s, int l) __attribute__((always_inline)) {
    // first linear >= l with work for this workgroup
    for (; l < n_lin; ++l) {
      s = S::sched(desc(l));
      if (s.my_rb > 0) {
        cur = Cursor{l, 0, 0, true};
        return;
      }
    }
    cur.valid = false;
    cur.l = n_lin;
  };
  auto advance = [&](Cursor& cur, LinSched& s) __attribute__((always_inline)) {
    if (++cur.it < s.n_it) return;
    cur.it = 0;
    if (++cur.j < s.my_rb) return;
    seek(cur, s, cur.l + 1);
  };

  // ---- activation staging: x[:, chunk] straight into LDS (global_load_lds,
  // one 1 KB block per wave instruction, no registers). LDS row m of the
  // chunk holds s.xs / 8 16-byte units, a whole number of blocks; units past
  // the end of x load a clamped valid address and are never read. The
  // staging is complete (vmcnt) and visible to all waves (barrier) on
  // return.
  auto stage_x = [&](const LinSched& s, int chunk) __attribute__((always_inline)) {
    const int k0 = chunk * s.kc;
    const int units = min(s.kc, s.K - k0) / 8;  // valid units per row
    const int blocks = s.xs / 512;              // 64-unit blocks per LDS row
    const uint16_t* xs = s.x;
    for (int m = 0; m < M; ++m) {
      for (int b = wave; b < blocks; b += kStreamWaves) {
        const int cc = min(b * 64 + lane, units - 1);
        const SPECV_GLOBAL void* src = gptr<void>(xs + (size_t)m * s.K + k0 + cc * 8);
        __attribute__((address_space(3))) void* dst =
            (__attribute__((address_space(3))) void*)(lds + (m * blocks + b) * 64);
        if (is_chain)  // x may be the previous linear's output: device scope
          __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kCachePolicyDevice);
        else
          __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  };

  // element offset of this lane's F::kEpl weights for segment u of stage it
  auto kofs = [&](int it, int u) __attribute__((always_inline)) {
    return ((it * U + u) * kStreamWaves + wave) * F::kSeg + sub * F::kEpl;
  };

  // Weight loads are branch-free: rows past N and reduction elements past K
  // read a clamped valid address. Rows past N feed outputs that are never
  // stored, and the compute zeroes the activation for elements past K, so
  // no loaded value needs a select (a select right after a load would make
  // the wave wait for it). An exhausted cursor also loads a valid clamped
  // address; its values are never used. Issuing the same loads on every
  // path keeps the compiler's vmcnt waits exact, so DEPTH stages really are
  // in flight.
  // An exhausted cursor points every lane at the first 16 bytes of the
  // weights, so its loads are served by the cache instead of HBM.
  auto load = [&](u32x4 (&buf)[U][RPL], const LinSched& s, const Cursor& cur)
      __attribute__((always_inline)) {
    const int rb = cur.j < s.q ? bid + cur.j * G : s.extra;
    const int live = -(int)cur.valid;  // all ones, or zero for an exhausted cursor
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int row = min(rb * NR + grp * RPL + r, s.N - 1) & live;
      const SPECV_GLOBAL u32x4* base =
          gptr<u32x4>(static_cast<const char*>(s.w) + (size_t)row * s.K * F::kEsz);
#pragma unroll
      for (int u = 0; u < U; ++u)
        buf[u][r] = __builtin_nontemporal_load(
            base + ((min(kofs(cur.it, u), s.K - F::kEpl) >> F::kEplShift) & live));
    }
  };

  float acc[RPL][M];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
  };
  auto compute = [&](const u32x4 (&buf)[U][RPL], const LinSched& s, const Cursor& cur)
      __attribute__((always_inline)) {
    const int chunk_base = (cur.it / s.ipc) * s.kc;
    const int row_units = s.xs / 8;
    if constexpr (W8) {
      // 16 weights per register quad: widen to two bf16 octets (exact), then
      // two dot products against the matching activation units. On the
      // ragged last stage, activations past K are zeroed (d_in is a multiple
      // of 16, so a lane's 16 weights are all inside K or all outside).
      auto body = [&](auto RAG) __attribute__((always_inline)) {
        constexpr bool rag = decltype(RAG)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          u32x4 lo[RPL], hi[RPL];
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
            lo[r] = u32x4{widen_fp8x2(buf[u][r].x, false), widen_fp8x2(buf[u][r].x, true),
                          widen_fp8x2(buf[u][r].y, false), widen_fp8x2(buf[u][r].y, true)};
            hi[r] = u32x4{widen_fp8x2(buf[u][r].z, false), widen_fp8x2(buf[u][r].z, true),
                          widen_fp8x2(buf[u][r].w, false), widen_fp8x2(buf[u][r].w, true)};
          }
          const int k = kofs(cur.it, u);
          const bool ok = !rag || k < s.K;
          const int lu = ok ? (k - chunk_base) >> 3 : 0;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            u32x4 xa = lds[m * row_units + lu];
            u32x4 xb = lds[m * row_units + lu + 1];
            if constexpr (rag) {
              xa = ok ? xa : u32x4{0u, 0u, 0u, 0u};
              xb = ok ? xb : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r)
              acc[r][m] = dot8_bf16(hi[r], xb, dot8_bf16(lo[r], xa, acc[r][m]));
          }
        }
      };
      if (s.ragged_k && cur.it == s.n_it - 1)
        body(std::true_type{});
      else
        body(std::false_type{});
      return;
    }
    if (s.ragged_k && cur.it == s.n_it - 1) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kofs(cur.it, u);
        const bool ok = k < s.K;
        const int lu = ok ? (k - chunk_base) >> 3 : 0;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          u32x4 xv = lds[m * row_units + lu];
          xv = ok ? xv : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int r = 0; r < RPL; ++r) acc[r][m] = dot8_bf16(buf[u][r], xv, acc[r][m]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int lu = (kofs(cur.it, u) - chunk_base) >> 3;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 xv = lds[m * row_units + lu];
#pragma unroll
          for (int r = 0; r < RPL; ++r) acc[r][m] = dot8_bf16(buf[u][r], xv, acc[r][m]);
        }
      }
    }
  };
  // One row block's outputs v of one position, held by the 16 consecutive
  // threads of its rows (rows past N are left out), folded into the running
  // statistics of the group's row-0 thread. Sums are fp64, relative to the
  // running maximum, in row-block order: deterministic.
  auto fold_stats = [&](float v, bool ok, int row, int rr) __attribute__((always_inline)) {
    const float lv = ok ? v : -INFINITY;
    float bm = lv;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 16));
    if (st.greedy) {
      int a = (ok && lv == bm) ? row : INT_MAX;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) a = min(a, __shfl_xor(a, o, 16));
      if (rr == 0 && bm != -INFINITY) {
        if (bm > st_max) {
          st_max = bm;
          st_arg = a;
        } else if (bm == st_max) {
          st_arg = min(st_arg, a);
        }
      }
    } else {
      double e = ok ? exp(((double)lv - (double)bm) * st.inv) : 0.0;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) e += __shfl_xor(e, o, 16);
      if (rr == 0 && bm != -INFINITY) {
        if (bm > st_max) {
          st_sum = st_sum * exp(((double)st_max - (double)bm) * st.inv) + e;
          st_max = bm;
        } else {
          st_sum += e * exp(((double)bm - (double)st_max) * st.inv);
        }
      }
    }
  };

  // Row block done: partial sums reduced within each lane group (DPP), then
  // across the waves through LDS in wave order, and stored. Alternate row
  // blocks use alternate LDS buffers, so one barrier per row block suffices:
  // a buffer is written again only two row blocks later, after every thread
  // has passed the barrier of the row block in between, which follows its
  // reads.
  auto finish = [&](const LinSched& s, const Cursor& cur) __attribute__((always_inline)) {
    float* const red = red_base + red_par * S::kRedFloats;
    red_par ^= 1;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = row16_sum(acc[r][m]);
    if (sub == 0) {
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) red[(wave * NR + grp * RPL + r) * M + m] = acc[r][m];
    }
    __syncthreads();
    const int rb = cur.j < s.q ? bid + cur.j * G : s.extra;
    // FP8 weights: the row block's scales through the scalar cache (uniform
    // addresses, counted on lgkmcnt), so no wait on the weight loads in
    // flight; each thread then picks its row's scale.
    float scl[W8 ? NR : 1];
    if constexpr (W8) {
      // pointer and row made visibly uniform, or the compiler emits vector
      // loads whose waits would drain the weight loads in flight
      const __attribute__((address_space(4))) float* sp =
          (const __attribute__((address_space(4))) float*)uniform_ptr(s.scale);
      const int row0 = __builtin_amdgcn_readfirstlane(rb * NR);
      const int last = __builtin_amdgcn_readfirstlane(s.N - 1);
#pragma unroll
      for (int j = 0; j < NR; ++j) scl[j] = sp[min(row0 + j, last)];
    }
    for (int i = tid; i < NR * M; i += kStreamThreads) {
      const int m = i / NR, rr = i - m * NR;
      const int row = rb * NR + rr;
      float v = 0.0f;
      if (row < s.N) {
        v = red[rr * M + m];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) v += red[(w * NR + rr) * M + m];  // wave order
        if constexpr (W8) {
          float sc = scl[0];
#pragma unroll
          for (int j = 1; j < NR; ++j) sc = rr == j ? scl[j] : sc;
          v *= sc;
        }
        const size_t o = (size_t)m * s.N + row;
        if (is_chain) {  // visible at device scope without a cache write-back
          if (s.bf16)
            __hip_atomic_store(gptr_mut<uint16_t>(s.y) + o, f32_to_bf16_bits(v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            __hip_atomic_store(gptr_mut<float>(s.y) + o, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        } else if (s.bf16) {
          gptr_mut<uint16_t>(s.y)[o] = f32_to_bf16_bits(v);
        } else {
          gptr_mut<float>(s.y)[o] = v;
        }
      }
      if (want_stats) fold_stats(v, row < s.N, row, rr);
    }
    zero_acc();
  };

  // Arrive at the counters of linears [from, to) in which this workgroup
  // has no row block (nothing to wait for, nothing to compute).
  auto arrive_empty = [&](int from, int to) __attribute__((always_inline)) {
    if (!is_chain) return;
    for (int l = from; l < to; ++l) arrive(l);
  };

  // Waves that write outputs (the reduced row block is stored by the first
  // NR * M threads) wait for their stores before the workgroup arrives at a
  // linear's counter; the other waves never wait before the barrier, so the
  // refills they issued for the next linear keep streaming through it.
  const bool storer = wave * kWave < NR * M;
  u32x4 wbuf[DEPTH][U][RPL];

  // One pipeline step on buffer IB: compute stage c, refill the buffer with
  // stage p (DEPTH stages ahead), close the row block / linear if c was its
  // last stage, advance c. Once c is exhausted a step only issues its
  // (cache-served) refill. Every step issues the same loads on every path,
  // so between the refill of a buffer and its next use exactly DEPTH - 1
  // other stages' loads are issued on every path through the loop, and the
  // compiler's wait before the products leaves those in flight.
  auto step = [&](auto IB) __attribute__((always_inline)) {
    constexpr int ib = decltype(IB)::value;
    auto& buf = wbuf[ib];
    const bool live = c.valid;
    bool closes_rb = false;
    if (live) {
      if (c.it == 0 && c.j == 0) {
        // first stage of a linear: its x may depend on the previous linear
        if (is_chain && c.l > 0) wait(c.l - 1);
        stage_x(cs, 0);
        if (trace && tid == 0) trace[((size_t)c.l * G + bid) * 4 + 2] = wall_clock64();
      } else if (c.it % cs.ipc == 0 && cs.ipc < cs.n_it) {
        // next activation chunk (chunk 0 again for a new row block), once
        // every wave is done with the previous one
        __syncthreads();
        stage_x(cs, c.it / cs.ipc);
      }
      compute(buf, cs, c);
      closes_rb = c.it == cs.n_it - 1;
    }
    // The refill goes out before the row block's reduction: with FP8 weights
    // a 4096-wide row block is a single stage, so a refill issued after the
    // reduction's workgroup barrier would reach HBM late at every stage
    // (measured: FP8 chain 1.93 against 2.03 ms, 70B bf16 5.16 against 5.24).
    load(buf, ps, p);  // unconditional (see load)
    if (p.valid) advance(p, ps);
    if (live && closes_rb) finish(cs, c);
    if (live) {
      if (closes_rb && c.j == cs.my_rb - 1 && is_chain) {
        if (trace && tid == 0) trace[((size_t)c.l * G + bid) * 4 + 3] = wall_clock64();
        if (storer) wait_vmcnt<0>();  // output stores complete (and, in order, older loads)
        arrive(c.l);
      }
      const int l_before = c.l;
      advance(c, cs);
      arrive_empty(l_before + 1, c.valid ? c.l : n_lin);
    }
  };

  zero_acc();
  seek(c, cs, 0);
  arrive_empty(0, c.valid ? c.l : n_lin);
  p = c;
  ps = cs;
  // DEPTH register stages of weights are in flight ahead of the compute.
  static_for<DEPTH>([&](auto D) __attribute__((always_inline)) {
    load(wbuf[decltype(D)::value], ps, p);
    if (p.valid) advance(p, ps);
  });
  // Whole rounds of DEPTH steps only: a round that c leaves mid-way still
  // issues its remaining refills, so no path re-enters the loop with fewer
  // loads in flight than the waits assume.
  while (c.valid) {
    static_for<DEPTH>([&](auto D) __attribute__((always_inline)) { step(D); });
  }
  // Refills past the end are never consumed; let them land before exit.
  wait_vmcnt<0>();
  if (want_stats && tid < NR * M && tid % NR == 0) {
    const size_t o = (size_t)(tid / NR) * st.stride + bid;
    gptr_mut<float>(st.pmax)[o] = st_max;
    gptr_mut<double>(st.psum)[o] = st_sum;
    gptr_mut<int32_t>(st.parg)[o] = st_arg;
  }

  // exit: the last workgroup out advances the generation
  if (is_chain) {
    __syncthreads();
    if (tid == 0) {
      const unsigned prev =
          __hip_atomic_fetch_add(&sync->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev + 1u == target)
        __hip_atomic_fetch_add(&sync->gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Launch: per-M tile choice and the persistent grid
// ---------------------------------------------------------------------------

template <int M, int RPL, int U, int KCMAX, int DEPTH, bool W8>
static hipError_t launch_m(const StreamLinear& single, const StreamLinear* chain, int n_lin,
                           ChainSync* sync, const LogitStats& st, int grid, hipStream_t s) {
  using S = Stream<M, RPL, U, KCMAX, W8>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_stream_kernel<M, RPL, U, KCMAX, DEPTH, W8>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_stream_kernel<M, RPL, U, KCMAX, DEPTH, W8>), dim3(grid),
                     dim3(kStreamThreads), S::kLdsBytes, s, single, chain, n_lin, sync, st);
  return hipGetLastError();
}

// Tile parameters per M: (RPL, U, KCMAX, DEPTH). Rows per row block =
// 4 * RPL; activation chunk KCMAX elements (M * KCMAX * 2 bytes of LDS, at
// most about 150 KB so that whole activations of d_in up to 14336 stay
// resident at M = 5); DEPTH register stages of U * RPL 16-byte loads per
// lane in flight (8 KB per wave per stage; two-wave-per-SIMD register
// budget).
#if !defined(SPECV_DIAGNOSTICS) || !defined(SPECV_T5)
#undef SPECV_T5
#define SPECV_T5(X) X(5, 4, 2, 14336, 4)
#endif
#define SPECV_STREAM_TABLE(X) \
  X(1, 4, 2, 32768, 4)         \
  X(2, 4, 2, 32768, 4)         \
  X(3, 4, 2, 24576, 4)         \
  X(4, 4, 2, 18432, 4)         \
  SPECV_T5(X)                  \
  X(6, 4, 2, 12288, 4)         \
  X(7, 4, 2, 10240, 4)         \
  X(8, 4, 2, 8192, 4)          \
  X(9, 4, 2, 6144, 4)          \
  X(10, 4, 2, 6144, 4)         \
  X(11, 4, 2, 6144, 4)         \
  X(12, 4, 2, 6144, 4)         \
  X(13, 4, 2, 4096, 3)         \
  X(14, 4, 2, 4096, 3)         \
  X(15, 4, 2, 4096, 3)         \
  X(16, 4, 2, 4096, 3)

// FP8 weights: a segment holds 256 weights (16 bytes per lane), so a stage
// of U = 2 segments covers 4096 reduction elements in the same 8 loads per
// lane as a bf16 stage (half the bytes each). KCMAX as for bf16 (the LDS
// holds bf16 activations either way).
#if defined(SPECV_DIAGNOSTICS) && defined(SPECV_STREAM_W8_TABLE)
// (diagnostic build: table given on the command line)
#else
#undef SPECV_STREAM_W8_TABLE
#define SPECV_STREAM_W8_TABLE(X) \
  X(1, 4, 2, 32768, 4)            \
  X(2, 4, 2, 32768, 4)            \
  X(3, 4, 2, 24576, 4)            \
  X(4, 4, 2, 18432, 4)            \
  X(5, 4, 2, 14336, 4)            \
  X(6, 4, 2, 12288, 3)            \
  X(7, 4, 2, 10240, 3)            \
  X(8, 4, 2, 8192, 3)             \
  X(9, 4, 2, 6144, 2)             \
  X(10, 4, 2, 6144, 2)            \
  X(11, 4, 2, 6144, 2)            \
  X(12, 4, 2, 6144, 2)            \
  X(13, 4, 2, 4096, 2)            \
  X(14, 4, 2, 4096, 2)            \
  X(15, 4, 1, 4096, 3)            \
  X(16, 4, 1, 4096, 2)
#endif

// Both tables use 16-row blocks (RPL = 4).
size_t stream_rows_per_block(int M) { return M >= 1 && M <= kMaxStreamM ? 16 : 0; }

template <int M, int RPL, int U, int KCMAX, int DEPTH, bool W8>
static int max_wgs_m() {
  using S = Stream<M, RPL, U, KCMAX, W8>;
  static_assert(S::NR == 16, "row block size shared by both weight formats");
  int n = 0;
  (void)hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_stream_kernel<M, RPL, U, KCMAX, DEPTH, W8>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::kLdsBytes);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, gemm_stream_kernel<M, RPL, U, KCMAX, DEPTH, W8>, kStreamThreads, S::kLdsBytes) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

int stream_max_wgs_per_cu(int M, bool w8) {
  if (w8) {
    switch (M) {
#define SPECV_OCC8(MM, RPL, U, KC, D) \
  case MM:                            \
    return max_wgs_m<MM, RPL, U, KC, D, true>();
      SPECV_STREAM_W8_TABLE(SPECV_OCC8)
#undef SPECV_OCC8
      default:
        return 1;
    }
  }
  switch (M) {
#define SPECV_OCC(MM, RPL, U, KC, D) \
  case MM:                           \
    return max_wgs_m<MM, RPL, U, KC, D, false>();
    SPECV_STREAM_TABLE(SPECV_OCC)
#undef SPECV_OCC
    default:
      return 1;
  }
}

static hipError_t launch_gemm_stream_any(const StreamLinear& single, const StreamLinear* chain,
                                         int n_lin, ChainSync* sync, const LogitStats& st, int M,
                                         bool w8, int grid, hipStream_t s) {
  if (w8) {
    switch (M) {
#define SPECV_CASE8(MM, RPL, U, KC, D) \
  case MM:                             \
    return launch_m<MM, RPL, U, KC, D, true>(single, chain, n_lin, sync, st, grid, s);
      SPECV_STREAM_W8_TABLE(SPECV_CASE8)
#undef SPECV_CASE8
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (M) {
#define SPECV_CASE(MM, RPL, U, KC, D) \
  case MM:                            \
    return launch_m<MM, RPL, U, KC, D, false>(single, chain, n_lin, sync, st, grid, s);
    SPECV_STREAM_TABLE(SPECV_CASE)
#undef SPECV_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_stream(const uint16_t* x, const void* w, const float* w_scale, void* y,
                              bool out_bf16, bool w8, int M, int K, int N, int grid,
                              hipStream_t s, const LogitStats* stats) {
  StreamLinear d{x, w, w_scale, y, K, N, out_bf16 ? 1 : 0, 0};
  const int n_rb = (N + (int)stream_rows_per_block(M) - 1) / (int)stream_rows_per_block(M);
  LogitStats st{};
  if (stats && stats->pmax && !out_bf16) {
    // every workgroup writes its partials, so keep the whole grid (those
    // without row blocks write empty ones)
    if (grid > stats->stride) return hipErrorInvalidValue;
    st = *stats;
  } else if (grid > n_rb) {
    grid = n_rb;
  }
  return launch_gemm_stream_any(d, nullptr, 1, nullptr, st, M, w8, grid, s);
}

hipError_t launch_gemm_chain(const StreamLinear* chain, int n_lin, ChainSync* sync, int M, bool w8,
                             int grid, hipStream_t s) {
  StreamLinear none{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0};
  return launch_gemm_stream_any(none, chain, n_lin, sync, LogitStats{}, M, w8, grid, s);
}

}  // namespace specv
