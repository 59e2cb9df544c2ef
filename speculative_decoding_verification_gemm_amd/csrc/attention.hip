// Verify attention: the K+1 verify positions of each sequence attend, through
// the causal mask, over its KV cache ("Speculative Decoding: Guess Several
// Tokens, Check Them in One Pass", Step 1: the pass is a tiny prefill and
// reads the cache once for all K+1 positions).
//
// Shapes: q [B][K+1][H][D], k/v cache [B][T][Hkv][D] (the K+1 verify
// positions are the last K+1 entries), out [B][K+1][H][D]; D = 128. Query
// position i sits at absolute position T-K-1+i; head h reads key/value head
// h / G, G = H / Hkv.
//
// The cache is read once and the work per byte is small (R = (K+1) * G query
// rows share every key/value row of a head), so HBM bounds the kernel:
//
//  * Grid (split, kv head, sequence): a split is a range of the cache's
//    tokens; splits give small batches enough workgroups. Within a
//    workgroup, teams of waves walk their own 32-token tiles, each wave with
//    its own running softmax (max, sum, output), and the waves are merged at
//    the end, then the splits in a second kernel, in a fixed order. Large
//    batches run four waves per workgroup, two workgroups per CU; small ones
//    eight, one per CU, so that a split's few tiles are spread over more
//    waves.
//  * A tile's keys and values come in as whole 256-byte rows (16 lanes x
//    16 bytes per row, 4 rows per load instruction) into registers, one or
//    two tiles ahead, and go to the team's LDS tile with an XOR swizzle of
//    the 16-byte units.
//  * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, A = 16 keys,
//    B = 16 query rows, reduction over D). The keys enter the A operand in
//    an order that leaves each lane with one query row's scores of 8
//    consecutive tokens: exactly the 8 reduction slots it supplies to the P
//    operand of the next product, so the probabilities need no shuffle. The
//    row's maximum and sum over its four lanes use the row-swap permutes
//    (VALU, no LDS).
//  * O^T += V^T P^T on the matrix cores: the A operand (16 value columns x
//    8 consecutive tokens per lane) comes from the token-major tile through
//    LDS transpose reads, two per 16 columns.
//  * Softmax in base 2 (scale * log2 e folded into the scores), masked
//    entries -inf; a running max of -inf is replaced by 0 in the exponents
//    so that no -inf - -inf arises. P is rounded to bf16 for the product
//    and the row sums add the same rounded values.

#include <math.h>

#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kAttD = 128;
constexpr int kAttTile = 32;                     // tokens per tile
constexpr int kAttRowBytes = kAttD * 2;          // 256 bytes per token and head
constexpr int kAttTileBytes = kAttTile * kAttRowBytes;      // 8 KB
constexpr int kAttQBytes = 32 * kAttRowBytes;                // query rows, after the tiles
constexpr int kAttPartStride = kAttD + 2;        // o[D], m, l per partial row

#define SPECV_ATT_GLOBAL __attribute__((address_space(1)))

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* part;  // split partials [B][Hkv][n_split][R][kAttPartStride], or null
  int B, K1, T, H, Hkv, G, R;
  // Split s covers tiles [s * split_tiles + min(s, split_rem), ...) of the
  // cache: split_tiles + 1 tiles for s < split_rem, split_tiles after.
  int n_split, split_tiles, split_rem;
  float scale_log2;        // scale * log2(e)
  int out_bf16;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_round(float v) {
  return __uint_as_float((uint32_t)f32_to_bf16_bits(v) << 16);
}

// Maximum and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes
// holding one query row's scores), with the gfx950 row-swap permutes: a
// swap of a value with itself hands every lane the pair (lane with the bit
// clear, lane with it set), so both lanes of a pair combine the same two
// values in the same order and every lane ends with the same result.
__device__ __forceinline__ float att_row_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float att_row_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Stored position of 16-byte unit u of token t in an LDS tile: u ^ swz(t),
// swz(t) = (t0, t0, t1, t1 ^ t3) as bits 0..3 (t0 = bit 0 of t, ...). With
// the sixteen lanes that one 16-byte access serves together (lanes 0-7 with
// 32-39, and so on) needing sixteen distinct 16-byte slots of a 256-byte
// window, this is conflict-free for the three patterns on a tile: the
// stores from registers (units 0-7 of tokens 4k and 4k + 2), the key reads
// in the permuted row order (tokens 8a + 4tt + b, units u and u ^ 2), and
// the value transpose reads (tokens 8g + 4h + c, units u and u ^ 1).
__device__ __forceinline__ int att_swz(int t) {
  const int b0 = t & 1, b1 = (t >> 1) & 1, b3 = (t >> 3) & 1;
  return b0 | (b0 << 1) | (b1 << 2) | ((b1 ^ b3) << 3);
}

// LDS transpose read (ds_read_b64_tr_b16): within each 16 lanes, lane j
// receives element j % 4 of the 8-byte chunks addressed by lanes j / 4,
// j / 4 + 4, j / 4 + 8 and j / 4 + 12 (measured on MI355X), i.e. a 4 x 4
// transpose of 16-bit elements.
typedef short att_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 att_read_tr(const char* p) {
  const att_v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) att_v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Waves and query rows: every wave computes one 16-row tile of the group's
// query rows. With up to 16 rows (RT = 1) each of the NW waves walks its own
// token tiles; with 17..32 rows (RT = 2) teams of two waves share token
// tiles, each wave of a team loading half of a tile (keys or values) into
// the team's double-buffered LDS tile, one barrier per tile step. The
// registers allow two waves per SIMD: two four-wave workgroups per CU, or
// one of eight.
template <int RT, int NW>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void verify_attention_kernel(AttnArgs a) {
  extern __shared__ u32x4 att_lds[];
  constexpr int kThreads = NW * kWave;
  constexpr int kTeams = NW / RT;                // groups of waves sharing token tiles
  constexpr int kLoads = 16 / RT;                // 16-byte loads per lane per tile and wave
  constexpr int kBufs = RT == 1 ? 1 : 2;         // LDS tiles per team
  constexpr int kLds = kTeams * kBufs * 2 * kAttTileBytes;  // the tiles; then the query rows
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, grp = lane >> 4;
  const int team = wave % kTeams, rtw = wave / kTeams;  // token team, row tile of this wave
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int ts = (split * a.split_tiles + min(split, a.split_rem)) * kAttTile;
  const int te = min(ts + (a.split_tiles + (split < a.split_rem ? 1 : 0)) * kAttTile, a.T);
  const int n_tiles = ts < te ? (te - ts + kAttTile - 1) / kAttTile : 0;
  const int team_tiles = n_tiles > team ? (n_tiles - team + kTeams - 1) / kTeams : 0;
  const int trips = n_tiles > 0 ? (n_tiles + kTeams - 1) / kTeams : 0;  // team 0's count

  char* team_lds = reinterpret_cast<char*>(att_lds) + team * kBufs * 2 * kAttTileBytes;
  const size_t head_stride = (size_t)a.Hkv * kAttD;  // elements per token
  const uint16_t* kbase = a.k + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;
  const uint16_t* vbase = a.v + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;

  // Tile j of a team covers tokens ts + (team + kTeams j) * 32 + 0..31. Its
  // 16 load instructions (8 of keys, 8 of values; 4 whole token rows each)
  // are split over the team's waves. Tiles past the team's last one, and
  // tokens past T, load clamped valid rows that are never used. With 17..32
  // query rows (RT = 2: 8 loads per lane and tile) two tiles are in flight
  // in registers (buffers ra, rb) while a third is computed; with up to 16
  // (16 loads per lane and tile) one, as two would not fit in registers.
  u32x4 ra[kLoads], rb[kLoads];
  auto load = [&](u32x4(&regs)[kLoads], int j) __attribute__((always_inline)) {
    const int jc = team_tiles > 0 ? min(j, team_tiles - 1) : 0;
    const int t0 = ts + (team + kTeams * jc) * kAttTile;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ni = rtw * kLoads + n;  // instruction of the tile: 0..7 keys, 8..15 values
      const int t = min(t0 + 4 * (ni & 7) + grp, a.T - 1);
      const uint16_t* base = ni < 8 ? kbase : vbase;
      regs[n] = __builtin_nontemporal_load(
          (const SPECV_ATT_GLOBAL u32x4*)(base + (size_t)t * head_stride) + row16);
    }
  };
  load(ra, 0);
  if (RT == 2 && trips > 1) load(rb, 1);

  // The group's query rows r = i * G + qh (zero past R) go to LDS once, in
  // the same swizzled layout as the tiles (their loads are issued after the
  // first tiles', so all are in flight together); the B operand of S^T is
  // read from there per tile.
  char* qlds = reinterpret_cast<char*>(att_lds) + kLds;
  for (int x = tid; x < 16 * RT * 16; x += kThreads) {
    const int r = x >> 4, u = x & 15;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < a.R) {
      const int i = r / a.G, qh = r - i * a.G;
      v = *reinterpret_cast<const u32x4*>(
          a.q + ((size_t)(b * a.K1 + i) * a.H + kvh * a.G + qh) * kAttD + u * 8);
    }
    *reinterpret_cast<u32x4*>(qlds + r * kAttRowBytes + ((u ^ (r & 7)) << 4)) = v;
  }
  __syncthreads();
  const int my_row = rtw * 16 + row16;  // this lane's query row
  const int limit = my_row < a.R ? a.T - a.K1 + my_row / a.G : a.T - 1;  // last visible key

  // 16-byte unit u of token t sits at t * 256 + ((u ^ att_swz(t)) * 16); the
  // values follow the keys
  auto store_lds = [&](const u32x4(&regs)[kLoads], char* tile) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ni = rtw * kLoads + n;
      const int t = 4 * (ni & 7) + grp;
      *reinterpret_cast<u32x4*>(tile + (ni < 8 ? 0 : kAttTileBytes) + t * kAttRowBytes +
                                ((row16 ^ att_swz(t)) << 4)) = regs[n];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int j, const char* tile) __attribute__((always_inline)) {
    const int t0 = ts + (team + kTeams * j) * kAttTile;
    // S^T for this lane's query row and the 8 consecutive tokens
    // 8 grp + 4 tt + e of the tile: block tt takes as its A-operand row i
    // the key of token 8 (i / 4) + 4 tt + i % 4, so that the scores a lane
    // holds are exactly the 8 reduction slots it supplies to P^T below.
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = 8 * (row16 >> 2) + 4 * tt + (row16 & 3);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const int u = ds * 4 + grp;
        const u32x4 kv =
            *reinterpret_cast<const u32x4*>(tile + t * kAttRowBytes + ((u ^ att_swz(t)) << 4));
        const u32x4 qv = *reinterpret_cast<const u32x4*>(qlds + my_row * kAttRowBytes +
                                                         ((u ^ (my_row & 7)) << 4));
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kv), __builtin_bit_cast(bf16x8, qv), s[tt], 0, 0, 0);
      }
    }
    // masked, scaled scores; running max and sum of the row
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ta = t0 + 8 * grp + 4 * tt + e;
        const bool vis = ta < te && ta <= limit;
        s[tt][e] = vis ? s[tt][e] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[tt][e]);
      }
    mx = att_row_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float p[8];
    float sum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = bf16_round(__builtin_amdgcn_exp2f(s[tt][e] - m_use));
        p[tt * 4 + e] = pv;
        sum += pv;
      }
    sum = att_row_sum(sum);
    l_run = l_run * corr + sum;
    // P^T slots of this lane: tokens 8 grp + 0..7 in order
    const u32x4 pf{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])};
    // O^T[d][r] = corr * O^T + sum over the tile's tokens of V[t][d] P[r][t].
    // The A operand V^T (row d = 16 dt + row16, tokens 8 grp + 0..7) comes
    // from two transpose reads of the token-major tile: for tokens
    // 8 grp + 4 h + 0..3 this lane addresses the 8-byte chunk 4 dt + row16 % 4
    // of token 8 grp + 4 h + row16 / 4.
    const char* vt_lds = tile + kAttTileBytes;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int ch = 4 * dt + (row16 & 3);
      uint2 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int t = 8 * grp + 4 * hh + (row16 >> 2);
        h[hh] = att_read_tr(vt_lds + t * kAttRowBytes + (((ch >> 1) ^ att_swz(t)) << 4) + (ch & 1) * 8);
      }
      const u32x4 vt{h[0].x, h[0].y, h[1].x, h[1].y};
      f32x4 c = acc_o[dt];
      c[0] *= corr;
      c[1] *= corr;
      c[2] *= corr;
      c[3] *= corr;
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, vt), __builtin_bit_cast(bf16x8, pf), c, 0, 0, 0);
    }
  };

  // In the main loops every step issues its reload unconditionally (tiles
  // past a team's last one are clamped), so the compiler's waits on them are
  // exact: storing tile j waits for its own loads only while the next
  // tile's stay in flight. The last steps reload nothing past the split, so
  // a split of few tiles reads each of its bytes once.
  if constexpr (RT == 1) {
    // a wave's LDS accesses run in order: no barrier between its own tiles
    int j = 0;
    for (; j + 1 < team_tiles; ++j) {
      store_lds(ra, team_lds);
      load(ra, j + 1);
      compute(j, team_lds);
    }
    if (j < team_tiles) {
      store_lds(ra, team_lds);
      compute(j, team_lds);
    }
  } else {
    // the team's two waves fill one tile together: a barrier before it is
    // read; alternate buffers make a second barrier unnecessary (a buffer is
    // refilled two steps later, after every wave passed the barrier between)
    auto step = [&](u32x4(&regs)[kLoads], int j, bool reload) __attribute__((always_inline)) {
      char* tile = team_lds + (j & 1) * 2 * kAttTileBytes;
      store_lds(regs, tile);
      if (reload) load(regs, j + 2);
      __syncthreads();
      if (j < team_tiles) compute(j, tile);
    };
    int j = 0;
    for (; j + 3 < trips; j += 2) {
      step(ra, j, true);
      step(rb, j + 1, true);
    }
    // at most three steps left; only the first may have a tile to reload
    if (j < trips) step(ra, j, j + 2 < trips);
    if (j + 1 < trips) step(rb, j + 1, false);
    if (j + 2 < trips) step(ra, j + 2, false);
  }

  // ---- merge the waves of each row tile (fixed order), then store or write
  // the split's partial
  __builtin_amdgcn_s_waitcnt(0);  // the unused loads past the last tile have landed
  __syncthreads();  // every wave is done with its tiles; LDS is reused below
  // wave w's row r of the output at wo + (w * 16 + r) * kAttWoStride: rows
  // padded by 4 floats (16 bytes) so that the 16 rows a store instruction
  // writes fall in distinct banks; each lane stores 4 consecutive columns
  constexpr int kAttWoStride = kAttD + 4;
  float* wm = reinterpret_cast<float*>(att_lds);  // [wave][16]
  float* wlsum = wm + NW * 16;                     // [wave][16]
  float* wo = wlsum + NW * 16;                     // [wave][16][kAttWoStride]
  static_assert((2 * NW * 16 + NW * 16 * kAttWoStride) * 4 <= kLds,
                "the merge buffers fit in the tiles");
  if (grp == 0) {
    wm[wave * 16 + row16] = m_run;
    wlsum[wave * 16 + row16] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4*>(wo + (wave * 16 + row16) * kAttWoStride + dt * 16 + 4 * grp) =
        acc_o[dt];
  // per query row: the maximum over the teams' maxima, each team's factor
  // and the row's sum (one thread per row), then every output from the
  // teams' partial rows in team order
  float* rfac = wo + NW * 16 * kAttWoStride;  // [32][kTeams]
  float* rmax = rfac + 32 * kTeams;            // [32]
  float* rsum = rmax + 32;                     // [32]
  static_assert((2 * NW * 16 + NW * 16 * kAttWoStride + 32 * (kTeams + 2)) * 4 <= kLds,
                "the merge buffers fit in the tiles");
  __syncthreads();
  if (tid < a.R) {
    const int r = tid, w0 = (r >> 4) * kTeams, rl = r & 15;  // waves w0 .. w0 + kTeams - 1
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTeams; ++t) m = fmaxf(m, wm[(w0 + t) * 16 + rl]);
    const float m_use = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < kTeams; ++t) {
      const float f = __builtin_amdgcn_exp2f(wm[(w0 + t) * 16 + rl] - m_use);
      rfac[r * kTeams + t] = f;
      l += wlsum[(w0 + t) * 16 + rl] * f;
    }
    rmax[r] = m;
    rsum[r] = l;
  }
  __syncthreads();
  constexpr int kPhases = kThreads / kAttD;  // rows handled side by side
  const int d = tid % kAttD, r0 = tid / kAttD;
#pragma unroll
  for (int k = 0; k < 32 / kPhases; ++k) {
    const int r = r0 + k * kPhases;
    if (r < a.R) {
      const int w0 = (r >> 4) * kTeams, rl = r & 15;
      float o = 0.f;
#pragma unroll
      for (int t = 0; t < kTeams; ++t)
        o += wo[((w0 + t) * 16 + rl) * kAttWoStride + d] * rfac[r * kTeams + t];
      if (a.part) {
        float* pr = a.part +
                    ((((size_t)b * a.Hkv + kvh) * a.n_split + split) * a.R + r) * kAttPartStride;
        pr[d] = o;
        if (d == 0) {
          pr[kAttD] = rmax[r];
          pr[kAttD + 1] = rsum[r];
        }
      } else {
        const int i = r / a.G, h = kvh * a.G + (r - i * a.G);
        const size_t oi = ((size_t)(b * a.K1 + i) * a.H + h) * kAttD + d;
        const float v = o / rsum[r];
        if (a.out_bf16)
          reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(v);
        else
          reinterpret_cast<float*>(a.out)[oi] = v;
      }
    }
  }
}

// Merge the splits of one (sequence, kv head, query row) in split order.
// Each thread merges one output column. Its partial outputs are requested
// kAttMergeChunk splits at a time, the first chunk before the splits'
// maxima and sums (which go to LDS), so that both are in flight together.
constexpr int kAttMaxSplit = 4096;
constexpr int kAttMergeChunk = 64;
__global__ __launch_bounds__(kAttD) void verify_attention_merge_kernel(AttnArgs a) {
  __shared__ float sm[kAttMaxSplit], sl[kAttMaxSplit];
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const float* base = a.part + (((size_t)b * a.Hkv + kvh) * a.n_split * a.R + r) * kAttPartStride;
  const size_t step = (size_t)a.R * kAttPartStride;
  float ov[kAttMergeChunk];
  auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAttMergeChunk; ++i)
      ov[i] = s0 + i < a.n_split ? base[(size_t)(s0 + i) * step + d] : 0.f;
  };
  fetch(0);
  for (int s = d; s < a.n_split; s += kAttD) {
    sm[s] = base[s * step + kAttD];
    sl[s] = base[s * step + kAttD + 1];
  }
  __syncthreads();
  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, sm[s]);
  const float m_use = m == -INFINITY ? 0.f : m;
  float o = 0.f, l = 0.f;
  for (int s0 = 0; s0 < a.n_split; s0 += kAttMergeChunk) {
    if (s0 > 0) fetch(s0);
#pragma unroll
    for (int i = 0; i < kAttMergeChunk; ++i) {
      if (s0 + i < a.n_split) {
        const float f = __builtin_amdgcn_exp2f(sm[s0 + i] - m_use);
        o += ov[i] * f;
        l += sl[s0 + i] * f;
      }
    }
  }
  const int i = r / a.G, h = kvh * a.G + (r - i * a.G);
  const size_t oi = ((size_t)(b * a.K1 + i) * a.H + h) * kAttD + d;
  const float v = o / l;
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(a.out)[oi] = v;
}

// Workgroups and splits. With at least 256 (sequence, kv head) groups the
// four-wave kernel runs two workgroups per CU: one split per group from 512
// groups up, two below. With fewer groups the eight-wave kernel (one
// workgroup per CU, two waves per SIMD) splits each group's cache so that
// about 256 workgroups run, a split keeping at least one tile per team:
// at B = 1 (8 groups, a cache of 129 tiles) 32 splits of 4 or 5 tiles, one
// step per team, where four waves per workgroup would leave one wave per
// SIMD to walk two tiles each. Splits differ by at most one tile. The plan
// depends on the shape only, so results do not depend on the device.
struct AttnPlan {
  int nw, n_split, split_tiles, split_rem;
};
static AttnPlan attention_plan(int B, int K1, int H, int Hkv, int T) {
  const int n_t = (T + kAttTile - 1) / kAttTile;
  const long long groups = (long long)B * Hkv;
  const int rt = K1 * (H / Hkv) <= 16 ? 1 : 2;
  AttnPlan p;
  if (groups >= 256) {
    p.nw = 4;
    p.n_split = groups >= 512 ? 1 : max(1, min(2, n_t / (4 / rt)));
  } else {
    p.nw = 8;
    p.n_split = max(1, min((int)(256 / groups), n_t / (8 / rt)));
  }
  p.n_split = min(p.n_split, kAttMaxSplit);
  p.split_tiles = n_t / p.n_split;
  p.split_rem = n_t % p.n_split;
  return p;
}

int attention_splits(int B, int K1, int H, int Hkv, int T) {
  return attention_plan(B, K1, H, Hkv, T).n_split;
}

size_t attention_workspace_bytes(int B, int K1, int H, int Hkv, int n_split) {
  if (n_split <= 1) return 0;
  const int R = K1 * (H / Hkv);
  return (size_t)B * Hkv * n_split * R * kAttPartStride * sizeof(float);
}

template <int RT, int NW>
static hipError_t launch_att(const AttnArgs& a, hipStream_t s) {
  constexpr int kTeams = NW / RT, kBufs = RT == 1 ? 1 : 2;
  const size_t lds = kTeams * kBufs * 2 * kAttTileBytes + kAttQBytes;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_attention_kernel<RT, NW>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((verify_attention_kernel<RT, NW>), dim3(a.n_split, a.Hkv, a.B),
                     dim3(NW * kWave), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split <= 1) return e;
  hipLaunchKernelGGL(verify_attention_merge_kernel, dim3(a.R, a.Hkv, a.B), dim3(kAttD), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   void* out, bool out_bf16, int B, int K1, int T, int H, int Hkv,
                                   float scale, void* workspace, hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.B = B;
  a.K1 = K1;
  a.T = T;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.R = K1 * a.G;
  const AttnPlan p = attention_plan(B, K1, H, Hkv, T);
  a.n_split = p.n_split;
  a.split_tiles = p.split_tiles;
  a.split_rem = p.split_rem;
  a.part = a.n_split > 1 ? static_cast<float*>(workspace) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_bf16 ? 1 : 0;
  if (p.nw == 8) return a.R <= 16 ? launch_att<1, 8>(a, s) : launch_att<2, 8>(a, s);
  return a.R <= 16 ? launch_att<1, 4>(a, s) : launch_att<2, 4>(a, s);
}

}  // namespace specv
